// scan_fwd.hip -- prefill selective scan for gfx950.
//
// Computes, per batch row b, channel d and state n (Mamba model notes sections
// 2.2, 4.1 and 4.4; Mamba paper notes section 2.3 for the discretisation):
//   Delta_t = softplus(delta_t + bias[d])
//   h_t[n]  = exp(Delta_t A[d,n]) h_{t-1}[n] + Delta_t B[b,n,t] u_t
//   out_t   = (sum_n C[b,n,t] h_t[n] + D[d] u_t) * silu(z_t)
//
// Work decomposition (one workgroup = 16 channels of one batch row x 16 states,
// 256 lanes, walking the whole sequence in blocks of 16 tokens):
//   scan role   lane (n = tid/16, c = tid%16) owns the fp32 state h[n] of
//               channel d0+c.  The state never leaves the register file.
//   owner role  lane (c = tid/16, j = tid%16) owns token t0+j of channel d0+c:
//               it loads u/delta/z, computes Delta and Delta*u once, and at the
//               end of the block reduces the readout over n, applies the skip
//               term and the gate, and stores out.
// B and C depend on (b, n, t) only, so each 16-lane row (one state n) needs the
// same 16 values per block: lane j of the row loads token t0+j and a DPP
// row_newbcast hands it to every lane of the row inside the consuming VALU op.
// Delta and Delta*u travel from owners to scan lanes through LDS, and so do
// the per-state readout partials on their way back to the owners.
// The state recurrence itself is sequential per lane: no scan operator, no
// recomputation, one exp per (t, n).
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kN = 16;              // states per channel = rows of the workgroup
constexpr int kCh = 16;             // channels per workgroup = lanes per row
constexpr int kT = 16;              // tokens per block
constexpr int kThreads = kN * kCh;  // 256
constexpr int kPitch = 20;          // LDS row pitch in floats: b128 accesses hit distinct banks

struct ScanParams {
  const void* u;
  const void* delta;
  const void* z;
  const void* B;
  const void* C;
  const float* A;
  const float* D;
  const float* bias;
  const float* h0;
  float* last_state;
  void* out;
  int64_t usb, usd, dsb, dsd, zsb, zsd, Bsb, Bsn, Csb, Csn, Asd, Asn, osb, osd;
  int64_t batch, dim, L;
  int64_t dgroups;
  int softplus;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void scan_fwd_kernel(ScanParams p) {
  __shared__ __align__(16) float s_dl[kCh][kPitch];
  __shared__ __align__(16) float s_du[kCh][kPitch];
  __shared__ __align__(16) float s_part[kN][kCh][kPitch];

  const int tid = threadIdx.x;
  const int row = tid >> 4;
  const int col = tid & 15;
  const int64_t b = blockIdx.x / p.dgroups;
  const int64_t d0 = (blockIdx.x % p.dgroups) * kCh;

  // scan role: state n = row of channel d0 + col
  const int64_t dS = d0 + col;
  const bool vS = dS < p.dim;
  const float a2 = vS ? p.A[dS * p.Asd + row * p.Asn] * kLog2e : 0.0f;
  float h = (vS && p.h0) ? p.h0[(b * p.dim + dS) * kN + row] : 0.0f;
  const T* Bp = static_cast<const T*>(p.B) + b * p.Bsb + row * p.Bsn;
  const T* Cp = static_cast<const T*>(p.C) + b * p.Csb + row * p.Csn;

  // owner role: token t0 + col of channel d0 + row
  const int64_t dO = d0 + row;
  const bool vO = dO < p.dim;
  const float bias = (vO && p.bias) ? p.bias[dO] : 0.0f;
  const float Dd = (vO && p.D) ? p.D[dO] : 0.0f;
  const T* uO = static_cast<const T*>(p.u) + b * p.usb + dO * p.usd;
  const T* dlO = static_cast<const T*>(p.delta) + b * p.dsb + dO * p.dsd;
  const T* zO = p.z ? static_cast<const T*>(p.z) + b * p.zsb + dO * p.zsd : nullptr;
  T* oO = static_cast<T*>(p.out) + b * p.osb + dO * p.osd;

  for (int64_t t0 = 0; t0 < p.L; t0 += kT) {
    const int64_t t = t0 + col;
    const bool inT = t < p.L;
    const bool okO = vO && inT;
    float uo = 0.0f, zo = 0.0f, dl = 0.0f;
    if (okO) {
      uo = io<T>::load(uO + t);
      const float x = io<T>::load(dlO + t) + bias;
      dl = p.softplus ? softplus_f32(x) : x;
      if (zO) zo = io<T>::load(zO + t);
    }
    s_dl[row][col] = dl;
    s_du[row][col] = dl * uo;
    const float bv = inT ? io<T>::load(Bp + t) : 0.0f;
    const float cv = inT ? io<T>::load(Cp + t) : 0.0f;
    __syncthreads();

    float dlr[kT], dur[kT];
#pragma unroll
    for (int k = 0; k < kT / 4; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(&s_dl[col][4 * k]);
      const float4 c = *reinterpret_cast<const float4*>(&s_du[col][4 * k]);
      dlr[4 * k + 0] = a.x; dlr[4 * k + 1] = a.y; dlr[4 * k + 2] = a.z; dlr[4 * k + 3] = a.w;
      dur[4 * k + 0] = c.x; dur[4 * k + 1] = c.y; dur[4 * k + 2] = c.z; dur[4 * k + 3] = c.w;
    }
    float part[kT];
    static_for<0, kT>([&](auto J) {
      constexpr int j = decltype(J)::value;
      const float e = __builtin_amdgcn_exp2f(dlr[j] * a2);   // Abar = exp(Delta A)
      const float w = dur[j] * row_bcast<j>(bv);            // Bbar u = Delta u B
      h = fmaf(e, h, w);
      part[j] = row_bcast<j>(cv) * h;                       // C_n h_n
    });
#pragma unroll
    for (int k = 0; k < kT / 4; ++k)
      *reinterpret_cast<float4*>(&s_part[row][col][4 * k]) =
          make_float4(part[4 * k], part[4 * k + 1], part[4 * k + 2], part[4 * k + 3]);
    __syncthreads();

    if (okO) {
      float y = 0.0f;
#pragma unroll
      for (int n = 0; n < kN; ++n) y += s_part[n][row][col];
      y = fmaf(Dd, uo, y);
      if (zO) y *= silu_f32(zo);
      io<T>::store(oO + t, y);
    }
  }
  if (vS && p.last_state) p.last_state[(b * p.dim + dS) * kN + row] = h;
}

// seqlen == 0: the final state is the initial one.
__global__ void copy_state_kernel(const float* h0, float* last, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) last[i] = h0 ? h0[i] : 0.0f;
}

}  // namespace

hipError_t launch_scan_fwd(const ssm_scan_args& a, hipStream_t stream) {
  if (a.seqlen == 0) {
    if (!a.last_state || a.last_state == a.h0) return hipSuccess;
    const int64_t n = a.batch * a.dim * a.dstate;
    copy_state_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(
        a.h0, a.last_state, n);
    return hipGetLastError();
  }
  ScanParams p;
  p.u = a.u; p.delta = a.delta; p.z = a.z; p.B = a.B; p.C = a.C;
  p.A = a.A; p.D = a.D; p.bias = a.delta_bias; p.h0 = a.h0; p.last_state = a.last_state;
  p.out = a.out;
  p.usb = a.u_batch_stride; p.usd = a.u_dim_stride;
  p.dsb = a.delta_batch_stride; p.dsd = a.delta_dim_stride;
  p.zsb = a.z_batch_stride; p.zsd = a.z_dim_stride;
  p.Bsb = a.B_batch_stride; p.Bsn = a.B_state_stride;
  p.Csb = a.C_batch_stride; p.Csn = a.C_state_stride;
  p.Asd = a.A_dim_stride; p.Asn = a.A_state_stride;
  p.osb = a.out_batch_stride; p.osd = a.out_dim_stride;
  p.batch = a.batch; p.dim = a.dim; p.L = a.seqlen;
  p.dgroups = (a.dim + kCh - 1) / kCh;
  p.softplus = a.delta_softplus ? 1 : 0;
  const dim3 grid((unsigned)(a.batch * p.dgroups));
  if (a.io_dtype == SSM_BF16)
    scan_fwd_kernel<uint16_t><<<grid, dim3(kThreads), 0, stream>>>(p);
  else
    scan_fwd_kernel<float><<<grid, dim3(kThreads), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace ssm

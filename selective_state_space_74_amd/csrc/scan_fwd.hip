// scan_fwd.hip -- prefill selective scan for gfx950.
//
// Computes, per batch row b, channel d and state n (Mamba model notes sections
// 2.2, 4.1 and 4.4; Mamba paper notes section 2.3 for the discretisation):
//   Delta_t = softplus(delta_t + bias[d])
//   h_t[n]  = exp(Delta_t A[d,n]) h_{t-1}[n] + Delta_t B[b,n,t] u_t
//   out_t   = (sum_n C[b,n,t] h_t[n] + D[d] u_t) * silu(z_t)
//
// Work decomposition.  One workgroup = 16 channels of one batch row x 16
// states (256 lanes, 4 wavefronts), walking its token range in blocks of 16:
//   scan role   lane (n = tid/16, c = tid%16) owns the fp32 state h[n] of
//               channel d0+c.  The state never leaves the register file.
//   owner role  lane (c = tid/16, j = tid%16) owns token t0+j of channel d0+c:
//               it loads u/delta/z, computes Delta and Delta*u once, and one
//               block later reduces the readout over n, applies the skip term
//               and the gate, and stores out.
// B and C depend on (b, n, t) only, so each 16-lane row (one state n) needs the
// same 16 values per block: lane j of the row loads token t0+j and a DPP
// row_newbcast hands it to every lane of the row inside the consuming VALU op.
// Delta and Delta*u travel from owners to scan lanes through LDS, and so do
// the per-state readout partials on their way back to the owners.  The state
// recurrence is sequential per lane: one exp per (t, n), nothing recomputed.
//
// Long sequences with few channels.  The recurrence is linear in the state
// (Mamba paper notes, sections 5.3/5.4: a long input can be cut into chunks
// with the state handed from one chunk to the next), so the sequence may be
// cut into G segments processed by different workgroups:
//   pass 1 (aggregate)  segments 0..G-2 run from a zero state and record their
//                       end state b_g and the sum of their step sizes S_g;
//   pass 2 (scan)       segment g starts from
//                       h_in = fold_{i<g} (exp(A S_i) h + b_i) applied to h0,
//                       then runs exactly like the single-segment scan.
// The exact state entering segment g is exp(A S_{g-1}) h_in(g-1) + b_{g-1},
// so the fold reproduces the sequential result up to fp32 rounding.
#include <algorithm>

#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kN = 16;              // states per channel = rows of the workgroup
constexpr int kCh = 16;             // channels per workgroup = lanes per row
constexpr int kT = 16;              // tokens per block
constexpr int kThreads = kN * kCh;  // 256
constexpr int kPitch = 20;          // LDS row pitch in floats: b128 accesses hit distinct banks
constexpr int kAggStride = kN + 1;  // floats per (row, segment) aggregate: b[16], S

enum class Mode { kScan, kAggregate };

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
  float* agg;      // [batch * dim][nseg - 1][kAggStride] segment aggregates (nseg > 1)
  int64_t usb, usd, dsb, dsd, zsb, zsd, Bsb, Bsn, Csb, Csn, Asd, Asn, osb, osd;
  int64_t batch, dim;
  int L;
  int seg_len;     // tokens per segment (multiple of kT)
  int nseg;        // segments per sequence
  int64_t dgroups; // ceil(dim / kCh)
  int softplus;
};

// Raw inputs of one block as one lane sees them: the owner role's u, delta, z
// for its (channel, token) and the scan role's B, C for (its state, token).
struct BlockIn {
  float u, dt, z, b, c;
};

// Per-lane constants and pointers shared by every block.
template <typename T>
struct Lane {
  const T* u;   // owner row of u (channel clamped into range)
  const T* dl;  // owner row of delta
  const T* z;   // owner row of z (u's row when there is no gate: loaded, never used)
  const T* B;   // scan row of B (state n)
  const T* C;   // scan row of C
  T* out;       // owner row of out
  float a2;     // A[d, n] * log2(e)
  float bias, Dd;
  bool vO;      // owner channel exists
  bool gate;    // z given
};

// Pipeline of one workgroup over blocks of kT tokens of its segment
// [t_beg, t_end).  Block j's raw inputs are loaded two iterations before the
// scan uses them, its step sizes are published one iteration before, and it is
// finished (readout, skip, gate, store) one iteration after its scan.  Four
// register buffers rotate with the iteration index; the loop is unrolled by
// four so every buffer is a fixed set of registers and no load result is
// copied while still in flight.
template <typename T, Mode M>
struct Pipe {
  const ScanParams& p;
  const Lane<T>& ln;
  int row, col;
  int t_beg, t_end;
  int nblk;
  float (*s_dl)[kCh][kPitch];
  float (*s_du)[kCh][kPitch];
  float (*s_part)[kN][kCh][kPitch];
  double* ssum;  // aggregate mode: this owner lane's running sum of Delta

  __device__ __forceinline__ int tok(int k) const { return t_beg + k * kT + col; }

  __device__ __forceinline__ BlockIn load(int k) const {
    // Clamped token index: every address is in bounds; values of tokens past
    // the segment end are masked where they are consumed.
    const int t = min(tok(k), t_end - 1);
    BlockIn in;
    in.b = io<T>::load(ln.B + t);
    in.c = M == Mode::kScan ? io<T>::load(ln.C + t) : 0.0f;
    in.u = io<T>::load(ln.u + t);
    in.dt = io<T>::load(ln.dl + t);
    in.z = M == Mode::kScan ? io<T>::load(ln.z + t) : 0.0f;
    return in;
  }

  __device__ __forceinline__ bool owns(int k) const { return ln.vO && tok(k) < t_end; }

  // Owner: Delta and Delta*u of block k into LDS slot k & 1 (zero past the end).
  __device__ __forceinline__ void publish(int k, const BlockIn& in) const {
    const float x = in.dt + ln.bias;
    const float dl = p.softplus ? softplus_f32(x) : x;
    const bool own = owns(k);
    s_dl[k & 1][row][col] = own ? dl : 0.0f;
    s_du[k & 1][row][col] = own ? dl * in.u : 0.0f;
    if (M == Mode::kAggregate && own) *ssum += static_cast<double>(dl);
  }

  // Owner: readout of block k from the partials, skip term, gate, store.
  __device__ __forceinline__ void finish(int k, const BlockIn& in, const float (&part)[kN]) const {
    float y = 0.0f;
#pragma unroll
    for (int n = 0; n < kN; ++n) y += part[n];
    y = fmaf(ln.Dd, in.u, y);
    if (ln.gate) y *= silu_f32(in.z);
    if (owns(k)) io<T>::store(ln.out + tok(k), y);
  }

  // Iteration k.  Buffers: P = block k-1 (finish), Q = block k (scan),
  // R = block k+1 (publish), S = block k+2 (load target).
  __device__ __forceinline__ void iter(int k, float& h, const BlockIn& P, const BlockIn& Q,
                                       const BlockIn& R, BlockIn& S) const {
    const int slot = k & 1;
    // LDS reads first: this block's step sizes and the previous block's partials.
    float dlr[kT], dur[kT], part[kN];
#pragma unroll
    for (int q = 0; q < kT / 4; ++q) {
      const float4 a = *reinterpret_cast<const float4*>(&s_dl[slot][col][4 * q]);
      const float4 c = *reinterpret_cast<const float4*>(&s_du[slot][col][4 * q]);
      dlr[4 * q + 0] = a.x; dlr[4 * q + 1] = a.y; dlr[4 * q + 2] = a.z; dlr[4 * q + 3] = a.w;
      dur[4 * q + 0] = c.x; dur[4 * q + 1] = c.y; dur[4 * q + 2] = c.z; dur[4 * q + 3] = c.w;
    }
    if (M == Mode::kScan) {
      // unconditional: at k = 0 the values are never used
#pragma unroll
      for (int n = 0; n < kN; ++n) part[n] = s_part[slot ^ 1][n][row][col];
    }
    S = load(k + 2);   // unconditional: past the end the clamped index stays in bounds

    // scan role: 16 sequential steps of this lane's state
    const float bv = tok(k) < t_end ? Q.b : 0.0f;
    const float cv = Q.c;
    float pk[kT];
    static_for<0, kT>([&](auto J) {
      constexpr int j = decltype(J)::value;
      const float e = __builtin_amdgcn_exp2f(dlr[j] * ln.a2);   // Abar = exp(Delta A)
      const float w = dur[j] * row_bcast<j>(bv);               // Bbar u = Delta u B
      h = fmaf(e, h, w);
      if (M == Mode::kScan) pk[j] = row_bcast<j>(cv) * h;      // C_n h_n
    });
    if (M == Mode::kScan) {
#pragma unroll
      for (int q = 0; q < kT / 4; ++q)
        *reinterpret_cast<float4*>(&s_part[slot][row][col][4 * q]) =
            make_float4(pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]);
      if (k > 0) finish(k - 1, P, part);
    }
    if (k + 1 < nblk) publish(k + 1, R);
    __syncthreads();
  }
};

template <typename T, Mode M>
__global__ __launch_bounds__(kThreads) void scan_fwd_kernel(ScanParams p) {
  // Double-buffered by block parity, so one barrier per block is enough.
  __shared__ __align__(16) float s_dl[2][kCh][kPitch];
  __shared__ __align__(16) float s_du[2][kCh][kPitch];
  __shared__ __align__(16) float s_part[M == Mode::kScan ? 2 : 1][kN][kCh][kPitch];
  __shared__ double s_sum[kCh][kCh];

  const int tid = threadIdx.x;
  const int row = tid >> 4;
  const int col = tid & 15;
  // blockIdx.x = (b * dgroups + dg) * nseg_grid + g; the aggregate pass skips
  // the last segment (its end state is never needed by a later segment)
  const int nseg_grid = M == Mode::kScan ? p.nseg : p.nseg - 1;
  const int g = static_cast<int>(blockIdx.x % nseg_grid);
  const int64_t bd = blockIdx.x / nseg_grid;
  const int64_t b = bd / p.dgroups;
  const int64_t d0 = (bd % p.dgroups) * kCh;
  const int t_beg = g * p.seg_len;
  const int t_end = min(p.L, t_beg + p.seg_len);
  const int nblk = (t_end - t_beg + kT - 1) / kT;

  Lane<T> ln;
  // scan role: state n = row of channel d0 + col
  const int64_t dS = d0 + col;
  const bool vS = dS < p.dim;
  const int64_t dSc = vS ? dS : p.dim - 1;
  ln.a2 = p.A[dSc * p.Asd + row * p.Asn] * kLog2e;
  ln.B = static_cast<const T*>(p.B) + b * p.Bsb + row * p.Bsn;
  ln.C = static_cast<const T*>(p.C) + b * p.Csb + row * p.Csn;
  // owner role: token t0 + col of channel d0 + row
  const int64_t dO = d0 + row;
  ln.vO = dO < p.dim;
  const int64_t dOc = ln.vO ? dO : p.dim - 1;
  ln.bias = p.bias ? p.bias[dOc] : 0.0f;
  ln.Dd = p.D ? p.D[dOc] : 0.0f;
  ln.u = static_cast<const T*>(p.u) + b * p.usb + dOc * p.usd;
  ln.dl = static_cast<const T*>(p.delta) + b * p.dsb + dOc * p.dsd;
  ln.gate = p.z != nullptr;
  ln.z = ln.gate ? static_cast<const T*>(p.z) + b * p.zsb + dOc * p.zsd : ln.u;
  ln.out = static_cast<T*>(p.out) + b * p.osb + dOc * p.osd;

  // Initial state: zero for an aggregate segment; otherwise h0 (or zero) carried
  // through the aggregates of every earlier segment.
  float h = 0.0f;
  if (M == Mode::kScan) {
    h = (vS && p.h0) ? p.h0[(b * p.dim + dS) * kN + row] : 0.0f;
    if (g > 0) {
      const float* ag = p.agg + ((b * p.dim + dSc) * (p.nseg - 1)) * kAggStride;
      for (int i = 0; i < g; ++i) {
        const float decay = __builtin_amdgcn_exp2f(ln.a2 * ag[i * kAggStride + kN]);
        h = fmaf(decay, h, ag[i * kAggStride + row]);
      }
    }
  }

  double ssum = 0.0;
  Pipe<T, M> pp{p, ln, row, col, t_beg, t_end, nblk, s_dl, s_du, s_part, &ssum};
  // block j lives in buffer j % 4; iteration k loads block k + 2
  BlockIn buf0 = pp.load(0), buf1 = pp.load(1), buf2 = buf0, buf3 = buf0;
  pp.publish(0, buf0);
  __syncthreads();

  int k = 0;
  for (; k + 4 <= nblk; k += 4) {
    pp.iter(k + 0, h, buf3, buf0, buf1, buf2);
    pp.iter(k + 1, h, buf0, buf1, buf2, buf3);
    pp.iter(k + 2, h, buf1, buf2, buf3, buf0);
    pp.iter(k + 3, h, buf2, buf3, buf0, buf1);
  }
  if (k < nblk) pp.iter(k, h, buf3, buf0, buf1, buf2);
  if (k + 1 < nblk) pp.iter(k + 1, h, buf0, buf1, buf2, buf3);
  if (k + 2 < nblk) pp.iter(k + 2, h, buf1, buf2, buf3, buf0);

  if (M == Mode::kScan) {
    // finish the last block: its partials are in slot (nblk - 1) & 1
    const int kl = nblk - 1;
    const int r = kl & 3;
    const BlockIn last = r == 0 ? buf0 : r == 1 ? buf1 : r == 2 ? buf2 : buf3;
    float part[kN];
#pragma unroll
    for (int n = 0; n < kN; ++n) part[n] = s_part[kl & 1][n][row][col];
    pp.finish(kl, last, part);
    if (vS && p.last_state && g == p.nseg - 1) p.last_state[(b * p.dim + dS) * kN + row] = h;
  } else {
    // segment aggregate: end state from zero and the step-size sum (fp64 partial
    // sums of the 16 owner lanes of each channel, added in a fixed order)
    s_sum[row][col] = ssum;
    __syncthreads();
    float* ag = p.agg + ((b * p.dim + dSc) * (p.nseg - 1) + g) * kAggStride;
    if (vS) ag[row] = h;
    if (vS && row == 0) {
      double s = 0.0;
      for (int j = 0; j < kCh; ++j) s += s_sum[col][j];
      ag[kN] = static_cast<float>(s);
    }
  }
}

// seqlen == 0: the final state is the initial one.
__global__ void copy_state_kernel(const float* h0, float* last, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) last[i] = h0 ? h0[i] : 0.0f;
}

// Segments per sequence: cut only when the batch x channel groups alone leave
// the machine short of workgroups, and keep segments long enough that the
// extra aggregate pass and the fold stay small.
constexpr int64_t kTargetGroups = 768;    // 3 workgroups per CU on 256 CUs
constexpr int64_t kMinSegLen = 8192;
constexpr int kMaxSeg = 64;

int choose_segments(int64_t groups, int64_t L) {
  if (groups >= kTargetGroups / 2) return 1;
  int64_t g = (kTargetGroups + groups - 1) / groups;
  g = std::min<int64_t>(g, std::max<int64_t>(1, L / kMinSegLen));
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(g, kMaxSeg)));
}

}  // namespace

size_t scan_workspace_bytes(const ssm_scan_args& a) {
  if (a.batch <= 0 || a.dim <= 0 || a.seqlen <= 0) return 0;
  const int64_t groups = a.batch * ((a.dim + kCh - 1) / kCh);
  const int nseg = choose_segments(groups, a.seqlen);
  if (nseg <= 1) return 0;
  return static_cast<size_t>(a.batch * a.dim * (nseg - 1) * kAggStride) * sizeof(float);
}

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
  p.batch = a.batch; p.dim = a.dim; p.L = static_cast<int>(a.seqlen);
  p.dgroups = (a.dim + kCh - 1) / kCh;
  p.softplus = a.delta_softplus ? 1 : 0;

  // Segmenting needs the caller's workspace; without enough of it the whole
  // sequence runs as one segment (same result, less parallelism).
  const int64_t groups = a.batch * p.dgroups;
  const size_t need = scan_workspace_bytes(a);
  int nseg = 1;
  if (need > 0 && a.workspace && a.workspace_bytes >= need)
    nseg = choose_segments(groups, a.seqlen);
  const int64_t seg = (a.seqlen + nseg - 1) / nseg;
  p.seg_len = static_cast<int>((seg + kT - 1) / kT * kT);
  p.nseg = static_cast<int>((a.seqlen + p.seg_len - 1) / p.seg_len);
  p.agg = p.nseg > 1 ? static_cast<float*>(a.workspace) : nullptr;

  if (p.nseg > 1) {
    const dim3 g1((unsigned)(groups * (p.nseg - 1)));
    if (a.io_dtype == SSM_BF16)
      scan_fwd_kernel<uint16_t, Mode::kAggregate><<<g1, dim3(kThreads), 0, stream>>>(p);
    else
      scan_fwd_kernel<float, Mode::kAggregate><<<g1, dim3(kThreads), 0, stream>>>(p);
  }
  const dim3 g2((unsigned)(groups * p.nseg));
  if (a.io_dtype == SSM_BF16)
    scan_fwd_kernel<uint16_t, Mode::kScan><<<g2, dim3(kThreads), 0, stream>>>(p);
  else
    scan_fwd_kernel<float, Mode::kScan><<<g2, dim3(kThreads), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace ssm

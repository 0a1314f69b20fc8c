// state_update.hip -- single-token decode update for gfx950.
//
// Same recurrence as the prefill scan, one token per (batch, channel), with
// the fp32 state resident in HBM (Mamba paper notes section 4.3: the step form
// keeps only a fixed-size state and updates it per generated token):
//   Delta = softplus(dt + bias[d])
//   s[n]  = exp(Delta A[d,n]) s[n] + Delta B[b,n] x        (in place)
//   out   = (sum_n C[b,n] s[n] + D[d] x) * silu(z)
//
// The step is bound by HBM traffic on the state (read + write 128 B per
// channel).  Four consecutive lanes share one channel and own four states
// each, so a wavefront moves 1 KiB of contiguous state per vector access.
// The readout is reduced over the quad with two DPP quad permutations.
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kThreads = 256;

struct UpdateParams {
  float* state;
  const void* x;
  const void* dt;
  const void* z;
  const void* B;
  const void* C;
  const float* A;
  const float* D;
  const float* bias;
  void* out;
  int64_t ssb, ssd, xsb, dtsb, zsb, Bsb, Csb, Asd, osb;
  int64_t batch, dim;
  int softplus;
  int vec_state;  // state rows 16-byte aligned: float4 path
  int vec_A;      // A rows 16-byte aligned: float4 path
};

template <typename T>
__global__ __launch_bounds__(kThreads) void state_update_kernel(UpdateParams p) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int q = threadIdx.x & 3;
  const int64_t r = gid >> 2;
  const bool valid = r < p.batch * p.dim;
  const int64_t b = valid ? r / p.dim : 0;
  const int64_t d = valid ? r - b * p.dim : 0;
  float y = 0.0f, xv = 0.0f, zv = 0.0f;
  if (valid) {
    xv = io<T>::load(static_cast<const T*>(p.x) + b * p.xsb + d);
    float dl = io<T>::load(static_cast<const T*>(p.dt) + b * p.dtsb + d);
    if (p.bias) dl += p.bias[d];
    if (p.softplus) dl = softplus_f32(dl);
    if (p.z) zv = io<T>::load(static_cast<const T*>(p.z) + b * p.zsb + d);
    float* sp = p.state + b * p.ssb + d * p.ssd + 4 * q;
    const float* ap = p.A + d * p.Asd + 4 * q;
    float s[4], a[4];
    if (p.vec_state) {
      const float4 v = *reinterpret_cast<const float4*>(sp);
      s[0] = v.x; s[1] = v.y; s[2] = v.z; s[3] = v.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = sp[i];
    }
    if (p.vec_A) {
      const float4 v = *reinterpret_cast<const float4*>(ap);
      a[0] = v.x; a[1] = v.y; a[2] = v.z; a[3] = v.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = ap[i];
    }
    const T* Bq = static_cast<const T*>(p.B) + b * p.Bsb + 4 * q;
    const T* Cq = static_cast<const T*>(p.C) + b * p.Csb + 4 * q;
    const float dlx = dl * xv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __builtin_amdgcn_exp2f(dl * (a[i] * kLog2e));
      s[i] = fmaf(e, s[i], dlx * io<T>::load(Bq + i));
      y = fmaf(io<T>::load(Cq + i), s[i], y);
    }
    if (p.vec_state) {
      *reinterpret_cast<float4*>(sp) = make_float4(s[0], s[1], s[2], s[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) sp[i] = s[i];
    }
  }
  // quad sum: lanes (0,1,2,3) <- (1,0,3,2), then <- (2,3,0,1)
  y += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y), 0xB1, 0xf, 0xf, true));
  y += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y), 0x4E, 0xf, 0xf, true));
  if (valid && q == 0) {
    if (p.D) y = fmaf(p.D[d], xv, y);
    if (p.z) y *= silu_f32(zv);
    io<T>::store(static_cast<T*>(p.out) + b * p.osb + d, y);
  }
}

}  // namespace

hipError_t launch_state_update(const ssm_update_args& a, hipStream_t stream) {
  UpdateParams p;
  p.state = a.state; p.x = a.x; p.dt = a.dt; p.z = a.z; p.B = a.B; p.C = a.C;
  p.A = a.A; p.D = a.D; p.bias = a.dt_bias; p.out = a.out;
  p.ssb = a.state_batch_stride; p.ssd = a.state_dim_stride;
  p.xsb = a.x_batch_stride; p.dtsb = a.dt_batch_stride; p.zsb = a.z_batch_stride;
  p.Bsb = a.B_batch_stride; p.Csb = a.C_batch_stride; p.Asd = a.A_dim_stride;
  p.osb = a.out_batch_stride;
  p.batch = a.batch; p.dim = a.dim;
  p.softplus = a.dt_softplus ? 1 : 0;
  p.vec_state = (reinterpret_cast<uintptr_t>(a.state) % 16 == 0) && (a.state_batch_stride % 4 == 0) &&
                (a.state_dim_stride % 4 == 0);
  p.vec_A = (reinterpret_cast<uintptr_t>(a.A) % 16 == 0) && (a.A_dim_stride % 4 == 0);
  const int64_t lanes = a.batch * a.dim * 4;
  const dim3 grid((unsigned)((lanes + kThreads - 1) / kThreads));
  if (a.io_dtype == SSM_BF16)
    state_update_kernel<uint16_t><<<grid, dim3(kThreads), 0, stream>>>(p);
  else
    state_update_kernel<float><<<grid, dim3(kThreads), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace ssm

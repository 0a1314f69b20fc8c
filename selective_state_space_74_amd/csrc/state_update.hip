// state_update.hip -- single-token decode update for gfx950.
//
// Same recurrence as the prefill scan, one token per (batch, channel), with
// the fp32 state resident in device memory (Mamba paper notes section 4.3:
// the step form keeps only a fixed-size state and updates it per generated
// token):
//   Delta = softplus(dt + bias[d])
//   s[n]  = exp(Delta A[d,n]) s[n] + Delta B[b,n] x        (in place)
//   out   = (sum_n C[b,n] s[n] + D[d] x) * silu(z)
//
// The step is bound by memory traffic on the state (read + write 8N bytes per
// channel).  Four consecutive lanes share one channel and own R = N/4
// consecutive states each (R rounded up to 1, 2, 4, 8 or 16 for N up to 64),
// so every state access of a wavefront is one contiguous run (one lane per
// channel with 64 B per lane measured ~35% slower on gfx950).  The grid is
// (blocks of 64 channels, batch rows or pairs of them): no thread divides to
// find its (batch, channel).  With a large enough grid a thread takes two
// batch rows of its channel: A, bias and D are loaded once for both, and
// both rows' state and inputs are in flight together.  Aligned layouts with N = 4R (the usual contiguous ones) take a
// branch-free instantiation with vector accesses; others take the
// element-wise one, masked to the N real states.  The readout is reduced
// over the quad with two DPP quad permutations.  B and C are those of the
// channel's group (one group: shared by every channel of the batch row).
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kThreads = 256;
constexpr int kChannelsPerBlock = kThreads / 4;
constexpr int kMaxConv = SSM_MAX_CONV;
// batch rows per thread for the plain update (vector path, up to 16 states
// per channel), when the grid keeps enough workgroups
constexpr int kRowsPerThread = 2;
constexpr int64_t kMinBlocksRows = 2048;

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
  int64_t ssb, ssd, xsb, dtsb, zsb, Bsb, Bsg, Csb, Csg, Asd, osb;
  int64_t batch, dim, cpg;
  int N;
  int softplus;
  // fused conv branch: [batch][dim][K] state shifted in place, [dim][K]
  // weights, [dim] bias (or NULL)
  float* conv_state;
  const float* conv_w;
  const float* conv_b;
  int K;
  int conv_silu;
};

// R consecutive values from p as fp32: vector accesses (VEC: all R real and
// aligned to min(R, 4) elements) or element-wise ones masked to the first
// nvalid.
template <typename T, bool VEC, int R>
__device__ __forceinline__ void loadR(const T* p, float (&v)[R], int nvalid) {
  if constexpr (VEC && R >= 4) {
#pragma unroll
    for (int c = 0; c < R / 4; ++c) {
      if constexpr (sizeof(T) == 4) {
        const float4 q = reinterpret_cast<const float4*>(p)[c];
        v[4 * c] = q.x; v[4 * c + 1] = q.y; v[4 * c + 2] = q.z; v[4 * c + 3] = q.w;
      } else {
        const uint2 q = reinterpret_cast<const uint2*>(p)[c];
        v[4 * c] = __uint_as_float(q.x << 16); v[4 * c + 1] = __uint_as_float(q.x & 0xffff0000u);
        v[4 * c + 2] = __uint_as_float(q.y << 16); v[4 * c + 3] = __uint_as_float(q.y & 0xffff0000u);
      }
    }
  } else if constexpr (VEC && R == 2) {
    if constexpr (sizeof(T) == 4) {
      const float2 q = *reinterpret_cast<const float2*>(p);
      v[0] = q.x; v[1] = q.y;
    } else {
      const uint32_t q = *reinterpret_cast<const uint32_t*>(p);
      v[0] = __uint_as_float(q << 16); v[1] = __uint_as_float(q & 0xffff0000u);
    }
  } else if constexpr (VEC) {
    v[0] = io<T>::load(p);
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i) v[i] = i < nvalid ? io<T>::load(p + i) : 0.0f;
  }
}

template <bool VEC, int R>
__device__ __forceinline__ void storeR(float* p, const float (&v)[R], int nvalid) {
  if constexpr (VEC && R >= 4) {
#pragma unroll
    for (int c = 0; c < R / 4; ++c)
      reinterpret_cast<float4*>(p)[c] = make_float4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
  } else if constexpr (VEC && R == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  } else if constexpr (VEC) {
    *p = v[0];
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (i < nvalid) p[i] = v[i];
  }
}

// VEC: N == 4R and state rows, A rows and B/C rows are aligned for vector
// accesses.
// CONV: x is the conv input.  CONV == 1 (width <= 4): lane q of the channel's
// quad holds conv state element q, takes element q+1 from its neighbour by a
// DPP quad permute (the newest, x, at q = K-1), and the quad sums the four
// weighted taps.  CONV == 2 (width 5..8): every lane of the quad forms the
// whole sum and lane q writes back the elements k = q, q + 4.
// NBB: batch rows per thread (without the conv branch or with a width of at
// most 4).  The channel's A, bias, D and conv weights are loaded once for
// all of them, and every row's loads are issued before the first row is
// computed, so a wavefront keeps NBB times the bytes in flight.
template <typename T, bool VEC, int CONV, int R, int NBB>
__global__ __launch_bounds__(kThreads) void state_update_kernel(UpdateParams p) {
  static_assert(CONV != 2 || NBB == 1, "widths above 4 run one batch row per thread");
  const int q = threadIdx.x & 3;
  const int64_t b0 = static_cast<int64_t>(blockIdx.y) * NBB;
  const int64_t d0 = static_cast<int64_t>(blockIdx.x) * kChannelsPerBlock + (threadIdx.x >> 2);
  const bool ok = d0 < p.dim;
  const int64_t d = ok ? d0 : p.dim - 1;   // clamped: loads stay in bounds

  const int nv = min(R, max(0, p.N - R * q));   // real states of this lane
  // B/C group of the channel (a uniform branch: no division with one group)
  int64_t g = 0;
  if (p.cpg != p.dim) g = d / p.cpg;
  float a[R];
  loadR<float, VEC, R>(p.A + d * p.Asd + R * q, a, nv);
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float Dd = p.D ? p.D[d] : 0.0f;
  float s[NBB][R], bb[NBB][R], cc[NBB][R], xv[NBB], dtv[NBB], zv[NBB];
#pragma unroll
  for (int i = 0; i < NBB; ++i) {
    const int64_t b = min(b0 + i, p.batch - 1);   // rows past the batch repeat the last
    loadR<float, VEC, R>(p.state + b * p.ssb + d * p.ssd + R * q, s[i], nv);
    loadR<T, VEC, R>(static_cast<const T*>(p.B) + b * p.Bsb + g * p.Bsg + R * q, bb[i], nv);
    loadR<T, VEC, R>(static_cast<const T*>(p.C) + b * p.Csb + g * p.Csg + R * q, cc[i], nv);
    xv[i] = io<T>::load(static_cast<const T*>(p.x) + b * p.xsb + d);
    dtv[i] = io<T>::load(static_cast<const T*>(p.dt) + b * p.dtsb + d);
    zv[i] = p.z ? io<T>::load(static_cast<const T*>(p.z) + b * p.zsb + d) : 0.0f;
  }
  if constexpr (CONV == 1) {
    // causal conv of the block's conv branch: shift in x, then the weighted
    // sum of the K newest inputs (Mamba model notes, section 4.3)
    const int K = p.K;
    const int qk = min(q, K - 1);                     // lanes past K stay in the row
    const float wq = q < K ? p.conv_w[d * K + q] : 0.0f;
    const float cb = p.conv_b ? p.conv_b[d] : 0.0f;
    float old[NBB];
#pragma unroll
    for (int i = 0; i < NBB; ++i)
      old[i] = p.conv_state[(min(b0 + i, p.batch - 1) * p.dim + d) * K + qk];
#pragma unroll
    for (int i = 0; i < NBB; ++i) {
      const float nb = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(old[i]), 0xF9, 0xf, 0xf, true));
      const float nvx = q == K - 1 ? xv[i] : nb;      // element q of the shifted state
      float acc = q < K ? wq * nvx : 0.0f;
      acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0xB1, 0xf, 0xf, true));
      acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0x4E, 0xf, 0xf, true));
      acc += cb;
      if (ok && b0 + i < p.batch && q < K) p.conv_state[((b0 + i) * p.dim + d) * K + q] = nvx;
      xv[i] = p.conv_silu ? silu_f32(acc) : acc;
    }
  } else if constexpr (CONV == 2) {
    const int K = p.K;
    float* cs = p.conv_state + (b0 * p.dim + d) * K;
    const float* cw = p.conv_w + d * K;
    float acc = p.conv_b ? p.conv_b[d] : 0.0f;
    float nvx[kMaxConv];
#pragma unroll
    for (int k = 0; k < kMaxConv; ++k) {
      if (k < K) {
        nvx[k] = k + 1 < K ? cs[k + 1] : xv[0];
        acc = fmaf(cw[k], nvx[k], acc);
      }
    }
    // all four lanes have read the old state before any lane writes
    __builtin_amdgcn_wave_barrier();
    if (ok) {
#pragma unroll
      for (int k = 0; k < kMaxConv; ++k)
        if (k < K && (k & 3) == q) cs[k] = nvx[k];
    }
    xv[0] = p.conv_silu ? silu_f32(acc) : acc;
  }

#pragma unroll
  for (int i = 0; i < NBB; ++i) {
    const int64_t b = b0 + i;
    float dl = dtv[i] + bias;
    if (p.softplus) dl = softplus_f32(dl);
    const float dlx = dl * xv[i];
    float y = 0.0f;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float e = __builtin_amdgcn_exp2f(dl * (a[j] * kLog2e));
      s[i][j] = fmaf(e, s[i][j], dlx * bb[i][j]);
      y = fmaf(cc[i][j], s[i][j], y);   // padding states are 0 with C = 0
    }
    const bool okb = ok && b < p.batch;
    if (okb) storeR<VEC, R>(p.state + b * p.ssb + d * p.ssd + R * q, s[i], nv);
    // quad sum: lanes (0,1,2,3) <- (1,0,3,2), then <- (2,3,0,1)
    y += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y), 0xB1, 0xf, 0xf, true));
    y += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y), 0x4E, 0xf, 0xf, true));
    if (okb && q == 0) {
      y = fmaf(Dd, xv[i], y);
      if (p.z) y *= silu_f32(zv[i]);
      io<T>::store(static_cast<T*>(p.out) + b * p.osb + d, y);
    }
  }
}

template <typename T, bool VEC, int R>
void launch_v(int conv, bool rows, dim3 grid, dim3 block, const UpdateParams& p,
              hipStream_t stream) {
  if (conv == 0) {
    if constexpr (VEC && R <= 4) {
      if (rows) {
        state_update_kernel<T, VEC, 0, R, kRowsPerThread><<<grid, block, 0, stream>>>(p);
        return;
      }
    }
    state_update_kernel<T, VEC, 0, R, 1><<<grid, block, 0, stream>>>(p);
  } else if (conv == 1) {
    if constexpr (VEC && R <= 4) {
      if (rows) {
        state_update_kernel<T, VEC, 1, R, kRowsPerThread><<<grid, block, 0, stream>>>(p);
        return;
      }
    }
    state_update_kernel<T, VEC, 1, R, 1><<<grid, block, 0, stream>>>(p);
  } else {
    state_update_kernel<T, VEC, 2, R, 1><<<grid, block, 0, stream>>>(p);
  }
}

template <typename T, int R>
void launch_r(bool vec, int conv, bool rows, dim3 grid, dim3 block, const UpdateParams& p,
              hipStream_t stream) {
  if (vec) launch_v<T, true, R>(conv, rows, grid, block, p, stream);
  else launch_v<T, false, R>(conv, rows, grid, block, p, stream);
}

template <typename T>
void launch_t(int r, bool vec, int conv, bool rows, dim3 grid, dim3 block,
              const UpdateParams& p, hipStream_t stream) {
  switch (r) {
    case 1: launch_r<T, 1>(vec, conv, rows, grid, block, p, stream); break;
    case 2: launch_r<T, 2>(vec, conv, rows, grid, block, p, stream); break;
    case 4: launch_r<T, 4>(vec, conv, rows, grid, block, p, stream); break;
    case 8: launch_r<T, 8>(vec, conv, rows, grid, block, p, stream); break;
    default: launch_r<T, 16>(vec, conv, rows, grid, block, p, stream); break;
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
  const int64_t G = a.ngroups > 1 ? a.ngroups : 1;
  p.cpg = a.dim / G;
  p.Bsg = G > 1 ? a.B_group_stride : 0;
  p.Csg = G > 1 ? a.C_group_stride : 0;
  p.N = static_cast<int>(a.dstate);
  p.softplus = a.dt_softplus ? 1 : 0;
  // states per lane: N / 4 rounded up to a power of two
  int r = 1;
  while (4 * r < a.dstate) r *= 2;
  const int esz = a.io_dtype == SSM_BF16 ? 2 : 4;
  const int64_t w = r < 4 ? r : 4;   // elements per vector access
  auto al = [&](const void* ptr, int64_t bytes) {
    return reinterpret_cast<uintptr_t>(ptr) % static_cast<uintptr_t>(bytes) == 0;
  };
  const bool vec = a.dstate == 4 * r && al(a.state, 4 * w) && a.state_batch_stride % w == 0 &&
                   a.state_dim_stride % w == 0 && al(a.A, 4 * w) && a.A_dim_stride % w == 0 &&
                   al(a.B, esz * w) && al(a.C, esz * w) && a.B_batch_stride % w == 0 &&
                   a.C_batch_stride % w == 0 && p.Bsg % w == 0 && p.Csg % w == 0;
  p.conv_state = a.conv_weight ? a.conv_state : nullptr;
  p.conv_w = a.conv_weight; p.conv_b = a.conv_bias;
  p.K = a.conv_weight ? a.d_conv : 0;
  p.conv_silu = a.conv_silu;
  const int64_t xblocks = (a.dim + kChannelsPerBlock - 1) / kChannelsPerBlock;
  if (xblocks > 0x7fffffff || a.batch > 65535) return hipErrorInvalidConfiguration;
  const bool rows = (a.conv_weight == nullptr || a.d_conv <= 4) && vec && r <= 4 &&
                    xblocks * ((a.batch + kRowsPerThread - 1) / kRowsPerThread) >= kMinBlocksRows;
  const int64_t ybl = rows ? (a.batch + kRowsPerThread - 1) / kRowsPerThread : a.batch;
  const dim3 grid(static_cast<unsigned>(xblocks), static_cast<unsigned>(ybl));
  const dim3 block(kThreads);
  const int conv = a.conv_weight == nullptr ? 0 : (a.d_conv <= 4 ? 1 : 2);
  if (a.io_dtype == SSM_BF16) launch_t<uint16_t>(r, vec, conv, rows, grid, block, p, stream);
  else launch_t<float>(r, vec, conv, rows, grid, block, p, stream);
  return hipGetLastError();
}

}  // namespace ssm

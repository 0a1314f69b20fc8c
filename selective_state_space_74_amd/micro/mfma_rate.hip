// mfma_rate.hip -- issue rate of gfx950's two bf16 matrix instructions of
// 16 x 16 output tiles: v_mfma_f32_16x16x16_bf16 (k = 16, the form the SSD
// chunk products use) and v_mfma_f32_16x16x32_bf16 (k = 32, new in gfx950).
// A register-only kernel: each wavefront runs eight independent accumulator
// chains (enough to cover the dependent-issue latency), so the figure is the
// matrix cores' throughput, not latency.  bench.py --micro-mfma times it.
// Built into libssm_micro.so (not part of the libssm.so boundary).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) float v4f;
typedef __attribute__((ext_vector_type(4))) short v4s;
typedef __attribute__((ext_vector_type(8))) __bf16 v8bf;

constexpr int kChains = 8;

template <int K>
__global__ __launch_bounds__(256) void mfma_rate_kernel(float* out, int iters) {
  const int lane = threadIdx.x + blockIdx.x * blockDim.x;
  v4f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) {   // distinct chains (none can be merged)
    const float f = static_cast<float>(c) + 1e-3f * static_cast<float>(lane & 63);
    acc[c] = v4f{f, f, f, f};
  }
  // operands: small bf16 values that depend on the lane (0x3c00 + i is about
  // 2^-7 (1 + i/128))
  const short s = static_cast<short>(0x3c00 + (lane & 7));
  if constexpr (K == 16) {
    const v4s a = {s, s, s, s};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, a, acc[c], 0, 0, 0);
    }
  } else {
    v8bf a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = __builtin_bit_cast(__bf16, s);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, acc[c], 0, 0, 0);
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) sum += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[lane] = sum;
}

}  // namespace

extern "C" {

// Launches `lanes` / 256 workgroups of 256 lanes; each wavefront issues
// iters * 8 matrix instructions of k = `k` (16 or 32), each 2 * 16 * 16 * k
// flops.  out: device buffer of `lanes` floats.  Returns a hipError_t.
int ssm_micro_mfma_rate(float* out, int64_t lanes, int32_t iters, int32_t k, void* stream) {
  if (!out || lanes <= 0 || lanes % 256 != 0 || iters <= 0 || (k != 16 && k != 32))
    return static_cast<int>(hipErrorInvalidValue);
  const dim3 grid(static_cast<unsigned>(lanes / 256)), block(256);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (k == 16) mfma_rate_kernel<16><<<grid, block, 0, st>>>(out, iters);
  else mfma_rate_kernel<32><<<grid, block, 0, st>>>(out, iters);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"

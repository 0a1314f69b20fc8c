// Internal declarations shared by the HIP sources of libssm.so (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm.h"

namespace ssm {

// Launches; arguments already validated by the ABI layer.
hipError_t launch_scan_fwd(const ssm_scan_args& a, hipStream_t stream);
hipError_t launch_state_update(const ssm_update_args& a, hipStream_t stream);

// ---------------------------------------------------------------------------
// Device helpers.

// bf16 <-> fp32.  bf16 is the upper half of an fp32 word, so widening is a
// shift; narrowing rounds to nearest-even and keeps NaNs quiet.
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct io;
template <> struct io<float> {
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct io<uint16_t> {
  __device__ static __forceinline__ float load(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ static __forceinline__ void store(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};

constexpr float kLog2e = 1.4426950408889634f;

// softplus(x) = log(1 + e^x); above 20 the correction e^-x < 2.1e-9 is below
// fp32 resolution of x, so x itself is returned.
__device__ __forceinline__ float softplus_f32(float x) {
  return x > 20.0f ? x : log1pf(expf(x));
}

// silu(z) = z * sigmoid(z)
__device__ __forceinline__ float silu_f32(float z) {
  return z / (1.0f + expf(-z));
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Lane J of each 16-lane row, broadcast to the whole row (DPP row_newbcast).
template <int J>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + J, 0xf, 0xf, true));
}

}  // namespace ssm

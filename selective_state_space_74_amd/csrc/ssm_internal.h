// Internal declarations shared by the HIP sources of libssm.so (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm.h"

namespace ssm {

// Launches; arguments already validated by the ABI layer.
hipError_t launch_scan_fwd(const ssm_scan_args& a, hipStream_t stream);
// The same scan with its segment scratch in the library's static device
// buffer (validated arguments; returns an ssm_status).
int scan_fwd_noalloc(const ssm_scan_args& a, hipStream_t stream);
size_t scan_workspace_bytes(const ssm_scan_args& a);
// The scan addresses each wavefront's rows through 32-bit byte windows.
bool scan_windows_fit(const ssm_scan_args& a);
hipError_t launch_state_update(const ssm_update_args& a, hipStream_t stream);
hipError_t launch_scan_bwd(const ssm_scan_bwd_args& a, hipStream_t stream);
bool scan_bwd_windows_fit(const ssm_scan_bwd_args& a);
size_t scan_bwd_workspace_bytes(const ssm_scan_bwd_args& a);
hipError_t launch_ssd_fwd(const ssm_ssd_args& a, hipStream_t stream);
size_t ssd_workspace_bytes(const ssm_ssd_args& a);

// ---------------------------------------------------------------------------
// Device helpers.

// bf16 <-> fp32.  bf16 is the upper half of an fp32 word, so widening is a
// shift; narrowing rounds to nearest-even and keeps NaNs quiet.
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}
// fp32 -> bf16, round to nearest even, NaN stays NaN (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
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

constexpr float kLn2 = 0.6931471805599453f;

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^-|x|), on the hardware
// exp2/log2.  log1p(y) for y in (0, 1] is log(u) for u = 1 + y rounded, plus
// the part of y that the rounding dropped, e = y - (u - 1) (exact):
// log1p(y) = log(u) + log(1 + e/u) = log(u) + e/u to first order, as
// |e| <= 2^-24.  e is added in place of e/u: the two differ by e y / (1 + y),
// under 2^-24 y / (1 + y), while log1p(y) >= y ln 2, so the result moves by
// at most about one unit in its last place and no reciprocal is spent.  This
// keeps full relative accuracy for small y (Delta around 1e-3 sits there), and
// when 1 + y rounds to 1 it gives y itself.
__device__ __forceinline__ float softplus_f32(float x) {
  const float y = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
  const float u = 1.0f + y;
  const float e = y - (u - 1.0f);
  const float lp = fmaf(__builtin_amdgcn_logf(u), kLn2, e);
  return fmaxf(x, 0.0f) + lp;
}

// silu(z) = z * sigmoid(z) = z / (1 + 2^(-z log2 e))
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// Workgroup order.  The dispatcher hands the i-th workgroup of a launch to
// XCD i % 8; xcd_order(i, n) is the logical workgroup that kernels work on,
// chosen so that each XCD receives a contiguous logical range (XCD x gets
// n / 8 workgroups, one more for x < n % 8, slots i / 8 in order, after the
// ranges of the XCDs before it): neighbouring logical workgroups (the
// channel groups of one segment, which read the same B/C tile) then share
// one XCD's L2 and translation caches.  A bijection of [0, n).
constexpr uint32_t kXcds = 8;
__device__ __forceinline__ uint32_t xcd_order(uint32_t i, uint32_t n) {
  const uint32_t x = i % kXcds, slot = i / kXcds, q = n / kXcds, r = n % kXcds;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + slot;
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

// An opaque register copy.  Broadcasting the copy instead of the original
// keeps the compiler from merging two broadcasts of one value (which would
// leave a separate DPP move, live across everything between its two uses).
__device__ __forceinline__ float opaque_copy(float v) {
  float r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

// ---------------------------------------------------------------------------
// Buffer-descriptor access (raw buffers, gfx9 family descriptor word 3).

constexpr int kRsrcWord3 = 0x00020000;

// One IO element through a buffer descriptor: loads return the raw bits
// (widened later), stores round to the IO type.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kSize = 4;
  __device__ static __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  __device__ static __forceinline__ float f32(uint32_t v) { return __uint_as_float(v); }
  __device__ static __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
  }
};
template <> struct Elem<uint16_t> {
  static constexpr int kSize = 2;
  __device__ static __forceinline__ uint32_t load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  }
  __device__ static __forceinline__ float f32(uint32_t v) { return __uint_as_float(v << 16); }
  __device__ static __forceinline__ void store(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, off, 0, 0);
  }
};

// A wavefront-uniform byte window [base, base + bytes) of one tensor.  Host
// validation keeps every window below 4 GiB, so all offsets are 32-bit.
struct Window {
  const char* base;
  uint32_t bytes;
  // The window moved `skip` bytes forward; skip never exceeds bytes (block
  // starts stay inside the sequence).
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t at(uint32_t skip) const {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + skip), 0,
                                             static_cast<int>(bytes - skip), kRsrcWord3);
  }
};

}  // namespace ssm

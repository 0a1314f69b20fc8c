// valu_mix.hip -- the arithmetic ceiling of the selective scan on gfx950,
// measured: a register-only kernel that executes, per 16 (token, state)
// steps of one lane, the instruction mix the scan cannot avoid, with no
// memory traffic.  bench.py times it to report the fraction of this ceiling
// that the scan kernels reach next to their fraction of HBM bandwidth.
// Built into libssm_micro.so (not part of the libssm.so boundary).
//
// Per state n and token t (Mamba paper notes, section 2.3: Abar = exp(Delta A),
// Bbar u = Delta B u; Mamba model notes, section 2.2: h = Abar h + Bbar u,
// y = sum_n C h):
//   one multiply Delta * A[n] log2(e), one v_exp_f32, one multiply
//   (Delta u) * B[n], the state FMA and the readout FMA.
// Per token (once per 16 steps here, as a lane owns one token of each
// 16-token block): delta + bias; softplus as max(x,0) + log2(1 + 2^(-|x|
// log2 e)) ln 2 (2 transcendentals, 4 VALU); silu(z) = z / (1 + 2^(-z log2
// e)) (2 transcendentals, 3 VALU); Delta u; D u + y; the gate product; and
// one operation per loaded input (u, delta, z), as the bf16 widening costs.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kS = 16;

__global__ __launch_bounds__(256) void valu_mix_kernel(float* out, int blocks) {
  const int lane = threadIdx.x + blockIdx.x * blockDim.x;
  const float fl = static_cast<float>(lane & 1023) * 1e-4f;
  float a2[kS], bv[kS], cv[kS];
#pragma unroll
  for (int j = 0; j < kS; ++j) {
    a2[j] = -(1.0f + j + fl) * 1.4426950408889634f;
    bv[j] = 0.25f + 0.01f * j - fl;
    cv[j] = 0.5f - 0.02f * j + fl;
  }
  float h = fl, acc = 0.0f;
  for (int k = 0; k < blocks; ++k) {
    const float fk = static_cast<float>(k);
    // the token's inputs (one operation each, like widening a bf16 load)
    const float u = fmaf(fk, 1e-7f, fl);
    const float dt = fmaf(fk, -3e-8f, 0.01f);
    const float z = fmaf(fk, 2e-7f, -fl);
    const float x = dt + fl;  // + bias
    const float sp = fmaf(__builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f)),
                          0.6931471805599453f, fmaxf(x, 0.0f));
    const float g = z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
    const float du = sp * u;
    float y = 0.0f;
#pragma unroll
    for (int j = 0; j < kS; ++j) {
      const float e = __builtin_amdgcn_exp2f(sp * a2[j]);
      const float w = du * bv[j];
      h = fmaf(e, h, w);
      y = fmaf(cv[j], h, y);
    }
    y = fmaf(fl, u, y);  // D u
    acc += y * g;        // gate (and a sum that keeps every step live)
  }
  out[lane] = h + acc;
}

}  // namespace

extern "C" {

// Launches `lanes` / 256 workgroups of 256 lanes, each lane running `blocks`
// iterations of 16 steps (lanes * blocks * 16 (token, state) steps in all).
// out: device buffer of `lanes` floats.  Returns a hipError_t.
int ssm_micro_valu_mix(float* out, int64_t lanes, int32_t blocks, void* stream) {
  if (!out || lanes <= 0 || lanes % 256 != 0 || blocks <= 0) return static_cast<int>(hipErrorInvalidValue);
  valu_mix_kernel<<<dim3(static_cast<unsigned>(lanes / 256)), dim3(256), 0,
                    static_cast<hipStream_t>(stream)>>>(out, blocks);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"

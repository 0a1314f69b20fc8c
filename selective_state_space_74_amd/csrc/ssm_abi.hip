// ssm_abi.hip -- the extern "C" surface of libssm.so: host-side validation
// and dispatch to the gfx950 kernels.  Validation is pure host code (no HIP
// call) so it can be exercised on a machine without a GPU.
#include <stdint.h>
#include <string.h>

#include "ssm_internal.h"

namespace {

struct Span {  // byte range [lo, hi)
  uintptr_t lo = 0, hi = 0;
  bool empty() const { return hi <= lo; }
};

bool overlap(const Span& a, const Span& b) {
  return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

// Bytes touched by a (n0, n1, n2) tensor with strides (s0, s1, 1).
Span span3(const void* p, int64_t n0, int64_t s0, int64_t n1, int64_t s1, int64_t n2,
           int64_t esz) {
  Span s;
  if (!p || n0 <= 0 || n1 <= 0 || n2 <= 0) return s;
  s.lo = reinterpret_cast<uintptr_t>(p);
  s.hi = s.lo + static_cast<uintptr_t>(((n0 - 1) * s0 + (n1 - 1) * s1 + n2) * esz);
  return s;
}

Span span1(const void* p, int64_t n, int64_t esz) { return span3(p, 1, 0, 1, 0, n, esz); }

// Bytes touched by a (n0, n1, n2, n3) tensor with strides (s0, s1, s2, 1).
Span span4(const void* p, int64_t n0, int64_t s0, int64_t n1, int64_t s1, int64_t n2,
           int64_t s2, int64_t n3, int64_t esz) {
  Span s;
  if (!p || n0 <= 0 || n1 <= 0 || n2 <= 0 || n3 <= 0) return s;
  s.lo = reinterpret_cast<uintptr_t>(p);
  s.hi = s.lo + static_cast<uintptr_t>(((n0 - 1) * s0 + (n1 - 1) * s1 + (n2 - 1) * s2 + n3) * esz);
  return s;
}

// B/C groups: 0 or 1 is one group; otherwise it must divide dim.
int64_t groups_of(int64_t ngroups) { return ngroups > 1 ? ngroups : 1; }
bool bad_groups(int64_t ngroups, int64_t dim) {
  return ngroups < 0 || (dim > 0 && dim % groups_of(ngroups) != 0);
}

bool misaligned(const void* p, int64_t align) {
  return p && (reinterpret_cast<uintptr_t>(p) % static_cast<uintptr_t>(align)) != 0;
}

int64_t io_size(int32_t dt) { return dt == SSM_BF16 ? 2 : 4; }

// Token indices are 32-bit inside the scan kernel.
constexpr int64_t kMaxSeqlen = (int64_t{1} << 31) - 64;
constexpr int64_t kCkptTokens = SSM_CHECKPOINT_TOKENS;

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }
size_t ssm_scan_args_size(void) { return sizeof(ssm_scan_args); }
size_t ssm_scan_bwd_args_size(void) { return sizeof(ssm_scan_bwd_args); }
size_t ssm_update_args_size(void) { return sizeof(ssm_update_args); }
size_t ssm_ssd_args_size(void) { return sizeof(ssm_ssd_args); }

size_t ssm_scan_workspace_size(const ssm_scan_args* a) {
  if (!a || a->dstate < 1 || a->dstate > SSM_MAX_DSTATE || a->seqlen > kMaxSeqlen) return 0;
  return ssm::scan_workspace_bytes(*a);
}

size_t ssm_ssd_workspace_size(const ssm_ssd_args* a) {
  if (!a || a->seqlen > kMaxSeqlen || a->batch < 0 || a->seqlen < 0) return 0;
  return ssm::ssd_workspace_bytes(*a);
}

size_t ssm_scan_bwd_workspace_size(const ssm_scan_bwd_args* a) {
  if (!a || a->dstate < 1 || a->dstate > SSM_MAX_DSTATE || a->seqlen > kMaxSeqlen || a->batch < 0 ||
      a->dim < 0 || a->seqlen < 0)
    return 0;
  return ssm::scan_bwd_workspace_bytes(*a);
}

const char* ssm_status_string(int status) {
  switch (status) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "a required pointer is NULL";
    case SSM_ERR_SHAPE: return "invalid size (negative, dstate < 1, or ngroups not dividing dim)";
    case SSM_ERR_STRIDE: return "invalid stride (negative)";
    case SSM_ERR_DTYPE: return "io_dtype must be SSM_F32 or SSM_BF16";
    case SSM_ERR_ALIGN: return "pointer not aligned to its element size";
    case SSM_ERR_ALIAS: return "an output overlaps an input";
    case SSM_ERR_UNSUPPORTED: return "unsupported configuration (dstate or B/C groups outside what is built, or a size past the limits in ssm.h)";
    case SSM_ERR_HIP: return "HIP runtime error at launch";
    case SSM_ERR_SCRATCH: return "the scan needs more segment scratch than the no-allocation entry point's static buffer (SSM_NOALLOC_SCRATCH_BYTES) holds";
    default: return "unknown status";
  }
}

int ssm_validate_scan(const ssm_scan_args* a) {
  if (!a) return SSM_ERR_NULL;
  if (a->batch < 0 || a->dim < 0 || a->seqlen < 0 || a->dstate < 1) return SSM_ERR_SHAPE;
  if (bad_groups(a->ngroups, a->dim)) return SSM_ERR_SHAPE;
  if (a->io_dtype != SSM_F32 && a->io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (a->dstate > SSM_MAX_DSTATE) return SSM_ERR_UNSUPPORTED;
  if (a->seqlen > kMaxSeqlen) return SSM_ERR_UNSUPPORTED;
  if (a->batch == 0 || a->dim == 0) return SSM_OK;
  const int64_t B = a->batch, Dm = a->dim, L = a->seqlen, N = a->dstate;
  const int64_t G = groups_of(a->ngroups);
  const int64_t esz = io_size(a->io_dtype);
  if (L > 0) {
    if (!a->u || !a->delta || !a->B || !a->C || !a->A || !a->out) return SSM_ERR_NULL;
    const int64_t strides[] = {a->u_batch_stride, a->u_dim_stride, a->delta_batch_stride,
                               a->delta_dim_stride, a->B_batch_stride, a->B_state_stride,
                               a->C_batch_stride, a->C_state_stride, a->A_dim_stride,
                               a->A_state_stride, a->out_batch_stride, a->out_dim_stride,
                               a->z ? a->z_batch_stride : 0, a->z ? a->z_dim_stride : 0,
                               G > 1 ? a->B_group_stride : 0, G > 1 ? a->C_group_stride : 0};
    for (int64_t s : strides)
      if (s < 0) return SSM_ERR_STRIDE;
    if (misaligned(a->u, esz) || misaligned(a->delta, esz) || misaligned(a->z, esz) ||
        misaligned(a->B, esz) || misaligned(a->C, esz) || misaligned(a->out, esz))
      return SSM_ERR_ALIGN;
    if (!ssm::scan_windows_fit(*a)) return SSM_ERR_UNSUPPORTED;
  }
  if (misaligned(a->A, 4) || misaligned(a->D, 4) || misaligned(a->delta_bias, 4) ||
      misaligned(a->h0, 4) || misaligned(a->last_state, 4) || misaligned(a->workspace, 4))
    return SSM_ERR_ALIGN;

  if (misaligned(a->checkpoints, 4) || misaligned(a->conv_weight, 4) ||
      misaligned(a->conv_bias, 4) || misaligned(a->conv_state_in, 4) ||
      misaligned(a->conv_state_out, 4))
    return SSM_ERR_ALIGN;
  int64_t K = 0;
  if (a->conv_weight) {
    K = a->d_conv;
    if (K < 1) return SSM_ERR_SHAPE;
    if (K > SSM_MAX_CONV) return SSM_ERR_UNSUPPORTED;
    if (L > 0 && a->conv_out) {
      if (a->conv_out_batch_stride < 0 || a->conv_out_dim_stride < 0) return SSM_ERR_STRIDE;
      if (misaligned(a->conv_out, esz)) return SSM_ERR_ALIGN;
    }
  }

  const Span sA = L > 0 ? Span{reinterpret_cast<uintptr_t>(a->A),
                               reinterpret_cast<uintptr_t>(a->A) +
                                   static_cast<uintptr_t>(((Dm - 1) * a->A_dim_stride +
                                                           (N - 1) * a->A_state_stride + 1) * 4)}
                        : Span{};
  const Span sh0 = span1(a->h0, B * Dm * N, 4);
  const Span inputs[] = {
      span3(a->u, B, a->u_batch_stride, Dm, a->u_dim_stride, L, esz),
      span3(a->delta, B, a->delta_batch_stride, Dm, a->delta_dim_stride, L, esz),
      span3(a->z, B, a->z_batch_stride, Dm, a->z_dim_stride, L, esz),
      span4(a->B, B, a->B_batch_stride, G, a->B_group_stride, N, a->B_state_stride, L, esz),
      span4(a->C, B, a->C_batch_stride, G, a->C_group_stride, N, a->C_state_stride, L, esz),
      sA, span1(a->D, Dm, 4), span1(a->delta_bias, Dm, 4), sh0,
      span1(a->conv_weight, Dm * K, 4), span1(a->conv_bias, Dm, 4),
      span1(a->conv_state_in, B * Dm * K, 4)};
  const Span sls = span1(a->last_state, B * Dm * N, 4);
  const Span outputs[] = {
      span3(a->out, B, a->out_batch_stride, Dm, a->out_dim_stride, L, esz), sls,
      span1(a->workspace, static_cast<int64_t>(a->workspace_bytes), 1),
      span1(a->checkpoints, B * Dm * ((L + kCkptTokens - 1) / kCkptTokens) * N, 4),
      K ? span1(a->conv_state_out, B * Dm * K, 4) : Span{},
      K ? span3(a->conv_out, B, a->conv_out_batch_stride, Dm, a->conv_out_dim_stride, L, esz)
        : Span{}};
  for (const Span& o : outputs) {
    for (const Span& i : inputs) {
      // last_state may be exactly h0 (the state carried in place)
      if (&o == &outputs[1] && &i == &inputs[8] && a->last_state == a->h0) continue;
      if (overlap(o, i)) return SSM_ERR_ALIAS;
    }
    for (const Span& o2 : outputs)
      if (&o2 != &o && overlap(o, o2)) return SSM_ERR_ALIAS;
  }
  return SSM_OK;
}

int ssm_validate_scan_bwd(const ssm_scan_bwd_args* a) {
  if (!a) return SSM_ERR_NULL;
  if (a->batch < 0 || a->dim < 0 || a->seqlen < 0 || a->dstate < 1) return SSM_ERR_SHAPE;
  if (bad_groups(a->ngroups, a->dim)) return SSM_ERR_SHAPE;
  if (a->io_dtype != SSM_F32 && a->io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (a->dstate > SSM_MAX_DSTATE) return SSM_ERR_UNSUPPORTED;
  // every block of 16 channels must sit in one group
  if (groups_of(a->ngroups) > 1 && (a->dim / groups_of(a->ngroups)) % 16 != 0)
    return SSM_ERR_UNSUPPORTED;
  if (a->seqlen > kMaxSeqlen) return SSM_ERR_UNSUPPORTED;
  if (a->batch == 0 || a->dim == 0) return SSM_OK;
  if (!a->A || !a->dA) return SSM_ERR_NULL;
  const int64_t B = a->batch, Dm = a->dim, L = a->seqlen, N = a->dstate;
  const int64_t G = groups_of(a->ngroups);
  const int64_t esz = io_size(a->io_dtype);
  if (L > 0) {
    if (!a->u || !a->delta || !a->B || !a->C || !a->checkpoints || !a->dout || !a->du ||
        !a->ddelta || !a->dB || !a->dC || (a->z && !a->dz))
      return SSM_ERR_NULL;
    const int64_t strides[] = {a->u_batch_stride, a->u_dim_stride, a->delta_batch_stride,
                               a->delta_dim_stride, a->B_batch_stride, a->B_state_stride,
                               a->C_batch_stride, a->C_state_stride, a->A_dim_stride,
                               a->A_state_stride, a->dout_batch_stride, a->dout_dim_stride,
                               a->du_batch_stride, a->du_dim_stride, a->ddelta_batch_stride,
                               a->ddelta_dim_stride, a->z ? a->z_batch_stride : 0,
                               a->z ? a->z_dim_stride : 0, a->z ? a->dz_batch_stride : 0,
                               a->z ? a->dz_dim_stride : 0, G > 1 ? a->B_group_stride : 0,
                               G > 1 ? a->C_group_stride : 0};
    for (int64_t s : strides)
      if (s < 0) return SSM_ERR_STRIDE;
    if (misaligned(a->u, esz) || misaligned(a->delta, esz) || misaligned(a->z, esz) ||
        misaligned(a->B, esz) || misaligned(a->C, esz) || misaligned(a->dout, esz) ||
        misaligned(a->du, esz) || misaligned(a->ddelta, esz) || (a->z && misaligned(a->dz, esz)))
      return SSM_ERR_ALIGN;
    if (!ssm::scan_bwd_windows_fit(*a)) return SSM_ERR_UNSUPPORTED;
  }
  if (misaligned(a->A, 4) || misaligned(a->D, 4) || misaligned(a->delta_bias, 4) ||
      misaligned(a->h0, 4) || misaligned(a->checkpoints, 4) || misaligned(a->dlast, 4) ||
      misaligned(a->dB, 4) || misaligned(a->dC, 4) || misaligned(a->dA, 4) ||
      misaligned(a->dD, 4) || misaligned(a->ddelta_bias, 4) || misaligned(a->dh0, 4) ||
      misaligned(a->workspace, 4))
    return SSM_ERR_ALIGN;
  const int64_t nbk = (L + kCkptTokens - 1) / kCkptTokens;
  const Span inputs[] = {
      span3(a->u, B, a->u_batch_stride, Dm, a->u_dim_stride, L, esz),
      span3(a->delta, B, a->delta_batch_stride, Dm, a->delta_dim_stride, L, esz),
      span3(a->z, B, a->z_batch_stride, Dm, a->z_dim_stride, L, esz),
      span4(a->B, B, a->B_batch_stride, G, a->B_group_stride, N, a->B_state_stride, L, esz),
      span4(a->C, B, a->C_batch_stride, G, a->C_group_stride, N, a->C_state_stride, L, esz),
      L > 0 ? Span{reinterpret_cast<uintptr_t>(a->A),
                   reinterpret_cast<uintptr_t>(a->A) +
                       static_cast<uintptr_t>(((Dm - 1) * a->A_dim_stride +
                                               (N - 1) * a->A_state_stride + 1) * 4)}
            : Span{},
      span1(a->D, Dm, 4), span1(a->delta_bias, Dm, 4), span1(a->h0, B * Dm * N, 4),
      span1(a->checkpoints, B * Dm * nbk * N, 4),
      span3(a->dout, B, a->dout_batch_stride, Dm, a->dout_dim_stride, L, esz),
      span1(a->dlast, B * Dm * N, 4)};
  const Span outputs[] = {
      span3(a->du, B, a->du_batch_stride, Dm, a->du_dim_stride, L, esz),
      span3(a->ddelta, B, a->ddelta_batch_stride, Dm, a->ddelta_dim_stride, L, esz),
      a->z ? span3(a->dz, B, a->dz_batch_stride, Dm, a->dz_dim_stride, L, esz) : Span{},
      span1(a->dB, B * G * N * L, 4), span1(a->dC, B * G * N * L, 4), span1(a->dA, Dm * N, 4),
      span1(a->dD, Dm, 4), span1(a->ddelta_bias, Dm, 4), span1(a->dh0, B * Dm * N, 4),
      span1(a->workspace, static_cast<int64_t>(a->workspace_bytes), 1)};
  for (const Span& o : outputs) {
    for (const Span& i : inputs)
      if (overlap(o, i)) return SSM_ERR_ALIAS;
    for (const Span& o2 : outputs)
      if (&o2 != &o && overlap(o, o2)) return SSM_ERR_ALIAS;
  }
  return SSM_OK;
}

int ssm_validate_update(const ssm_update_args* a) {
  if (!a) return SSM_ERR_NULL;
  if (a->batch < 0 || a->dim < 0 || a->dstate < 1) return SSM_ERR_SHAPE;
  if (bad_groups(a->ngroups, a->dim)) return SSM_ERR_SHAPE;
  if (a->io_dtype != SSM_F32 && a->io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (a->dstate > SSM_MAX_DSTATE) return SSM_ERR_UNSUPPORTED;
  if (a->batch > 65535) return SSM_ERR_UNSUPPORTED;
  if (a->batch == 0 || a->dim == 0) return SSM_OK;
  if (!a->state || !a->x || !a->dt || !a->B || !a->C || !a->A || !a->out) return SSM_ERR_NULL;
  const int64_t strides[] = {a->state_batch_stride, a->state_dim_stride, a->x_batch_stride,
                             a->dt_batch_stride, a->z ? a->z_batch_stride : 0,
                             a->B_batch_stride, a->C_batch_stride, a->A_dim_stride,
                             a->out_batch_stride,
                             a->ngroups > 1 ? a->B_group_stride : 0,
                             a->ngroups > 1 ? a->C_group_stride : 0};
  for (int64_t s : strides)
    if (s < 0) return SSM_ERR_STRIDE;
  const int64_t esz = io_size(a->io_dtype);
  const int64_t B = a->batch, Dm = a->dim, N = a->dstate;
  if (misaligned(a->x, esz) || misaligned(a->dt, esz) || misaligned(a->z, esz) ||
      misaligned(a->B, esz) || misaligned(a->C, esz) || misaligned(a->out, esz))
    return SSM_ERR_ALIGN;
  if (misaligned(a->state, 4) || misaligned(a->A, 4) || misaligned(a->D, 4) ||
      misaligned(a->dt_bias, 4))
    return SSM_ERR_ALIGN;
  const Span sst = span3(a->state, B, a->state_batch_stride, Dm, a->state_dim_stride, N, 4);
  const Span sx = span3(a->x, 1, 0, B, a->x_batch_stride, Dm, esz);
  const Span sdt = span3(a->dt, 1, 0, B, a->dt_batch_stride, Dm, esz);
  const Span sz = span3(a->z, 1, 0, B, a->z_batch_stride, Dm, esz);
  const int64_t G = groups_of(a->ngroups);
  const Span sB = span3(a->B, B, a->B_batch_stride, G, a->B_group_stride, N, esz);
  const Span sC = span3(a->C, B, a->C_batch_stride, G, a->C_group_stride, N, esz);
  const Span sA = span3(a->A, 1, 0, Dm, a->A_dim_stride, N, 4);
  const Span sD = span1(a->D, Dm, 4), sbias = span1(a->dt_bias, Dm, 4);
  const Span sout = span3(a->out, 1, 0, B, a->out_batch_stride, Dm, esz);
  int64_t K = 0;
  if (a->conv_weight) {
    K = a->d_conv;
    if (K < 1) return SSM_ERR_SHAPE;
    if (K > SSM_MAX_CONV) return SSM_ERR_UNSUPPORTED;
    if (!a->conv_state) return SSM_ERR_NULL;
    if (misaligned(a->conv_state, 4) || misaligned(a->conv_weight, 4) ||
        misaligned(a->conv_bias, 4))
      return SSM_ERR_ALIGN;
  }
  const Span scs = span1(K ? a->conv_state : nullptr, B * Dm * K, 4);
  const Span inputs[] = {sx, sdt, sz, sB, sC, sA, sD, sbias,
                         span1(K ? a->conv_weight : nullptr, Dm * K, 4),
                         span1(K ? a->conv_bias : nullptr, Dm, 4)};
  for (const Span& s : inputs)
    if (overlap(sout, s) || overlap(sst, s) || overlap(scs, s)) return SSM_ERR_ALIAS;
  if (overlap(sout, sst) || overlap(sout, scs) || overlap(sst, scs)) return SSM_ERR_ALIAS;
  return SSM_OK;
}

int ssm_validate_ssd(const ssm_ssd_args* a) {
  if (!a) return SSM_ERR_NULL;
  if (a->batch < 0 || a->seqlen < 0 || a->nheads < 1 || a->headdim < 1 || a->dstate < 1 ||
      a->ngroups < 0)
    return SSM_ERR_SHAPE;
  const int64_t G = groups_of(a->ngroups);
  if (a->nheads % G != 0) return SSM_ERR_SHAPE;
  if (a->io_dtype != SSM_F32 && a->io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (a->dstate > (a->io_dtype == SSM_BF16 ? 128 : 64)) return SSM_ERR_UNSUPPORTED;
  if (a->seqlen > kMaxSeqlen) return SSM_ERR_UNSUPPORTED;
  if (a->batch * a->nheads * ((a->headdim + 15) / 16) > 0x7fffffff) return SSM_ERR_UNSUPPORTED;
  if (a->batch == 0) return SSM_OK;
  const int64_t Bt = a->batch, L = a->seqlen, H = a->nheads, P = a->headdim, N = a->dstate;
  const int64_t esz = io_size(a->io_dtype);
  if (!a->A) return SSM_ERR_NULL;
  if (L > 0) {
    if (!a->x || !a->dt || !a->B || !a->C || !a->out) return SSM_ERR_NULL;
    const int64_t strides[] = {a->x_batch_stride, a->x_seq_stride, a->x_head_stride,
                               a->dt_batch_stride, a->dt_seq_stride,
                               a->B_batch_stride, a->B_seq_stride, G > 1 ? a->B_group_stride : 0,
                               a->C_batch_stride, a->C_seq_stride, G > 1 ? a->C_group_stride : 0,
                               a->out_batch_stride, a->out_seq_stride, a->out_head_stride,
                               a->z ? a->z_batch_stride : 0, a->z ? a->z_seq_stride : 0,
                               a->z ? a->z_head_stride : 0};
    for (int64_t s : strides)
      if (s < 0) return SSM_ERR_STRIDE;
    if (misaligned(a->x, esz) || misaligned(a->dt, esz) || misaligned(a->z, esz) ||
        misaligned(a->B, esz) || misaligned(a->C, esz) || misaligned(a->out, esz))
      return SSM_ERR_ALIGN;
    // the kernel reads a chunk (64 tokens) of x, dt, B and C through 31-bit
    // byte windows
    auto fits = [&](int64_t seq_stride, int64_t inner) {
      return (63 * seq_stride + inner) * esz < (int64_t{1} << 31);
    };
    if (!fits(a->x_seq_stride, P) || !fits(a->dt_seq_stride, 1) || !fits(a->B_seq_stride, N) ||
        !fits(a->C_seq_stride, N) || !fits(a->out_seq_stride, P) ||
        (a->z && !fits(a->z_seq_stride, P)))
      return SSM_ERR_UNSUPPORTED;
  }
  if (misaligned(a->A, 4) || misaligned(a->D, 4) || misaligned(a->dt_bias, 4) ||
      misaligned(a->h0, 4) || misaligned(a->last_state, 4) || misaligned(a->workspace, 4))
    return SSM_ERR_ALIGN;
  const Span sh0 = span1(a->h0, Bt * H * P * N, 4);
  const Span inputs[] = {
      span4(a->x, Bt, a->x_batch_stride, L, a->x_seq_stride, H, a->x_head_stride, P, esz),
      span3(a->dt, Bt, a->dt_batch_stride, L, a->dt_seq_stride, H, esz),
      span4(a->z, Bt, a->z_batch_stride, L, a->z_seq_stride, H, a->z_head_stride, P, esz),
      span4(a->B, Bt, a->B_batch_stride, L, a->B_seq_stride, G, a->B_group_stride, N, esz),
      span4(a->C, Bt, a->C_batch_stride, L, a->C_seq_stride, G, a->C_group_stride, N, esz),
      span1(a->A, H, 4), span1(a->D, H, 4), span1(a->dt_bias, H, 4), sh0};
  const Span sout = span4(a->out, Bt, a->out_batch_stride, L, a->out_seq_stride, H,
                          a->out_head_stride, P, esz);
  const Span slast = span1(a->last_state, Bt * H * P * N, 4);
  const Span sws = span1(a->workspace, static_cast<int64_t>(a->workspace_bytes), 1);
  for (const Span& i : inputs) {
    if (overlap(sout, i) || overlap(sws, i)) return SSM_ERR_ALIAS;
    if (&i == &inputs[8] && a->last_state == a->h0) continue;
    if (overlap(slast, i)) return SSM_ERR_ALIAS;
  }
  if (overlap(sout, slast) || overlap(sws, sout) || overlap(sws, slast)) return SSM_ERR_ALIAS;
  return SSM_OK;
}

int ssm_selective_scan_fwd(const ssm_scan_args* a, void* stream) {
  const int st = ssm_validate_scan(a);
  if (st != SSM_OK) return st;
  if (a->batch == 0 || a->dim == 0) return SSM_OK;
  if (ssm::launch_scan_fwd(*a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SSM_ERR_HIP;
  return SSM_OK;
}

int ssm_selective_scan_fwd_noalloc(const ssm_scan_args* a, void* stream) {
  if (!a) return SSM_ERR_NULL;
  // the caller's workspace is not used: validate without it
  ssm_scan_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  const int st = ssm_validate_scan(&b);
  if (st != SSM_OK) return st;
  if (b.batch == 0 || b.dim == 0) return SSM_OK;
  return ssm::scan_fwd_noalloc(b, static_cast<hipStream_t>(stream));
}

int ssm_selective_scan_bwd(const ssm_scan_bwd_args* a, void* stream) {
  const int st = ssm_validate_scan_bwd(a);
  if (st != SSM_OK) return st;
  if (a->batch == 0 || a->dim == 0) return SSM_OK;
  if (ssm::launch_scan_bwd(*a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SSM_ERR_HIP;
  return SSM_OK;
}

int ssm_ssd_scan_fwd(const ssm_ssd_args* a, void* stream) {
  const int st = ssm_validate_ssd(a);
  if (st != SSM_OK) return st;
  if (a->batch == 0) return SSM_OK;
  if (ssm::launch_ssd_fwd(*a, static_cast<hipStream_t>(stream)) != hipSuccess) return SSM_ERR_HIP;
  return SSM_OK;
}

int ssm_selective_state_update(const ssm_update_args* a, void* stream) {
  const int st = ssm_validate_update(a);
  if (st != SSM_OK) return st;
  if (a->batch == 0 || a->dim == 0) return SSM_OK;
  if (ssm::launch_state_update(*a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SSM_ERR_HIP;
  return SSM_OK;
}

}  // extern "C"

// scan_fwd_kernel.h -- the prefill selective-scan kernel for gfx950, as a
// template instantiated by scan_fwd_s1/s2/s4.hip (one translation unit per
// number of states a lane holds, so that the variants compile in parallel).
//
// Computes, per batch row b, channel d and state n (Mamba model notes sections
// 2.2, 4.1 and 4.4; Mamba paper notes section 2.3 for the discretisation):
//   Delta_t = softplus(delta_t + bias[d])
//   h_t[n]  = exp(Delta_t A[d,n]) h_{t-1}[n] + Delta_t B[b,g,n,t] u_t
//   out_t   = (sum_n C[b,g,n,t] h_t[n] + D[d] u_t) * silu(z_t)
// with g the B/C group of channel d (one group: B and C shared by every
// channel of the batch row).
//
// Work decomposition.  A workgroup is 4 wavefronts; a wavefront is 4
// channels of one batch row, each a 16-lane row whose lane c holds the fp32
// states n = c, c + 16, ... (S of them, S = 1, 2 or 4 for up to 16, 32 or 64
// states; states past dstate are padding that stays exactly zero) in
// registers for the whole sequence.  The workgroup walks its token range in
// blocks of 16:
//   owner role  lane (row r, col j) loads u/delta/z of token t0+j of channel r
//               and computes Delta and Delta*u once; a DPP row_newbcast:j
//               inside the consuming VALU op hands them to the 16 state lanes
//               of the same row.
//   B/C         shared mode (all 16 channels of the workgroup in one group):
//               every 2 blocks the workgroup loads the next 16S x 32 tile of
//               B and of C (one state row per 16 lanes, coalesced) into a
//               double-buffered LDS tile and synchronises once; every lane
//               then reads back its states' rows for each block.
//               lane mode (groups smaller than a workgroup, down to one
//               channel per group): each lane loads the 16 tokens of its own
//               group's rows for each block straight from memory (16-byte
//               loads when the rows are aligned); no LDS tile and no barrier.
//   readout     each state lane leaves sum_s C_n h_n per token in its
//               wavefront's LDS; one block later the owner of the token sums
//               the 16 partials, adds D*u, applies the gate and stores.
// Apart from the B/C tile, LDS is private to a wavefront, whose LDS operations
// complete in issue order, so the per-block exchange needs no barrier.  Every
// global access goes through a buffer descriptor whose window ends where the
// wavefront's data ends: lanes of a partial last block that reach past it
// read zero instead of touching memory, so no lane clamps its address; the
// B/C rows of padding states and the checkpoint stores of padding states
// start at the window's end and read zero / are dropped the same way (the
// host keeps every window 256 bytes short of 4 GiB, so these offsets plus a
// block's reach never wrap).
//
// Long sequences with few channels.  The recurrence is linear in the state
// (Mamba paper notes, sections 5.3/5.4: a long input can be cut into chunks
// with the state handed from one chunk to the next), so the sequence may be
// cut into G segments processed by different workgroups:
//   pass 1  every segment runs the full scan (outputs, checkpoints) from a
//           zero state (segment 0 from h0) and records its end state b_g and
//           the sum of its step sizes S_g, and, at the start of each window
//           of its head (below), its state and the step sizes summed so far;
//   plan    (scan_fwd.hip) the exact state entering segment g >= 1,
//           h_in = fold_{i<g} (exp(A S_i) h + b_i), with the associative
//           combine (a1,b1).(a2,b2) = (a1 a2, a2 b1 + b2) kept in factored
//           form; the exact state at each window start; and, per channel,
//           the windows still to rescan;
//   pass 2  one workgroup per 16 channels (of one B/C group) and window
//           rescans the window from its exact start state, rewriting
//           outputs and checkpoints, only while the incoming state's
//           contribution still counts.
// Pass 1's state inside segment g differs from the exact one by
// d_t = exp(A (S_0 + ... + S_t)) h_in (the free response of h_in), so once
// |d_t| falls below fp32 resolution of the state (2^-24 max_n |h_t[n]|, over
// each channel's states) pass 1's values are the sequential result up to
// rounding.  With A < 0 the contribution decays: a channel's windows end at
// the first window start where it holds, and a workgroup stops inside its
// window once it holds for all 16 of its channels (checked every 64 tokens).
// With A >= 0 it never decays and the whole segment is rescanned.  Windows
// start 0, 528, 1040, 2064, ... tokens into a segment (win_blk), short at the
// head where most channels drop out and longer behind it, so that both the
// rescanned tokens and the longest window stay small; channels that need
// the same window are gathered across the B/C group, so one slow channel
// does not hold fifteen converged ones.
#pragma once

#include <algorithm>

#include "ssm_internal.h"

namespace ssm {
namespace fwd {

constexpr int kN = 16;              // lanes per channel row (states per slot)
constexpr int kRows = 4;            // channels per wavefront
constexpr int kWaves = 4;           // wavefronts per workgroup
constexpr int kCh = kRows * kWaves; // channels per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kT = 16;              // tokens per block
constexpr int kGB = 2;              // blocks per B/C staging group
constexpr int kGT = kT * kGB;       // tokens per group
static_assert(4 % kGB == 0, "the steady-state loop runs four blocks at a time");
constexpr int kGPitch = kGT + 4;    // LDS pitch (floats) of one state's group of B / C
constexpr int kPitch = 20;          // LDS pitch (floats) of one state's readout partials
constexpr int kCPitch = kN + 4;     // LDS pitch (floats) of one token's C (token-major tile)
constexpr int kPartRow = kN * kPitch + 16;  // floats per channel of readout partials

// Segmented scan: the windows of a segment's head that pass 2 rescans.
// Window j starts win_blk(j) blocks into the segment, at the top of a
// steady-state round (1 mod 4 blocks), where pass 1 records its state; it
// ends where the next window present starts, the last one present at the
// segment's end.  Window j >= 1 is present when pass 1 runs that round:
// win_blk(j) + 4 <= the segment's full blocks.
constexpr int kWin = 10;
__host__ __device__ constexpr int win_blk(int j) {
  return j <= 0 ? 0 : j == 1 ? 33 : j == 2 ? 65 : j == 3 ? 129 : j == 4 ? 257
       : j == 5 ? 385 : j == 6 ? 513 : j == 7 ? 769 : j == 8 ? 1025 : 1537;
}
__host__ __device__ constexpr int seg_windows(int nfull) {
  int n = 1;
  while (n < kWin && win_blk(n) + 4 <= nfull) ++n;
  return n;
}

// kScan: one segment per sequence.  kSeg, kFix: passes 1 and 2 of a
// segmented sequence.
enum class Mode { kScan, kSeg, kFix };

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
  // segmented scan (nseg > 1)
  float* agg;      // [batch * dim][nseg][N + 1] segment end states and step-size sums
  float* rec;      // [nseg][kWin][batch * dim][N + 1] window start states and step sums
  const int* counts;  // [batch][nseg][kWin][dim] channels to rescan, at each chunk's first
  const int* lists;   // the same shape: those channels, ascending, from the chunk's first
  float* ckpt;     // [batch][dim][nbk][N] states entering each block, or NULL
  const float* conv_w;      // [dim][K] conv weights (the conv path only)
  const float* conv_b;      // [dim] or NULL
  const float* conv_in;     // [batch][dim][K] inputs before the sequence, or NULL
  float* conv_stout;        // [batch][dim][K] last K inputs, or NULL
  void* conv_out;           // (batch, dim, L) SSM input u, or NULL
  int64_t usb, usd, dsb, dsd, zsb, zsd, Bsb, Bsg, Bsn, Csb, Csg, Csn, Asd, Asn, osb, osd,
      cosb, cosd;
  int K;                    // conv width
  int conv_silu;
  int N;                    // states per channel (dstate)
  int64_t cpg;              // channels per B/C group
  int64_t batch, dim;
  int L;
  int seg_len;     // tokens per segment (multiple of kGT)
  int nseg;        // segments per sequence
  int nbk;         // blocks per sequence, ceil(L / kT)
  int64_t cgroups; // ceil(dim / kCh)
  int64_t scope;   // pass 2: channels per B/C scope, the group (shared tile) or dim
  int64_t cw;      // pass 2: channels per chunk (a scope is cut into chunks of cw)
  int64_t nchunk;  // pass 2: chunks per batch row
  int maxi;        // pass 2: workgroups per chunk and window, ceil(cw / 16)
};

// Owner role raw inputs of one block: token t0 + col of the lane's channel
// (bit patterns, widened where they are used); with the conv path, u holds
// the conv input x.
struct Raw {
  uint32_t u, dt, z;
};

// Shared mode, stage role raw inputs of one group: B and C of states
// 4w + row + 16s at tokens tg + col + 16i.
template <int S>
struct GroupRaw {
  uint32_t b[S][kGB], c[S][kGB];
};

// Lane (J - m) mod 16 of the 16-lane row (DPP row_ror:m).
template <int M>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 + M, 0xf, 0xf, true));
}

template <typename T, Mode M, bool kSoftplus, int KP, int S, int kLane, bool kDefer>
struct Wave {
  const ScanParams& p;
  int wave, row, col;
  int t_beg, t_end, nblk, ngrp;
  Window wu, wdt, wz, wB, wC, wout, wck;
  uint32_t ou, odt, oz, oout;       // per-lane byte offsets inside the windows
  // per state slot; B/C offsets of padding states (n >= dstate) point past
  // their window, so those loads read zero
  uint32_t oB[S], oC[S], ock[S];
  uint32_t ckstep;    // checkpoint bytes per block of a channel row (0: none kept)
  int blk0;           // global index of this segment's first block
  float a2[S], bias, Dd;
  // conv path (KP > 0: the width padded to KP): tap weights by lag m,
  // wl[m] multiplies x_{t-m} (zero past the real width), and the bias
  float wl[KP > 0 ? KP : 1], cb;
  bool silu_in;
  Window wco;                 // conv_out window (empty when not wanted)
  uint32_t oco;
  float (*sB)[kN * S][kGPitch];   // [2][16S][kGPitch], shared by the workgroup
  float (*sC)[kN * S][kGPitch];
  float (*sCt)[kGT][kCPitch];     // [2][kGT][kCPitch] token-major C (kOwnerC)
  float (*sP)[kPartRow];          // this wavefront's [kRows][kPartRow]

  static constexpr int E = Elem<T>::kSize;
  // One state slot with the shared tile: the state lanes hand their h to
  // LDS and the owner of each token contracts it with the token's C column
  // (16 FMAs in place of 16 products on the state lanes and a 15-add sum);
  // C is then staged token-major.
  static constexpr bool kOwnerC = S == 1 && !kLane;
  static constexpr bool kSegm = M != Mode::kScan;
  static constexpr bool kFixp = M == Mode::kFix;
  // token of the scan after which the owner's C column is read, so that the
  // read is in flight during the rest of the scan: at the top of the block
  // in the compact one-segment form (its 84 registers still leave five
  // wavefronts per SIMD), after token 7 where registers are tight (the
  // segmented passes at 96) or the read is carried over (deferred form)
  static constexpr int kCRead = (M == Mode::kScan && !kDefer) ? 0 : 7;
  // Owner-C readout deferred to the top of the next block (kDefer): the
  // block's states are read back from LDS there and contracted after the
  // next block's owner work, which covers the LDS round trip; the C column
  // is carried in registers across the block boundary.  Costs about 30
  // VGPRs (128), so it is launched only where the grid leaves three
  // wavefronts per SIMD anyway.
  static_assert(!kDefer || (kOwnerC && !kSegm),
                "the deferred readout is an owner-C form of the one-segment scan");

  __device__ __forceinline__ uint32_t skip(int k) const {
    return static_cast<uint32_t>(t_beg + k * kT) * E;
  }

  // Pass 2 of a segmented sequence: has the free response of the incoming
  // state, |h_in[n]| exp(A[n] S) with S the step sizes of the tokens done so
  // far, fallen to 2^-24 max_n |h[n]| or below in every channel of the
  // workgroup?  (ssum: this owner's share of S; a non-finite state or
  // h_in never compares true.)  Every wavefront of the workgroup calls it
  // at the same point: it ends with a workgroup barrier.
  __device__ __forceinline__ bool converged(const float (&h)[S], const float (&hin)[S],
                                            double ssum) const {
    float sacc = static_cast<float>(ssum);
    float hm = 0.0f;
#pragma unroll
    for (int q = 0; q < S; ++q) hm = fmaxf(hm, fabsf(h[q]));
#pragma unroll
    for (int m = 1; m < kN; m <<= 1) {
      sacc += __shfl_xor(sacc, m, kN);
      hm = fmaxf(hm, __shfl_xor(hm, m, kN));
    }
    bool ok = true;
#pragma unroll
    for (int q = 0; q < S; ++q)
      ok = ok && __builtin_amdgcn_exp2f(a2[q] * sacc) * hin[q] <= 0x1p-24f * hm;
    return __syncthreads_and(ok) != 0;
  }

  // Owner raw inputs of block k; blocks past the last one reload the last one
  // (the pipeline prefetches two blocks ahead and never uses those).
  __device__ __forceinline__ Raw load(int k) const {
    Raw r;
    const uint32_t s = skip(min(k, nblk - 1));
    r.u = Elem<T>::load(wu.at(s), ou);
    r.dt = Elem<T>::load(wdt.at(s), odt);
    // without a gate the z window is u's: the load is a cache hit, never used
    r.z = Elem<T>::load(wz.at(s), oz);
    return r;
  }

  // Shared mode, stage raw inputs of group g (clamped to the last group like
  // load()).
  __device__ __forceinline__ GroupRaw<S> load_group(int g) const {
    GroupRaw<S> r;
    const uint32_t s = skip(min(g, ngrp - 1) * kGB);
    const __amdgpu_buffer_rsrc_t rb = wB.at(s);
    const __amdgpu_buffer_rsrc_t rc = wC.at(s);
#pragma unroll
    for (int q = 0; q < S; ++q) {
#pragma unroll
      for (int i = 0; i < kGB; ++i) {
        r.b[q][i] = Elem<T>::load(rb, oB[q] + i * kT * E);
        r.c[q][i] = Elem<T>::load(rc, oC[q] + i * kT * E);
      }
    }
    return r;
  }

  // Shared mode, stage role: group g's B (and C) into LDS buffer g & 1, as
  // loaded: tokens past the end hold whatever lies beyond them (the next
  // segment, or the next state's row), which bc() keeps from h in the masked
  // blocks, the only ones that reach past the end; rows of padding states
  // load as zero.
  __device__ __forceinline__ void stage(int g, const GroupRaw<S>& r) const {
    const int st = kRows * wave + row;
#pragma unroll
    for (int q = 0; q < S; ++q) {
#pragma unroll
      for (int i = 0; i < kGB; ++i) {
        sB[g & 1][st + kN * q][col + i * kT] = Elem<T>::f32(r.b[q][i]);
        if constexpr (kOwnerC) sCt[g & 1][col + i * kT][st] = Elem<T>::f32(r.c[q][i]);
        else sC[g & 1][st + kN * q][col + i * kT] = Elem<T>::f32(r.c[q][i]);
      }
    }
  }

  // B and C of state slot q for the 16 tokens of block k: from the LDS tile
  // (shared mode) or from this lane's own rows (lane mode).  In a masked
  // block B of the tokens past the end reads as zero, so that a non-finite
  // value lying beyond them cannot reach h (their step is then exactly the
  // identity: Delta and Delta u are zero there).
  template <bool kMask>
  __device__ __forceinline__ void bc(int k, int q, float (&bv)[kT], float (&cv)[kT]) const {
    if constexpr (!kLane) {
      const int buf = (k / kGB) & 1;
      const int tb = (k % kGB) * kT;
#pragma unroll
      for (int i = 0; i < kT / 4; ++i) {
        const float4 x = *reinterpret_cast<const float4*>(&sB[buf][col + kN * q][tb + 4 * i]);
        bv[4 * i] = x.x; bv[4 * i + 1] = x.y; bv[4 * i + 2] = x.z; bv[4 * i + 3] = x.w;
        if constexpr (!kOwnerC) {
          const float4 y = *reinterpret_cast<const float4*>(&sC[buf][col + kN * q][tb + 4 * i]);
          cv[4 * i] = y.x; cv[4 * i + 1] = y.y; cv[4 * i + 2] = y.z; cv[4 * i + 3] = y.w;
        }
      }
      if constexpr (kMask) {
        const int tleft = t_end - (t_beg + k * kT);
#pragma unroll
        for (int j = 0; j < kT; ++j) bv[j] = j < tleft ? bv[j] : 0.0f;
      }
    } else {
      const uint32_t s = skip(k);
      const __amdgpu_buffer_rsrc_t rb = wB.at(s);
      const __amdgpu_buffer_rsrc_t rc = wC.at(s);
      const int tleft = t_end - (t_beg + k * kT);
      if constexpr (kLane == 2) {
        // 16-byte aligned rows: the block's 16 tokens in 16-byte loads
        constexpr int kV = kT * E / 16;  // loads per tensor
        uint32_t rbw[kT * E / 4], rcw[kT * E / 4];
#pragma unroll
        for (int v = 0; v < kV; ++v) {
          const auto xb = __builtin_amdgcn_raw_buffer_load_b128(rb, oB[q] + 16 * v, 0, 0);
          const auto xc = __builtin_amdgcn_raw_buffer_load_b128(rc, oC[q] + 16 * v, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            rbw[4 * v + i] = xb[i];
            rcw[4 * v + i] = xc[i];
          }
        }
#pragma unroll
        for (int j = 0; j < kT; ++j) {
          float b, cc;
          if constexpr (E == 2) {
            b = __uint_as_float(j % 2 ? rbw[j / 2] & 0xffff0000u : rbw[j / 2] << 16);
            cc = __uint_as_float(j % 2 ? rcw[j / 2] & 0xffff0000u : rcw[j / 2] << 16);
          } else {
            b = __uint_as_float(rbw[j]);
            cc = __uint_as_float(rcw[j]);
          }
          bv[j] = !kMask || j < tleft ? b : 0.0f;
          cv[j] = cc;
        }
      } else {
#pragma unroll
        for (int j = 0; j < kT; ++j) {
          const float b = Elem<T>::f32(Elem<T>::load(rb, oB[q] + j * E));
          bv[j] = !kMask || j < tleft ? b : 0.0f;
          cv[j] = Elem<T>::f32(Elem<T>::load(rc, oC[q] + j * E));
        }
      }
    }
  }

  // Owner role: readout of block k (y = the sum of its 16 partials, uv its
  // SSM input), skip term, gate, store.  Rows past dim repeat the last channel bit for bit, so in full
  // blocks every lane may store (duplicates write identical values); with
  // kMask only tokens before the end are stored.
  template <bool kMask>
  __device__ __forceinline__ void finish(int k, const Raw& r, float uv, float y) const {
    y = fmaf(Dd, uv, y);
    const float g = silu_f32(Elem<T>::f32(r.z));
    y *= p.z ? g : 1.0f;  // a select, not a branch
    const __amdgpu_buffer_rsrc_t ro = wout.at(skip(k));
    if (!kMask || t_beg + k * kT + col < t_end) Elem<T>::store(ro, oout, y);
  }

  // Iteration k.  Buffers: P = block k-1 (finish), Q = block k (scan),
  // R = block k+2 (load target); G holds the next group's B/C.
  // kMask = false is the steady state, valid when blocks k-1 and k are full:
  // it has no branch, so the scan's DPP broadcasts stay fused into the ops
  // that use them.  kEnd (steady state only) marks the last block of a group,
  // after which the workgroup synchronises; the other blocks are first blocks
  // (two per group), after which the next group is staged.  In the masked
  // form both are decided at run time.
  // ssum: the owner's step-size sum, fp64 (masked blocks) or an fp32 sum of
  // one steady-state round's four steps that the caller adds to it.
  template <bool kMask, bool kEnd, typename Acc>
  __device__ __forceinline__ void iter(int k, float (&h)[S], Acc& ssum, const Raw& P,
                                       const Raw& Q, Raw& R, GroupRaw<S>& G, float& uprev,
                                       float& xprev, float (&cl)[kN]) const {
    // B/C of the first state slot and the previous block's partials first
    float bv[kT], cv[kT];
    bc<kMask>(k, 0, bv, cv);
    float ysum = 0.0f;
    float part[kN];
    if constexpr (!kOwnerC || kDefer) {
      // The previous block's readout inputs from this wavefront's LDS region,
      // read before this block's own stores there (a wavefront's LDS
      // operations complete in order); unconditional: at k = 0 they are never
      // used.  Without owner-C they are summed right away so that one
      // register, not sixteen, lives across the scan.
#pragma unroll
      for (int n = 0; n < kN; ++n) part[n] = sP[row][n * kPitch + col];
      if constexpr (!kOwnerC) {
#pragma unroll
        for (int n = 0; n < kN; ++n) ysum += part[n];
      }
    }
    R = load(k + 2);

    // owner role: the SSM input u of this token (through the causal conv on
    // the conv path), Delta and Delta*u (zero past the end)
    float uv;
    if constexpr (KP > 0) {
      // x_{t-m} is lane col-m of this block for m <= col, else lane col-m+16
      // of the previous one: a DPP row rotation of each and a select
      const float xc = Elem<T>::f32(Q.u);
      float pre = fmaf(wl[0], xc, cb);
      static_for<1, KP>([&](auto Mm) {
        constexpr int m = decltype(Mm)::value;
        const float xcur = row_ror<m>(xc), xold = row_ror<m>(xprev);
        pre = fmaf(wl[m], col >= m ? xcur : xold, pre);
      });
      const float act = silu_f32(pre);
      uv = silu_in ? act : pre;  // a select, not a branch
      xprev = xc;
      if (!kMask || t_beg + k * kT + col < t_end)
        Elem<T>::store(wco.at(p.conv_out ? skip(k) : 0u), oco, uv);
    } else {
      uv = Elem<T>::f32(Q.u);
    }
    const float x = Elem<T>::f32(Q.dt) + bias;
    float dl = kSoftplus ? softplus_f32(x) : x;
    float du = dl * uv;
    if (kMask) {
      const bool own = t_beg + k * kT + col < t_end;
      dl = own ? dl : 0.0f;
      du = own ? du : 0.0f;
    }
    // segmented: the step sizes of this owner's tokens, summed in fp64
    if constexpr (kSegm) ssum += static_cast<Acc>(dl);
    if constexpr (kDefer) {
      // the previous block's readout: its states (read above) against its
      // token's C column (read during its scan), after this block's owner
      // work so that the LDS reads above are not waited on right away
#pragma unroll
      for (int n = 0; n < kN; ++n) ysum = fmaf(cl[n], part[n], ysum);
    }

    // checkpoint: the states entering this block (an empty window when none
    // are kept, and an offset past the window for padding slots, so the
    // stores are dropped without a branch)
#pragma unroll
    for (int q = 0; q < S; ++q) Elem<float>::store(wck.at((blk0 + k) * ckstep), ock[q], h[q]);

    // state role: 16 sequential steps of each state slot; the readout
    // partials sum_q C_n h_n go to LDS four tokens at a time after the last
    // slot
    // one slot: a rolling 4-register buffer; several: one sum per token
    float pk[S == 1 ? 4 : kT];
    static_for<0, S>([&](auto Qs) {
      constexpr int q = decltype(Qs)::value;
      if constexpr (q > 0) {
        // compiler-only fence: one slot's B/C live at a time, not all S
        asm volatile("" ::: "memory");
        bc<kMask>(k, q, bv, cv);
      }
      static_for<0, kT>([&](auto J) {
        constexpr int j = decltype(J)::value;
        const float e = __builtin_amdgcn_exp2f(row_bcast<j>(dl) * a2[q]);  // Abar = exp(Delta A)
        const float w = row_bcast<j>(du) * bv[j];                          // Bbar u = Delta u B
        h[q] = fmaf(e, h[q], w);
        {
          constexpr int i = S == 1 ? j % 4 : j;
          if constexpr (kOwnerC) pk[i] = h[q];                               // h_n
          else pk[i] = q == 0 ? cv[j] * h[q] : fmaf(cv[j], h[q], pk[i]);   // C_n h_n
          if constexpr (q == S - 1 && j % 4 == 3)
            *reinterpret_cast<float4*>(&sP[row][col * kPitch + j - 3]) =
                make_float4(pk[i - 3], pk[i - 2], pk[i - 1], pk[i]);
        }
        if constexpr (kOwnerC && j == kCRead) {
          const float* cc = &sCt[(k / kGB) & 1][(k % kGB) * kT + col][0];
#pragma unroll
          for (int ii = 0; ii < kN / 4; ++ii) {
            const float4 c4 = *reinterpret_cast<const float4*>(cc + 4 * ii);
            cl[4 * ii] = c4.x; cl[4 * ii + 1] = c4.y; cl[4 * ii + 2] = c4.z; cl[4 * ii + 3] = c4.w;
          }
        }
      });
    });
    if constexpr (kOwnerC && !kDefer) {
      // this block's readout right away: y = sum_n C_n h_n from the h the
      // state lanes just left in LDS and this token's C column of the tile
      // (read during the scan; still this group's buffer: the other one is
      // staged next)
#pragma unroll
      for (int n = 0; n < kN; ++n) part[n] = sP[row][n * kPitch + col];
#pragma unroll
      for (int n = 0; n < kN; ++n) ysum = fmaf(cl[n], part[n], ysum);
      finish<kMask>(k, Q, uv, ysum);
    } else {
      if (!kMask) finish<false>(k - 1, P, uprev, ysum);
      else if (k > 0) finish<true>(k - 1, P, uprev, ysum);
    }
    uprev = uv;
    // Compiler-only fence: keep this block's LDS traffic in program order with
    // the next block's (the hardware already keeps one wavefront's in order).
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    if constexpr (!kLane) {
      // Group g + 1 goes into the other buffer at the end of group g's first
      // block: that buffer held group g - 1, which every wavefront finished
      // reading before the barrier that closed group g - 1.  The barrier at
      // the end of group g's last block orders these stores before group
      // g + 1's reads; issued a block earlier, they no longer hold it up.
      static_assert(kGB == 2, "each block is the first or the last of its group");
      const bool first = kMask ? (k % kGB == 0) : !kEnd;
      const bool last = kMask ? (k % kGB == kGB - 1) : kEnd;
      const int g = k / kGB + 1;
      // (the steady state may stage one group past the end: clamped data into
      // a buffer that nothing reads again)
      if (kMask ? first && g < ngrp : first) {
        stage(g, G);
        G = load_group(g + 1);
      }
      if (last && k + 1 < nblk) __syncthreads();
    }
  }
};

template <typename T, Mode M, bool kSoftplus, int KP, int S, int kLane, bool kDefer>
__global__ __launch_bounds__(kThreads) void scan_fwd_kernel(ScanParams p) {
  constexpr int kTile = kLane ? 1 : 2;
  __shared__ __align__(16) float sB[kTile][kN * S][kGPitch];
  using W = Wave<T, M, kSoftplus, KP, S, kLane, kDefer>;
  constexpr bool kOC = W::kOwnerC;
  constexpr bool kSegm = W::kSegm;
  __shared__ __align__(16) float sC[!kOC ? kTile : 1][kN * S][kGPitch];
  __shared__ __align__(16) float sCt[kOC ? 2 : 1][kOC ? kGT : 1][kCPitch];
  __shared__ __align__(16) float sP[kWaves][kRows][kPartRow];

  // wavefront index, made visibly uniform so that windows stay in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = (threadIdx.x >> 4) & 3;
  const int col = threadIdx.x & 15;
  // Logical workgroup (XCD-aware order, ssm_internal.h), segment-major: one
  // XCD runs every channel group of a few segments.  Those workgroups start
  // together and walk the same tokens at about the same pace, so each line of
  // a segment's B/C tile is fetched into that XCD's L2 once and read there by
  // all of them; in channel-major order every XCD streamed the B/C of all
  // segments once per channel group it held (at 1M tokens, 1.5x the input
  // bytes read instead of 1.1x).
  constexpr bool fix = W::kFixp;
  const int N = p.N;
  const int aggs = N + 1;  // floats per aggregate and per window record: h[N], S
  const int64_t BD = p.batch * p.dim;
  int g, jw = 0, t_beg, t_end;
  int64_t b, d, dc, dw0, dw3, grp_tile;
  bool vrow;
  if constexpr (!fix) {
    // wg = g * (batch * cgroups) + b * cgroups + cg: 16 consecutive
    // channels, one segment
    const uint32_t wg = xcd_order(blockIdx.x, gridDim.x);
    const int64_t ncg = p.batch * p.cgroups;
    g = static_cast<int>(wg / ncg);
    const int64_t bc = wg % ncg;
    b = bc / p.cgroups;
    const int64_t cg0 = (bc % p.cgroups) * kCh;
    d = cg0 + kRows * wave + row;
    vrow = d < p.dim;
    // rows past dim repeat the last channel exactly (same inputs, same state)
    dc = vrow ? d : p.dim - 1;
    // this wavefront's first and last (clamped) rows
    dw0 = std::min<int64_t>(cg0 + kRows * wave, p.dim - 1);
    dw3 = std::min<int64_t>(dw0 + kRows - 1, p.dim - 1);
    grp_tile = cg0 / p.cpg;
    t_beg = g * p.seg_len;
    t_end = std::min(p.L, t_beg + p.seg_len);
  } else {
    // Pass 2: wg = (((j' * batch + b) * nchunk + chunk) * (nseg - 1) + g - 1)
    // * maxi + i, the i-th 16 channels of the list of window j = kWin-1-j'
    // of segment g in one chunk of a batch row (windows outermost, the
    // longest first, so that they do not trail the launch).  Entries past
    // the list repeat its last channel (identical values, identical
    // stores); a wavefront's windows run from the smallest to the largest
    // channel of its rows, all in one chunk.  The workgroup index is taken
    // as is, not in XCD order: the windows hold very different amounts of
    // work (most list slots of the later windows are empty), and the
    // dispatcher's round robin spreads each window over all XCDs, where
    // contiguous ranges per XCD would give one XCD the later windows and
    // another the dense first ones.
    uint32_t wg = blockIdx.x;
    const int i = static_cast<int>(wg % static_cast<uint32_t>(p.maxi));
    wg /= static_cast<uint32_t>(p.maxi);
    g = static_cast<int>(wg % static_cast<uint32_t>(p.nseg - 1)) + 1;
    wg /= static_cast<uint32_t>(p.nseg - 1);
    const int64_t chunk = wg % p.nchunk;
    const int64_t wr = wg / p.nchunk;
    b = wr % p.batch;
    jw = kWin - 1 - static_cast<int>(wr / p.batch);
    const int s0 = g * p.seg_len;
    const int send = std::min(p.L, s0 + p.seg_len);
    const int nwin = seg_windows((send - s0) / kT);
    if (jw >= nwin) return;
    const int64_t cps = (p.scope + p.cw - 1) / p.cw;  // chunks per scope
    const int64_t c0 = (chunk / cps) * p.scope + (chunk % cps) * p.cw;
    const int64_t key = ((b * p.nseg + g) * kWin + jw) * p.dim + c0;
    const int cnt = __builtin_amdgcn_readfirstlane(p.counts[key]);
    if (i * kCh >= cnt) return;
    const int ch = p.lists[key + std::min(i * kCh + kRows * wave + row, cnt - 1)];
    const int ch0 = __builtin_amdgcn_readlane(ch, 0), ch1 = __builtin_amdgcn_readlane(ch, 16);
    const int ch2 = __builtin_amdgcn_readlane(ch, 32), ch3 = __builtin_amdgcn_readlane(ch, 48);
    dw0 = std::min(std::min(ch0, ch1), std::min(ch2, ch3));
    dw3 = std::max(std::max(ch0, ch1), std::max(ch2, ch3));
    dc = ch;
    d = dc;
    vrow = true;
    // shared tile: a chunk never straddles a group
    grp_tile = dw0 / p.cpg;
    t_beg = s0 + kT * win_blk(jw);
    t_end = jw + 1 < nwin ? s0 + kT * win_blk(jw + 1) : send;
  }

  constexpr int E = Elem<T>::kSize;
  W w{p};
  w.wave = wave; w.row = row; w.col = col;
  w.t_beg = t_beg;
  w.t_end = t_end;
  w.nblk = (w.t_end - w.t_beg + kT - 1) / kT;
  w.ngrp = (w.nblk + kGB - 1) / kGB;

  // Windows run from this wavefront's first row to the end of its last row.
  auto rows_window = [&](const void* base, int64_t sb, int64_t sd, uint32_t& off) {
    off = static_cast<uint32_t>(((dc - dw0) * sd + col) * E);
    return Window{static_cast<const char*>(base) + (b * sb + dw0 * sd) * E,
                  static_cast<uint32_t>(((dw3 - dw0) * sd + p.L) * E)};
  };
  w.wu = rows_window(p.u, p.usb, p.usd, w.ou);
  w.wdt = rows_window(p.delta, p.dsb, p.dsd, w.odt);
  if (p.z) {
    w.wz = rows_window(p.z, p.zsb, p.zsd, w.oz);
  } else {
    w.wz = w.wu;
    w.oz = w.ou;
  }
  w.wout = rows_window(p.out, p.osb, p.osd, w.oout);
  // checkpoints: rows of nbk * N floats, [b][d][block][n]
  const int64_t ckrow = static_cast<int64_t>(p.nbk) * N;
  w.blk0 = w.t_beg / kT;
  w.ckstep = p.ckpt ? N * 4 : 0;
  w.wck = Window{reinterpret_cast<const char*>(p.ckpt ? p.ckpt + (b * p.dim + dw0) * ckrow : nullptr),
                 p.ckpt ? static_cast<uint32_t>((dw3 - dw0 + 1) * ckrow * 4) : 0u};
#pragma unroll
  for (int q = 0; q < S; ++q) {
    const int n = col + kN * q;
    w.ock[q] = n < N ? static_cast<uint32_t>(((dc - dw0) * ckrow + n) * 4) : w.wck.bytes;
  }
  if constexpr (!kLane) {
    // B/C: the workgroup's group; this lane stages states 4 wave + row + 16q
    // of tokens col, col + 16 of each staging group
    const int st = kRows * wave + row;
    w.wB = Window{static_cast<const char*>(p.B) + (b * p.Bsb + grp_tile * p.Bsg) * E,
                  static_cast<uint32_t>(((N - 1) * p.Bsn + p.L) * E)};
    w.wC = Window{static_cast<const char*>(p.C) + (b * p.Csb + grp_tile * p.Csg) * E,
                  static_cast<uint32_t>(((N - 1) * p.Csn + p.L) * E)};
#pragma unroll
    for (int q = 0; q < S; ++q) {
      const int n = st + kN * q;
      w.oB[q] = n < N ? static_cast<uint32_t>((n * p.Bsn + col) * E) : w.wB.bytes;
      w.oC[q] = n < N ? static_cast<uint32_t>((n * p.Csn + col) * E) : w.wC.bytes;
    }
  } else {
    // B/C: this lane reads its own states' rows in its channel's group; the
    // window spans the groups of the wavefront's four rows
    const int64_t g0 = dw0 / p.cpg, g3 = dw3 / p.cpg, gl = dc / p.cpg;
    w.wB = Window{static_cast<const char*>(p.B) + (b * p.Bsb + g0 * p.Bsg) * E,
                  static_cast<uint32_t>(((g3 - g0) * p.Bsg + (N - 1) * p.Bsn + p.L) * E)};
    w.wC = Window{static_cast<const char*>(p.C) + (b * p.Csb + g0 * p.Csg) * E,
                  static_cast<uint32_t>(((g3 - g0) * p.Csg + (N - 1) * p.Csn + p.L) * E)};
#pragma unroll
    for (int q = 0; q < S; ++q) {
      const int n = col + kN * q;
      w.oB[q] = n < N ? static_cast<uint32_t>(((gl - g0) * p.Bsg + n * p.Bsn) * E) : w.wB.bytes;
      w.oC[q] = n < N ? static_cast<uint32_t>(((gl - g0) * p.Csg + n * p.Csn) * E) : w.wC.bytes;
    }
  }

#pragma unroll
  for (int q = 0; q < S; ++q) {
    const int n = col + kN * q;
    w.a2[q] = n < N ? p.A[dc * p.Asd + n * p.Asn] * kLog2e : 0.0f;
  }
  w.bias = p.bias ? p.bias[dc] : 0.0f;
  w.Dd = p.D ? p.D[dc] : 0.0f;
  w.sB = sB; w.sC = sC; w.sP = sP[wave];
  w.sCt = reinterpret_cast<float (*)[kGT][kCPitch]>(&sCt[0][0][0]);

  // conv path: tap weights by lag, bias, the inputs just before this
  // segment (x_{t_beg-16+col}: from the conv state at the sequence start,
  // else from x itself), and the conv_out window
  float xprev = 0.0f;
  if constexpr (KP > 0) {
    const int K = p.K;
#pragma unroll
    for (int m = 0; m < KP; ++m) w.wl[m] = m < K ? p.conv_w[dc * K + (K - 1 - m)] : 0.0f;
    w.cb = p.conv_b ? p.conv_b[dc] : 0.0f;
    w.silu_in = p.conv_silu != 0;
    if (w.t_beg == 0) {
      const int t = col - kT;  // token index before the sequence, -16 .. -1
      xprev = (p.conv_in && t >= -K) ? p.conv_in[(b * p.dim + dc) * K + K + t] : 0.0f;
    } else {
      xprev = Elem<T>::f32(Elem<T>::load(w.wu.at(static_cast<uint32_t>(w.t_beg - kT) * E), w.ou));
    }
    if (p.conv_out) {
      w.wco = rows_window(p.conv_out, p.cosb, p.cosd, w.oco);
    } else {
      w.wco = Window{nullptr, 0u};
      w.oco = 0;
    }
  }
  float uprev = 0.0f;

  // Initial state: h0 (or zero) for the one segment of kScan and for segment
  // 0 of pass 1; zero for the other segments of pass 1; in pass 2, the
  // window's exact start state (written by the plan), and hin, the size of
  // the incoming state's free response there, |h_in| exp(A S) with S the
  // step sizes before the window (slot 0 holds h_in itself, with S = 0).
  float h[S], hin[S];
  const size_t arow = static_cast<size_t>(b * p.dim + dc) * p.nseg;  // aggregates of this channel
#pragma unroll
  for (int q = 0; q < S; ++q) {
    const int n = col + kN * q;
    h[q] = 0.0f;
    hin[q] = 0.0f;
    if (n < N) {
      if constexpr (!fix) {
        if (g == 0 && p.h0) h[q] = p.h0[(b * p.dim + dc) * N + n];
      } else {
        const size_t c = static_cast<size_t>(b * p.dim + dc);
        const float* rs = p.rec + ((static_cast<size_t>(g) * kWin + jw) * BD + c) * aggs;
        const float* r0 = p.rec + (static_cast<size_t>(g) * kWin * BD + c) * aggs;
        h[q] = rs[n];
        hin[q] = fabsf(r0[n]) * __builtin_amdgcn_exp2f(w.a2[q] * rs[N]);
      }
    }
  }

  double ssum = 0.0;
  // group 0 staged before the loop, group 1 in flight; block j's owner inputs
  // live in buffer j % 4 and iteration k loads block k + 2
  GroupRaw<S> grp;
  if constexpr (!kLane) grp = w.load_group(0);
  Raw buf0 = w.load(0), buf1 = w.load(1), buf2 = buf0, buf3 = buf0;
  if constexpr (!kLane) {
    w.stage(0, grp);
    grp = w.load_group(1);
    __syncthreads();
  }

  // Steady state: iterations 1 .. nfull-1 (blocks k-1 and k full), four at a
  // time so that buffer j % 4 is a fixed set of registers; a group ends at
  // k % kGB == kGB - 1.  The first iteration and the last few take the masked
  // form.  Pass 2 checks at the top of each four-block round whether it can
  // stop (block k - 1 is then the last one done).
  const int nblk = w.nblk;
  const int nfull = (w.t_end - w.t_beg) / kT;
  // owner-C: the C column of each block's token, read during the block's scan
  // (deferred form: used in the next block's readout)
  float cl[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n) cl[n] = 0.0f;
  w.template iter<true, false>(0, h, ssum, buf3, buf0, buf2, grp, uprev, xprev, cl);
  int k = 1;
  bool done = false;
  // pass 1: the next window start to record (segment 0 needs none)
  int rj = 1, rblk = g > 0 ? win_blk(1) : 0x7fffffff;
  for (; k + 4 <= nfull; k += 4) {
    if constexpr (fix) {
      if (w.converged(h, hin, ssum)) {
        done = true;
        break;
      }
    }
    if constexpr (M == Mode::kSeg) {
      if (k == rblk) {
        // window rj starts at block k: the state entering it and the step
        // sizes before it (this channel's 16 owner sums added up)
        double sk = ssum;
#pragma unroll
        for (int m = 1; m < kN; m <<= 1) sk += __shfl_xor(sk, m, kN);
        if (vrow) {
          float* rs = p.rec + ((static_cast<size_t>(g) * kWin + rj) * BD + b * p.dim + d) * aggs;
#pragma unroll
          for (int q = 0; q < S; ++q) {
            const int n = col + kN * q;
            if (n < N) rs[n] = h[q];
          }
          if (col == 0) rs[N] = static_cast<float>(sk);
        }
        ++rj;
        rblk = rj < kWin ? win_blk(rj) : 0x7fffffff;
      }
    }
    // k % 4 == 1 here, and 4 is a multiple of kGB; the round's four step
    // sizes are summed in fp32 and then added to the fp64 sum
    float sq = 0.0f;
    w.template iter<false, (1 % kGB == kGB - 1)>(k + 0, h, sq, buf0, buf1, buf3, grp, uprev, xprev, cl);
    w.template iter<false, (2 % kGB == kGB - 1)>(k + 1, h, sq, buf1, buf2, buf0, grp, uprev, xprev, cl);
    w.template iter<false, (3 % kGB == kGB - 1)>(k + 2, h, sq, buf2, buf3, buf1, grp, uprev, xprev, cl);
    w.template iter<false, (4 % kGB == kGB - 1)>(k + 3, h, sq, buf3, buf0, buf2, grp, uprev, xprev, cl);
    if constexpr (kSegm) ssum += static_cast<double>(sq);
  }
  if (!done) {
    if (k < nblk) w.template iter<true, false>(k, h, ssum, buf0, buf1, buf3, grp, uprev, xprev, cl);
    if (k + 1 < nblk) w.template iter<true, false>(k + 1, h, ssum, buf1, buf2, buf0, grp, uprev, xprev, cl);
    if (k + 2 < nblk) w.template iter<true, false>(k + 2, h, ssum, buf2, buf3, buf1, grp, uprev, xprev, cl);
    if (k + 3 < nblk) w.template iter<true, false>(k + 3, h, ssum, buf3, buf0, buf2, grp, uprev, xprev, cl);
  }

  if constexpr (!kOC || kDefer) {
    // finish the last block done: its partials (owner-C: states) are in LDS,
    // its raw inputs in buffer kl % 4 (block k - 1 after an early stop:
    // buffer 0)
    const int kl = done ? k - 1 : nblk - 1;
    const int r = kl & 3;
    const Raw last = r == 0 ? buf0 : r == 1 ? buf1 : r == 2 ? buf2 : buf3;
    float ysum = 0.0f;
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      const float v = w.sP[row][n * kPitch + col];
      ysum = kOC ? fmaf(cl[n], v, ysum) : ysum + v;
    }
    w.template finish<true>(kl, last, uprev, ysum);
  }
  if constexpr (fix) return;
  if (vrow && p.last_state && !kSegm) {
#pragma unroll
    for (int q = 0; q < S; ++q) {
      const int n = col + kN * q;
      if (n < N) p.last_state[(b * p.dim + d) * N + n] = h[q];
    }
  }
  if constexpr (KP > 0) {
    // the last K inputs, for the decode update to continue from
    const int K = p.K;
    if (vrow && p.conv_stout && g == p.nseg - 1 && col < K) {
      const int t = p.L - K + col;
      float v;
      if (t >= 0) {
        const uint32_t orow = w.ou - static_cast<uint32_t>(col * E);
        v = Elem<T>::f32(Elem<T>::load(w.wu.at(0), orow + static_cast<uint32_t>(t * E)));
      } else {
        v = p.conv_in ? p.conv_in[(b * p.dim + d) * K + K + t] : 0.0f;
      }
      p.conv_stout[(b * p.dim + d) * K + col] = v;
    }
  }
  if constexpr (kSegm) {
    // pass 1: segment aggregate, the end state and the step-size sum (the
    // fp64 partial sums of the 16 owner lanes of each channel, added by a
    // lane butterfly in registers: the workgroup's LDS stays that of the
    // one-segment scan, five workgroups per CU)
#pragma unroll
    for (int m = 1; m < kN; m <<= 1) ssum += __shfl_xor(ssum, m, kN);
    float* ag = p.agg + (arow + g) * aggs;
    if (vrow) {
#pragma unroll
      for (int q = 0; q < S; ++q) {
        const int n = col + kN * q;
        if (n < N) ag[n] = h[q];
      }
    }
    if (vrow && col == 0) ag[N] = static_cast<float>(ssum);
  }
}

// Launch of one variant family: the dtype, softplus and conv width choose
// among the instantiations with S state slots per lane and the B/C mode.
template <Mode M, int KP, int S, int kLane, bool kDefer = false>
void launch_kp(bool bf16, bool softplus, dim3 grid, const ScanParams& p, hipStream_t stream) {
  const dim3 block(kThreads);
  if (bf16) {
    if (softplus) scan_fwd_kernel<uint16_t, M, true, KP, S, kLane, kDefer><<<grid, block, 0, stream>>>(p);
    else scan_fwd_kernel<uint16_t, M, false, KP, S, kLane, kDefer><<<grid, block, 0, stream>>>(p);
  } else {
    if (softplus) scan_fwd_kernel<float, M, true, KP, S, kLane, kDefer><<<grid, block, 0, stream>>>(p);
    else scan_fwd_kernel<float, M, false, KP, S, kLane, kDefer><<<grid, block, 0, stream>>>(p);
  }
}

// The conv width is padded to 4 or 8 taps (zero weights); only the
// one-slot shared-B/C kernels, the common Mamba-1 shape, get the 4-tap form.
// B/C modes: 0 shared tile, 1 per-lane element loads, 2 per-lane 16-byte
// loads (aligned rows; without the conv branch).  `defer` picks the
// deferred owner-C readout for the one-slot shared-tile scan without the
// conv branch (with it the form measured slower: 137 -> 149 us on the
// 130m-like layer, at 146-151 VGPRs).
template <Mode M, int S>
void launch_mode(int lane, bool bf16, bool softplus, int K, bool defer, dim3 grid,
                 const ScanParams& p, hipStream_t stream) {
  if constexpr (M == Mode::kScan && S == 1) {
    if (defer && lane == 0 && K == 0) {
      launch_kp<M, 0, S, 0, true>(bf16, softplus, grid, p, stream);
      return;
    }
  }
  if (lane == 0) {
    if (K == 0) launch_kp<M, 0, S, 0>(bf16, softplus, grid, p, stream);
    else if (K <= 4 && S == 1) launch_kp<M, 4, S, 0>(bf16, softplus, grid, p, stream);
    else launch_kp<M, 8, S, 0>(bf16, softplus, grid, p, stream);
  } else if (lane == 2 && K == 0) {
    launch_kp<M, 0, S, 2>(bf16, softplus, grid, p, stream);
  } else {
    if (K == 0) launch_kp<M, 0, S, 1>(bf16, softplus, grid, p, stream);
    else launch_kp<M, 8, S, 1>(bf16, softplus, grid, p, stream);
  }
}

// Launches for S state slots per lane (defined in scan_fwd_s<S>.hip): pass 0
// is the one-segment scan, passes 1 and 2 those of a segmented sequence.
template <int S>
void launch_slots(int pass, int lane, bool bf16, bool softplus, int K, bool defer, dim3 grid,
                  const ScanParams& p, hipStream_t stream);
// Passes 1 and 2 of a segmented sequence (defined in scan_fwd_seg_s<S>.hip).
template <int S>
void launch_slots_seg(int pass, int lane, bool bf16, bool softplus, int K, dim3 grid,
                      const ScanParams& p, hipStream_t stream);

}  // namespace fwd
}  // namespace ssm

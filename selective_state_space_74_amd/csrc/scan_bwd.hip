// scan_bwd.hip -- backward of the prefill selective scan for gfx950.
//
// Reverse-mode derivative of the recurrence of scan_fwd.hip (Mamba model
// notes sections 2.2 and 4.4; zero-order-hold step of the Mamba paper notes
// section 2.3), per batch row b, channel d, state n:
//   gate     out = y silu(z):   dy = dout silu(z),
//                               dz = dout y s(z) (1 + z (1 - s(z)))
//   readout  y = sum_n C h_t + D u:   dC += dy h_t,  dD += dy u,  du = dy D + ...
//   step     h_t = e_t h_{t-1} + Delta B u,  e_t = exp(Delta A); with g the
//            adjoint of h_t (g_t = dy_t C_t + e_{t+1} g_{t+1}):
//            dB += g Delta u,  du += Delta sum_n g B,
//            dDelta = u sum_n g B + sum_n g A e_t h_{t-1},  dA += g Delta e_t h_{t-1}
//   Delta    Delta = softplus(x):  ddelta = dDelta s(x),  dbias += ddelta
//   h0       dh0 = e_0 g_0
// Back-propagation needs every h_{t-1}; the forward keeps only the state
// entering each 16-token block (Mamba paper notes section 5.4: recompute the
// intermediate states from the forward instead of storing them), and the
// backward recomputes the 16 steps of a block from its checkpoint.
//
// Work decomposition (the forward's): a workgroup is 4 wavefronts x 4
// channels of one batch row, lane (row c, col n) holds states n, n + 16, ...
// (S slots for up to 16 S states; states past dstate are padding that stays
// zero) of channel c, and lane (row c, col j), as owner, handles token j of
// each block.  Blocks are walked from the last to the first; per block (one
// slot; with several, see block_slots):
//   1. state lanes recompute e_t and h_t for the 16 tokens from the
//      checkpoint (registers) and leave C_n h_t in LDS;
//   2. owners sum those into y, form dy and dz (dy reaches the state lanes
//      by DPP row broadcast);
//   3. state lanes run the adjoint from token 15 down to 0, accumulating dA in
//      a register and leaving per-token terms in LDS: g B and g A e h_{t-1}
//      (summed over n by the owners, who finish du and ddelta), g Delta u and
//      dy h_t (summed over the workgroup's 16 channels); this runs in two
//      halves of 8 tokens so that the LDS holds half a block of terms.
// The workgroup's dB/dC sums go, with a caller workspace (the default of the
// binding), to the workgroup's own slot of a partial-sum buffer that a second
// kernel adds up per group in a fixed order (deterministic); without one,
// they are added into dB and dC with one device atomic per (n, t) and
// workgroup.  dA, dD and the bias gradient are summed over batch rows the
// same way: per-row slots and an ordered sum with the workspace, device
// atomics without.  B/C tiles are staged as in the forward (16 states x 32
// tokens, double buffered), walking backwards.
//
// Long sequences with few channels (with the workspace) are cut into
// segments, as the forward does.  The adjoint recurrence
// g_{t-1} = e_t (dy_t C_t + g_t) is linear in g and needs no forward state, so
//   pass 1 (bwd_aggregate_kernel) runs it over segments 1..G-1 from a zero
//          adjoint and records what leaves each segment at its start,
//          alpha_s, and the segment's step-size sum S_s;
//   pass 2 (scan_bwd_kernel) runs the full backward of segment s from the
//          exact adjoint entering it from the right,
//          K_s = alpha_{s+1} + exp(A S_{s+1}) K_{s+1},  K_{G-1} = dlast,
//          with dA, dD and the bias gradient in per-segment slots.
// Every output is then the single-segment result up to fp32 rounding.
#include <algorithm>

#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kN = 16;               // lanes per row = states per slot
constexpr int kRows = 4;             // channels per wavefront
constexpr int kWaves = 4;            // wavefronts per workgroup
constexpr int kCh = kRows * kWaves;  // channels per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kT = 16;               // tokens per block (= checkpoint interval)
constexpr int kGB = 2;               // blocks per B/C tile
constexpr int kGT = kT * kGB;        // tokens per tile
constexpr int kGPitch = kGT + 4;     // LDS pitch (floats) of one state's tile row
constexpr int kPitch = 20;           // LDS pitch (floats) of one state's 16 token terms

// The value held by lane col ^ 8 of the same 16-lane row (DPP row_ror:8).
__device__ __forceinline__ float row_swap8(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xf, 0xf, true));
}

// Sums over the four 16-lane rows of a wavefront by lane swaps (no LDS).
// swap_add32(a, b): rows 0..3 hold a0+a2, a1+a3, b0+b2, b1+b3.
__device__ __forceinline__ float swap_add32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// swap_add16(x, y): rows 0..3 hold x0+x1, y0+y1, x2+x3, y2+y3.  Applied to
// x = swap_add32(a, b) and y = swap_add32(c, d) it leaves the four-row sums
// of a, c, b, d in rows 0, 1, 2, 3.
__device__ __forceinline__ float swap_add16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct BwdParams {
  const void* u;
  const void* delta;
  const void* z;
  const void* B;
  const void* C;
  const float* A;
  const float* D;
  const float* bias;
  const float* ckpt;
  const void* dout;
  const float* dlast;
  void* du;
  void* ddelta;
  void* dz;
  float* dB;
  float* dC;
  float* dA;
  float* dD;
  float* dbias;
  float* dh0;
  float* part;          // [batch][cgroups][2][N][L] dB/dC partial sums, or NULL (atomics)
  float* pdA;           // with part: [nseg][batch][dim][N] dA, [nseg][batch][dim] dD and
  float* pdD;           // bias gradient per segment and batch row, summed over both
  float* pdb;           // by a second kernel (NULL: device atomics into dA, dD, dbias)
  float* agg;           // segmented: [batch][dim][nseg][N + 1] adjoint aggregates
  int seg_len;          // tokens per segment (a multiple of kGT)
  int nseg;             // segments per sequence (1: the whole sequence)
  int64_t usb, usd, dsb, dsd, zsb, zsd, Bsb, Bsn, Csb, Csn, Asd, Asn, gsb, gsd;
  int64_t dusb, dusd, ddsb, ddsd, dzsb, dzsd;
  int64_t Bsg, Csg;     // B/C group strides
  int64_t ngroups, cpg; // groups, channels per group (a multiple of kCh, or dim)
  int64_t batch, dim;
  int L;
  int N;            // states per channel (dstate)
  int nbk;          // ceil(L / kT)
  int64_t cgroups;  // ceil(dim / kCh)
};

// Owner inputs of one block: token t0 + col of the lane's channel.
struct Raw {
  uint32_t u, dt, z, dout;
};

// Tile inputs: B and C of states 4 wave + row + 16 q at tokens tg + col + 16 i.
template <int S>
struct TileRaw {
  uint32_t b[S][kGB], c[S][kGB];
};

// LDS pitch (floats) of one state's per-token terms: 16 tokens (one slot:
// readout partials, then half a block of g B and g A e h terms), or 32 (slots:
// a whole block of both terms).
template <int S>
constexpr int kXPitch = S == 1 ? kPitch : 2 * kT + 4;
template <int S>
constexpr int kXRow = kN * kXPitch<S> + 16;   // floats per channel
// Buffers of the dB/dC exchange (sQ).  One slot: four, a pair per block in
// turn (half h8 of block k in buffer 2 (k % 2) + h8), so that one barrier
// per block orders both halves' writes before their sums, and the previous
// pair's sums before the next writes into it (one block later, past the
// next block's barrier).  Two slots: two, one per half in turn, one barrier
// per half.  Four slots: one, and a second barrier per half (more LDS would
// leave a single workgroup per CU).
template <int S>
constexpr int kQBuf = S == 1 ? 4 : S == 2 ? 2 : 1;

template <typename T, bool kSoftplus, int S>
struct BwdWave {
  const BwdParams& p;
  int wave, row, col;
  int nbk, ntile;
  Window wu, wdt, wz, wg, wdu, wdd, wdz, wB, wC, wck, wdB, wdC;
  uint32_t ou, odt, oz, og, odu, odd, odz;
  // per state slot; B/C and checkpoint offsets of padding states point past
  // their window (loads read zero)
  uint32_t oB[S], oC[S], ock[S];
  float a[S], a2[S], bias, Dd;
  // one slot: A of the lane's channel at states (col & 8) + 0..7, the
  // weights of the owner's half of the sum over states for ddelta
  float ah[kN / 2];
  bool gate;
  bool partials;      // dB/dC sums stored to this workgroup's slots, not added
  int nvalid;         // channels of this workgroup below dim
  float (*sB)[kN * S][kGPitch];   // [2][kN S][kGPitch], shared
  float (*sC)[kN * S][kGPitch];
  float (*sX)[kXRow<S>];      // this wavefront's [kRows][kXRow]: readout, then the
                              // per-state du/ddelta terms
  float (*sQ)[kWaves][kRows][kN][4];  // [kQBuf][kWaves][kRows][kN][4], shared: dB/dC terms
                              // of half a block (one slot) summed over each wavefront's
                              // channels (buffers: kQBuf); row r holds
                              // tensor r / 2 (dB, dC), tokens 4 (r % 2) + 0..3

  static constexpr int E = Elem<T>::kSize;

  __device__ __forceinline__ uint32_t skip(int k) const { return static_cast<uint32_t>(k * kT) * E; }

  // Owner inputs of block k (clamped into [0, nbk), like the forward's).
  __device__ __forceinline__ Raw load(int k) const {
    Raw r;
    const uint32_t s = skip(max(k, 0));
    r.u = Elem<T>::load(wu.at(s), ou);
    r.dt = Elem<T>::load(wdt.at(s), odt);
    r.z = Elem<T>::load(wz.at(s), oz);
    r.dout = Elem<T>::load(wg.at(s), og);
    return r;
  }

  __device__ __forceinline__ TileRaw<S> load_tile(int g) const {
    TileRaw<S> r;
    const uint32_t s = skip(max(g, 0) * kGB);
    const __amdgpu_buffer_rsrc_t rb = wB.at(s), rc = wC.at(s);
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

  // Tile g into LDS buffer g & 1; B of tokens past the end is zeroed.
  __device__ __forceinline__ void stage(int g, const TileRaw<S>& r) const {
    const int st = kRows * wave + row;
    const int t = g * kGT + col;
#pragma unroll
    for (int q = 0; q < S; ++q) {
#pragma unroll
      for (int i = 0; i < kGB; ++i) {
        sB[g & 1][st + kN * q][col + i * kT] = t + i * kT < p.L ? Elem<T>::f32(r.b[q][i]) : 0.0f;
        sC[g & 1][st + kN * q][col + i * kT] = Elem<T>::f32(r.c[q][i]);
      }
    }
  }

  // B and C of slot q for the 16 tokens of block k, from the LDS tile.
  __device__ __forceinline__ void tile_rows(int k, int q, float (&bv)[kT], float (&cv)[kT]) const {
    const int buf = (k / kGB) & 1;
    const int tb = (k % kGB) * kT;
#pragma unroll
    for (int i = 0; i < kT / 4; ++i) {
      const float4 x = *reinterpret_cast<const float4*>(&sB[buf][col + kN * q][tb + 4 * i]);
      bv[4 * i] = x.x; bv[4 * i + 1] = x.y; bv[4 * i + 2] = x.z; bv[4 * i + 3] = x.w;
      const float4 y = *reinterpret_cast<const float4*>(&sC[buf][col + kN * q][tb + 4 * i]);
      cv[4 * i] = y.x; cv[4 * i + 1] = y.y; cv[4 * i + 2] = y.z; cv[4 * i + 3] = y.w;
    }
  }

  // The checkpoint of slot q: the state entering block k.
  __device__ __forceinline__ float checkpoint(int k, int q) const {
    return Elem<float>::f32(__builtin_amdgcn_raw_buffer_load_b32(
        wck.at(static_cast<uint32_t>(k) * p.N * 4), ock[q], 0, 0));
  }

  // dB/dC of half h8 of block k, slot q: thread (tensor, n, t) sums the
  // workgroup's channels from sQ (filled and synchronised by the caller) and
  // stores or adds the sum.  Tokens past the end, and padding states,
  // address the window's end, where the store or atomic is dropped: their
  // offsets would otherwise reach into later states' rows, and a plain store
  // there (the partial sums) races with the real value when the sequence is
  // shorter than a block.
  __device__ __forceinline__ void dbdc_sum(int k, int h8, int q, int qb) const {
    const int tid = threadIdx.x;
    // the tensor (dB, dC) is one per wavefront pair: made visibly uniform so
    // that the buffer descriptor is selected in scalar registers
    const int ten = __builtin_amdgcn_readfirstlane(tid >> 7);
    const int n = (tid >> 3) & 15, t = tid & 7;
    const int qr = 2 * ten + (t >> 2), qt = t & 3;
    const auto& sq = sQ[qb];
    float sum = sq[0][qr][n][qt];
#pragma unroll
    for (int v = 1; v < kWaves; ++v) sum += sq[v][qr][n][qt];
    const int tok = k * kT + 8 * h8 + t;
    const int na = n + kN * q;
    const uint32_t off =
        static_cast<uint32_t>((tok < p.L && na < p.N ? na * p.L + tok : p.N * p.L) * 4);
    // (a uniform branch)
    if (partials)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sum), ten ? wdC.at(0) : wdB.at(0), off, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(sum, ten ? wdC.at(0) : wdB.at(0), off, 0, 0);
  }

  // Block k (all of it; k runs from nbk - 1 down to 0), one state slot.  Q
  // holds its owner inputs; g is the state lane's adjoint of the state
  // leaving the block.
  __device__ __forceinline__ void block(int k, const Raw& Q, float (&ga)[S], float (&dAa)[S],
                                        float& dDs, float& dbs) const {
    static_assert(S == 1, "one state slot");
    float& g = ga[0];
    float& dA = dAa[0];
    const float a2 = this->a2[0];
    const int t0 = k * kT;
    float bv[kT], cv[kT];
    tile_rows(k, 0, bv, cv);
    const float hck = checkpoint(k, 0);

    // owner: Delta, Delta u (zero past the end, so those steps are identities).
    // The mask is applied to the inputs (softplus(-inf) = 0) so that Delta
    // and Delta u, the DPP broadcast sources, come from arithmetic, not from
    // a select: that keeps the broadcasts foldable into their consumers.
    const bool own = t0 + col < p.L;
    const float uv = own ? Elem<T>::f32(Q.u) : 0.0f;
    const float x = Elem<T>::f32(Q.dt) + bias;
    const float xm = own ? x : (kSoftplus ? -__builtin_inff() : 0.0f);
    const float dl = kSoftplus ? softplus_f32(xm) : xm;
    const float du = dl * uv;

    // 1. forward again from the checkpoint; readout terms to LDS
    float e[kT], hs[kT];
    {
      float h = hck;
      float pk[4];
      static_for<0, kT>([&](auto J) {
        constexpr int j = decltype(J)::value;
        e[j] = __builtin_amdgcn_exp2f(row_bcast<j>(dl) * a2);
        h = fmaf(e[j], h, row_bcast<j>(du) * bv[j]);
        hs[j] = h;
        pk[j % 4] = cv[j] * h;
        if (j % 4 == 3)
          *reinterpret_cast<float4*>(&sX[row][col * kPitch + j - 3]) =
              make_float4(pk[0], pk[1], pk[2], pk[3]);
      });
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");

    // 2. owner: y, dy, dz
    float y = 0.0f;
#pragma unroll
    for (int n = 0; n < kN; ++n) y += sX[row][n * kPitch + col];
    y = fmaf(Dd, uv, y);
    const float zv = Elem<T>::f32(Q.z);
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zv * kLog2e));
    const float go = own ? Elem<T>::f32(Q.dout) : 0.0f;
    const float dy = gate ? go * zv * sg : go;
    const float dzv = go * y * sg * fmaf(zv, 1.0f - sg, 1.0f);  // stored below
    dDs = fmaf(dy, uv, dDs);
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");

    // 3. adjoint, token 15 down to 0, in two halves of 8 tokens (second
    // broadcasts of Delta, Delta u and dy go through opaque copies so that
    // each broadcast folds into its one consumer).  After each half: the
    // owners of its 8 tokens finish du/ddelta from the per-state terms, and
    // the workgroup's 256 threads sum the dB/dC terms over its channels.
    // channels past dim (their rows repeat the last channel) add nothing to
    // dB/dC: their Delta u and dy copies for those terms are zero
    const bool rv = kRows * wave + row < nvalid;
    const float dl2 = opaque_copy(dl), du2 = opaque_copy(rv ? du : 0.0f),
                dy2 = opaque_copy(rv ? dy : 0.0f);
    float sxm = 0.0f;  // softplus'(x) for this owner's token
    if (kSoftplus) sxm = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
    float s1[4], s2[4], yq[4], rq[4];
    // The adjoint of h_t itself is carried from token to token,
    // adj_t = exp(Delta_{t+1} A) adj_{t+1} + dy_t C_t (the adjoint of the
    // state leaving the block, g, enters at token 15 and leaves as
    // exp(Delta_0 A) adj_0): one DPP-fused multiply and one FMA per token.
    float adj = 0.0f;
    static_for<0, kT>([&](auto J) {
      constexpr int j = kT - 1 - decltype(J)::value;
      constexpr int h8 = j / 8;          // which half
      constexpr int jj = j % 8;          // token within the half
      const float dyc = row_bcast<j>(dy) * cv[j];
      if constexpr (j == kT - 1) adj = g + dyc;                    // adjoint of h_t
      else adj = fmaf(e[j + 1], adj, dyc);
      const float hp = j > 0 ? hs[j > 0 ? j - 1 : 0] : hck;        // h_{t-1}
      const float q = adj * (e[j] * hp);
      s1[j % 4] = adj * bv[j];                                     // -> du, ddelta
      s2[j % 4] = q;                                               // x A by the owner -> ddelta
      const float rb = row_bcast<j>(du2) * adj;                    // -> dB
      const float rc = row_bcast<j>(dy2) * hs[j];                  // -> dC
      // summed over the wavefront's four channels as they come: tokens 4..7
      // of the half pair with tokens 0..3 (row layout of sQ)
      if constexpr (jj >= 4) yq[jj - 4] = swap_add32(rb, rc);
      else rq[jj] = swap_add16(swap_add32(rb, rc), yq[jj]);
      dA = fmaf(row_bcast<j>(dl2), q, dA);
      if constexpr (j == 0) g = e[0] * adj;                        // adjoint of h_{t-1}
      if constexpr (j % 4 == 0) {
        // per-wave region: [c][n][0..7] g B, [c][n][8..15] g e h_{t-1}
        *reinterpret_cast<float4*>(&sX[row][col * kPitch + jj]) = make_float4(s1[0], s1[1], s1[2], s1[3]);
        *reinterpret_cast<float4*>(&sX[row][col * kPitch + 8 + jj]) =
            make_float4(s2[0], s2[1], s2[2], s2[3]);
      }
      if constexpr (jj == 0) {
        const int qb = 2 * (k & 1);   // this block's pair of exchange buffers
        *reinterpret_cast<float4*>(&sQ[qb + h8][wave][row][col][0]) =
            make_float4(rq[0], rq[1], rq[2], rq[3]);
        // one barrier per block, after both halves' stores
        if constexpr (h8 == 0) __syncthreads();
        // owners of tokens 8 h8 .. 8 h8 + 7: du, ddelta.  The sums over the
        // 16 states for token ti: lanes col and col ^ 8 each add 8 states'
        // terms and then exchange, so both hold the sum (the owner is the
        // one in this half; the other discards it)
        const int tj = col - 8 * h8;
        const bool mine = own && tj >= 0 && tj < 8;
        const int ti = col & 7, n0 = col & 8;
        float S1 = 0.0f, S2 = 0.0f;
#pragma unroll
        for (int n = 0; n < kN / 2; ++n) {
          S1 += sX[row][(n0 + n) * kPitch + ti];
          S2 = fmaf(ah[n], sX[row][(n0 + n) * kPitch + 8 + ti], S2);
        }
        S1 += row_swap8(S1);
        S2 += row_swap8(S2);
        const float duv = fmaf(dl, S1, dy * Dd);
        float dx = fmaf(uv, S1, S2);
        if (kSoftplus) dx *= sxm;
        dx = mine ? dx : 0.0f;
        dbs += dx;
        if (mine) {
          Elem<T>::store(wdu.at(skip(k)), odu, duv);
          Elem<T>::store(wdd.at(skip(k)), odd, dx);
          // without a gate the dz window is empty and stays at offset 0, so
          // the store is dropped
          Elem<T>::store(wdz.at(gate ? skip(k) : 0u), odz, dzv);
        }
        // dB, dC of both halves: summed over the workgroup's channels; the
        // next block writes the other pair, and the block after it this pair
        // again only past the next block's barrier, which every thread
        // reaches after these reads
        if constexpr (h8 == 0) {
          dbdc_sum(k, 1, 0, qb + 1);
          dbdc_sum(k, 0, 0, qb);
        }
      }
    });
  }

  // Block k with several state slots.  The adjoint of each state needs every
  // h_{t-1} and e_t of the block, 32 registers per slot, so the slots are
  // taken one at a time (a loop that is not unrolled; the per-slot values
  // rotate through index 0 of their arrays, so that every index stays
  // static) and the forward is recomputed twice: once over all slots for the
  // readout (y needs every state), once per slot right before its adjoint.
  // The per-token sums over the states (for du and ddelta) accumulate over
  // the slots in registers and go through LDS once per block; dB/dC go out
  // per slot and half block as in the one-slot form.
  template <typename V>
  __device__ __forceinline__ static void rotate(V (&v)[S]) {
    const V first = v[0];
#pragma unroll
    for (int q = 0; q + 1 < S; ++q) v[q] = v[q + 1];
    v[S - 1] = first;
  }

  __device__ __forceinline__ void block_slots(int k, const Raw& Q, float (&g)[S], float (&dA)[S],
                                              float& dDs, float& dbs) {
    const int t0 = k * kT;
    float hck[S];
#pragma unroll
    for (int q = 0; q < S; ++q) hck[q] = checkpoint(k, q);

    // owner: Delta, Delta u (zero past the end, as in the one-slot form)
    const bool own = t0 + col < p.L;
    const float uv = own ? Elem<T>::f32(Q.u) : 0.0f;
    const float x = Elem<T>::f32(Q.dt) + bias;
    const float xm = own ? x : (kSoftplus ? -__builtin_inff() : 0.0f);
    const float dl = kSoftplus ? softplus_f32(xm) : xm;
    const float du = dl * uv;

    // 1. readout partials sum_q C h_t of this lane's states, to LDS
    {
      float acc[kT];
#pragma unroll
      for (int j = 0; j < kT; ++j) acc[j] = 0.0f;
#pragma unroll 1
      for (int q = 0; q < S; ++q) {
        float bv[kT], cv[kT];
        tile_rows(k, q, bv, cv);
        float h = hck[0];
        static_for<0, kT>([&](auto J) {
          constexpr int j = decltype(J)::value;
          const float e = __builtin_amdgcn_exp2f(row_bcast<j>(dl) * a2[0]);
          h = fmaf(e, h, row_bcast<j>(du) * bv[j]);
          acc[j] = fmaf(cv[j], h, acc[j]);
        });
        rotate(hck);
        rotate(a2);
      }
#pragma unroll
      for (int i = 0; i < kT / 4; ++i)
        *reinterpret_cast<float4*>(&sX[row][col * kXPitch<S> + 4 * i]) =
            make_float4(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");

    // 2. owner: y, dy, dz
    float y = 0.0f;
#pragma unroll
    for (int n = 0; n < kN; ++n) y += sX[row][n * kXPitch<S> + col];
    y = fmaf(Dd, uv, y);
    const float zv = Elem<T>::f32(Q.z);
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zv * kLog2e));
    const float go = own ? Elem<T>::f32(Q.dout) : 0.0f;
    const float dy = gate ? go * zv * sg : go;
    const float dzv = go * y * sg * fmaf(zv, 1.0f - sg, 1.0f);
    dDs = fmaf(dy, uv, dDs);
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");

    // 3. adjoint per slot, token 15 down to 0; channels past dim add nothing
    // to dB/dC (their Delta u and dy copies for those terms are zero)
    const bool rv = kRows * wave + row < nvalid;
    const float du2 = rv ? du : 0.0f, dy2 = rv ? dy : 0.0f;
    float s1[kT], s2[kT];   // sums over this lane's states of g B and g A e h_{t-1}
#pragma unroll
    for (int j = 0; j < kT; ++j) s1[j] = s2[j] = 0.0f;
#pragma unroll 1
    for (int q = 0; q < S; ++q) {
      float bv[kT], cv[kT];
      tile_rows(k, q, bv, cv);
      float e[kT], hs[kT];
      {
        float h = hck[0];
        static_for<0, kT>([&](auto J) {
          constexpr int j = decltype(J)::value;
          e[j] = __builtin_amdgcn_exp2f(row_bcast<j>(dl) * a2[0]);
          h = fmaf(e[j], h, row_bcast<j>(du) * bv[j]);
          hs[j] = h;
        });
      }
      float yq[4], rq[4];
      // the adjoint of h_t carried from token to token, as in the one-slot
      // form
      float adj = 0.0f;
      static_for<0, kT>([&](auto J) {
        constexpr int j = kT - 1 - decltype(J)::value;
        constexpr int h8 = j / 8;
        constexpr int jj = j % 8;
        const float dyc = row_bcast<j>(dy) * cv[j];
        if constexpr (j == kT - 1) adj = g[0] + dyc;                      // adjoint of h_t
        else adj = fmaf(e[j + 1], adj, dyc);
        const float hp = j > 0 ? hs[j > 0 ? j - 1 : 0] : hck[0];          // h_{t-1}
        const float qv = adj * (e[j] * hp);
        s1[j] = fmaf(adj, bv[j], s1[j]);
        s2[j] = fmaf(qv, a[0], s2[j]);
        const float rb = row_bcast<j>(du2) * adj;                         // -> dB
        const float rc = row_bcast<j>(dy2) * hs[j];                       // -> dC
        if constexpr (jj >= 4) yq[jj - 4] = swap_add32(rb, rc);
        else rq[jj] = swap_add16(swap_add32(rb, rc), yq[jj]);
        dA[0] = fmaf(row_bcast<j>(dl), qv, dA[0]);
        if constexpr (j == 0) g[0] = e[0] * adj;                          // adjoint of h_{t-1}
        if constexpr (jj == 0) {
          *reinterpret_cast<float4*>(&sQ[h8 % kQBuf<S>][wave][row][col][0]) =
              make_float4(rq[0], rq[1], rq[2], rq[3]);
          __syncthreads();
          dbdc_sum(k, h8, q, h8 % kQBuf<S>);
          if constexpr (kQBuf<S> == 1) __syncthreads();
        }
      });
      rotate(g);
      rotate(dA);
      rotate(hck);
      rotate(a2);
      rotate(a);
    }

    // 4. per-state terms of the 16 tokens to LDS ([c][n][0..15] g B,
    // [c][n][16..31] g A e h_{t-1}); the owner of each token sums its 16
    // lanes' terms into du and ddelta
#pragma unroll
    for (int i = 0; i < kT / 4; ++i) {
      *reinterpret_cast<float4*>(&sX[row][col * kXPitch<S> + 4 * i]) =
          make_float4(s1[4 * i], s1[4 * i + 1], s1[4 * i + 2], s1[4 * i + 3]);
      *reinterpret_cast<float4*>(&sX[row][col * kXPitch<S> + kT + 4 * i]) =
          make_float4(s2[4 * i], s2[4 * i + 1], s2[4 * i + 2], s2[4 * i + 3]);
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    float S1 = 0.0f, S2 = 0.0f;
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      S1 += sX[row][n * kXPitch<S> + col];
      S2 += sX[row][n * kXPitch<S> + kT + col];
    }
    const float duv = fmaf(dl, S1, dy * Dd);
    float dx = fmaf(uv, S1, S2);
    if (kSoftplus) dx *= __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
    dx = own ? dx : 0.0f;
    dbs += dx;
    if (own) {
      Elem<T>::store(wdu.at(skip(k)), odu, duv);
      Elem<T>::store(wdd.at(skip(k)), odd, dx);
      Elem<T>::store(wdz.at(gate ? skip(k) : 0u), odz, dzv);
    }
    // the next block's readout rewrites sX
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  }
};

template <typename T, bool kSoftplus, int S>
__global__ __launch_bounds__(kThreads) void scan_bwd_kernel(BwdParams p) {
  __shared__ __align__(16) float sB[2][kN * S][kGPitch];
  __shared__ __align__(16) float sC[2][kN * S][kGPitch];
  __shared__ __align__(16) float sX[kWaves][kRows][kXRow<S>];
  __shared__ __align__(16) float sQ[kQBuf<S>][kWaves][kRows][kN][4];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = (threadIdx.x >> 4) & 3;
  const int col = threadIdx.x & 15;
  // logical workgroup wg = (b * cgroups + cg) * nseg + seg: channel-major
  // (segment-major, which lets the channel groups of a segment share its B/C
  // lines in one XCD's L2 as the forward does, measured 2.7% slower on the
  // 1M-token backward)
  const uint32_t wg = xcd_order(blockIdx.x, gridDim.x);
  const int seg = static_cast<int>(wg % p.nseg);
  const int64_t bcg = wg / p.nseg;
  const int64_t b = bcg / p.cgroups;
  const int64_t cg = bcg % p.cgroups;
  const int64_t d = cg * kCh + kRows * wave + row;
  const bool vrow = d < p.dim;
  const int64_t dc = vrow ? d : p.dim - 1;
  const int64_t dw0 = std::min<int64_t>(cg * kCh + kRows * wave, p.dim - 1);
  const int64_t dw3 = std::min<int64_t>(dw0 + kRows - 1, p.dim - 1);
  const int N = p.N;

  constexpr int E = Elem<T>::kSize;
  BwdWave<T, kSoftplus, S> w{p};
  w.wave = wave; w.row = row; w.col = col;
  w.nbk = p.nbk;
  w.ntile = (p.nbk + kGB - 1) / kGB;
  w.gate = p.z != nullptr;
  w.nvalid = static_cast<int>(std::min<int64_t>(kCh, p.dim - cg * kCh));

  auto rows_window = [&](const void* base, int64_t sb, int64_t sd, uint32_t& off) {
    off = static_cast<uint32_t>(((dc - dw0) * sd + col) * E);
    return Window{static_cast<const char*>(base) + (b * sb + dw0 * sd) * E,
                  static_cast<uint32_t>(((dw3 - dw0) * sd + p.L) * E)};
  };
  w.wu = rows_window(p.u, p.usb, p.usd, w.ou);
  w.wdt = rows_window(p.delta, p.dsb, p.dsd, w.odt);
  w.wg = rows_window(p.dout, p.gsb, p.gsd, w.og);
  w.wdu = rows_window(p.du, p.dusb, p.dusd, w.odu);
  w.wdd = rows_window(p.ddelta, p.ddsb, p.ddsd, w.odd);
  if (w.gate) {
    w.wz = rows_window(p.z, p.zsb, p.zsd, w.oz);
    w.wdz = rows_window(p.dz, p.dzsb, p.dzsd, w.odz);
  } else {
    w.wz = w.wu; w.oz = w.ou;      // loaded, never used
    w.wdz = Window{nullptr, 0u}; w.odz = 0;
  }
  // the workgroup's 16 channels share one B/C group
  const int64_t grp = (cg * kCh) / p.cpg;
  const int st = kRows * wave + row;
  w.wB = Window{static_cast<const char*>(p.B) + (b * p.Bsb + grp * p.Bsg) * E,
                static_cast<uint32_t>(((N - 1) * p.Bsn + p.L) * E)};
  w.wC = Window{static_cast<const char*>(p.C) + (b * p.Csb + grp * p.Csg) * E,
                static_cast<uint32_t>(((N - 1) * p.Csn + p.L) * E)};
  const int64_t ckrow = static_cast<int64_t>(p.nbk) * N;
  w.wck = Window{reinterpret_cast<const char*>(p.ckpt + (b * p.dim + dw0) * ckrow),
                 static_cast<uint32_t>((dw3 - dw0 + 1) * ckrow * 4)};
#pragma unroll
  for (int q = 0; q < S; ++q) {
    const int ns = st + kN * q;     // the state this lane stages
    w.oB[q] = ns < N ? static_cast<uint32_t>((ns * p.Bsn + col) * E) : w.wB.bytes;
    w.oC[q] = ns < N ? static_cast<uint32_t>((ns * p.Csn + col) * E) : w.wC.bytes;
    const int n = col + kN * q;     // the state this lane carries
    w.ock[q] = n < N ? static_cast<uint32_t>(((dc - dw0) * ckrow + n) * 4) : w.wck.bytes;
    w.a[q] = n < N ? p.A[dc * p.Asd + n * p.Asn] : 0.0f;
    w.a2[q] = w.a[q] * kLog2e;
  }
  if constexpr (S == 1) {
#pragma unroll
    for (int n = 0; n < kN / 2; ++n) {
      const int na = (col & 8) + n;
      w.ah[n] = na < N ? p.A[dc * p.Asd + na * p.Asn] : 0.0f;
    }
  }
  // dB/dC: this workgroup's slots of the partial sums, or the group's rows
  // of dB/dC themselves (atomics)
  const int64_t NL = static_cast<int64_t>(N) * p.L;
  const float* pB = p.part ? p.part + ((b * p.cgroups + cg) * 2 + 0) * NL : p.dB + (b * p.ngroups + grp) * NL;
  const float* pC = p.part ? p.part + ((b * p.cgroups + cg) * 2 + 1) * NL : p.dC + (b * p.ngroups + grp) * NL;
  w.wdB = Window{reinterpret_cast<const char*>(pB), static_cast<uint32_t>(NL * 4)};
  w.wdC = Window{reinterpret_cast<const char*>(pC), static_cast<uint32_t>(NL * 4)};
  w.partials = p.part != nullptr;

  w.bias = p.bias ? p.bias[dc] : 0.0f;
  w.Dd = p.D ? p.D[dc] : 0.0f;
  w.sB = sB; w.sC = sC; w.sX = sX[wave]; w.sQ = sQ;

  // The adjoint entering the segment from the right: dlast, folded with the
  // aggregates of the later segments (segment i turns K into
  // alpha_i + exp(A S_i) K).
  float g[S], dA[S];
#pragma unroll
  for (int q = 0; q < S; ++q) {
    const int n = col + kN * q;
    g[q] = 0.0f;
    dA[q] = 0.0f;
    if (n < N) {
      g[q] = p.dlast ? p.dlast[(b * p.dim + dc) * N + n] : 0.0f;
      if (seg < p.nseg - 1) {
        const float* ag = p.agg + (b * p.dim + dc) * p.nseg * (N + 1);
        for (int i = p.nseg - 1; i > seg; --i)
          g[q] = fmaf(__builtin_amdgcn_exp2f(w.a2[q] * ag[i * (N + 1) + N]), g[q], ag[i * (N + 1) + n]);
      }
    }
  }
  float dDs = 0.0f, dbs = 0.0f;

  // this segment's blocks [kbeg, kend), walked from the last; segment
  // starts are multiples of a tile
  const int kbeg = seg * (p.seg_len / kT);
  const int kend = std::min(p.nbk, kbeg + p.seg_len / kT);
  // the last tile first; owner inputs of block k in buffer k % 2, the next
  // (earlier) one loading meanwhile
  const int tl = (kend - 1) / kGB;
  TileRaw<S> tile = w.load_tile(tl);
  w.stage(tl, tile);
  tile = w.load_tile(tl - 1);
  __syncthreads();
  Raw cur = w.load(kend - 1);
  for (int k = kend - 1; k >= kbeg; --k) {
    const Raw next = w.load(k - 1);
    if constexpr (S == 1) {
      // one slot: tile (k / kGB) - 1 goes into the other buffer at the top
      // of block k (every wavefront finished reading that buffer, tile
      // k / kGB + 1, before the barrier at the end of block k + 1), and the
      // barrier at the end of block k publishes it to block k - 1
      if (k % kGB == 0 && k > kbeg) {
        w.stage(k / kGB - 1, tile);
        tile = w.load_tile(k / kGB - 2);
      }
      w.block(k, cur, g, dA, dDs, dbs);
    } else {
      w.block_slots(k, cur, g, dA, dDs, dbs);
      if (k % kGB == 0 && k > kbeg) {
        // tile (k / kGB) - 1 into the other buffer; every wavefront finished
        // reading it before the barrier at the end of the previous block
        w.stage(k / kGB - 1, tile);
        tile = w.load_tile(k / kGB - 2);
        __syncthreads();
      }
    }
    cur = next;
  }

  const int64_t slot = seg * p.batch * p.dim + b * p.dim + d;   // per segment and batch row
#pragma unroll
  for (int q = 0; q < S; ++q) {
    const int n = col + kN * q;
    if (vrow && n < N) {
      if (p.dh0 && seg == 0) p.dh0[(b * p.dim + d) * N + n] = g[q];
      if (p.pdA) p.pdA[slot * N + n] = dA[q];
      else atomicAdd(&p.dA[d * N + n], dA[q]);
    }
  }
  // dD and the bias gradient: sum the 16 owner lanes of the row
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) {
    dDs += __shfl_xor(dDs, m, 16);
    dbs += __shfl_xor(dbs, m, 16);
  }
  if (vrow && col == 0) {
    if (p.pdA) {
      p.pdD[slot] = dDs;
      p.pdb[slot] = dbs;
    } else {
      if (p.dD) atomicAdd(&p.dD[d], dDs);
      if (p.dbias) atomicAdd(&p.dbias[d], dbs);
    }
  }
}

// Pass 1 of a segmented backward: the adjoint recurrence alone over segment
// s (1..nseg-1) from a zero adjoint at its end.  Lane (row c, col n) carries
// the adjoints of states n, n + 16, ... of channel c; owner lane (row c, col
// j) forms dy (dout through the gate) and Delta of token j of each block,
// handed to the state lanes by DPP row broadcasts; C comes through the same
// double-buffered LDS tiles as in the full backward.  Per token t, walking
// down: g <- exp(Delta_t A) (dy_t C_t + g).  What leaves the segment at its
// start, alpha_s = g, and the step-size sum S_s (fp64 per owner, summed by a
// lane butterfly) go to agg[b][d][s].
template <typename T, bool kSoftplus, int S>
__global__ __launch_bounds__(kThreads) void bwd_aggregate_kernel(BwdParams p) {
  __shared__ __align__(16) float sC[2][kN * S][kGPitch];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = (threadIdx.x >> 4) & 3;
  const int col = threadIdx.x & 15;
  // logical workgroup lw = (b * cgroups + cg) * (nseg - 1) + seg - 1
  const uint32_t lw = xcd_order(blockIdx.x, gridDim.x);
  const int seg = 1 + static_cast<int>(lw % (p.nseg - 1));
  const int64_t bcg = lw / (p.nseg - 1);
  const int64_t b = bcg / p.cgroups;
  const int64_t cg = bcg % p.cgroups;
  const int64_t d = cg * kCh + kRows * wave + row;
  const bool vrow = d < p.dim;
  const int64_t dc = vrow ? d : p.dim - 1;
  const int64_t dw0 = std::min<int64_t>(cg * kCh + kRows * wave, p.dim - 1);
  const int64_t dw3 = std::min<int64_t>(dw0 + kRows - 1, p.dim - 1);
  constexpr int E = Elem<T>::kSize;
  const bool gate = p.z != nullptr;
  const int N = p.N;

  auto rows_window = [&](const void* base, int64_t sb, int64_t sd, uint32_t& off) {
    off = static_cast<uint32_t>(((dc - dw0) * sd + col) * E);
    return Window{static_cast<const char*>(base) + (b * sb + dw0 * sd) * E,
                  static_cast<uint32_t>(((dw3 - dw0) * sd + p.L) * E)};
  };
  uint32_t odt, oz, og;
  const Window wdt = rows_window(p.delta, p.dsb, p.dsd, odt);
  const Window wg = rows_window(p.dout, p.gsb, p.gsd, og);
  const Window wz = gate ? rows_window(p.z, p.zsb, p.zsd, oz) : wdt;
  if (!gate) oz = odt;   // loaded, never used
  const int64_t grp = (cg * kCh) / p.cpg;
  const int st = kRows * wave + row;
  const Window wC{static_cast<const char*>(p.C) + (b * p.Csb + grp * p.Csg) * E,
                  static_cast<uint32_t>(((N - 1) * p.Csn + p.L) * E)};
  uint32_t oC[S];
  float a2[S];
#pragma unroll
  for (int q = 0; q < S; ++q) {
    const int ns = st + kN * q, n = col + kN * q;
    oC[q] = ns < N ? static_cast<uint32_t>((ns * p.Csn + col) * E) : wC.bytes;
    a2[q] = n < N ? p.A[dc * p.Asd + n * p.Asn] * kLog2e : 0.0f;
  }
  const float bias = p.bias ? p.bias[dc] : 0.0f;

  auto skip = [](int k) { return static_cast<uint32_t>(k * kT) * E; };
  struct In { uint32_t dt, z, go; };
  auto load = [&](int k) {
    const uint32_t s = skip(max(k, 0));
    return In{Elem<T>::load(wdt.at(s), odt), Elem<T>::load(wz.at(s), oz),
              Elem<T>::load(wg.at(s), og)};
  };
  auto load_tile = [&](int t, uint32_t (&c)[S][kGB]) {
    const __amdgpu_buffer_rsrc_t rc = wC.at(skip(max(t, 0) * kGB));
#pragma unroll
    for (int q = 0; q < S; ++q)
#pragma unroll
      for (int i = 0; i < kGB; ++i) c[q][i] = Elem<T>::load(rc, oC[q] + i * kT * E);
  };
  auto stage = [&](int t, const uint32_t (&c)[S][kGB]) {
#pragma unroll
    for (int q = 0; q < S; ++q)
#pragma unroll
      for (int i = 0; i < kGB; ++i) sC[t & 1][st + kN * q][col + i * kT] = Elem<T>::f32(c[q][i]);
  };

  const int kbeg = seg * (p.seg_len / kT);
  const int kend = std::min(p.nbk, kbeg + p.seg_len / kT);
  const int tl = (kend - 1) / kGB;
  uint32_t tile[S][kGB];
  load_tile(tl, tile);
  stage(tl, tile);
  load_tile(tl - 1, tile);
  __syncthreads();
  float g[S];
#pragma unroll
  for (int q = 0; q < S; ++q) g[q] = 0.0f;
  double ssum = 0.0;
  In cur = load(kend - 1);
  for (int k = kend - 1; k >= kbeg; --k) {
    if ((k + 1) % kGB == 0 && k + 1 > kbeg && k + 1 < kend) {
      // tile (k + 1) / kGB - 1 (blocks k - 1, k) into the other buffer, at
      // the top of block k, the first of them: that buffer held tile
      // (k + 1) / kGB + 1, which every wavefront finished before the barrier
      // that followed the previous staging.  (Staged here rather than after
      // block k + 1, so that the block's token loop and the broadcasts that
      // feed it stay in one basic block and the broadcasts fold into their
      // multiplies.)
      stage((k + 1) / kGB - 1, tile);
      load_tile((k + 1) / kGB - 2, tile);
      __syncthreads();
    }
    const In next = load(k - 1);
    const int t0 = k * kT;
    const int buf = (k / kGB) & 1;
    const int tb = (k % kGB) * kT;
    // owner: Delta (zero past the end: softplus(-inf) = 0) and dy
    const bool own = t0 + col < p.L;
    const float x = Elem<T>::f32(cur.dt) + bias;
    const float xm = own ? x : (kSoftplus ? -__builtin_inff() : 0.0f);
    const float dl = kSoftplus ? softplus_f32(xm) : xm;
    const float zv = Elem<T>::f32(cur.z);
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zv * kLog2e));
    const float go = own ? Elem<T>::f32(cur.go) : 0.0f;
    const float dy = gate ? go * zv * sg : go;
    ssum += static_cast<double>(dl);
    static_for<0, S>([&](auto Qs) {
      constexpr int q = decltype(Qs)::value;
      float cv[kT];
#pragma unroll
      for (int i = 0; i < kT / 4; ++i) {
        const float4 y = *reinterpret_cast<const float4*>(&sC[buf][col + kN * q][tb + 4 * i]);
        cv[4 * i] = y.x; cv[4 * i + 1] = y.y; cv[4 * i + 2] = y.z; cv[4 * i + 3] = y.w;
      }
      // the adjoint of h_t carried from token to token (the backward's
      // form): adj_t = exp(Delta_{t+1} A) adj_{t+1} + dy_t C_t, and what
      // leaves the block is exp(Delta_0 A) adj_0; each broadcast folds into
      // a two-operand multiply
      float adj = 0.0f, enext = 1.0f;
      static_for<0, kT>([&](auto J) {
        constexpr int j = kT - 1 - decltype(J)::value;
        const float dyc = row_bcast<j>(dy) * cv[j];
        adj = j == kT - 1 ? g[q] + dyc : fmaf(enext, adj, dyc);
        enext = __builtin_amdgcn_exp2f(row_bcast<j>(dl) * a2[q]);
      });
      g[q] = enext * adj;
    });
    cur = next;
  }
#pragma unroll
  for (int m = 1; m < kN; m <<= 1) ssum += __shfl_xor(ssum, m, kN);
  if (vrow) {
    float* ag = p.agg + ((b * p.dim + d) * p.nseg + seg) * (N + 1);
#pragma unroll
    for (int q = 0; q < S; ++q) {
      const int n = col + kN * q;
      if (n < N) ag[n] = g[q];
    }
    if (col == 0) ag[N] = static_cast<float>(ssum);
  }
}

// dA, dD and the bias gradient from the partials per segment and batch row
// (`rows` = nseg * batch of them), summed in slot order.
__global__ void param_sum_kernel(const float* pdA, const float* pdD, const float* pdb, float* dA,
                                 float* dD, float* dbias, int64_t rows, int64_t dim, int64_t N) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < dim * N) {
    float s = 0.0f;
    for (int64_t b = 0; b < rows; ++b) s += pdA[b * dim * N + i];
    dA[i] = s;
  }
  if (i < dim) {
    float sd = 0.0f, sb = 0.0f;
    for (int64_t b = 0; b < rows; ++b) {
      sd += pdD[b * dim + i];
      sb += pdb[b * dim + i];
    }
    if (dD) dD[i] = sd;
    if (dbias) dbias[i] = sb;
  }
}

// dB/dC from the partial sums: element i of group g's (n, t) plane is the
// sum over the group's channel blocks.  V consecutive elements per thread
// (float4 when the buffers are 16-byte aligned); the four thread rows of a
// workgroup each sum a quarter of the blocks in block order, and row 0 adds
// the quarters in row order, so the result does not depend on scheduling.
constexpr int kSumCols = 64, kSumRows = 4;

template <typename V>
__global__ __launch_bounds__(kSumCols* kSumRows) void partial_sum_kernel(
    const float* part, float* dB, float* dC, int64_t NL, int64_t cgroups, int64_t G) {
  constexpr int kV = sizeof(V) / sizeof(float);
  __shared__ V sB[kSumRows - 1][kSumCols], sC[kSumRows - 1][kSumCols];
  const int x = threadIdx.x, q = threadIdx.y;
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * kSumCols + x) * kV;
  const int64_t bg = blockIdx.y;   // b * G + g
  const int64_t b = bg / G, g = bg % G, per = cgroups / G;
  const int64_t lo = g * per + q * per / kSumRows, hi = g * per + (q + 1) * per / kSumRows;
  V sb{}, sc{};
  if (i < NL) {
#pragma unroll 4
    for (int64_t cg = lo; cg < hi; ++cg) {
      const float* r = part + (b * cgroups + cg) * 2 * NL + i;
      sb += *reinterpret_cast<const V*>(r);
      sc += *reinterpret_cast<const V*>(r + NL);
    }
  }
  if (q > 0) {
    sB[q - 1][x] = sb;
    sC[q - 1][x] = sc;
  }
  __syncthreads();
  if (q == 0 && i < NL) {
#pragma unroll
    for (int r = 0; r < kSumRows - 1; ++r) {
      sb += sB[r][x];
      sc += sC[r][x];
    }
    *reinterpret_cast<V*>(dB + bg * NL + i) = sb;
    *reinterpret_cast<V*>(dC + bg * NL + i) = sc;
  }
}

// Zero the outputs that are accumulated with atomics (a plain kernel, not a
// memset, so the launch sequence can be captured in a graph).
__global__ void zero_kernel(float* p0, int64_t n0, float* p1, int64_t n1, float* p2, int64_t n2,
                            float* p3, int64_t n3, float* p4, int64_t n4) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (p0 && i < n0) p0[i] = 0.0f;
  if (p1 && i < n1) p1[i] = 0.0f;
  if (p2 && i < n2) p2[i] = 0.0f;
  if (p3 && i < n3) p3[i] = 0.0f;
  if (p4 && i < n4) p4[i] = 0.0f;
}

}  // namespace

bool scan_bwd_windows_fit(const ssm_scan_bwd_args& a) {
  const int64_t esz = a.io_dtype == SSM_BF16 ? 2 : 4;
  const int64_t rows = std::min<int64_t>(kRows, a.dim) - 1;
  const int64_t lim = int64_t{1} << 32;
  auto fits = [&](int64_t span, int64_t es) { return span * es < lim; };
  const int64_t nbk = (a.seqlen + kT - 1) / kT;
  bool ok = fits(rows * a.u_dim_stride + a.seqlen, esz) &&
            fits(rows * a.delta_dim_stride + a.seqlen, esz) &&
            fits(rows * a.dout_dim_stride + a.seqlen, esz) &&
            fits(rows * a.du_dim_stride + a.seqlen, esz) &&
            fits(rows * a.ddelta_dim_stride + a.seqlen, esz) &&
            fits((a.dstate - 1) * a.B_state_stride + a.seqlen, esz) &&
            fits((a.dstate - 1) * a.C_state_stride + a.seqlen, esz) &&
            fits(a.dstate * a.seqlen, 4) && fits((rows + 1) * nbk * a.dstate, 4);
  if (a.z) ok = ok && fits(rows * a.z_dim_stride + a.seqlen, esz) &&
                fits(rows * a.dz_dim_stride + a.seqlen, esz);
  return ok;
}

// The partial-sum path is taken whenever the caller gives a workspace.  The
// atomics' speed depends on where dB and dC sit relative to each other:
// every workgroup adds into dB(n, t) and dC(n, t) at the same moment, and at
// some offsets between the two buffers those addresses share memory channels
// (measured on the 130m-like layer: 561 us at 1 or 3 MiB apart, 713-729 us
// at 2 or 8 MiB or 1 MiB + 4 KiB; the partial sums take 605 us at every
// offset, and on the 2.8b-like layer they beat the atomics at any offset).
namespace {

// Segments of the backward: as in the forward, cut only when the batch x
// channel groups leave the machine short of workgroups, here as many as fill
// one residency round of the backward kernel (three workgroups of 4 waves
// per CU at its register count), with segments of at least 8192 tokens.
constexpr int64_t kBwdTargetGroups = 768;
constexpr int64_t kBwdMinSegLen = 8192;
constexpr int kBwdMaxSeg = 64;

int bwd_segments(int64_t groups, int64_t L) {
  if (groups >= kBwdTargetGroups / 2) return 1;
  int64_t g = std::min<int64_t>(kBwdTargetGroups / groups, std::max<int64_t>(1, L / kBwdMinSegLen));
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(g, kBwdMaxSeg)));
}

}  // namespace

size_t scan_bwd_workspace_bytes(const ssm_scan_bwd_args& a) {
  const int64_t G = a.ngroups > 1 ? a.ngroups : 1;
  const int64_t cgroups = (a.dim + kCh - 1) / kCh;
  if (a.batch <= 0 || a.dim <= 0 || a.seqlen <= 0) return 0;
  if (a.batch * G > 65535) return 0;   // the sum pass runs one grid row per (batch, group)
  const int64_t nseg = bwd_segments(a.batch * cgroups, a.seqlen);
  // dB/dC partials per channel block, then dA, dD and the bias gradient per
  // segment and batch row, then (segmented) the adjoint aggregates
  const int64_t N = a.dstate;
  return static_cast<size_t>(a.batch * cgroups * 2 * N * a.seqlen +
                             nseg * a.batch * a.dim * (N + 2) +
                             (nseg > 1 ? a.batch * a.dim * nseg * (N + 1) : 0)) *
         sizeof(float);
}

namespace {

// The backward (or, kAgg, its segment aggregate pass) with S state slots.
template <int S, bool kAgg>
void launch_bwd(bool bf16, bool softplus, dim3 grid, const BwdParams& p, hipStream_t stream) {
  const dim3 block(kThreads);
  if constexpr (kAgg) {
    if (bf16) {
      if (softplus) bwd_aggregate_kernel<uint16_t, true, S><<<grid, block, 0, stream>>>(p);
      else bwd_aggregate_kernel<uint16_t, false, S><<<grid, block, 0, stream>>>(p);
    } else {
      if (softplus) bwd_aggregate_kernel<float, true, S><<<grid, block, 0, stream>>>(p);
      else bwd_aggregate_kernel<float, false, S><<<grid, block, 0, stream>>>(p);
    }
  } else {
    if (bf16) {
      if (softplus) scan_bwd_kernel<uint16_t, true, S><<<grid, block, 0, stream>>>(p);
      else scan_bwd_kernel<uint16_t, false, S><<<grid, block, 0, stream>>>(p);
    } else {
      if (softplus) scan_bwd_kernel<float, true, S><<<grid, block, 0, stream>>>(p);
      else scan_bwd_kernel<float, false, S><<<grid, block, 0, stream>>>(p);
    }
  }
}

}  // namespace

hipError_t launch_scan_bwd(const ssm_scan_bwd_args& a, hipStream_t stream) {
  const int64_t G = a.ngroups > 1 ? a.ngroups : 1;
  const int64_t nbc = a.batch * G * a.dstate * a.seqlen;
  const size_t wneed = scan_bwd_workspace_bytes(a);
  const bool partials = wneed > 0 && a.workspace && a.workspace_bytes >= wneed;
  // Without the workspace, zero what the kernel adds into with atomics (with
  // it, every output is written whole by plain stores).
  if (!partials) {
    const int64_t nmax = std::max<int64_t>(nbc, a.dim * a.dstate);
    zero_kernel<<<dim3(static_cast<unsigned>((nmax + 255) / 256)), dim3(256), 0, stream>>>(
        a.dB, nbc, a.dC, nbc, a.dA, a.dim * a.dstate, a.dD, a.dim, a.ddelta_bias, a.dim);
  }
  if (a.seqlen == 0) {
    // no token: the gradient reaching h0 is dlast itself
    if (a.dh0) {
      if (a.dlast)
        return hipMemcpyAsync(a.dh0, a.dlast, sizeof(float) * a.batch * a.dim * a.dstate,
                              hipMemcpyDeviceToDevice, stream);
      zero_kernel<<<dim3(static_cast<unsigned>((a.batch * a.dim * a.dstate + 255) / 256)),
                    dim3(256), 0, stream>>>(a.dh0, a.batch * a.dim * a.dstate, nullptr, 0,
                                            nullptr, 0, nullptr, 0, nullptr, 0);
    }
    return hipGetLastError();
  }
  BwdParams p;
  p.u = a.u; p.delta = a.delta; p.z = a.z; p.B = a.B; p.C = a.C;
  p.A = a.A; p.D = a.D; p.bias = a.delta_bias; p.ckpt = a.checkpoints;
  p.dout = a.dout; p.dlast = a.dlast;
  p.du = a.du; p.ddelta = a.ddelta; p.dz = a.dz;
  p.dB = a.dB; p.dC = a.dC; p.dA = a.dA; p.dD = a.dD; p.dbias = a.ddelta_bias; p.dh0 = a.dh0;
  p.part = partials ? static_cast<float*>(a.workspace) : nullptr;
  const int64_t cgroups = (a.dim + kCh - 1) / kCh;
  // segments only with the workspace (the aggregates and per-segment
  // partial sums live there); without it, one segment and atomics
  p.nseg = partials ? bwd_segments(a.batch * cgroups, a.seqlen) : 1;
  {
    const int64_t seg = (a.seqlen + p.nseg - 1) / p.nseg;
    p.seg_len = static_cast<int>((seg + kGT - 1) / kGT * kGT);
    p.nseg = static_cast<int>((a.seqlen + p.seg_len - 1) / p.seg_len);
  }
  p.pdA = partials ? p.part + a.batch * cgroups * 2 * a.dstate * a.seqlen : nullptr;
  p.pdD = partials ? p.pdA + p.nseg * a.batch * a.dim * a.dstate : nullptr;
  p.pdb = partials ? p.pdD + p.nseg * a.batch * a.dim : nullptr;
  p.agg = partials && p.nseg > 1 ? p.pdb + p.nseg * a.batch * a.dim : nullptr;
  p.usb = a.u_batch_stride; p.usd = a.u_dim_stride;
  p.dsb = a.delta_batch_stride; p.dsd = a.delta_dim_stride;
  p.zsb = a.z_batch_stride; p.zsd = a.z_dim_stride;
  p.Bsb = a.B_batch_stride; p.Bsn = a.B_state_stride;
  p.Csb = a.C_batch_stride; p.Csn = a.C_state_stride;
  p.Bsg = G > 1 ? a.B_group_stride : 0; p.Csg = G > 1 ? a.C_group_stride : 0;
  p.ngroups = G; p.cpg = a.dim / G;
  p.Asd = a.A_dim_stride; p.Asn = a.A_state_stride;
  p.gsb = a.dout_batch_stride; p.gsd = a.dout_dim_stride;
  p.dusb = a.du_batch_stride; p.dusd = a.du_dim_stride;
  p.ddsb = a.ddelta_batch_stride; p.ddsd = a.ddelta_dim_stride;
  p.dzsb = a.dz_batch_stride; p.dzsd = a.dz_dim_stride;
  p.batch = a.batch; p.dim = a.dim; p.L = static_cast<int>(a.seqlen);
  p.N = static_cast<int>(a.dstate);
  p.nbk = static_cast<int>((a.seqlen + kT - 1) / kT);
  p.cgroups = (a.dim + kCh - 1) / kCh;
  const dim3 grid(static_cast<unsigned>(a.batch * p.cgroups * p.nseg));
  const bool sp = a.delta_softplus != 0, bf = a.io_dtype == SSM_BF16;
  const int S = a.dstate <= 16 ? 1 : a.dstate <= 32 ? 2 : 4;   // state slots per lane
  if (p.nseg > 1) {
    // pass 1: the adjoint aggregates of segments 1..nseg-1
    const dim3 agrid(static_cast<unsigned>(a.batch * p.cgroups * (p.nseg - 1)));
    if (S == 1) launch_bwd<1, true>(bf, sp, agrid, p, stream);
    else if (S == 2) launch_bwd<2, true>(bf, sp, agrid, p, stream);
    else launch_bwd<4, true>(bf, sp, agrid, p, stream);
  }
  if (S == 1) launch_bwd<1, false>(bf, sp, grid, p, stream);
  else if (S == 2) launch_bwd<2, false>(bf, sp, grid, p, stream);
  else launch_bwd<4, false>(bf, sp, grid, p, stream);
  if (partials) {
    // NL = dstate * seqlen; float4 when the bases are 16-byte aligned and NL
    // is a multiple of 4
    const int64_t NL = a.dstate * a.seqlen;
    auto al16 = [](const void* ptr) { return reinterpret_cast<uintptr_t>(ptr) % 16 == 0; };
    const dim3 sblock(kSumCols, kSumRows);
    if (al16(p.part) && al16(a.dB) && al16(a.dC) && NL % 4 == 0) {
      const int64_t cols = (NL / 4 + kSumCols - 1) / kSumCols;
      partial_sum_kernel<float4><<<dim3(static_cast<unsigned>(cols), static_cast<unsigned>(a.batch * G)),
                                   sblock, 0, stream>>>(p.part, a.dB, a.dC, NL, p.cgroups, G);
    } else {
      const int64_t cols = (NL + kSumCols - 1) / kSumCols;
      partial_sum_kernel<float><<<dim3(static_cast<unsigned>(cols), static_cast<unsigned>(a.batch * G)),
                                  sblock, 0, stream>>>(p.part, a.dB, a.dC, NL, p.cgroups, G);
    }
    param_sum_kernel<<<dim3(static_cast<unsigned>((a.dim * a.dstate + 255) / 256)), dim3(256), 0, stream>>>(
        p.pdA, p.pdD, p.pdb, a.dA, a.dD, a.ddelta_bias, p.nseg * a.batch, a.dim, a.dstate);
  }
  return hipGetLastError();
}

}  // namespace ssm

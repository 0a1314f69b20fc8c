// ssd_fwd.hip -- the Mamba-2 SSM (SSD layer) prefill on gfx950, chunked and
// on the matrix cores.
//
// Per batch row b, head h (group g of its B/C), head channel p and state n
// (Mamba-2 section of the mamba_ssm notes; skill page, Mamba-2 configuration:
// multi-head, headdim, ngroups; the printed Mamba-2 parameter count: one A,
// D and step bias per head):
//   Delta_t  = softplus(dt[b,t,h] + bias[h])
//   S_t[p,n] = exp(Delta_t A[h]) S_{t-1}[p,n] + Delta_t B[b,t,g,n] x[b,t,h,p]
//   y_t[p]   = sum_n C[b,t,g,n] S_t[p,n] + D[h] x[b,t,h,p],  out = y silu(z)
//
// The same map is a structured matrix (state space duality): with
// a_t = A * (Delta_0 + ... + Delta_t) inside a chunk of Q = 64 tokens and
// H_in the state entering the chunk,
//   y_t   = sum_{s<=t} (C_t . B_s) exp(a_t - a_s) Delta_s x_s + exp(a_t) C_t H_in
//   H_out = exp(a_{Q-1}) H_in + sum_s exp(a_{Q-1} - a_s) Delta_s B_s x_s^T
// which are four small matrix products per chunk:
//   scores  G[s][t]  = sum_n B_s[n] C_t[n]                      (Q x Q, k = N)
//   intra   Y1[t][p] = sum_s M[t][s] x_s[p],  M = G^T * decay mask * Delta
//   state   Y2[t][p] = exp(a_t) sum_n C_t[n] H_in[n][p]         (k = N)
//   update  H_out^T[p][n] = exp(a_{Q-1}) H_in^T + sum_s w_s x_s[p] B_s[n]  (k = Q),
//           w_s = exp(a_{Q-1} - a_s) Delta_s
//
// Work decomposition.  A workgroup (4 wavefronts) owns one (batch, head,
// PB blocks of 16 head channels) and walks the sequence chunk by chunk,
// keeping the fp32 state H^T (16 PB channels x N states) in MFMA accumulator
// registers: wavefront w holds state columns n in blocks w, w+4, ... .  The
// chunk's step scan, B/C staging, score tiles and masks are formed once and
// used for all PB channel blocks.  Wavefront w also
// owns output tokens 16w..16w+15 of each chunk: it forms the score tiles for
// source blocks 0..w (causal), masks them, and feeds them straight into the
// next product: the accumulator layout of a 16x16 tile (lane l holds rows
// 4(l/16)+i, column l%16) is exactly the operand layout of the following
// 16x16x16 product (lane l supplies row l%16, k = 4(l/16)+i), so the scores
// never leave registers.  B, C and x of a chunk are staged in LDS by the
// whole workgroup; the state goes through LDS once per chunk for the state
// product.  bf16 IO uses v_mfma_f32_16x16x32_bf16 where two 16-wide k blocks
// pair up (the scores, the state product, the state update) and
// v_mfma_f32_16x16x16_bf16 for the causal intra-chunk product (fp32
// accumulation; the masked scores and the decay-weighted x are rounded to
// bf16, and the state operand is split into a bf16 value and its bf16
// remainder);
// fp32 IO uses v_mfma_f32_16x16x4_f32 four times per 16-wide k block, each
// lane supplying the same four consecutive k values one per instruction.
//
// Long sequences with few heads.  The state recurrence is linear (Mamba paper
// notes, sections 5.3/5.4: a long input is cut into chunks with the state
// handed on), and a head's decay exp(Delta A) is one scalar per token, so
// with a caller workspace the sequence is cut into G segments of whole
// chunks, in two launches of this kernel:
//   pass 1  every segment from a zero state (segment 0 from h0), writing
//           every output, and recording its end state H_g and its step-size
//           sum S_g;
//   pass 2  segment g >= 1 from the exact state entering it, h_in =
//           fold_{i<g} (exp(A S_i) h + H_i), rewriting outputs while the
//           free response exp(A S) |h_in| (S: the step sizes since the
//           segment start) exceeds 2^-24 of the largest state entry of the
//           workgroup's channels, checked once per chunk; the last segment's
//           workgroups also write last_state = exp(A S_g) h_in + H_g.
// Past that point pass 1's values are the sequential result up to rounding.
#include <algorithm>

#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kQ = 64;          // tokens per chunk
constexpr int kPB = 16;         // head channels per channel block
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));

struct SsdParams {
  const void* x;
  const void* dt;
  const void* z;
  const void* B;
  const void* C;
  const float* A;
  const float* D;
  const float* bias;
  const float* h0;
  float* last;
  void* out;
  int64_t xsb, xsh, dsb, zsb, zsh, Bsb, Bsg, Csb, Csg, osb, osh;
  // byte strides between consecutive tokens (a chunk's 64 rows span less
  // than 2^31 bytes, so these and every in-chunk offset are 32-bit)
  uint32_t xsl, dsl, zsl, Bsl, Csl, osl;
  int L, H, P, G, N;
  int pblocks;   // workgroups per head: ceil(P / (16 PB))
  // segmented sequences: mode 0 one segment, 1 and 2 the two passes
  int mode, nseg, seg_chunks;   // segments, chunks per segment
  float* aggH;   // [batch * H][nseg][P][N] segment end states (from a zero start)
  float* aggS;   // [batch * H][nseg] segment step-size sums
};

// Storage of one IO element in LDS and its widening.
template <typename T> struct Lds;
template <> struct Lds<float> {
  using E = float;
  __device__ static __forceinline__ float f(E v) { return v; }
  __device__ static __forceinline__ E from(float v) { return v; }
};
template <> struct Lds<uint16_t> {
  using E = uint16_t;
  __device__ static __forceinline__ float f(E v) { return bf16_to_f32(v); }
  // round to nearest even in hardware (v_cvt_pk_bf16_f32)
  __device__ static __forceinline__ E from(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
  }
};

// A lane's operand fragment of one 16x16 tile step over a 16-wide k block:
// four consecutive k values (k = 4 (l/16) + i) of its A row or B column, as
// the product instruction takes them (four bf16, or four fp32).
template <typename T> struct Frag;
template <> struct Frag<uint16_t> { using V = v4s; };
template <> struct Frag<float> { using V = v4f; };

template <typename T>
__device__ __forceinline__ v4f mma16(typename Frag<T>::V a, typename Frag<T>::V b, v4f c) {
  if constexpr (sizeof(T) == 2) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], c, 0, 0, 0);
    return c;
  }
}

// bf16, k = 32 (v_mfma_f32_16x16x32_bf16, twice the work of the k = 16 form
// at the same issue rate on gfx950).  The instruction sums over its 32 k
// slots, pairing slot v of A's lane 16 g + i with slot v of B's lane
// 16 g + j, so any placement of the k values into (lane group, slot) that A
// and B share gives the same sum: two k = 16 fragments side by side (slots
// 0-3 and 4-7) give the sum of their two k = 16 products, and eight
// consecutive k values per lane (slots 0-7 of lane group g holding k = 8 g
// .. 8 g + 7) one 32-wide k block.
__device__ __forceinline__ v4f mma32(v8s a, v8s b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b),
                                                 c, 0, 0, 0);
}
__device__ __forceinline__ v4f mma32(v4s a0, v4s a1, v4s b0, v4s b1, v4f c) {
  return mma32(__builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7),
               __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7), c);
}

// Four consecutive LDS elements (8 or 16 bytes, aligned) as a fragment.
template <typename T>
__device__ __forceinline__ typename Frag<T>::V ldsf(const typename Lds<T>::E* p) {
  return *reinterpret_cast<const typename Frag<T>::V*>(p);
}

// bf16 operand fragment through the LDS transpose read (ds_read_b64_tr_b16).
// Within each group of 16 lanes, lane i receives element k from the chunk
// (four consecutive elements) that lane 4k + i / 4 of the group addresses,
// its element i % 4 (lane layout checked on the device with an in-bounds
// probe).  So when lane r of group g addresses row 4g + r / 4, columns
// 4 (r % 4) .. + 3 of a row-major tile X[k][c], lane 16 g + i receives
// X[4g + k][i] for k = 0..3: the operand fragment of column i (k = 4g + k')
// of a 16x16x16 product, equally the A fragment of row i of X^T.
__device__ __forceinline__ v4s lds_tr(const uint16_t* row_chunk) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (v4s __attribute__((address_space(3)))*)(row_chunk));
}

// Two fp32 values rounded to bf16 (nearest even) in one word, a low.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Four LDS elements (already in the fragment's element type) as a fragment.
template <typename T>
__device__ __forceinline__ typename Frag<T>::V tofrag_bits(typename Lds<T>::E a, typename Lds<T>::E b,
                                                           typename Lds<T>::E c, typename Lds<T>::E d) {
  if constexpr (sizeof(T) == 2) {
    v4s v;
    v[0] = static_cast<short>(a); v[1] = static_cast<short>(b);
    v[2] = static_cast<short>(c); v[3] = static_cast<short>(d);
    return v;
  } else {
    return v4f{a, b, c, d};
  }
}

// Four fp32 values as a fragment (rounded to bf16 for bf16 IO).
template <typename T>
__device__ __forceinline__ typename Frag<T>::V tofrag(float a, float b, float c, float d) {
  if constexpr (sizeof(T) == 2) {
    v4s v;
    v[0] = __builtin_bit_cast(short, static_cast<__bf16>(a));
    v[1] = __builtin_bit_cast(short, static_cast<__bf16>(b));
    v[2] = __builtin_bit_cast(short, static_cast<__bf16>(c));
    v[3] = __builtin_bit_cast(short, static_cast<__bf16>(d));
    return v;
  } else {
    return v4f{a, b, c, d};
  }
}

// The one-block bf16 kernel with 64 states and vector staging fits four
// wavefronts per SIMD (128 registers) without spilling; asking for that keeps
// a grid of 4 x 256 workgroups in one wave of residency.
// One DPP step on a float: lanes outside the row and bank masks, and lanes
// whose source lies outside their row, read 0.
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ float dpp0(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xf, true));
}

// Inclusive prefix sum over the 64 lanes of a wavefront in registers: row
// shifts by 1, 2, 4 and 8 sum each 16-lane row, then row_bcast:15 adds row
// 0's total to row 1 and row 2's to row 3, and row_bcast:31 adds lane 31's
// (rows 0 and 1) to rows 2 and 3.
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += dpp0<0x111>(v);         // row_shr:1
  v += dpp0<0x112>(v);         // row_shr:2
  v += dpp0<0x114>(v);         // row_shr:4
  v += dpp0<0x118>(v);         // row_shr:8
  v += dpp0<0x142, 0xa>(v);    // row_bcast:15 into rows 1 and 3
  v += dpp0<0x143, 0xc>(v);    // row_bcast:31 into rows 2 and 3
  return v;
}

template <typename T, int NMAX, bool kVec, int PB>
constexpr bool kFourWaves() { return sizeof(T) == 2 && NMAX == 64 && kVec && PB == 1; }

// kVec: B/C rows, x rows and their strides are 16-byte (x: 8-byte for bf16)
// aligned and dstate is a multiple of NMAX / 4, so staging uses vector loads
// and 16-byte LDS stores; otherwise element-wise loads.  PB: blocks of 16
// head channels per workgroup (the score tiles, masks and B/C staging of a
// chunk are shared by all of them).  kSegd: the passes of a segmented
// sequence (p.mode 1 or 2); without it, one segment and none of their code.
template <typename T, int NMAX, bool kSoftplus, bool kVec, int PB, bool kSegd>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(kFourWaves<T, NMAX, kVec, PB>() ? 4 : 1)))
void ssd_fwd_kernel(SsdParams p) {
  using L = Lds<T>;
  using E = typename L::E;
  constexpr int kPadE = 16 / sizeof(E);        // 16 bytes of padding per row
  constexpr int NP = NMAX + kPadE;             // LDS pitch of a B / C row
  constexpr int QP = kQ + kPadE;               // LDS pitch of an x^T row
  constexpr int NB = NMAX / 16;                // 16-wide state blocks
  constexpr int NBW = (NB + kWaves - 1) / kWaves;  // state blocks per wavefront
  constexpr int PC = kPB * PB;                 // head channels per workgroup
  constexpr bool kBF = sizeof(E) == 2;
  __shared__ __align__(16) E sB[kQ][NP];       // B_s[n]
  __shared__ __align__(16) E sC[kQ][NP];       // C_t[n]
  // fp32: x, the decay-weighted x and the state operand stored transposed
  // (the fragments then read four consecutive k values); bf16: stored as
  // they are, [channel block][token or state][16 channels] (32-byte rows),
  // with 8-byte stores, and read through the transpose read (lds_tr)
  constexpr int kFP = kBF ? 1 : PC;
  __shared__ __align__(16) E sXT[kFP][kBF ? 1 : QP];      // x_s[p], transposed
  __shared__ __align__(16) E sXW[kFP][kBF ? 1 : QP];      // exp(a_{Q-1} - a_s) Delta_s x_s[p], transposed
  __shared__ __align__(16) E sHT[kFP][kBF ? 1 : NP];      // H_in^T[p][n] (operand copy)
  constexpr int kBP = kBF ? PB : 1;
  __shared__ __align__(16) E sXb[kBP][kBF ? kQ : 1][kPB];     // x_s[p]
  __shared__ __align__(16) E sXWb[kBP][kBF ? kQ : 1][kPB];    // exp(a_{Q-1} - a_s) Delta_s x_s[p]
  __shared__ __align__(16) E sHb[kBP][kBF ? NMAX : 1][kPB];   // H_in[n][p], bf16 value
  // bf16: the rounding remainder H - bf16(H), so that the state product
  // carries the fp32 state to about 16 bits (two bf16 products)
  __shared__ __align__(16) E sHL[kBP][kBF ? NMAX : 1][kPB];
  __shared__ __align__(16) float sDl[kQ];      // Delta_s (0 past the end)
  __shared__ __align__(16) float sLa[kQ];      // a_t * log2(e)
  // segmented passes (kept in LDS, not in registers across the chunk loop):
  __shared__ float sRed[kWaves];               // per-wavefront state maxima (pass 2 check)
  __shared__ float sHin[kWaves];               // per-wavefront maxima of |h_in| (pass 2)
  __shared__ double sSum;                      // step sizes of the chunks done

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;    // row / column and k quarter
  // workgroup = ((b * nseg' + seg') * H + h) * pblocks + pb; pass 2 skips
  // segment 0 (seg = seg' + 1)
  const int nsg = kSegd ? (p.mode == 2 ? p.nseg - 1 : p.nseg) : 1;
  const int pb = blockIdx.x % p.pblocks;
  const int h = (blockIdx.x / p.pblocks) % p.H;
  const int64_t bs = blockIdx.x / (static_cast<int64_t>(p.pblocks) * p.H);
  const int seg = kSegd ? static_cast<int>(bs % nsg) + (p.mode == 2 ? 1 : 0) : 0;
  const int64_t b = bs / nsg;
  const int g = h / (p.H / p.G);
  const int p0 = pb * PC;
  const int N = p.N;
  const float a2 = p.A[h] * kLog2e;
  const float bias = p.bias ? p.bias[h] : 0.0f;
  const float Dh = p.D ? p.D[h] : 0.0f;

  const T* xg = static_cast<const T*>(p.x) + b * p.xsb + static_cast<int64_t>(h) * p.xsh + p0;
  const T* dtg = static_cast<const T*>(p.dt) + b * p.dsb + h;
  const T* zg = p.z ? static_cast<const T*>(p.z) + b * p.zsb + static_cast<int64_t>(h) * p.zsh + p0
                    : nullptr;
  const T* Bg = static_cast<const T*>(p.B) + b * p.Bsb + static_cast<int64_t>(g) * p.Bsg;
  const T* Cg = static_cast<const T*>(p.C) + b * p.Csb + static_cast<int64_t>(g) * p.Csg;
  T* og = static_cast<T*>(p.out) + b * p.osb + static_cast<int64_t>(h) * p.osh + p0;

  // State H^T tiles: lane holds H^T[p = 16 q + 4 lq + i][n = 16 m + lr] for
  // channel block q and state block m = wave + 4 j.
  v4f Hs[NBW][PB];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const int n = 16 * (wave + kWaves * j) + lr;
#pragma unroll
    for (int q = 0; q < PB; ++q) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pp = p0 + kPB * q + 4 * lq + i;
        Hs[j][q][i] = (p.h0 && seg == 0 && n < N && pp < p.P)
                          ? p.h0[((b * p.H + h) * p.P + pp) * static_cast<int64_t>(N) + n]
                          : 0.0f;
      }
    }
  }
  const int64_t bh = b * p.H + h;
  // pass 2: the exact state entering the segment, folded from the end
  // states of segments 0..seg-1 (segment 0's includes h0), and its largest
  // entry over this workgroup's channels; the last segment also writes the
  // final state
  float hin_max = 0.0f;
  if (kSegd && p.mode == 2) {
    const float* aS = p.aggS + bh * p.nseg;
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int n = 16 * (wave + kWaves * j) + lr;
#pragma unroll
      for (int q = 0; q < PB; ++q) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pp = p0 + kPB * q + 4 * lq + i;
          if (n < N && pp < p.P) {
            const float* aH = p.aggH + (bh * p.nseg * p.P + pp) * static_cast<int64_t>(N) + n;
            const int64_t sst = static_cast<int64_t>(p.P) * N;   // from one segment to the next
            float hv = aH[0];
            for (int k = 1; k < seg; ++k) hv = fmaf(__builtin_amdgcn_exp2f(a2 * aS[k]), hv, aH[k * sst]);
            Hs[j][q][i] = hv;
            // a non-finite entry never lets the rescan stop
            hin_max = fmaxf(hin_max, hv == hv ? fabsf(hv) : __builtin_huge_valf());
            if (p.last && seg == p.nseg - 1)
              p.last[(bh * p.P + pp) * static_cast<int64_t>(N) + n] =
                  fmaf(__builtin_amdgcn_exp2f(a2 * aS[seg]), hv, aH[seg * sst]);
          }
        }
      }
    }
  }
  if (kSegd && p.mode == 2) {
    // per wavefront; the workgroup's maximum is taken where it is used (the
    // chunk loop's barriers order these stores before those reads)
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) hin_max = fmaxf(hin_max, __shfl_xor(hin_max, m, 64));
    if (lane == 0) sHin[wave] = hin_max;
  }
  if (kSegd && tid == 0) sSum = 0.0;
  // operand copy of the state (bf16: value and remainder)
  auto store_ht = [&]() {
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int m = wave + kWaves * j;
      if (m < NB) {
#pragma unroll
        for (int q = 0; q < PB; ++q) {
          if constexpr (kBF) {
            // lane holds H[n = 16 m + lr][p = 16 q + 4 lq + i], i = 0..3:
            // one 8-byte store of the four values and one of the remainders
            E hi[4], lo[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              hi[i] = L::from(Hs[j][q][i]);
              lo[i] = L::from(Hs[j][q][i] - L::f(hi[i]));
            }
            *reinterpret_cast<uint2*>(&sHb[q][16 * m + lr][4 * lq]) =
                make_uint2(hi[0] | static_cast<uint32_t>(hi[1]) << 16, hi[2] | static_cast<uint32_t>(hi[3]) << 16);
            *reinterpret_cast<uint2*>(&sHL[q][16 * m + lr][4 * lq]) =
                make_uint2(lo[0] | static_cast<uint32_t>(lo[1]) << 16, lo[2] | static_cast<uint32_t>(lo[3]) << 16);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) sHT[kPB * q + 4 * lq + i][16 * m + lr] = L::from(Hs[j][q][i]);
          }
        }
      }
    }
  };
  store_ht();

  // Staging of one chunk.  Thread tid covers B/C row s = tid / 4, quarter
  // (tid % 4) of the NMAX states, and x row s, channels 16 q + 4 (tid % 4)
  // .. +3 of each channel block q; every thread also loads the step of token
  // (tid % 64) for its wavefront's scan.  Every load goes through a buffer
  // window that starts at the chunk and ends where the chunk's rows of the
  // tensor's (batch, head or group) slice end, so the loads are issued
  // unconditionally (past the end they read zero) and all at once; validity
  // is applied by selects when the values are written to LDS.
  const int srow = tid >> 2, squart = tid & 3;
  constexpr int kQn = NMAX / 4;               // states per thread per row
  constexpr int ES = Elem<T>::kSize;
  const int nchunks = (p.L + kQ - 1) / kQ;
  constexpr int kQw = kQn * ES / 4;            // dwords per thread per B/C row
  constexpr int kXw = 4 * ES / 4;              // dwords of a thread's 4 x values
  struct Stage {
    // element bits (scalar path) or packed dwords (vector path)
    uint32_t b[kVec ? kQw : kQn], c[kVec ? kQw : kQn], x[PB][kVec ? kXw : 4], dt, z[PB][4];
  };
  auto window = [&](const T* base, uint32_t seq_bytes, int inner, int t0) {
    // bytes from token t0's row to the end of the chunk's last row (at most
    // 64 rows; the host keeps that below 2^31); empty past the sequence
    const int rows = std::min(p.L - 1 - t0, kQ - 1);
    const uint32_t bytes = rows < 0 ? 0u : static_cast<uint32_t>(rows) * seq_bytes + inner * ES;
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(base) + static_cast<int64_t>(t0) * seq_bytes),
        0, static_cast<int>(bytes), kRsrcWord3);
  };
  // per-lane byte offsets inside a chunk's windows (the same every chunk)
  const uint32_t ob = srow * p.Bsl + squart * kQn * ES;
  const uint32_t oc = srow * p.Csl + squart * kQn * ES;
  const uint32_t ox0 = srow * p.xsl + 4 * squart * ES;     // + 16 q ES for block q
  const uint32_t odt = lane * p.dsl;
  const uint32_t oz0 = (16 * wave + 4 * lq) * p.zsl + lr * ES;   // + i zsl + 16 q ES
  const uint32_t oo0 = (16 * wave + 4 * lq) * p.osl + lr * ES;   // likewise for out
  auto load_stage = [&](int c) {
    Stage st;
    const int t0 = c * kQ;
    const __amdgpu_buffer_rsrc_t rb = window(Bg, p.Bsl, N, t0);
    const __amdgpu_buffer_rsrc_t rc = window(Cg, p.Csl, N, t0);
    const __amdgpu_buffer_rsrc_t rx = window(xg, p.xsl, p.P - p0, t0);
    const __amdgpu_buffer_rsrc_t rd = window(dtg, p.dsl, 1, t0);
    if constexpr (kVec) {
#pragma unroll
      for (int k = 0; k < kQw / 4; ++k) {
        const v4u vb = __builtin_amdgcn_raw_buffer_load_b128(rb, ob + 16 * k, 0, 0);
        const v4u vc = __builtin_amdgcn_raw_buffer_load_b128(rc, oc + 16 * k, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          st.b[4 * k + j] = vb[j];
          st.c[4 * k + j] = vc[j];
        }
      }
#pragma unroll
      for (int q = 0; q < PB; ++q) {
        const uint32_t ox = ox0 + kPB * q * ES;
        if constexpr (kXw == 4) {
          const v4u vx = __builtin_amdgcn_raw_buffer_load_b128(rx, ox, 0, 0);
#pragma unroll
          for (int j = 0; j < 4; ++j) st.x[q][j] = vx[j];
        } else {
          const v2u vx = __builtin_amdgcn_raw_buffer_load_b64(rx, ox, 0, 0);
          st.x[q][0] = vx[0];
          st.x[q][1] = vx[1];
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < kQn; ++k) {
        st.b[k] = Elem<T>::load(rb, ob + k * ES);
        st.c[k] = Elem<T>::load(rc, oc + k * ES);
      }
#pragma unroll
      for (int q = 0; q < PB; ++q) {
        const uint32_t ox = ox0 + kPB * q * ES;
#pragma unroll
        for (int k = 0; k < 4; ++k) st.x[q][k] = Elem<T>::load(rx, ox + k * ES);
      }
    }
    st.dt = Elem<T>::load(rd, odt);
    // the gate at this lane's output positions (t = 16 w + 4 lq + i,
    // p = 16 q + lr)
    if (zg) {
      const __amdgpu_buffer_rsrc_t rz = window(zg, p.zsl, p.P - p0, t0);
#pragma unroll
      for (int q = 0; q < PB; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          st.z[q][i] = Elem<T>::load(rz, oz0 + i * p.zsl + kPB * q * ES);
    } else {
#pragma unroll
      for (int q = 0; q < PB; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) st.z[q][i] = 0u;
    }
    return st;
  };
  // raw bits as an LDS element, or zero: a mask, not a branch
  auto raw = [](uint32_t v, bool keep) -> E {
    const uint32_t m = v & (keep ? 0xffffffffu : 0u);
    if constexpr (sizeof(E) == 2) return static_cast<E>(m);
    else return __uint_as_float(m);
  };
  // this segment's chunks
  const int c_beg = kSegd ? seg * p.seg_chunks : 0;
  const int c_end = kSegd ? std::min(nchunks, c_beg + p.seg_chunks) : nchunks;
  Stage st;
  if (c_beg < c_end) st = load_stage(c_beg);
  for (int c = c_beg; c < c_end; ++c) {
    if (kSegd && p.mode == 2 && c > c_beg) {
      // pass 2: stop once the incoming state's free response is below fp32
      // resolution of this workgroup's state (the chunk's loads in flight
      // are simply dropped)
      float hm = 0.0f;
#pragma unroll
      for (int j = 0; j < NBW; ++j)
#pragma unroll
        for (int q = 0; q < PB; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) hm = fmaxf(hm, fabsf(Hs[j][q][i]));
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) hm = fmaxf(hm, __shfl_xor(hm, m, 64));
      if (lane == 0) sRed[wave] = hm;
      __syncthreads();
      hm = fmaxf(fmaxf(sRed[0], sRed[1]), fmaxf(sRed[2], sRed[3]));
      const float hi = fmaxf(fmaxf(sHin[0], sHin[1]), fmaxf(sHin[2], sHin[3]));
      const float fr = __builtin_amdgcn_exp2f(a2 * static_cast<float>(sSum)) * hi;
      if (fr <= 0x1p-24f * hm) break;   // the same values in every thread
    }
    const int t0 = c * kQ;
    const int nv = std::min(kQ, p.L - t0);
    // ---- B, C and x^T of this chunk into LDS, before the step-size scan so
    // that the stores are under way while it runs (the barrier closing the
    // previous chunk freed these buffers) ----
    uint2 xm[PB];   // bf16 vector staging: the masked words of x, for the weighted copy
    {
      const bool tv = srow < nv;
      if constexpr (kVec) {
        // a whole quarter row is real or padding (dstate % (NMAX/4) == 0)
        const uint32_t m = (tv && squart * kQn < N) ? 0xffffffffu : 0u;
#pragma unroll
        for (int k = 0; k < kQw / 4; ++k) {
          const int col = squart * kQn + k * (16 / ES);
          *reinterpret_cast<uint4*>(&sB[srow][col]) =
              make_uint4(st.b[4 * k] & m, st.b[4 * k + 1] & m, st.b[4 * k + 2] & m, st.b[4 * k + 3] & m);
          *reinterpret_cast<uint4*>(&sC[srow][col]) =
              make_uint4(st.c[4 * k] & m, st.c[4 * k + 1] & m, st.c[4 * k + 2] & m, st.c[4 * k + 3] & m);
        }
      } else {
#pragma unroll
        for (int k = 0; k < kQn; ++k) {
          const int n = squart * kQn + k;
          const bool ok = tv && n < N;
          sB[srow][n] = raw(st.b[k], ok);
          sC[srow][n] = raw(st.c[k], ok);
        }
      }
#pragma unroll
      for (int q = 0; q < PB; ++q) {
        if constexpr (kBF && kVec) {
          // the thread's four channels as loaded (two words), each half
          // kept where its row and channel are real: one 8-byte store
          const int vc = p.P - p0 - (kPB * q + 4 * squart);  // real channels from the first
          const uint32_t m0 = !tv ? 0u : vc >= 2 ? 0xffffffffu : vc == 1 ? 0xffffu : 0u;
          const uint32_t m1 = !tv ? 0u : vc >= 4 ? 0xffffffffu : vc == 3 ? 0xffffu : 0u;
          xm[q] = make_uint2(st.x[q][0] & m0, st.x[q][1] & m1);
          *reinterpret_cast<uint2*>(&sXb[q][srow][4 * squart]) = xm[q];
          continue;
        }
        E xv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int pp = kPB * q + 4 * squart + k;
          uint32_t v;
          if constexpr (kVec) v = ES == 2 ? (st.x[q][k / 2] >> (16 * (k % 2))) : st.x[q][k % kXw];
          else v = st.x[q][k];
          xv[k] = raw(v, tv && p0 + pp < p.P);
          if constexpr (!kBF) sXT[pp][srow] = xv[k];
        }
        // bf16: row s, channels 4 squart .. + 3 of block q, one 8-byte store
        if constexpr (kBF)
          *reinterpret_cast<uint2*>(&sXb[q][srow][4 * squart]) =
              make_uint2(xv[0] | static_cast<uint32_t>(xv[1]) << 16, xv[2] | static_cast<uint32_t>(xv[3]) << 16);
      }
    }
    // ---- the chunk's step sizes: every wavefront runs the 64-token scan
    // (lane = token), so that each staging thread has the weight of its row
    float w_row;
    {
      const bool tv = lane < nv;
      const float x = Elem<T>::f32(st.dt) + bias;
      float dl = kSoftplus ? softplus_f32(x) : x;
      dl = tv ? dl : 0.0f;
      const float cum = wave_prefix_sum(dl);
      const float la = cum * a2;
      const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(la), 63));
      if constexpr (kSegd) {
        // segmented: read at the next chunk's top and after the loop, past
        // this chunk's barriers
        const float csum = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), 63));
        if (tid == 0) sSum += static_cast<double>(csum);
      }
      const float w = __builtin_amdgcn_exp2f(last - la) * dl;   // exp(a_{Q-1} - a_s) Delta_s
      w_row = __shfl(w, srow, 64);
      if (wave == 0) {
        sDl[lane] = dl;
        sLa[lane] = la;
      }
    }
    // ---- decay-weighted x^T (needs the step sizes) ----
    {
      const bool tv = srow < nv;
#pragma unroll
      for (int q = 0; q < PB; ++q) {
        if constexpr (kBF && kVec) {
          const uint2 v = xm[q];
          *reinterpret_cast<uint2*>(&sXWb[q][srow][4 * squart]) = make_uint2(
              pack_bf16x2(__uint_as_float(v.x << 16) * w_row, __uint_as_float(v.x & 0xffff0000u) * w_row),
              pack_bf16x2(__uint_as_float(v.y << 16) * w_row, __uint_as_float(v.y & 0xffff0000u) * w_row));
          continue;
        }
        E xw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int pp = kPB * q + 4 * squart + k;
          uint32_t v;
          if constexpr (kVec) v = ES == 2 ? (st.x[q][k / 2] >> (16 * (k % 2))) : st.x[q][k % kXw];
          else v = st.x[q][k];
          const E xv = raw(v, tv && p0 + pp < p.P);
          xw[k] = L::from(L::f(xv) * w_row);
          if constexpr (!kBF) sXW[pp][srow] = xw[k];
        }
        if constexpr (kBF)
          *reinterpret_cast<uint2*>(&sXWb[q][srow][4 * squart]) =
              make_uint2(xw[0] | static_cast<uint32_t>(xw[1]) << 16, xw[2] | static_cast<uint32_t>(xw[3]) << 16);
      }
    }
    __syncthreads();
    // this chunk's gate, then the next chunk's loads fly while this one is
    // computed
    uint32_t zr[PB][4];
#pragma unroll
    for (int q = 0; q < PB; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) zr[q][i] = st.z[q][i];
    if (c + 1 < c_end) st = load_stage(c + 1);

    // ---- outputs of tokens 16 w .. 16 w + 15 ----
    {
      const int tb = 16 * wave;
      const float la_t = sLa[tb + lr];
      v4f y1[PB];
#pragma unroll
      for (int q = 0; q < PB; ++q) y1[q] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      for (int sbk = 0; sbk <= wave; ++sbk) {
        // scores G[s][t] for s in block sbk, t in block wave: A = B (row s,
        // k = n), B operand = C^T (k = n, column t)
        v4f sc = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (kBF) {   // 32-wide n blocks, eight consecutive n per lane
#pragma unroll
          for (int nb = 0; nb < NB / 2; ++nb)
            sc = mma32(*reinterpret_cast<const v8s*>(&sB[16 * sbk + lr][32 * nb + 8 * lq]),
                       *reinterpret_cast<const v8s*>(&sC[tb + lr][32 * nb + 8 * lq]), sc);
        } else {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            sc = mma16<T>(ldsf<T>(&sB[16 * sbk + lr][16 * nb + 4 * lq]),
                          ldsf<T>(&sC[tb + lr][16 * nb + 4 * lq]), sc);
        }
        // mask and scale: lane holds s = 16 sbk + 4 lq + i, t = tb + lr
        const int s0 = 16 * sbk + 4 * lq;
        const float4 la_s = *reinterpret_cast<const float4*>(&sLa[s0]);
        const float4 dl_s = *reinterpret_cast<const float4*>(&sDl[s0]);
        const int t = tb + lr;
        const float m0 = s0 + 0 <= t ? sc[0] * __builtin_amdgcn_exp2f(la_t - la_s.x) * dl_s.x : 0.0f;
        const float m1 = s0 + 1 <= t ? sc[1] * __builtin_amdgcn_exp2f(la_t - la_s.y) * dl_s.y : 0.0f;
        const float m2 = s0 + 2 <= t ? sc[2] * __builtin_amdgcn_exp2f(la_t - la_s.z) * dl_s.z : 0.0f;
        const float m3 = s0 + 3 <= t ? sc[3] * __builtin_amdgcn_exp2f(la_t - la_s.w) * dl_s.w : 0.0f;
        // intra: A = M (row t, k = s), B operand = x (k = s, column p) of
        // every channel block
        const auto mf = tofrag<T>(m0, m1, m2, m3);
#pragma unroll
        for (int q = 0; q < PB; ++q) {
          if constexpr (kBF) y1[q] = mma16<T>(mf, lds_tr(&sXb[q][s0 + lr / 4][4 * (lr % 4)]), y1[q]);
          else y1[q] = mma16<T>(mf, ldsf<T>(&sXT[kPB * q + lr][s0]), y1[q]);
        }
      }
      // state: A = C (row t, k = n), B operand = H_in (k = n, column p)
      v4f y2[PB];
#pragma unroll
      for (int q = 0; q < PB; ++q) y2[q] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const auto cf = ldsf<T>(&sC[tb + lr][16 * nb + 4 * lq]);
#pragma unroll
        for (int q = 0; q < PB; ++q) {
          if constexpr (kBF) {
            const int hr = 16 * nb + 4 * lq + lr / 4;   // C (H + H_lo) in one k = 32 product
            y2[q] = mma32(cf, cf, lds_tr(&sHb[q][hr][4 * (lr % 4)]), lds_tr(&sHL[q][hr][4 * (lr % 4)]), y2[q]);
          } else {
            y2[q] = mma16<T>(cf, ldsf<T>(&sHT[kPB * q + lr][16 * nb + 4 * lq]), y2[q]);
          }
        }
      }
      // lane holds t = tb + 4 lq + i, p = 16 q + lr; stores of tokens past
      // the end or channels past headdim go past the window's end and are
      // dropped
      const __amdgpu_buffer_rsrc_t ro = window(og, p.osl, p.P - p0, t0);
      const uint32_t oend = static_cast<uint32_t>(std::min(p.L - 1 - t0, kQ - 1)) * p.osl +
                            (p.P - p0) * ES;
      const float4 la_o = *reinterpret_cast<const float4*>(&sLa[tb + 4 * lq]);
      const float ea[4] = {__builtin_amdgcn_exp2f(la_o.x), __builtin_amdgcn_exp2f(la_o.y),
                           __builtin_amdgcn_exp2f(la_o.z), __builtin_amdgcn_exp2f(la_o.w)};
#pragma unroll
      for (int q = 0; q < PB; ++q) {
        const int pl = kPB * q + lr;
        // bf16: x at this lane's four tokens, one transpose read
        v4s xq = {0, 0, 0, 0};
        if constexpr (kBF) xq = lds_tr(&sXb[q][tb + 4 * lq + lr / 4][4 * (lr % 4)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tl = tb + 4 * lq + i;
          float xval;
          if constexpr (kBF) xval = L::f(static_cast<uint16_t>(xq[i]));
          else xval = L::f(sXT[pl][tl]);
          float y = fmaf(ea[i], y2[q][i], y1[q][i]);
          y = fmaf(Dh, xval, y);
          const float gz = silu_f32(Elem<T>::f32(zr[q][i]));
          y *= zg ? gz : 1.0f;
          const bool ok = tl < nv && p0 + pl < p.P;
          const uint32_t off = ok ? oo0 + i * p.osl + kPB * q * ES : oend;
          Elem<T>::store(ro, off, y);
        }
      }
    }

    // ---- state update: H_out^T = exp(a_last) H_in^T + (w x)^T B ----
    {
      const float decay = __builtin_amdgcn_exp2f(sLa[kQ - 1]);
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int m = wave + kWaves * j;
        if (m < NB) {
          v4f acc[PB];
#pragma unroll
          for (int q = 0; q < PB; ++q) acc[q] = Hs[j][q] * decay;
#pragma unroll
          for (int sbk = 0; sbk < kQ / 16; ++sbk) {
            // A = (w x)^T (row p, k = s); B operand = B (k = s, column n)
            const int s0 = 16 * sbk + 4 * lq, n = 16 * m + lr;
            if constexpr (kBF) {   // two 16-token blocks per k = 32 product
              if (sbk % 2 == 0) {
                const int s1 = s0 + 16;
                const auto bf0 = lds_tr(&sB[s0 + lr / 4][16 * m + 4 * (lr % 4)]);
                const auto bf1 = lds_tr(&sB[s1 + lr / 4][16 * m + 4 * (lr % 4)]);
#pragma unroll
                for (int q = 0; q < PB; ++q)
                  acc[q] = mma32(lds_tr(&sXWb[q][s0 + lr / 4][4 * (lr % 4)]),
                                 lds_tr(&sXWb[q][s1 + lr / 4][4 * (lr % 4)]), bf0, bf1, acc[q]);
              }
            } else {
              const auto bf = tofrag_bits<T>(sB[s0][n], sB[s0 + 1][n], sB[s0 + 2][n], sB[s0 + 3][n]);
#pragma unroll
              for (int q = 0; q < PB; ++q) acc[q] = mma16<T>(ldsf<T>(&sXW[kPB * q + lr][s0]), bf, acc[q]);
            }
          }
#pragma unroll
          for (int q = 0; q < PB; ++q) Hs[j][q] = acc[q];
        }
      }
    }
    __syncthreads();   // every wavefront is done with this chunk's LDS
    store_ht();
  }

  // pass 1: the segment's end state from its start state and its
  // step-size sum (equal in every workgroup of the head)
  if (kSegd && p.mode == 1) {
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int n = 16 * (wave + kWaves * j) + lr;
#pragma unroll
      for (int q = 0; q < PB; ++q) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pp = p0 + kPB * q + 4 * lq + i;
          if (n < N && pp < p.P)
            p.aggH[((bh * p.nseg + seg) * p.P + pp) * static_cast<int64_t>(N) + n] = Hs[j][q][i];
        }
      }
    }
    if (pb == 0 && tid == 0) p.aggS[bh * p.nseg + seg] = static_cast<float>(sSum);
  }
  // final state (one segment)
  if (!kSegd && p.last) {
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int n = 16 * (wave + kWaves * j) + lr;
#pragma unroll
      for (int q = 0; q < PB; ++q) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int pp = p0 + kPB * q + 4 * lq + i;
          if (n < N && pp < p.P)
            p.last[((b * p.H + h) * p.P + pp) * static_cast<int64_t>(N) + n] = Hs[j][q][i];
        }
      }
    }
  }
}

// seqlen == 0: the final state is the initial one (or zero).
__global__ void ssd_copy_state_kernel(const float* h0, float* last, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) last[i] = h0 ? h0[i] : 0.0f;
}

// Blocks of 16 head channels per workgroup: up to the whole head, as far as
// 64 KB of LDS allows (four with 64 bf16 states, else two), while the grid
// still holds kMinGroups workgroups.
#ifndef SSD_PB_FORCE
constexpr int64_t kMinGroups = 512;
int choose_pb(int P, int nmax, bool bf, int64_t heads) {
  const int cap = (bf && nmax == 64) ? 4 : 2;
  const int full = (P + kPB - 1) / kPB;
  int pb = 1;
  while (2 * pb <= cap && pb < full &&
         heads * ((P + 2 * pb * kPB - 1) / (2 * pb * kPB)) >= kMinGroups)
    pb *= 2;
  return pb;
}
#else
int choose_pb(int P, int nmax, bool bf, int64_t) {
  const int cap = (bf && nmax == 64) ? 4 : 2;
  return std::min(SSD_PB_FORCE, cap);
}
#endif

// Segments of a long sequence whose (batch, head, channel block) workgroups
// leave the machine short: as many as bring the grid to about 2,048
// workgroups (eight per CU, in rounds of what the kernel's registers let
// reside), each at least 32,768 tokens long (pass 2 rescans a segment's head
// until the incoming state has decayed, about 17 / (Delta |A|) tokens for
// the slowest head: 17,000 at Delta 1e-3, A = -1), at most 64.  Measured on
// batch 1, 32 heads of 64, L 1M (128 workgroups per segment): 13.9 ms at a
// target of 512 (4 segments), 12.1 at 1,024, 11.8 at 2,048, 12.1 at 4,096.
constexpr int64_t kSsdTargetGroups = 2048;
constexpr int64_t kSsdMinSegLen = 32768;
constexpr int kSsdMaxSeg = 64;

struct SsdPlan {
  int pbk, pblocks;   // channel blocks per workgroup, workgroups per head
  int nseg, seg_chunks;
};

// segments: whether the sequence may be cut (a workspace will hold the
// segments' end states).  A cut sequence fills the machine with segments,
// so it takes two channel blocks per workgroup where the head has them
// (the chunk's staging, step scan and score tiles shared by both): on
// batch 1, L 1M, 32 heads of 64, 11.05 ms with one block per workgroup in
// 16 segments against 9.18 ms with two in 32 (same-box A/B).
SsdPlan ssd_plan(const ssm_ssd_args& a, bool segments = true) {
  const bool bf = a.io_dtype == SSM_BF16;
  const int nmax = (bf && a.dstate > 64) ? 128 : 64;
  const int64_t nchunks = (a.seqlen + kQ - 1) / kQ;
  SsdPlan q;
  int64_t g = 1;
  auto plan_with = [&](int pbk) {
    q.pbk = pbk;
    q.pblocks = static_cast<int>((a.headdim + kPB * q.pbk - 1) / (kPB * q.pbk));
    const int64_t groups = a.batch * a.nheads * q.pblocks;
    g = 1;
    if (segments && groups > 0 && groups < kSsdTargetGroups / 2)
      g = std::max<int64_t>(1, std::min<int64_t>({kSsdTargetGroups / groups, a.seqlen / kSsdMinSegLen,
                                                  int64_t{kSsdMaxSeg}}));
  };
  plan_with(choose_pb(static_cast<int>(a.headdim), nmax, bf, a.batch * a.nheads));
#ifndef SSD_PB_FORCE
  const int full = static_cast<int>((a.headdim + kPB - 1) / kPB);
  if (g > 1 && q.pbk < 2 && full >= 2) plan_with(2);
#endif
  q.seg_chunks = static_cast<int>(std::max<int64_t>(1, (nchunks + g - 1) / g));
  q.nseg = static_cast<int>(std::max<int64_t>(1, (nchunks + q.seg_chunks - 1) / q.seg_chunks));
  return q;
}

// Workspace of a segmented sequence: the end states, [batch * H][nseg][P][N]
// fp32, then the step-size sums [batch * H][nseg] (offset rounded to 256
// bytes).
size_t ssd_agg_offset(const ssm_ssd_args& a, int nseg) {
  const size_t n = static_cast<size_t>(a.batch * a.nheads) * nseg * a.headdim * a.dstate * 4;
  return (n + 255) / 256 * 256;
}

template <typename T, int NMAX, int PB, bool kSegd>
void launch_s(bool softplus, bool vec, dim3 grid, const SsdParams& p, hipStream_t stream) {
  if (vec) {
    if (softplus) ssd_fwd_kernel<T, NMAX, true, true, PB, kSegd><<<grid, dim3(kThreads), 0, stream>>>(p);
    else ssd_fwd_kernel<T, NMAX, false, true, PB, kSegd><<<grid, dim3(kThreads), 0, stream>>>(p);
  } else {
    if (softplus) ssd_fwd_kernel<T, NMAX, true, false, PB, kSegd><<<grid, dim3(kThreads), 0, stream>>>(p);
    else ssd_fwd_kernel<T, NMAX, false, false, PB, kSegd><<<grid, dim3(kThreads), 0, stream>>>(p);
  }
}

template <typename T, int NMAX, int PB>
void launch_n(bool softplus, bool vec, dim3 grid, const SsdParams& p, hipStream_t stream) {
  if (p.mode != 0) launch_s<T, NMAX, PB, true>(softplus, vec, grid, p, stream);
  else launch_s<T, NMAX, PB, false>(softplus, vec, grid, p, stream);
}

}  // namespace

size_t ssd_workspace_bytes(const ssm_ssd_args& a) {
  if (a.batch <= 0 || a.seqlen <= 0 || a.nheads <= 0 || a.headdim <= 0 || a.dstate <= 0) return 0;
  const SsdPlan q = ssd_plan(a);
  if (q.nseg <= 1) return 0;
  return ssd_agg_offset(a, q.nseg) + static_cast<size_t>(a.batch * a.nheads) * q.nseg * 4;
}

hipError_t launch_ssd_fwd(const ssm_ssd_args& a, hipStream_t stream) {
  if (a.seqlen == 0) {
    if (a.last_state && a.last_state != a.h0) {
      const int64_t n = a.batch * a.nheads * a.headdim * a.dstate;
      ssd_copy_state_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream>>>(
          a.h0, a.last_state, n);
    }
    return hipGetLastError();
  }
  SsdParams p;
  p.x = a.x; p.dt = a.dt; p.z = a.z; p.B = a.B; p.C = a.C;
  p.A = a.A; p.D = a.D; p.bias = a.dt_bias; p.h0 = a.h0; p.last = a.last_state; p.out = a.out;
  const int64_t es = a.io_dtype == SSM_BF16 ? 2 : 4;
  auto seqb = [&](int64_t stride) { return static_cast<uint32_t>(stride * es); };
  p.xsb = a.x_batch_stride; p.xsl = seqb(a.x_seq_stride); p.xsh = a.x_head_stride;
  p.dsb = a.dt_batch_stride; p.dsl = seqb(a.dt_seq_stride);
  p.zsb = a.z_batch_stride; p.zsl = seqb(a.z_seq_stride); p.zsh = a.z_head_stride;
  p.Bsb = a.B_batch_stride; p.Bsl = seqb(a.B_seq_stride); p.Bsg = a.B_group_stride;
  p.Csb = a.C_batch_stride; p.Csl = seqb(a.C_seq_stride); p.Csg = a.C_group_stride;
  p.osb = a.out_batch_stride; p.osl = seqb(a.out_seq_stride); p.osh = a.out_head_stride;
  p.L = static_cast<int>(a.seqlen); p.H = static_cast<int>(a.nheads);
  p.P = static_cast<int>(a.headdim); p.G = static_cast<int>(a.ngroups > 1 ? a.ngroups : 1);
  p.N = static_cast<int>(a.dstate);
  const bool sp = a.dt_softplus != 0;
  const bool bf = a.io_dtype == SSM_BF16;
  const int nmax = (bf && a.dstate > 64) ? 128 : 64;
  // segments only with a workspace that holds their end states; without
  // one, the plan of a single segment
  const size_t need = ssd_workspace_bytes(a);
  const bool segd = need > 0 && a.workspace && a.workspace_bytes >= need;
  const SsdPlan q = ssd_plan(a, segd);
  const int pbk = q.pbk;
  p.pblocks = q.pblocks;
  p.nseg = segd ? q.nseg : 1;
  p.seg_chunks = segd ? q.seg_chunks : static_cast<int>((a.seqlen + kQ - 1) / kQ);
  p.mode = segd ? 1 : 0;
  p.aggH = segd ? static_cast<float*>(a.workspace) : nullptr;
  p.aggS = segd ? reinterpret_cast<float*>(static_cast<char*>(a.workspace) + ssd_agg_offset(a, q.nseg))
                : nullptr;
  const int64_t nblocks = a.batch * a.nheads * p.pblocks * p.nseg;
  if (nblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid(static_cast<unsigned>(nblocks));
  // vector staging: 16-byte B/C row quarters, 8- (bf16) or 16-byte (fp32) x
  // rows of four channels
  const int esz = bf ? 2 : 4;
  const int64_t bw = 16 / esz, xw = bf ? 4 : 4;
  auto al = [](const void* ptr, int64_t bytes) {
    return reinterpret_cast<uintptr_t>(ptr) % static_cast<uintptr_t>(bytes) == 0;
  };
  const int64_t G = p.G;
  const bool vec = a.dstate % (nmax / 4) == 0 && al(a.B, 16) && al(a.C, 16) &&
                   a.B_batch_stride % bw == 0 && a.B_seq_stride % bw == 0 &&
                   (G == 1 || a.B_group_stride % bw == 0) && a.C_batch_stride % bw == 0 &&
                   a.C_seq_stride % bw == 0 && (G == 1 || a.C_group_stride % bw == 0) &&
                   al(a.x, xw * esz) && a.x_batch_stride % xw == 0 && a.x_seq_stride % xw == 0 &&
                   a.x_head_stride % xw == 0 && a.headdim % xw == 0;
  auto run = [&](const SsdParams& pp, dim3 gr) {
    if (bf && nmax == 64) {
      switch (pbk) {
        case 4: launch_n<uint16_t, 64, 4>(sp, vec, gr, pp, stream); break;
        case 2: launch_n<uint16_t, 64, 2>(sp, vec, gr, pp, stream); break;
        default: launch_n<uint16_t, 64, 1>(sp, vec, gr, pp, stream); break;
      }
    } else if (bf) {
      if (pbk == 2) launch_n<uint16_t, 128, 2>(sp, vec, gr, pp, stream);
      else launch_n<uint16_t, 128, 1>(sp, vec, gr, pp, stream);
    } else {
      if (pbk == 2) launch_n<float, 64, 2>(sp, vec, gr, pp, stream);
      else launch_n<float, 64, 1>(sp, vec, gr, pp, stream);
    }
  };
  run(p, grid);
  if (segd) {
    // pass 2: segments 1.. from their folded incoming states (stream order
    // puts pass 1's end states, and its reads of h0, first)
    SsdParams p2 = p;
    p2.mode = 2;
    run(p2, dim3(static_cast<unsigned>(a.batch * a.nheads * p.pblocks * (p.nseg - 1))));
  }
  return hipGetLastError();
}

}  // namespace ssm

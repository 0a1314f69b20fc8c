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
// block of 16 head channels) and walks the sequence chunk by chunk, keeping
// the fp32 state H^T (16 channels x N states) in MFMA accumulator registers:
// wavefront w holds state columns n in blocks w, w+4, ... .  Wavefront w also
// owns output tokens 16w..16w+15 of each chunk: it forms the score tiles for
// source blocks 0..w (causal), masks them, and feeds them straight into the
// next product: the accumulator layout of a 16x16 tile (lane l holds rows
// 4(l/16)+i, column l%16) is exactly the operand layout of the following
// 16x16x16 product (lane l supplies row l%16, k = 4(l/16)+i), so the scores
// never leave registers.  B, C and x of a chunk are staged in LDS by the
// whole workgroup; the state goes through LDS once per chunk for the state
// product.  bf16 IO uses v_mfma_f32_16x16x16_bf16 (fp32 accumulation; the
// masked scores and the decay-weighted x are rounded to bf16, and the state
// operand is split into a bf16 value and its bf16 remainder);
// fp32 IO uses v_mfma_f32_16x16x4_f32 four times per 16-wide k block, each
// lane supplying the same four consecutive k values one per instruction.
#include <algorithm>

#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kQ = 64;          // tokens per chunk
constexpr int kPB = 16;         // head channels per workgroup
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
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
  int64_t xsb, xsl, xsh, dsb, dsl, zsb, zsl, zsh, Bsb, Bsl, Bsg, Csb, Csl, Csg, osb, osl, osh;
  int L, H, P, G, N;
  int pblocks;   // ceil(P / 16)
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

// Four consecutive LDS elements (8 or 16 bytes, aligned) as a fragment.
template <typename T>
__device__ __forceinline__ typename Frag<T>::V ldsf(const typename Lds<T>::E* p) {
  return *reinterpret_cast<const typename Frag<T>::V*>(p);
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

// kVec: B/C rows, x rows and their strides are 16-byte (x: 8-byte for bf16)
// aligned and dstate is a multiple of NMAX / 4, so staging uses vector loads
// and 16-byte LDS stores; otherwise element-wise loads.
template <typename T, int NMAX, bool kSoftplus, bool kVec>
__global__ __launch_bounds__(kThreads) void ssd_fwd_kernel(SsdParams p) {
  using L = Lds<T>;
  using E = typename L::E;
  constexpr int kPadE = 16 / sizeof(E);        // 16 bytes of padding per row
  constexpr int NP = NMAX + kPadE;             // LDS pitch of a B / C row
  constexpr int QP = kQ + kPadE;               // LDS pitch of an x^T row
  constexpr int NB = NMAX / 16;                // 16-wide state blocks
  constexpr int NBW = (NB + kWaves - 1) / kWaves;  // state blocks per wavefront
  __shared__ __align__(16) E sB[kQ][NP];       // B_s[n]
  __shared__ __align__(16) E sC[kQ][NP];       // C_t[n]
  __shared__ __align__(16) E sXT[kPB][QP];     // x_s[p], transposed
  __shared__ __align__(16) E sXW[kPB][QP];     // exp(a_{Q-1} - a_s) Delta_s x_s[p], transposed
  __shared__ __align__(16) E sHT[kPB][NP];     // H_in^T[p][n] (operand copy)
  // bf16: the rounding remainder H - bf16(H), so that the state product
  // carries the fp32 state to about 16 bits (two bf16 products)
  __shared__ __align__(16) E sHL[sizeof(E) == 2 ? kPB : 1][sizeof(E) == 2 ? NP : 1];
  __shared__ __align__(16) float sDl[kQ];      // Delta_s (0 past the end)
  __shared__ __align__(16) float sLa[kQ];      // a_t * log2(e)

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;    // row / column and k quarter
  const int pb = blockIdx.x % p.pblocks;
  const int h = (blockIdx.x / p.pblocks) % p.H;
  const int64_t b = blockIdx.x / (static_cast<int64_t>(p.pblocks) * p.H);
  const int g = h / (p.H / p.G);
  const int p0 = pb * kPB;
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

  // State H^T tiles: lane holds H^T[p = 4 lq + i][n = 16 m + lr], m = wave + 4 j.
  v4f Hs[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j) {
    const int n = 16 * (wave + kWaves * j) + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pp = 4 * lq + i;
      Hs[j][i] = (p.h0 && n < N && p0 + pp < p.P)
                     ? p.h0[((b * p.H + h) * p.P + p0 + pp) * static_cast<int64_t>(N) + n]
                     : 0.0f;
    }
  }
  // operand copy of the initial state
  auto store_ht = [&]() {
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int m = wave + kWaves * j;
      if (m < NB) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const E hi = L::from(Hs[j][i]);
          sHT[4 * lq + i][16 * m + lr] = hi;
          if constexpr (sizeof(E) == 2) sHL[4 * lq + i][16 * m + lr] = L::from(Hs[j][i] - L::f(hi));
        }
      }
    }
  };
  store_ht();

  // Staging of one chunk.  Thread tid covers B/C row s = tid / 4, quarter
  // (tid % 4) of the NMAX states, and x row s, channels 4 (tid % 4) .. +3;
  // the threads of wavefront 0 also load the step of token tid.  Every load
  // goes through a buffer window that starts at the chunk and ends where the
  // tensor's (batch, head or group) slice ends, so the loads are issued
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
    uint32_t b[kVec ? kQw : kQn], c[kVec ? kQw : kQn], x[kVec ? kXw : 4], dt, z[4];
  };
  auto window = [&](const T* base, int64_t seq_stride, int inner, int t0) {
    // bytes from token t0's row to the end of the chunk's last row (at most
    // 64 rows; the host keeps that below 2^31); empty past the sequence
    const int64_t rows = std::min(p.L - 1 - t0, kQ - 1);
    const int64_t bytes = rows < 0 ? 0 : (rows * seq_stride + inner) * ES;
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(base + static_cast<int64_t>(t0) * seq_stride), 0,
        static_cast<int>(bytes), kRsrcWord3);
  };
  auto load_stage = [&](int c) {
    Stage st;
    const int t0 = c * kQ;
    const __amdgpu_buffer_rsrc_t rb = window(Bg, p.Bsl, N, t0);
    const __amdgpu_buffer_rsrc_t rc = window(Cg, p.Csl, N, t0);
    const __amdgpu_buffer_rsrc_t rx = window(xg, p.xsl, p.P - p0, t0);
    const __amdgpu_buffer_rsrc_t rd = window(dtg, p.dsl, 1, t0);
    const uint32_t ob = static_cast<uint32_t>((srow * p.Bsl + squart * kQn) * ES);
    const uint32_t oc = static_cast<uint32_t>((srow * p.Csl + squart * kQn) * ES);
    const uint32_t ox = static_cast<uint32_t>((srow * p.xsl + 4 * squart) * ES);
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
      if constexpr (kXw == 4) {
        const v4u vx = __builtin_amdgcn_raw_buffer_load_b128(rx, ox, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) st.x[j] = vx[j];
      } else {
        const v2u vx = __builtin_amdgcn_raw_buffer_load_b64(rx, ox, 0, 0);
        st.x[0] = vx[0];
        st.x[1] = vx[1];
      }
    } else {
#pragma unroll
      for (int k = 0; k < kQn; ++k) {
        st.b[k] = Elem<T>::load(rb, ob + k * ES);
        st.c[k] = Elem<T>::load(rc, oc + k * ES);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) st.x[k] = Elem<T>::load(rx, ox + k * ES);
    }
    st.dt = Elem<T>::load(rd, static_cast<uint32_t>(lane * p.dsl * ES));
    // the gate at this lane's output positions (t = 16 w + 4 lq + i, p = lr)
    if (zg) {
      const __amdgpu_buffer_rsrc_t rz = window(zg, p.zsl, p.P - p0, t0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st.z[i] = Elem<T>::load(rz, static_cast<uint32_t>(((16 * wave + 4 * lq + i) * p.zsl + lr) * ES));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) st.z[i] = 0u;
    }
    return st;
  };
  // raw bits as an LDS element, or zero: a mask, not a branch
  auto raw = [](uint32_t v, bool keep) -> E {
    const uint32_t m = v & (keep ? 0xffffffffu : 0u);
    if constexpr (sizeof(E) == 2) return static_cast<E>(m);
    else return __uint_as_float(m);
  };
  Stage st;
  if (nchunks > 0) st = load_stage(0);
  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * kQ;
    const int nv = std::min(kQ, p.L - t0);
    // ---- the chunk's step sizes: every wavefront runs the 64-token scan
    // (lane = token), so that each staging thread has the weight of its row
    float w_row;
    {
      const bool tv = lane < nv;
      const float x = Elem<T>::f32(st.dt) + bias;
      float dl = kSoftplus ? softplus_f32(x) : x;
      dl = tv ? dl : 0.0f;
      float cum = dl;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(cum, off, 64);
        cum += lane >= off ? o : 0.0f;
      }
      const float la = cum * a2;
      const float last = __shfl(la, 63, 64);
      const float w = __builtin_amdgcn_exp2f(last - la) * dl;   // exp(a_{Q-1} - a_s) Delta_s
      w_row = __shfl(w, srow, 64);
      if (wave == 0) {
        sDl[lane] = dl;
        sLa[lane] = la;
      }
    }
    // ---- B (raw and decay-weighted), C, x^T of this chunk into LDS ----
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
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int pp = 4 * squart + k;
          const uint32_t v = ES == 2 ? (st.x[k / 2] >> (16 * (k % 2))) : st.x[k % kXw];
          const E xv = raw(v, tv && p0 + pp < p.P);
          sXT[pp][srow] = xv;
          sXW[pp][srow] = L::from(L::f(xv) * w_row);
        }
      } else {
#pragma unroll
        for (int k = 0; k < kQn; ++k) {
          const int n = squart * kQn + k;
          const bool ok = tv && n < N;
          sB[srow][n] = raw(st.b[k], ok);
          sC[srow][n] = raw(st.c[k], ok);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int pp = 4 * squart + k;
          const E xv = raw(st.x[k], tv && p0 + pp < p.P);
          sXT[pp][srow] = xv;
          sXW[pp][srow] = L::from(L::f(xv) * w_row);
        }
      }
    }
    __syncthreads();
    // this chunk's gate, then the next chunk's loads fly while this one is
    // computed
    uint32_t zr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) zr[i] = st.z[i];
    if (c + 1 < nchunks) st = load_stage(c + 1);

    // ---- outputs of tokens 16 w .. 16 w + 15 ----
    {
      const int tb = 16 * wave;
      const float la_t = sLa[tb + lr];
      v4f y1 = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int sbk = 0; sbk <= wave; ++sbk) {
        // scores G[s][t] for s in block sbk, t in block wave: A = B (row s,
        // k = n), B operand = C^T (k = n, column t)
        v4f sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          sc = mma16<T>(ldsf<T>(&sB[16 * sbk + lr][16 * nb + 4 * lq]),
                        ldsf<T>(&sC[tb + lr][16 * nb + 4 * lq]), sc);
        // mask and scale: lane holds s = 16 sbk + 4 lq + i, t = tb + lr
        const int s0 = 16 * sbk + 4 * lq;
        const float4 la_s = *reinterpret_cast<const float4*>(&sLa[s0]);
        const float4 dl_s = *reinterpret_cast<const float4*>(&sDl[s0]);
        const int t = tb + lr;
        const float m0 = s0 + 0 <= t ? sc[0] * __builtin_amdgcn_exp2f(la_t - la_s.x) * dl_s.x : 0.0f;
        const float m1 = s0 + 1 <= t ? sc[1] * __builtin_amdgcn_exp2f(la_t - la_s.y) * dl_s.y : 0.0f;
        const float m2 = s0 + 2 <= t ? sc[2] * __builtin_amdgcn_exp2f(la_t - la_s.z) * dl_s.z : 0.0f;
        const float m3 = s0 + 3 <= t ? sc[3] * __builtin_amdgcn_exp2f(la_t - la_s.w) * dl_s.w : 0.0f;
        // intra: A = M (row t, k = s), B operand = x (k = s, column p)
        y1 = mma16<T>(tofrag<T>(m0, m1, m2, m3), ldsf<T>(&sXT[lr][s0]), y1);
      }
      // state: A = C (row t, k = n), B operand = H_in (k = n, column p)
      v4f y2 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
      {
        const auto cf = ldsf<T>(&sC[tb + lr][16 * nb + 4 * lq]);
        y2 = mma16<T>(cf, ldsf<T>(&sHT[lr][16 * nb + 4 * lq]), y2);
        if constexpr (sizeof(E) == 2) y2 = mma16<T>(cf, ldsf<T>(&sHL[lr][16 * nb + 4 * lq]), y2);
      }
      // lane holds t = tb + 4 lq + i, p = lr; stores of tokens past the end
      // or channels past headdim go past the window's end and are dropped
      const __amdgpu_buffer_rsrc_t ro = window(og, p.osl, p.P - p0, t0);
      const uint32_t oend = static_cast<uint32_t>(
          (static_cast<int64_t>(std::min(p.L - 1 - t0, kQ - 1)) * p.osl + (p.P - p0)) * ES);
      const float4 la_o = *reinterpret_cast<const float4*>(&sLa[tb + 4 * lq]);
      const float lav[4] = {la_o.x, la_o.y, la_o.z, la_o.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tl = tb + 4 * lq + i;
        const float xval = L::f(sXT[lr][tl]);
        float y = y1[i] + __builtin_amdgcn_exp2f(lav[i]) * y2[i];
        y = fmaf(Dh, xval, y);
        const float gz = silu_f32(Elem<T>::f32(zr[i]));
        y *= zg ? gz : 1.0f;
        const bool ok = tl < nv && p0 + lr < p.P;
        const uint32_t off = ok ? static_cast<uint32_t>((tl * p.osl + lr) * ES) : oend;
        Elem<T>::store(ro, off, y);
      }
    }

    // ---- state update: H_out^T = exp(a_last) H_in^T + (w x)^T B ----
    {
      const float decay = __builtin_amdgcn_exp2f(sLa[kQ - 1]);
#pragma unroll
      for (int j = 0; j < NBW; ++j) {
        const int m = wave + kWaves * j;
        if (m < NB) {
          v4f acc = Hs[j] * decay;
#pragma unroll
          for (int sbk = 0; sbk < kQ / 16; ++sbk) {
            // A = (w x)^T (row p, k = s); B operand = B (k = s, column n)
            const int s0 = 16 * sbk + 4 * lq, n = 16 * m + lr;
            acc = mma16<T>(ldsf<T>(&sXW[lr][s0]),
                           tofrag_bits<T>(sB[s0][n], sB[s0 + 1][n], sB[s0 + 2][n], sB[s0 + 3][n]),
                           acc);
          }
          Hs[j] = acc;
        }
      }
    }
    __syncthreads();   // every wavefront is done with this chunk's LDS
    store_ht();
  }

  // final state
  if (p.last) {
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int n = 16 * (wave + kWaves * j) + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pp = 4 * lq + i;
        if (n < N && p0 + pp < p.P)
          p.last[((b * p.H + h) * p.P + p0 + pp) * static_cast<int64_t>(N) + n] = Hs[j][i];
      }
    }
  }
}

// seqlen == 0: the final state is the initial one (or zero).
__global__ void ssd_copy_state_kernel(const float* h0, float* last, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) last[i] = h0 ? h0[i] : 0.0f;
}

template <typename T, int NMAX>
void launch_n(bool softplus, bool vec, dim3 grid, const SsdParams& p, hipStream_t stream) {
  if (vec) {
    if (softplus) ssd_fwd_kernel<T, NMAX, true, true><<<grid, dim3(kThreads), 0, stream>>>(p);
    else ssd_fwd_kernel<T, NMAX, false, true><<<grid, dim3(kThreads), 0, stream>>>(p);
  } else {
    if (softplus) ssd_fwd_kernel<T, NMAX, true, false><<<grid, dim3(kThreads), 0, stream>>>(p);
    else ssd_fwd_kernel<T, NMAX, false, false><<<grid, dim3(kThreads), 0, stream>>>(p);
  }
}

}  // namespace

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
  p.xsb = a.x_batch_stride; p.xsl = a.x_seq_stride; p.xsh = a.x_head_stride;
  p.dsb = a.dt_batch_stride; p.dsl = a.dt_seq_stride;
  p.zsb = a.z_batch_stride; p.zsl = a.z_seq_stride; p.zsh = a.z_head_stride;
  p.Bsb = a.B_batch_stride; p.Bsl = a.B_seq_stride; p.Bsg = a.B_group_stride;
  p.Csb = a.C_batch_stride; p.Csl = a.C_seq_stride; p.Csg = a.C_group_stride;
  p.osb = a.out_batch_stride; p.osl = a.out_seq_stride; p.osh = a.out_head_stride;
  p.L = static_cast<int>(a.seqlen); p.H = static_cast<int>(a.nheads);
  p.P = static_cast<int>(a.headdim); p.G = static_cast<int>(a.ngroups > 1 ? a.ngroups : 1);
  p.N = static_cast<int>(a.dstate);
  p.pblocks = (p.P + kPB - 1) / kPB;
  const int64_t nblocks = a.batch * a.nheads * p.pblocks;
  if (nblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(nblocks));
  const bool sp = a.dt_softplus != 0;
  const bool bf = a.io_dtype == SSM_BF16;
  const int nmax = (bf && a.dstate > 64) ? 128 : 64;
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
  if (bf) {
    if (nmax == 64) launch_n<uint16_t, 64>(sp, vec, grid, p, stream);
    else launch_n<uint16_t, 128>(sp, vec, grid, p, stream);
  } else {
    launch_n<float, 64>(sp, vec, grid, p, stream);
  }
  return hipGetLastError();
}

}  // namespace ssm

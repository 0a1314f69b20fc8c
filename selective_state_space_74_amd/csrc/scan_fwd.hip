// scan_fwd.hip -- host side of the prefill selective scan: segment choice,
// B/C mode, workspace, window limits and the launches, and the static
// segment scratch of the no-allocation entry point.  The kernel itself is
// in scan_fwd_kernel.h (instantiated by scan_fwd_s1/s2/s4.hip).
#include <algorithm>
#include <atomic>
#include <mutex>

#include "scan_fwd_kernel.h"

// The no-allocation entry point's segment scratch: one copy per device, held
// until the process ends.  Host code never uses this name as an address; it
// takes the device address from hipGetSymbolAddress once per device.
static __device__ __align__(256) float scratch[SSM_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace ssm {
namespace {

using fwd::kCh;
using fwd::kGT;
using fwd::kN;
using fwd::kRows;
using fwd::kT;

// seqlen == 0: the final state is the initial one.
__global__ void copy_state_kernel(const float* h0, float* last, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) last[i] = h0 ? h0[i] : 0.0f;
}

// Segments per sequence: cut only when the batch x channel groups alone leave
// the machine short of wavefronts, as many as fit one residency round of the
// one-slot kernels (5 workgroups per CU), and keep segments long enough that
// the second pass (bounded by the decay of the incoming state, not by the
// segment length) and the fold stay small next to them.
// The minimum segment length keeps pass 2 well inside each segment: its
// rescan of a segment's head runs until the incoming state has decayed,
// about 17 / (Delta |A|) tokens for the slowest state (17,000 at Delta 1e-3,
// A = -1), and on segments not much longer than that the two passes cost
// more than one (at batch 1, d_inner 2048: 8192-token segments took L 16,384
// from 265 us at 8192 tokens to 624 us).
constexpr int64_t kTargetGroups = 1280;   // 5 wavefronts per SIMD on 256 CUs
constexpr int64_t kMinSegLen = 32768;
constexpr int kMaxSeg = 64;
// Grids of at most this many workgroups leave three wavefronts per SIMD on
// 256 CUs whatever a kernel's register count; there the one-slot scan takes
// the deferred owner-C readout (more registers, the LDS round trip of the
// readout covered).  Larger grids keep the compact form's occupancy.
constexpr int64_t kDeferMaxGroups = 768;

int choose_segments(int64_t groups, int64_t L) {
  if (groups >= kTargetGroups / 2) return 1;
  int64_t g = kTargetGroups / groups;
  g = std::min<int64_t>(g, std::max<int64_t>(1, L / kMinSegLen));
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(g, kMaxSeg)));
}

int64_t ngroups_of(const ssm_scan_args& a) { return a.ngroups > 1 ? a.ngroups : 1; }

// Shared B/C (one LDS tile per workgroup) needs the workgroup's 16 channels
// in one group; otherwise each lane reads its own group's rows.
bool lane_bc(const ssm_scan_args& a) {
  const int64_t G = ngroups_of(a);
  return G > 1 && (a.dim / G) % kCh != 0;
}

// State slots per lane: 16 states per slot.
int slots(int64_t dstate) { return dstate <= 16 ? 1 : dstate <= 32 ? 2 : 4; }

}  // namespace

namespace {

// Per-wavefront byte windows (and the lane offsets inside them) are 32-bit,
// with a margin: lanes of padding states address from a window's end.  A
// wavefront's rows lie within `rows + 1` consecutive channels; with per-lane
// B/C they reach `gspan + 1` groups.
bool spans_fit(const ssm_scan_args& a, int64_t rows, int64_t gspan) {
  const int64_t esz = a.io_dtype == SSM_BF16 ? 2 : 4;
  const int64_t lim = (int64_t{1} << 32) - 256;
  auto fits = [&](int64_t span) { return span * esz < lim; };
  bool ok = fits(rows * a.u_dim_stride + a.seqlen) && fits(rows * a.delta_dim_stride + a.seqlen) &&
            fits(rows * a.out_dim_stride + a.seqlen) &&
            fits(gspan * a.B_group_stride + (a.dstate - 1) * a.B_state_stride + a.seqlen) &&
            fits(gspan * a.C_group_stride + (a.dstate - 1) * a.C_state_stride + a.seqlen);
  if (a.z) ok = ok && fits(rows * a.z_dim_stride + a.seqlen);
  if (a.conv_weight && a.conv_out) ok = ok && fits(rows * a.conv_out_dim_stride + a.seqlen);
  // checkpoints: rows + 1 rows of ceil(L / 16) * dstate floats
  if (a.checkpoints)
    ok = ok && (rows + 1) * ((a.seqlen + kT - 1) / kT) * a.dstate * 4 < lim;
  return ok;
}

// Pass 2 of the segmented scan gathers the channels of a window from a chunk
// of `cw` consecutive channels of one B/C scope (the group with the shared
// tile, the whole row with per-lane B/C): the widest chunk whose windows fit,
// at least min(4, scope), which scan_windows_fit guarantees.
int64_t chunk_width(const ssm_scan_args& a, int64_t scope) {
  const int64_t cpg = a.dim / ngroups_of(a);
  auto fit = [&](int64_t cw) {
    // cw consecutive channels reach at most ceil((cw - 1) / cpg) + 1 groups
    const int64_t gs = lane_bc(a) ? std::min<int64_t>((cw - 1 + cpg - 1) / cpg, ngroups_of(a) - 1) : 0;
    return spans_fit(a, cw - 1, gs);
  };
  int64_t lo = std::min<int64_t>(kRows, scope), hi = scope;
  if (fit(hi)) return hi;
  while (hi - lo > 1) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (fit(mid)) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Workspace of a segmented scan (offsets in bytes, 256-byte aligned):
// segment aggregates [B*D][G][N+1] and window records [G][kWin][B*D][N+1]
// (fp32), then per (channel, segment) the number of windows to rescan, and
// per (batch row, segment, window) the channel counts and lists.
struct SegLayout {
  size_t agg, rec, jst, cnt, lst, total;
};

SegLayout seg_layout(const ssm_scan_args& a, int nseg) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t bd = static_cast<size_t>(a.batch * a.dim), ns = static_cast<size_t>(nseg);
  const size_t aggs = static_cast<size_t>(a.dstate + 1);
  SegLayout l;
  l.agg = 0;
  l.rec = l.agg + al(bd * ns * aggs * 4);
  l.jst = l.rec + al(ns * fwd::kWin * bd * aggs * 4);
  l.cnt = l.jst + al(ns * bd * 4);
  l.lst = l.cnt + al(ns * fwd::kWin * bd * 4);
  l.total = l.lst + al(ns * fwd::kWin * bd * 4);
  return l;
}

// Between the passes of a segmented scan, one 16-lane row per channel and
// segment g >= 1 (lane c holds states c, c + 16, ...):
//  - h_in, the exact state entering segment g, folded from the aggregates
//    of segments 0..g-1 (segment 0's end state already includes h0), goes
//    to window slot 0 (with S = 0); the last segment also folds its own
//    aggregate into last_state;
//  - each later window start's record (pass 1's state there) becomes the
//    exact state, the record plus the free response exp(A S) h_in;
//  - jst, the number of windows to rescan: up to the first window start
//    where the free response is at most 2^-24 max_n |h[n]| in every state
//    (a non-finite one never passes), else all of the segment's windows;
//    and, in bits 8.., where in its last window the channel is expected to
//    pass, 0..15 (log2 of the free response over that bound taken as
//    linear between the window's start and the next start; 15 when the
//    window runs to the segment's end): the lists' sort key.
struct PlanParams {
  const float* agg;
  float* rec;
  int* jst;
  float* last_state;
  const float* A;
  int64_t Asd, Asn, batch, dim;
  int N, nseg, L, seg_len;
};

__global__ __launch_bounds__(256) void seg_plan_kernel(PlanParams q) {
  const int64_t bd = q.batch * q.dim;
  const int64_t item = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) / kN;
  const int col = threadIdx.x % kN;
  if (item >= bd * (q.nseg - 1)) return;  // whole rows
  const int64_t c = item % bd;
  const int g = static_cast<int>(item / bd) + 1;
  const int64_t d = c % q.dim;
  const int N = q.N, aggs = N + 1;
  const int s0 = g * q.seg_len;
  const int nw = fwd::seg_windows((min(q.L, s0 + q.seg_len) - s0) / kT);
  const float* ag = q.agg + c * q.nseg * aggs;
  float* slot0 = q.rec + (static_cast<size_t>(g) * fwd::kWin * bd + c) * aggs;
  const size_t sstride = static_cast<size_t>(bd) * aggs;  // floats from one window slot to the next
  float fr[fwd::kWin], hm[fwd::kWin];
#pragma unroll
  for (int j = 0; j < fwd::kWin; ++j) fr[j] = hm[j] = 0.0f;
  for (int n = col; n < N; n += kN) {
    const float a2 = q.A[d * q.Asd + n * q.Asn] * kLog2e;
    float h = ag[n];
    for (int i = 1; i < g; ++i)
      h = fmaf(__builtin_amdgcn_exp2f(a2 * ag[i * aggs + N]), h, ag[i * aggs + n]);
    if (q.last_state && g == q.nseg - 1)
      q.last_state[c * N + n] = fmaf(__builtin_amdgcn_exp2f(a2 * ag[g * aggs + N]), h, ag[g * aggs + n]);
    slot0[n] = h;
#pragma unroll
    for (int j = 1; j < fwd::kWin; ++j) {
      if (j < nw) {
        float* r = slot0 + j * sstride;
        const float e = __builtin_amdgcn_exp2f(a2 * r[N]);
        const float hx = fmaf(e, h, r[n]);
        r[n] = hx;
        const float f = e * fabsf(h);
        fr[j] = fmaxf(fr[j], f == f ? f : __builtin_huge_valf());
        hm[j] = fmaxf(hm[j], fabsf(hx));
      }
    }
  }
  if (col == 0) slot0[N] = 0.0f;
#pragma unroll
  for (int j = 1; j < fwd::kWin; ++j) {
#pragma unroll
    for (int o = 1; o < kN; o <<= 1) {
      fr[j] = fmaxf(fr[j], __shfl_xor(fr[j], o, kN));
      hm[j] = fmaxf(hm[j], __shfl_xor(hm[j], o, kN));
    }
  }
  int js = nw;
#pragma unroll
  for (int j = fwd::kWin - 1; j >= 1; --j)
    if (j < nw && fr[j] <= 0x1p-24f * hm[j]) js = j;
  int tq = 15;
  if (js < nw) {
    // log2 of the free response over the bound: 24 at the segment start
    // (h = h_in there), > 0 at the start of window js - 1, <= 0 at js's
    float la = 24.0f, lb = 0.0f;
#pragma unroll
    for (int j = 1; j < fwd::kWin; ++j) {
      const float l = __builtin_amdgcn_logf(fr[j]) - __builtin_amdgcn_logf(hm[j]) + 24.0f;
      if (j == js - 1) la = l;
      if (j == js) lb = l;
    }
    const float f = la / (la - lb);
    tq = f == f ? static_cast<int>(fminf(fmaxf(16.0f * f, 0.0f), 15.0f)) : 15;
  }
  if (col == 0) q.jst[static_cast<size_t>(g) * bd + c] = js | tq << 8;
}

// Per (batch row, segment g >= 1, chunk, window j): the chunk's channels
// with more than j windows to rescan, and their count.  The list is sorted
// by how far into the window a channel is expected to run (the whole
// window unless it is the channel's last, else the plan's estimate), the
// longest first, so that the 16 channels of a pass 2 workgroup stop at
// about the same point; ties keep channel order (a stable counting sort:
// each thread takes a run of consecutive channels, one scan per key).
struct ListParams {
  const int* jst;
  int* counts;
  int* lists;
  int64_t batch, dim, scope, cw, nchunk;
  int nseg;
};

__global__ __launch_bounds__(256) void seg_list_kernel(ListParams q) {
  __shared__ int wsum[4];
  const int64_t bid = blockIdx.x;
  const int j = static_cast<int>(bid % fwd::kWin);
  const int64_t chunk = (bid / fwd::kWin) % q.nchunk;
  const int g = static_cast<int>((bid / fwd::kWin / q.nchunk) % (q.nseg - 1)) + 1;
  const int64_t b = bid / (fwd::kWin * q.nchunk * (q.nseg - 1));
  const int64_t cps = (q.scope + q.cw - 1) / q.cw;
  const int64_t c0 = (chunk / cps) * q.scope + (chunk % cps) * q.cw;
  const int64_t c1 = std::min(c0 + q.cw, (chunk / cps + 1) * q.scope);
  const int64_t per = (c1 - c0 + 255) / 256;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int64_t lo = std::min(c1, c0 + t * per), hi = std::min(c1, lo + per);
  const int* js = q.jst + static_cast<size_t>(g) * q.batch * q.dim + b * q.dim;
  const int64_t key = ((b * q.nseg + g) * fwd::kWin + j) * q.dim + c0;
  // key of a channel in this window: 16 for the whole window, else the
  // plan's 0..15; -1 when the channel is not rescanned here
  auto skey = [&](int v) { return (v & 255) <= j ? -1 : (v & 255) > j + 1 ? 16 : v >> 8; };
  int base = 0;
  for (int sk = 16; sk >= 0; --sk) {
    int cnt = 0;
    for (int64_t c = lo; c < hi; ++c) cnt += skey(js[c]) == sk;
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int pos = base + incl - cnt, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (w < wv) pos += wsum[w];
      total += wsum[w];
    }
    for (int64_t c = lo; c < hi; ++c)
      if (skey(js[c]) == sk) q.lists[key + pos++] = static_cast<int>(c);
    base += total;
    __syncthreads();  // wsum is rewritten for the next key
  }
  if (t == 0) q.counts[key] = base;
}

}  // namespace

bool scan_windows_fit(const ssm_scan_args& a) {
  // a wavefront's four rows reach at most four groups in lane mode
  const int64_t gspan = lane_bc(a) ? std::min<int64_t>(3, ngroups_of(a) - 1) : 0;
  return spans_fit(a, std::min<int64_t>(kRows, a.dim) - 1, gspan);
}

size_t scan_workspace_bytes(const ssm_scan_args& a) {
  if (a.batch <= 0 || a.dim <= 0 || a.seqlen <= 0) return 0;
  const int64_t groups = a.batch * ((a.dim + kCh - 1) / kCh);
  const int nseg = choose_segments(groups, a.seqlen);
  if (nseg <= 1) return 0;
  return seg_layout(a, nseg).total;
}

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// The device address of the current device's copy of `scratch`, looked up
// on the first call on that device (with it current) and kept.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!ptr) return hipErrorInvalidSymbol;
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return hipSuccess;
}

}  // namespace

// The scan with the segment aggregates in `scratch` instead of a caller
// workspace.  Pass 1 writes every aggregate that pass 2 reads, so nothing in
// the scratch needs clearing between calls.
int scan_fwd_noalloc(const ssm_scan_args& a, hipStream_t stream) {
  if (scan_workspace_bytes(a) > SSM_NOALLOC_SCRATCH_BYTES) return SSM_ERR_SCRATCH;
  ssm_scan_args b = a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  if (scan_workspace_bytes(a) > 0) {
    void* ptr = nullptr;
    if (scratch_address(&ptr) != hipSuccess) return SSM_ERR_HIP;
    b.workspace = ptr;
    b.workspace_bytes = SSM_NOALLOC_SCRATCH_BYTES;
  }
  return launch_scan_fwd(b, stream) == hipSuccess ? SSM_OK : SSM_ERR_HIP;
}

hipError_t launch_scan_fwd(const ssm_scan_args& a, hipStream_t stream) {
  if (a.seqlen == 0) {
    // no token: the final states are the initial ones
    if (a.last_state && a.last_state != a.h0) {
      const int64_t n = a.batch * a.dim * a.dstate;
      copy_state_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(
          a.h0, a.last_state, n);
    }
    if (a.conv_weight && a.conv_state_out) {
      const int64_t n = a.batch * a.dim * a.d_conv;
      copy_state_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(
          a.conv_state_in, a.conv_state_out, n);
    }
    return hipGetLastError();
  }
  fwd::ScanParams p;
  p.u = a.u; p.delta = a.delta; p.z = a.z; p.B = a.B; p.C = a.C;
  p.A = a.A; p.D = a.D; p.bias = a.delta_bias; p.h0 = a.h0; p.last_state = a.last_state;
  p.out = a.out;
  p.usb = a.u_batch_stride; p.usd = a.u_dim_stride;
  p.dsb = a.delta_batch_stride; p.dsd = a.delta_dim_stride;
  p.zsb = a.z_batch_stride; p.zsd = a.z_dim_stride;
  p.Bsb = a.B_batch_stride; p.Bsg = a.B_group_stride; p.Bsn = a.B_state_stride;
  p.Csb = a.C_batch_stride; p.Csg = a.C_group_stride; p.Csn = a.C_state_stride;
  p.Asd = a.A_dim_stride; p.Asn = a.A_state_stride;
  p.osb = a.out_batch_stride; p.osd = a.out_dim_stride;
  p.batch = a.batch; p.dim = a.dim; p.L = static_cast<int>(a.seqlen);
  p.N = static_cast<int>(a.dstate);
  p.cpg = a.dim / ngroups_of(a);
  p.cgroups = (a.dim + kCh - 1) / kCh;

  // Segmenting needs the caller's workspace; without enough of it the whole
  // sequence runs as one segment (same result, less parallelism).
  const int64_t groups = a.batch * p.cgroups;
  const size_t need = scan_workspace_bytes(a);
  int nseg = 1;
  if (need > 0 && a.workspace && a.workspace_bytes >= need)
    nseg = choose_segments(groups, a.seqlen);
  const int64_t seg = (a.seqlen + nseg - 1) / nseg;
  p.seg_len = static_cast<int>((seg + kGT - 1) / kGT * kGT);
  p.nseg = static_cast<int>((a.seqlen + p.seg_len - 1) / p.seg_len);
  p.agg = nullptr;
  p.rec = nullptr;
  p.counts = nullptr;
  p.lists = nullptr;
  p.scope = p.cw = p.nchunk = 1;
  p.maxi = 1;
  p.ckpt = a.checkpoints;
  p.K = a.conv_weight ? a.d_conv : 0;
  p.conv_w = a.conv_weight; p.conv_b = a.conv_bias; p.conv_in = a.conv_state_in;
  p.conv_stout = a.conv_state_out; p.conv_out = a.conv_out;
  p.cosb = a.conv_out_batch_stride; p.cosd = a.conv_out_dim_stride;
  p.conv_silu = a.conv_silu;
  p.nbk = static_cast<int>((a.seqlen + kT - 1) / kT);

  const bool bf16 = a.io_dtype == SSM_BF16, sp = a.delta_softplus != 0;
  // lane mode with 16-byte aligned B/C rows and blocks: vector loads.  The
  // rows' ends are 16-byte aligned too (seqlen a multiple of the vector
  // width), so no load straddles the end of a buffer window.
  const int64_t vw = bf16 ? 8 : 4;
  auto al16 = [](const void* ptr) { return reinterpret_cast<uintptr_t>(ptr) % 16 == 0; };
  const bool lvec = al16(a.B) && al16(a.C) && a.seqlen % vw == 0 && a.B_batch_stride % vw == 0 &&
                    a.B_group_stride % vw == 0 && a.B_state_stride % vw == 0 &&
                    a.C_batch_stride % vw == 0 && a.C_group_stride % vw == 0 &&
                    a.C_state_stride % vw == 0;
  const int lane = lane_bc(a) ? (lvec ? 2 : 1) : 0;
  const bool defer = p.nseg == 1 && groups <= kDeferMaxGroups;
  auto run = [&](int pass, dim3 grid) {
    switch (slots(a.dstate)) {
      case 1: fwd::launch_slots<1>(pass, lane, bf16, sp, p.K, defer, grid, p, stream); break;
      case 2: fwd::launch_slots<2>(pass, lane, bf16, sp, p.K, defer, grid, p, stream); break;
      default: fwd::launch_slots<4>(pass, lane, bf16, sp, p.K, defer, grid, p, stream); break;
    }
  };
  if (p.nseg > 1) {
    // pass 1: every segment from zero (segment 0 from h0), with aggregates
    // and window records; the plan: incoming and window start states, the
    // windows each channel still needs, and per window the channels to
    // rescan, gathered by chunk; pass 2: those windows from their exact
    // start states, until the incoming state has decayed.  Stream order
    // puts each launch's results before the next.
    const SegLayout lay = seg_layout(a, p.nseg);
    char* ws = static_cast<char*>(a.workspace);
    p.agg = reinterpret_cast<float*>(ws + lay.agg);
    p.rec = reinterpret_cast<float*>(ws + lay.rec);
    int* jst = reinterpret_cast<int*>(ws + lay.jst);
    int* counts = reinterpret_cast<int*>(ws + lay.cnt);
    int* lists = reinterpret_cast<int*>(ws + lay.lst);
    p.counts = counts;
    p.lists = lists;
    p.scope = lane ? a.dim : p.cpg;
    p.cw = chunk_width(a, p.scope);
    p.nchunk = (a.dim / p.scope) * ((p.scope + p.cw - 1) / p.cw);
    p.maxi = static_cast<int>((p.cw + kCh - 1) / kCh);
    run(1, dim3((unsigned)(groups * p.nseg)));

    PlanParams pq;
    pq.agg = p.agg; pq.rec = p.rec; pq.jst = jst; pq.last_state = a.last_state;
    pq.A = a.A; pq.Asd = a.A_dim_stride; pq.Asn = a.A_state_stride;
    pq.batch = a.batch; pq.dim = a.dim;
    pq.N = p.N; pq.nseg = p.nseg; pq.L = p.L; pq.seg_len = p.seg_len;
    const int64_t rows = a.batch * a.dim * (p.nseg - 1);
    seg_plan_kernel<<<dim3((unsigned)((rows * kN + 255) / 256)), dim3(256), 0, stream>>>(pq);

    ListParams lq;
    lq.jst = jst; lq.counts = counts; lq.lists = lists;
    lq.batch = a.batch; lq.dim = a.dim; lq.scope = p.scope; lq.cw = p.cw; lq.nchunk = p.nchunk;
    lq.nseg = p.nseg;
    seg_list_kernel<<<dim3((unsigned)(a.batch * (p.nseg - 1) * p.nchunk * fwd::kWin)), dim3(256), 0,
                      stream>>>(lq);

    run(2, dim3((unsigned)(fwd::kWin * a.batch * p.nchunk * (p.nseg - 1) * p.maxi)));
  } else {
    run(0, dim3((unsigned)groups));
  }
  return hipGetLastError();
}

}  // namespace ssm

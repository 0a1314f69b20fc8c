// scan_fwd.hip -- host side of the prefill selective scan: segment choice,
// B/C mode, workspace, window limits and the launches.  The kernel itself is
// in scan_fwd_kernel.h (instantiated by scan_fwd_s1/s2/s4.hip).
#include <algorithm>

#include "scan_fwd_kernel.h"

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
// the extra aggregate pass and the fold stay small.
constexpr int64_t kTargetGroups = 1280;   // 5 wavefronts per SIMD on 256 CUs
constexpr int64_t kMinSegLen = 8192;
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

bool scan_windows_fit(const ssm_scan_args& a) {
  // Per-wavefront byte windows (and the lane offsets inside them) are 32-bit,
  // with a margin: lanes of padding states address from a window's end.
  const int64_t esz = a.io_dtype == SSM_BF16 ? 2 : 4;
  const int64_t rows = std::min<int64_t>(kRows, a.dim) - 1;
  const int64_t lim = (int64_t{1} << 32) - 256;
  auto fits = [&](int64_t span) { return span * esz < lim; };
  // a wavefront's four rows reach at most four groups in lane mode
  const int64_t gspan = lane_bc(a) ? std::min<int64_t>(3, ngroups_of(a) - 1) : 0;
  bool ok = fits(rows * a.u_dim_stride + a.seqlen) && fits(rows * a.delta_dim_stride + a.seqlen) &&
            fits(rows * a.out_dim_stride + a.seqlen) &&
            fits(gspan * a.B_group_stride + (a.dstate - 1) * a.B_state_stride + a.seqlen) &&
            fits(gspan * a.C_group_stride + (a.dstate - 1) * a.C_state_stride + a.seqlen);
  if (a.z) ok = ok && fits(rows * a.z_dim_stride + a.seqlen);
  if (a.conv_weight && a.conv_out) ok = ok && fits(rows * a.conv_out_dim_stride + a.seqlen);
  // checkpoints: four rows of ceil(L / 16) * dstate floats
  if (a.checkpoints)
    ok = ok && (rows + 1) * ((a.seqlen + kT - 1) / kT) * a.dstate * 4 < lim;
  return ok;
}

size_t scan_workspace_bytes(const ssm_scan_args& a) {
  if (a.batch <= 0 || a.dim <= 0 || a.seqlen <= 0) return 0;
  const int64_t groups = a.batch * ((a.dim + kCh - 1) / kCh);
  const int nseg = choose_segments(groups, a.seqlen);
  if (nseg <= 1) return 0;
  return static_cast<size_t>(a.batch * a.dim * (nseg - 1) * (a.dstate + 1)) * sizeof(float);
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
  p.agg = p.nseg > 1 ? static_cast<float*>(a.workspace) : nullptr;
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
  const bool defer = groups * p.nseg <= kDeferMaxGroups;
  auto run = [&](bool aggregate, dim3 grid) {
    switch (slots(a.dstate)) {
      case 1: fwd::launch_slots<1>(aggregate, lane, bf16, sp, p.K, defer, grid, p, stream); break;
      case 2: fwd::launch_slots<2>(aggregate, lane, bf16, sp, p.K, defer, grid, p, stream); break;
      default: fwd::launch_slots<4>(aggregate, lane, bf16, sp, p.K, defer, grid, p, stream); break;
    }
  };
  if (p.nseg > 1) run(true, dim3((unsigned)(groups * (p.nseg - 1))));
  run(false, dim3((unsigned)(groups * p.nseg)));
  return hipGetLastError();
}

}  // namespace ssm

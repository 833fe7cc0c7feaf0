// Gather of the bf16 rows of the selected tokens, the caller side of the
// hybrid set: after a selection, the full-precision K and V rows of the
// chosen tokens are copied into the contiguous [B][H][max_sel][D] arrays the
// hybrid decode reads (HyQuant page, method paragraphs: the vertical-line
// tokens are kept in full precision beside the 4-bit cache).
//
// A plain copy, bound by HBM: every row is read once and written once, with
// 16-byte loads and stores (16 lanes per row at D = 128, 8 at D = 64).
#include "mx_device.h"
#include "kernels.h"

namespace mxattn {

constexpr int kGatherThreads = 256;

__global__ __launch_bounds__(kGatherThreads) void gather_rows_kernel(GatherArgs a) {
  const int bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  int n = a.n_sel[bh];
  n = n < 0 ? 0 : (n > a.max_sel ? a.max_sel : n);
  const int lanes_per_row = a.D / 8;                 // 8 bf16 per lane
  const int rows_per_wg = kGatherThreads / lanes_per_row;
  const int row = blockIdx.x * rows_per_wg + static_cast<int>(threadIdx.x) / lanes_per_row;
  const int part = static_cast<int>(threadIdx.x) % lanes_per_row;
  if (row >= n) return;
  const int t = a.idx[static_cast<int64_t>(bh) * a.max_sel + row];
  const bool ok = t >= 0 && t < a.T;
  const int64_t dst = (static_cast<int64_t>(bh) * a.max_sel + row) * a.D + part * 8;
  v4i kv = v4i{0, 0, 0, 0}, vv = v4i{0, 0, 0, 0};
  if (ok) {
    kv = *reinterpret_cast<const v4i*>(a.k + b * a.ks[0] + h * a.ks[1] + t * a.ks[2] + part * 8);
    vv = *reinterpret_cast<const v4i*>(a.v + b * a.vs[0] + h * a.vs[1] + t * a.vs[2] + part * 8);
  }
  *reinterpret_cast<v4i*>(a.k_out + dst) = kv;
  *reinterpret_cast<v4i*>(a.v_out + dst) = vv;
}

hipError_t launch_gather_rows(const GatherArgs& a, hipStream_t stream) {
  const int rows_per_wg = kGatherThreads / (a.D / 8);
  const dim3 grid((a.max_sel + rows_per_wg - 1) / rows_per_wg, a.B * a.H);
  hipLaunchKernelGGL(gather_rows_kernel, grid, dim3(kGatherThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mxattn

// MXFP4 quantisation of activations / KV rows, and the Smooth-QK calibration
// reduction.
//
// Format: BitDecoding-FP4 page, "The KV Cache Bottleneck in Long-Context LLM
// Serving" (32-element blocks, E8M0 scale, E2M1 elements).  Optional
// per-channel factor: the static Smooth-QK rescale of the HiFA4 page
// (Abstract), applied as one fp32 multiply before the block maximum.
//
// Both kernels are bandwidth-bound: every input element is read once and
// 0.53 bytes per element are written.
#include "mx_device.h"
#include "kernels.h"

namespace mxattn {

// ---------------------------------------------------------------------------
// Eight consecutive elements of a row, widened to fp32, from one 16-byte
// (16-bit types) or two 16-byte (fp32) loads.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t i, float* y) {
  if constexpr (DT == 0) {
    const v4f a = *reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(base) + i);
    const v4f b = *reinterpret_cast<const v4f*>(reinterpret_cast<const float*>(base) + i + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      y[k] = a[k];
      y[4 + k] = b[k];
    }
  } else {
    const v4i w = *reinterpret_cast<const v4i*>(reinterpret_cast<const uint16_t*>(base) + i);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t u = static_cast<uint32_t>(w[k]);
      if constexpr (DT == 2) {
        y[2 * k] = __uint_as_float(u << 16);
        y[2 * k + 1] = __uint_as_float(u & 0xFFFF0000u);
      } else {
        y[2 * k] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u & 0xFFFFu)));
        y[2 * k + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(u >> 16)));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Head-dim blocks.  Four lanes own one 32-element block (8 elements each, one
// 16-byte load for 16-bit inputs), so one load instruction of a wave covers
// 16 consecutive blocks contiguously.  Each lane handles kHdRows such
// groups, all loads issued before any arithmetic; the block maximum is
// combined over the four lanes with two quad permutes.  Workgroup x of
// (batch b, head h) covers blocks [x*64*kHdRows, (x+1)*64*kHdRows) of that
// head; the index arithmetic inside a head is 32-bit.
constexpr int kHdRows = 2;
constexpr int kHdBlocksPerGroup = 64 * kHdRows;   // 4 waves x 16 blocks x kHdRows

__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  // quad_perm [1,0,3,2] then [2,3,0,1]: after both, every lane of a quad
  // holds the maximum of the four.
  uint32_t o = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false));
  v = o > v ? o : v;
  o = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false));
  return o > v ? o : v;
}

template <int DT>
__device__ __forceinline__ void quantize_hd(const QuantArgs& a, int x, int64_t h, int64_t b, bool flat) {
  const int nblk_row = static_cast<int>(a.D) / 32;   // 2 or 4
  // Blocks this launch covers for the workgroup's range: those of one head,
  // or (flat) those of every row of the tensor in (batch, head, row) order.
  const int64_t total = flat ? a.B * a.H * a.S * nblk_row : a.S * nblk_row;
  const int lane = threadIdx.x & 63;
  const int wave = x * 4 + (threadIdx.x >> 6);
  const int part = lane & 3;

  // Per group r: its block, and the (batch, head, row) that block lies in.
  int64_t blk[kHdRows], hr[kHdRows], br[kHdRows], sr[kHdRows];
#pragma unroll
  for (int r = 0; r < kHdRows; ++r) {
    blk[r] = (static_cast<int64_t>(wave) * kHdRows + r) * 16 + (lane >> 2);
    const int64_t row = blk[r] / nblk_row;
    if (flat) {
      sr[r] = row % a.S;
      const int64_t bh = row / a.S;
      hr[r] = bh % a.H;
      br[r] = bh / a.H;
    } else {
      sr[r] = row;
      hr[r] = h;
      br[r] = b;
    }
  }
  float y[kHdRows][8];
#pragma unroll
  for (int r = 0; r < kHdRows; ++r) {
    if (blk[r] < total) {
      load8<DT>(a.x, br[r] * a.xs[0] + hr[r] * a.xs[1] + sr[r] * a.xs[2] + ((blk[r] & (nblk_row - 1)) * 32 + part * 8),
                y[r]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) y[r][k] = 0.0f;
    }
  }
  // Groups of 16 blocks start on a row boundary (nblk_row divides 16), so a
  // lane's channels are the same in every group it handles.
  const int db = (lane >> 2) & (nblk_row - 1);
  const int d0 = db * 32 + part * 8;
  if (a.chan_scale != nullptr) {
#pragma unroll
    for (int r = 0; r < kHdRows; ++r) {
      // One head per workgroup: both groups share the factors.
      const int64_t hh = (flat || r == 0) ? (blk[r] < total ? hr[r] : 0) : hr[0];
      const v4f c0 = *reinterpret_cast<const v4f*>(a.chan_scale + hh * a.D + d0);
      const v4f c1 = *reinterpret_cast<const v4f*>(a.chan_scale + hh * a.D + d0 + 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        y[r][k] = __fmul_rn(y[r][k], c0[k]);
        y[r][4 + k] = __fmul_rn(y[r][4 + k], c1[k]);
      }
    }
  }
  if (a.hadamard) {
    // Normalised Walsh-Hadamard transform of each row (BitDecoding-FP4,
    // key outliers): element d = 8 (lane % lanes_per_row) + i.  Butterflies
    // (a, b) -> (a + b, a - b) on pairs (d, d + h), h = 1, 2, 4 inside the
    // lane, then h = 8 ... D/2 between lane and lane ^ (h / 8); every sum is
    // rounded to fp32 in that stage order, then one multiply by
    // fp32(1/sqrt(D)).
    const int row_lanes = static_cast<int>(a.D) / 8;   // 16 or 8
#pragma unroll
    for (int r = 0; r < kHdRows; ++r) {
#pragma unroll
      for (int hs = 1; hs < 8; hs <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if ((i & hs) == 0) {
            const float u = y[r][i], w = y[r][i + hs];
            y[r][i] = u + w;
            y[r][i + hs] = u - w;
          }
      for (int m = 1; m < row_lanes; m <<= 1) {
        const bool high = (lane & m) != 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float other = __shfl_xor(y[r][i], m);
          y[r][i] = high ? other - y[r][i] : y[r][i] + other;
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) y[r][i] = __fmul_rn(y[r][i], a.rot_scale);
    }
  }
#pragma unroll
  for (int r = 0; r < kHdRows; ++r) {
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t m = __float_as_uint(y[r][i]) & 0x7FFFFFFFu;
      amax = m > amax ? m : amax;  // magnitudes order like their bit patterns
    }
    // Lanes of a quad share blk, so a quad past the end is dead as a whole.
    amax = quad_max(amax);
    const int sb = e8m0_byte(amax, a.uos, a.qmax_quarter);
    const uint32_t packed = encode8(y[r], sb);
    uint32_t packed2 = 0;
    int sb2 = 0;
    if (a.codes2 != nullptr) {
      // Dual residual: x - dequant(code), exact in fp32 (the dequantised value
      // is 0 or within a factor of two of x), encoded the same way.
      float res[8];
      uint32_t amax2 = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        res[i] = y[r][i] - e2m1_value((packed >> (4 * i)) & 0xFu, sb);
        const uint32_t m2 = __float_as_uint(res[i]) & 0x7FFFFFFFu;
        amax2 = m2 > amax2 ? m2 : amax2;
      }
      amax2 = quad_max(amax2);
      sb2 = e8m0_byte(amax2, a.uos, a.qmax_quarter);
      packed2 = encode8(res, sb2);
    }
    if (blk[r] >= total) continue;
    const int64_t bb = br[r], hh = hr[r], s = sr[r];
    uint8_t* crow = a.codes + bb * a.cs[0] + hh * a.cs[1] + s * a.cs[2];
    *reinterpret_cast<uint32_t*>(crow + d0 / 2) = packed;
    if (part == 0) a.scales[bb * a.ss[0] + hh * a.ss[1] + s * a.ss[2] + db] = static_cast<uint8_t>(sb);
    if (a.codes2 != nullptr) {
      uint8_t* crow2 = a.codes2 + bb * a.cs2[0] + hh * a.cs2[1] + s * a.cs2[2];
      *reinterpret_cast<uint32_t*>(crow2 + d0 / 2) = packed2;
      if (part == 0) a.scales2[bb * a.ss2[0] + hh * a.ss2[1] + s * a.ss2[2] + db] = static_cast<uint8_t>(sb2);
    }
  }
}


// The same encoding for the common case: a workgroup inside one (batch,
// head), no rotation, no residual.  The (batch, head) bases are then
// uniform, so each lane's addresses are its row and channel only; this
// takes the 4K step's Q launch from 12.5 to 10.8 us against the general
// form above (same codes).
template <int DT>
__device__ __forceinline__ void quantize_hd_head(const QuantArgs& a, int x, int64_t h, int64_t b) {
  const int nblk_row = static_cast<int>(a.D) / 32;   // 2 or 4
  const int total = static_cast<int>(a.S) * nblk_row;
  const int lane = threadIdx.x & 63, part = lane & 3;
  const int wave = x * 4 + (threadIdx.x >> 6);
  constexpr int kElem = DT == 0 ? 4 : 2;
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(a.x) + (b * a.xs[0] + h * a.xs[1]) * kElem;
  uint8_t* cb = a.codes + b * a.cs[0] + h * a.cs[1];
  uint8_t* sbp = a.scales + b * a.ss[0] + h * a.ss[1];
  // Groups of 16 blocks start on a row boundary, so a lane's channels are
  // the same in every group it handles.
  const int db = (lane >> 2) & (nblk_row - 1);
  const int d0 = db * 32 + part * 8;
  int row[kHdRows];
  bool on[kHdRows];
  float y[kHdRows][8];
#pragma unroll
  for (int r = 0; r < kHdRows; ++r) {
    const int blk = (wave * kHdRows + r) * 16 + (lane >> 2);
    on[r] = blk < total;
    row[r] = blk / nblk_row;
    if (on[r]) {
      load8<DT>(xb + static_cast<int64_t>(row[r]) * a.xs[2] * kElem, d0, y[r]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) y[r][k] = 0.0f;
    }
  }
  if (a.chan_scale != nullptr) {
    const v4f c0 = *reinterpret_cast<const v4f*>(a.chan_scale + h * a.D + d0);
    const v4f c1 = *reinterpret_cast<const v4f*>(a.chan_scale + h * a.D + d0 + 4);
#pragma unroll
    for (int r = 0; r < kHdRows; ++r)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        y[r][k] = __fmul_rn(y[r][k], c0[k]);
        y[r][4 + k] = __fmul_rn(y[r][4 + k], c1[k]);
      }
  }
#pragma unroll
  for (int r = 0; r < kHdRows; ++r) {
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t m = __float_as_uint(y[r][i]) & 0x7FFFFFFFu;
      amax = m > amax ? m : amax;
    }
    // Lanes of a quad share the block, so a quad past the end is dead as a whole.
    amax = quad_max(amax);
    const int sb = e8m0_byte(amax, a.uos, a.qmax_quarter);
    const uint32_t packed = encode8(y[r], sb);
    if (!on[r]) continue;
    *reinterpret_cast<uint32_t*>(cb + static_cast<int64_t>(row[r]) * a.cs[2] + d0 / 2) = packed;
    if (part == 0) sbp[static_cast<int64_t>(row[r]) * a.ss[2] + db] = static_cast<uint8_t>(sb);
  }
}

// ---------------------------------------------------------------------------
// Sequence blocks (the key-blocked V layout of prefill).  Workgroup x of
// (b, h) stages tokens [32x, 32x+32) x D channels in LDS as fp32 (16-byte
// loads along the channels, all issued before the first LDS store), then
// each of the first D threads encodes one (channel, 32-token block) and
// writes its 16 code bytes.  Tokens past S are +0 padding inside the last
// block.
constexpr int kKeyChunk = 32;
// gfx950 (MI355X): the workgroups of a launch are dealt round robin to 8
// XCDs, each with its own L2.
constexpr int kXcds = 8;
constexpr int kKeyLoads = kKeyChunk * 16 / 256;  // 8-element loads per thread at D = 128

template <int DT>
__device__ __forceinline__ void quantize_key(const QuantArgs& a, int x, int64_t h, int64_t b,
                                             float (*tile)[129]) {
  const int D = static_cast<int>(a.D);
  const int64_t t0 = static_cast<int64_t>(x) * kKeyChunk;
  const int groups = D / 8;  // 8-channel groups per token
  float y[kKeyLoads][8];
#pragma unroll
  for (int j = 0; j < kKeyLoads; ++j) {
    const int i = threadIdx.x + j * 256;
    const int tt = i / groups, d0 = (i % groups) * 8;
    const int64_t t = t0 + tt;
    if (i < kKeyChunk * groups && t < a.S) {
      load8<DT>(a.x, b * a.xs[0] + h * a.xs[1] + t * a.xs[2] + d0, y[j]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) y[j][k] = 0.0f;
    }
  }
#pragma unroll
  for (int j = 0; j < kKeyLoads; ++j) {
    const int i = threadIdx.x + j * 256;
    if (i >= kKeyChunk * groups) continue;
    const int tt = i / groups, d0 = (i % groups) * 8;
    if (a.chan_scale != nullptr) {
#pragma unroll
      for (int k = 0; k < 8; ++k) y[j][k] = __fmul_rn(y[j][k], a.chan_scale[h * a.D + d0 + k]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) tile[tt][d0 + k] = y[j][k];
  }
  __syncthreads();
  const int d = threadIdx.x;
  if (d >= D) return;
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t m = __float_as_uint(tile[i][d]) & 0x7FFFFFFFu;
    amax = m > amax ? m : amax;
  }
  const int sb = e8m0_byte(amax, a.uos, a.qmax_quarter);
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = tile[q * 8 + i][d];
    w[q] = encode8(v, sb);
  }
  uint8_t* crow = a.codes + b * a.cs[0] + h * a.cs[1] + static_cast<int64_t>(d) * a.cs[2];
  *reinterpret_cast<v4i*>(crow + x * 16) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
  a.scales[b * a.ss[0] + h * a.ss[1] + static_cast<int64_t>(d) * a.ss[2] + x] = static_cast<uint8_t>(sb);
}

// ---------------------------------------------------------------------------
// One launch for up to kMaxQuantJobs tensors.  The grid is the concatenation
// of the jobs' workgroup ranges; workgroup id -> (job, x, head, batch) is
// uniform scalar arithmetic.  A single small tensor does not fill the chip
// and pays a launch's ramp and drain on its own: batched, the tensors of one
// attention call share them.
__global__ __launch_bounds__(256) void quantize_kernel(QuantBatch p) {
  __shared__ float tile[kKeyChunk][129];
  const int bid = blockIdx.x;
  int j = 0;
#pragma unroll
  for (int i = 1; i < kMaxQuantJobs; ++i) j += (i < p.n && bid >= p.start[i]) ? 1 : 0;
  const QuantArgs& a = p.job[j];
  const int local = bid - p.start[j];
  if (p.flat[j]) {
    if (a.dtype == 2) quantize_hd<2>(a, local, 0, 0, true);
    else if (a.dtype == 1) quantize_hd<1>(a, local, 0, 0, true);
    else quantize_hd<0>(a, local, 0, 0, true);
    return;
  }
  const int gx = p.gx[j];
  // Key layout: a workgroup writes 16 code bytes and one scale byte to each
  // channel row, and the neighbouring chunks of the same rows fill the rest
  // of those lines.  Workgroups are dealt to the 8 XCDs round robin, so
  // consecutive ids land in different L2s and their partial lines reach HBM
  // one by one (2.35x the written bytes, measured).  Each XCD takes one
  // contiguous run of chunks instead, so the lines fill in its L2 first.
  // (A permutation of the work: the output is the same.)
  int item = local;
  if (a.key_layout) {
    const int n = p.start[j + 1] - p.start[j];
    if (p.start[j] % kXcds == 0 && n % kXcds == 0) item = (local % kXcds) * (n / kXcds) + local / kXcds;
  }
  const int x = item % gx;
  const int rest = item / gx;
  const int H = static_cast<int>(a.H);
  const int64_t h = rest % H, b = rest / H;
  if (a.key_layout) {
    if (a.dtype == 2) quantize_key<2>(a, x, h, b, tile);
    else if (a.dtype == 1) quantize_key<1>(a, x, h, b, tile);
    else quantize_key<0>(a, x, h, b, tile);
  } else if (!a.hadamard && a.codes2 == nullptr) {
    if (a.dtype == 2) quantize_hd_head<2>(a, x, h, b);
    else if (a.dtype == 1) quantize_hd_head<1>(a, x, h, b);
    else quantize_hd_head<0>(a, x, h, b);
  } else {
    if (a.dtype == 2) quantize_hd<2>(a, x, h, b, false);
    else if (a.dtype == 1) quantize_hd<1>(a, x, h, b, false);
    else quantize_hd<0>(a, x, h, b, false);
  }
}

// ---------------------------------------------------------------------------
// Smooth-QK calibration.  One workgroup per (KV head, channel chunk of 64):
// maxima of |q| over the group's query heads and |k| over the tokens, then
//   s = sqrt(kmax/qmax) in double (1 if either is 0), clamped to [2^-8, 2^8].
// Maxima are exact; the double division and square root are IEEE operations,
// so the float32 results are reproducible bit for bit.
__global__ __launch_bounds__(256) void smooth_calibrate_kernel(CalibArgs a) {
  __shared__ float red_q[4][64];
  __shared__ float red_k[4][64];
  const int h = blockIdx.x;
  const int c = blockIdx.y * 64 + (threadIdx.x & 63);
  const int part = threadIdx.x >> 6;  // 4 row-groups
  const int g = a.hq / a.hkv;
  float qm = 0.0f, km = 0.0f;
  if (c < a.dim) {
    for (int64_t r = part; r < static_cast<int64_t>(g) * a.tokens; r += 4) {
      const int64_t gq = h * g + r / a.tokens, t = r % a.tokens;
      qm = fmaxf(qm, fabsf(load_elem(a.q, (gq * a.tokens + t) * a.dim + c, a.dtype)));
    }
    for (int64_t t = part; t < a.tokens; t += 4)
      km = fmaxf(km, fabsf(load_elem(a.k, (static_cast<int64_t>(h) * a.tokens + t) * a.dim + c, a.dtype)));
  }
  red_q[part][threadIdx.x & 63] = qm;
  red_k[part][threadIdx.x & 63] = km;
  __syncthreads();
  if (part == 0 && c < a.dim) {
    for (int p = 1; p < 4; ++p) {
      qm = fmaxf(qm, red_q[p][threadIdx.x]);
      km = fmaxf(km, red_k[p][threadIdx.x]);
    }
    double s = 1.0;
    if (qm > 0.0f && km > 0.0f) s = __dsqrt_rn(__ddiv_rn(static_cast<double>(km), static_cast<double>(qm)));
    s = s < 0x1p-8 ? 0x1p-8 : (s > 0x1p8 ? 0x1p8 : s);
    a.k_scale[h * a.dim + c] = static_cast<float>(__ddiv_rn(1.0, s));
    for (int i = 0; i < g; ++i) a.q_scale[(static_cast<int64_t>(h) * g + i) * a.dim + c] = static_cast<float>(s);
  }
}

// Jobs with the sequence-blocked layout go first: their workgroups have the
// longer dependency chain (load, LDS, barrier, encode), so they should not
// form the tail of the launch.
hipError_t launch_quantize_batch(const QuantArgs* jobs, int n, hipStream_t stream) {
  if (n < 1 || n > kMaxQuantJobs) return hipErrorInvalidValue;
  QuantBatch p{};
  int64_t total = 0;
  int k = 0;
  for (int pass = 0; pass < 2; ++pass)
    for (int i = 0; i < n; ++i) {
      const QuantArgs& a = jobs[i];
      if ((a.key_layout != 0) != (pass == 0)) continue;
      const int64_t blocks_head = a.S * (a.D / 32);
      const bool flat = !a.key_layout && blocks_head < kHdBlocksPerGroup;
      const int64_t gx = a.key_layout ? (a.S + kKeyChunk - 1) / kKeyChunk
                                      : (blocks_head + kHdBlocksPerGroup - 1) / kHdBlocksPerGroup;
      const int64_t n_wg = flat ? (blocks_head * a.H * a.B + kHdBlocksPerGroup - 1) / kHdBlocksPerGroup
                                : gx * a.H * a.B;
      p.job[k] = a;
      p.gx[k] = static_cast<int>(gx);
      p.flat[k] = flat ? 1 : 0;
      p.start[k] = static_cast<int>(total);
      total += n_wg;
      if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
      ++k;
    }
  p.n = k;
  p.start[k] = static_cast<int>(total);
  if (total > 0) hipLaunchKernelGGL(quantize_kernel, dim3(static_cast<unsigned>(total)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_smooth_calibrate(const CalibArgs& a, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(a.hkv), static_cast<unsigned>((a.dim + 63) / 64));
  hipLaunchKernelGGL(smooth_calibrate_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mxattn

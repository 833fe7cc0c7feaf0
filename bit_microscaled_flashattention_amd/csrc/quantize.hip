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
// 16-byte load for 16-bit inputs), so a wave covers 16 consecutive blocks and
// every load and store is contiguous across the wave.
// Eight elements to eight packed E2M1 codes (element i in nibble i) under
// scale byte sb.  From byte 3 up the hardware convert does it: it rounds
// y/2^e to nearest even on the E2M1 grid, saturates and keeps the sign, and
// every fp32 subnormal element lands below 0.25 and codes to signed zero
// whatever the convert's denormal handling.  Bytes 0..2 take the
// integer-exact encoder.
__device__ __forceinline__ uint32_t encode8(const float* y, int sb) {
  uint32_t packed = 0;
  if (sb >= 3) {
    const float scl = scale_of_byte(sb);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[0], y[1], scl, 0);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[2], y[3], scl, 1);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[4], y[5], scl, 2);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, y[6], y[7], scl, 3);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) packed |= e2m1_code(y[i], sb) << (4 * i);
  }
  return packed;
}

template <int DT>
__global__ __launch_bounds__(256) void quantize_hd_kernel(QuantArgs a) {
  const int64_t nblk_row = a.D / 32;
  const int64_t total = a.B * a.H * a.S * nblk_row;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t blk = gid >> 2;
  const int part = static_cast<int>(gid & 3);
  // Lanes past the end still take part in the cross-lane maximum (with a
  // zero contribution) and then write nothing.
  const bool live = blk < total;
  const int64_t bb = live ? blk : 0;
  const int64_t db = bb % nblk_row;
  int64_t rest = bb / nblk_row;
  const int64_t s = rest % a.S;
  rest /= a.S;
  const int64_t h = rest % a.H;
  const int64_t b = rest / a.H;
  const int64_t d0 = db * 32 + part * 8;

  float y[8];
  if (live) {
    load8<DT>(a.x, b * a.xs[0] + h * a.xs[1] + s * a.xs[2] + d0, y);
    if (a.chan_scale != nullptr) {
      const v4f c0 = *reinterpret_cast<const v4f*>(a.chan_scale + h * a.D + d0);
      const v4f c1 = *reinterpret_cast<const v4f*>(a.chan_scale + h * a.D + d0 + 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        y[k] = __fmul_rn(y[k], c0[k]);
        y[4 + k] = __fmul_rn(y[4 + k], c1[k]);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = 0.0f;
  }
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t m = __float_as_uint(y[i]) & 0x7FFFFFFFu;
    amax = m > amax ? m : amax;  // magnitudes order like their bit patterns
  }
  uint32_t o1 = __shfl_xor(amax, 1, 4);
  amax = o1 > amax ? o1 : amax;
  uint32_t o2 = __shfl_xor(amax, 2, 4);
  amax = o2 > amax ? o2 : amax;
  const int sb = e8m0_byte(amax, a.uos, a.qmax_quarter);
  const uint32_t packed = encode8(y, sb);
  if (!live) return;
  uint8_t* crow = a.codes + b * a.cs[0] + h * a.cs[1] + s * a.cs[2];
  *reinterpret_cast<uint32_t*>(crow + d0 / 2) = packed;
  if (part == 0) a.scales[b * a.ss[0] + h * a.ss[1] + s * a.ss[2] + db] = static_cast<uint8_t>(sb);
}

// ---------------------------------------------------------------------------
// Sequence blocks (the key-blocked V layout of prefill).  A workgroup stages
// 64 tokens x D channels in LDS as fp32 (16-byte loads along the channels),
// then each thread encodes one (channel, 32-token block) and writes its 16
// code bytes.  Tokens past S are +0 padding inside the last block.
constexpr int kKeyChunk = 64;

template <int DT>
__global__ __launch_bounds__(256) void quantize_key_kernel(QuantArgs a) {
  __shared__ float tile[kKeyChunk][129];
  const int64_t nchunk = (a.S + kKeyChunk - 1) / kKeyChunk;
  const int64_t chunk = blockIdx.x % nchunk;
  const int64_t bh = blockIdx.x / nchunk;
  const int64_t h = bh % a.H;
  const int64_t b = bh / a.H;
  const int D = static_cast<int>(a.D);
  const int64_t t0 = chunk * kKeyChunk;
  const int groups = D / 8;  // 8-channel groups per token
  for (int i = threadIdx.x; i < kKeyChunk * groups; i += blockDim.x) {
    const int tt = i / groups, d0 = (i % groups) * 8;
    const int64_t t = t0 + tt;
    float y[8];
    if (t < a.S) {
      load8<DT>(a.x, b * a.xs[0] + h * a.xs[1] + t * a.xs[2] + d0, y);
      if (a.chan_scale != nullptr) {
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = __fmul_rn(y[k], a.chan_scale[h * a.D + d0 + k]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) y[k] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) tile[tt][d0 + k] = y[k];
  }
  __syncthreads();
  const int tasks = D * (kKeyChunk / 32);
  for (int task = threadIdx.x; task < tasks; task += blockDim.x) {
    const int d = task % D;
    const int sub = task / D;
    const int64_t tblk = t0 / 32 + sub;
    if (tblk * 32 >= a.S) continue;
    uint32_t amax = 0;
    for (int i = 0; i < 32; ++i) {
      uint32_t m = __float_as_uint(tile[sub * 32 + i][d]) & 0x7FFFFFFFu;
      amax = m > amax ? m : amax;
    }
    const int sb = e8m0_byte(amax, a.uos, a.qmax_quarter);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = tile[sub * 32 + q * 8 + i][d];
      w[q] = encode8(y, sb);
    }
    uint8_t* crow = a.codes + b * a.cs[0] + h * a.cs[1] + static_cast<int64_t>(d) * a.cs[2];
    *reinterpret_cast<v4i*>(crow + tblk * 16) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    a.scales[b * a.ss[0] + h * a.ss[1] + static_cast<int64_t>(d) * a.ss[2] + tblk] = static_cast<uint8_t>(sb);
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

template <int DT>
static void launch_quantize_t(const QuantArgs& a, hipStream_t stream) {
  if (a.key_layout) {
    const int64_t nchunk = (a.S + kKeyChunk - 1) / kKeyChunk;
    const int64_t grid = nchunk * a.B * a.H;
    if (grid > 0) hipLaunchKernelGGL(quantize_key_kernel<DT>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, a);
  } else {
    const int64_t threads = a.B * a.H * a.S * (a.D / 32) * 4;
    const int64_t grid = (threads + 255) / 256;
    if (grid > 0) hipLaunchKernelGGL(quantize_hd_kernel<DT>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, a);
  }
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream) {
  if (a.dtype == 0) launch_quantize_t<0>(a, stream);
  else if (a.dtype == 1) launch_quantize_t<1>(a, stream);
  else launch_quantize_t<2>(a, stream);
  return hipGetLastError();
}

hipError_t launch_smooth_calibrate(const CalibArgs& a, hipStream_t stream) {
  dim3 grid(static_cast<unsigned>(a.hkv), static_cast<unsigned>((a.dim + 63) / 64));
  hipLaunchKernelGGL(smooth_calibrate_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mxattn

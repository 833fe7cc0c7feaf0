// Decode: one query token per sequence against an MXFP4 KV cache, with the
// dequantisation fused into the scan, optionally with a bf16 hybrid token set
// under the same softmax.
//
// Method: HyQuant page (method paragraphs) -- the decode cache stays 4-bit and
// is dequantised inside the attention scan (no full-precision copy); the
// vertical-line tokens and the recent window are held in bf16 and share one
// online softmax with the 4-bit tokens.  BitDecoding-FP4 page ("System-Level
// Optimization") -- the query heads of a KV head are stacked into one MMA.
//
// gfx950 design
//   * One workgroup (4 waves) per (batch, KV head, split of split_len tokens);
//     each wave walks 32-token chunks.  The GQA group's query heads are the
//     N columns of the MFMAs.
//   * Logits: v_mfma_scale_f32_16x16x128_f8f6f4 with the K rows (E2M1 codes
//     and their E8M0 scales) loaded straight from HBM into the A operand.
//   * P stays fp32; it enters a bf16 MFMA as hi + lo bf16 parts (about 16
//     significant bits).  V rows are converted to bf16 with their scale
//     (v_cvt_scalef32_pk_bf16_fp4, exact) and staged in LDS, from where each
//     lane gathers the 8 tokens of its channel for the V^T operand.
//   * The next chunk's K and V bytes are loaded while the current one is
//     computed.  Partial (O, m, l) per split go to the workspace and a merge
//     kernel combines them in a fixed order (deterministic).
#include "mx_device.h"
#include "kernels.h"

namespace mxattn {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kDecThreads = 256;
constexpr int kChunk = 32;          // tokens per wave iteration
constexpr int kVRow = 256 + 16;     // LDS bytes per staged bf16 V row (128 ch + pad)

__device__ __forceinline__ v4f mfma16_bf16(v4i a, v4i b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0,
                                                  0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const __bf16 a = static_cast<__bf16>(lo), b = static_cast<__bf16>(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ float bf16_to_f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Token (within a 32-token chunk) held by lane group g at k-slot i of the
// 16x16 C / 16x16x32 operand layout: two 16-key logit tiles, 4 keys each.
__device__ __forceinline__ int chunk_tok(int g, int i) { return (i < 4 ? 0 : 16) + 4 * g + (i & 3); }

struct DecState {
  float m, l;
  v4f O[8];
};

// Online-softmax update for one chunk.  s[8]: raw logits (-inf = absent) of
// this lane's 8 tokens for query column j.  Produces the hi/lo bf16 B
// operands of the PV product.
__device__ __forceinline__ void softmax_chunk(DecState& st, const float* s, float c, v4i& bhi, v4i& blo,
                                              float& alpha) {
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, s[i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m, mx);
  // m_new = -inf only while nothing has been seen: keep the state at zero.
  const bool none = m_new == -__builtin_huge_valf();
  alpha = none ? 1.0f : fast_exp2((st.m - m_new) * c);
  const float mc = none ? 0.0f : m_new * c;
  float p[8];
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = fast_exp2(__builtin_fmaf(s[i], c, -mc));
    sum += p[i];
  }
  st.l = st.l * alpha + sum;
  st.m = m_new;
  uint32_t h[4], lo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16(p[2 * i], p[2 * i + 1]);
    const float r0 = p[2 * i] - bf16_to_f(h[i] & 0xFFFFu);
    const float r1 = p[2 * i + 1] - bf16_to_f(h[i] >> 16);
    lo[i] = pack_bf16(r0, r1);
  }
  bhi = v4i{(int)h[0], (int)h[1], (int)h[2], (int)h[3]};
  blo = v4i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3]};
}

// O^T += V^T P^T for one chunk from the staged bf16 rows (this wave's LDS).
__device__ __forceinline__ void pv_chunk(DecState& st, const uint8_t* vr, int lane, v4i bhi, v4i blo, float alpha,
                                         int D) {
  const int dl = lane & 15, g = lane >> 4;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    if (dt * 16 >= D) break;
    const int d = dt * 16 + dl;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t a = *reinterpret_cast<const uint16_t*>(vr + chunk_tok(g, 2 * i) * kVRow + d * 2);
      const uint32_t b = *reinterpret_cast<const uint16_t*>(vr + chunk_tok(g, 2 * i + 1) * kVRow + d * 2);
      w[i] = a | (b << 16);
    }
    const v4i aop = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    v4f o = st.O[dt] * alpha;
    o = mfma16_bf16(aop, bhi, o);
    st.O[dt] = mfma16_bf16(aop, blo, o);
  }
}

// Combine the four waves' partial states of one workgroup (through the LDS
// staging area, which is free once the scan is done) and write one (O, m, l)
// per query column into partial slot `slot`.
struct RedLds {
  float m[4][16];
  float l[4][16];
  float o[4][16][132];
};

template <int D>
__device__ __forceinline__ void combine_store(void* lds, const DecState& st, const DecodeArgs& a, int b, int hk,
                                              int slot, int n_slot) {
  RedLds* red = reinterpret_cast<RedLds*>(lds);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int G = a.Hq / a.Hkv;
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (g == 0) {
    red->m[wave][j] = st.m;
    red->l[wave][j] = l;
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red->o[wave][j][dt * 16 + 4 * g + r] = st.O[dt][r];
  __syncthreads();
  for (int e = threadIdx.x; e < G * (D + 2); e += kDecThreads) {
    const int col = e / (D + 2), k = e % (D + 2);
    float M = -__builtin_huge_valf();
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red->m[w][col]);
    float acc = 0.0f;
    for (int w = 0; w < 4; ++w) {
      const float mw = red->m[w][col];
      const float f = mw == -__builtin_huge_valf() ? 0.0f : fast_exp2((mw - M) * a.c);
      acc += f * (k < D ? red->o[w][col][k] : (k == D + 1 ? red->l[w][col] : 0.0f));
    }
    const int hq = hk * G + col;
    float* dst = a.part + ((static_cast<int64_t>(b) * a.Hq + hq) * n_slot + slot) * (D + 2);
    dst[k] = k == D ? M : acc;
  }
}

constexpr int kStageBytes = 4 * kChunk * kVRow;
static_assert(sizeof(RedLds) <= kStageBytes, "reduction must fit in the staging area");

// ---------------------------------------------------------------------------
// FP4 cache scan of one split.
template <int D>
__global__ __launch_bounds__(kDecThreads) void decode_fp4_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t vstage[kStageBytes];
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int G = a.Hq / a.Hkv;
  int ctx = a.ctx_len[b];
  ctx = ctx < 1 ? 1 : (ctx > a.Tcap ? a.Tcap : ctx);
  const int win = a.hybrid ? (a.window < ctx ? a.window : ctx) : 0;
  const int end4 = ctx - win;                    // 4-bit tokens are [0, end4)
  const int t_begin = split * a.split_len;
  const int t_end = min(t_begin + a.split_len, end4);
  const int n_slot = a.n_split + (a.hybrid ? 1 : 0);

  // Query operand: column j (query head hk*G + j), channels [32g, 32g+32).
  v4i qop = {0, 0, 0, 0};
  int qsc = 0;
  if (j < G) {
    const int hq = hk * G + j;
    const uint8_t* qc = a.q.codes + b * a.q.cs[0] + hq * a.q.cs[1];
    const uint8_t* qs = a.q.scales + b * a.q.ss[0] + hq * a.q.ss[1];
    if (g < D / 32) {
      qop = *reinterpret_cast<const v4i*>(qc + g * 16);
      qsc = qs[g];
    }
  }
  const uint8_t* kc = a.k.codes + b * a.k.cs[0] + hk * a.k.cs[1];
  const uint8_t* ks = a.k.scales + b * a.k.ss[0] + hk * a.k.ss[1];
  const uint8_t* vc = a.v.codes + b * a.v.cs[0] + hk * a.v.cs[1];
  const uint8_t* vs = a.v.scales + b * a.v.ss[0] + hk * a.v.ss[1];
  const uint32_t* mask = a.hybrid ? a.mask + (static_cast<int64_t>(b) * a.Hkv + hk) * ((a.Tcap + 31) / 32) : nullptr;
  uint8_t* vr = vstage + wave * kChunk * kVRow;

  DecState st;
  st.m = -__builtin_huge_valf();
  st.l = 0.0f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.O[dt] = v4f{0, 0, 0, 0};

  const int nblk_d = D / 32;
  // Per-lane loads of one chunk: K operands of the two 16-key tiles, and two
  // (token, 32-channel) V blocks for the bf16 staging.
  struct Loaded {
    v4i k[2];
    int ks[2];
    v4i v[2];
    int vs[2];
  } cur, nxt;
  auto load = [&](Loaded& L, int t0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = t0 + h * 16 + j;
      const bool ok = t < t_end && g < nblk_d;
      L.k[h] = ok ? *reinterpret_cast<const v4i*>(kc + static_cast<int64_t>(t) * a.k.cs[2] + g * 16) : v4i{0, 0, 0, 0};
      L.ks[h] = ok ? ks[static_cast<int64_t>(t) * a.k.ss[2] + g] : 0;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int bi = lane + 64 * h;               // (token, channel block) id in the chunk
      const int tt = bi / nblk_d, db = bi % nblk_d;
      const int t = t0 + tt;
      const bool ok = tt < kChunk && t < t_end;
      L.v[h] = ok ? *reinterpret_cast<const v4i*>(vc + static_cast<int64_t>(t) * a.v.cs[2] + db * 16) : v4i{0, 0, 0, 0};
      L.vs[h] = ok ? vs[static_cast<int64_t>(t) * a.v.ss[2] + db] : 127;
    }
  };

  const int n_chunks = t_end > t_begin ? (t_end - t_begin + kChunk - 1) / kChunk : 0;
  const int rounds = (n_chunks + 3) / 4;
  if (rounds > 0) load(cur, t_begin + wave * kChunk);
  for (int rd = 0; rd < rounds; ++rd) {
    const int ci = rd * 4 + wave;
    const int t0 = t_begin + ci * kChunk;
    const bool active = ci < n_chunks;
    if (rd + 1 < rounds) load(nxt, t0 + 4 * kChunk);
    // Stage V as bf16 rows (exact: code x 2^e).
    if (active) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int bi = lane + 64 * h;
        const int tt = bi / nblk_d, db = bi % nblk_d;
        if (tt < kChunk) {
          const float scl = cur.vs[h] > 0 ? scale_of_byte(cur.vs[h]) : 0.0f;
          uint32_t w[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t src = static_cast<uint32_t>(cur.v[h][q]);
            w[4 * q + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scl, 0));
            w[4 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scl, 1));
            w[4 * q + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scl, 2));
            w[4 * q + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(src, scl, 3));
          }
          uint8_t* dst = vr + tt * kVRow + db * 64;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<v4i*>(dst + 16 * q) = v4i{(int)w[4 * q], (int)w[4 * q + 1], (int)w[4 * q + 2], (int)w[4 * q + 3]};
        }
      }
    }
    __syncthreads();
    if (active) {
      // Logits for the two 16-key tiles.
      v4f s0 = mfma16_fp4(cur.k[0], qop, v4f{0, 0, 0, 0}, cur.ks[0], qsc);
      v4f s1 = mfma16_fp4(cur.k[1], qop, v4f{0, 0, 0, 0}, cur.ks[1], qsc);
      float s[8];
      const uint32_t mw = mask ? mask[t0 / 32] : 0u;   // chunks are 32-aligned
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int tk = chunk_tok(g, i);
        const float x = i < 4 ? s0[i] : s1[i - 4];
        const bool absent = (t0 + tk >= t_end) || ((mw >> tk) & 1u) || j >= G;
        s[i] = absent ? -__builtin_huge_valf() : x;
      }
      v4i bhi, blo;
      float alpha;
      softmax_chunk(st, s, a.c, bhi, blo, alpha);
      pv_chunk(st, vr, lane, bhi, blo, alpha, D);
    }
    __syncthreads();
    cur = nxt;
  }

  combine_store<D>(vstage, st, a, b, hk, split, n_slot);
}

// ---------------------------------------------------------------------------
// bf16 hybrid set: selected rows (idx < ctx - window) then the window rows.
template <int D>
__global__ __launch_bounds__(kDecThreads) void decode_bf16_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t vstage[kStageBytes];
  const int hk = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int G = a.Hq / a.Hkv;
  int ctx = a.ctx_len[b];
  ctx = ctx < 1 ? 1 : (ctx > a.Tcap ? a.Tcap : ctx);
  const int win = a.window < ctx ? a.window : ctx;
  const int64_t bh = static_cast<int64_t>(b) * a.Hkv + hk;
  int nsel = a.max_sel > 0 ? a.n_sel[bh] : 0;
  nsel = nsel < 0 ? 0 : (nsel > a.max_sel ? a.max_sel : nsel);
  const int32_t* idx = a.max_sel > 0 ? a.idx + bh * a.max_sel : nullptr;
  // Selected rows at or past ctx - window are not part of the set.
  const int limit = ctx - win;
  const int n_total = nsel + win;
  const int woff = a.window - win;   // window rows before ctx-window+0 are unused
  const int n_slot = a.n_split + 1;
  uint8_t* vr = vstage + wave * kChunk * kVRow;

  // bf16 query operand for the 16x16x32 bf16 MFMA: column j, channels
  // [32 kk + 8g, +8) for k-step kk.
  v4i qop[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    qop[kk] = v4i{0, 0, 0, 0};
    if (j < G && kk * 32 < D) {
      const uint16_t* q = a.q_bf16 + (static_cast<int64_t>(b) * a.Hq + hk * G + j) * D + kk * 32 + 8 * g;
      qop[kk] = *reinterpret_cast<const v4i*>(q);
    }
  }
  auto row_k = [&](int i) -> const uint16_t* {
    return i < nsel ? a.k_sel + (bh * a.max_sel + i) * D : a.k_win + (bh * a.window + woff + (i - nsel)) * D;
  };
  auto row_v = [&](int i) -> const uint16_t* {
    return i < nsel ? a.v_sel + (bh * a.max_sel + i) * D : a.v_win + (bh * a.window + woff + (i - nsel)) * D;
  };
  auto valid = [&](int i) -> bool { return i < n_total && (i >= nsel || idx[i] < limit); };

  DecState st;
  st.m = -__builtin_huge_valf();
  st.l = 0.0f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.O[dt] = v4f{0, 0, 0, 0};

  const int n_chunks = (n_total + kChunk - 1) / kChunk;
  const int rounds = (n_chunks + 3) / 4;
  for (int rd = 0; rd < rounds; ++rd) {
    const int ci = rd * 4 + wave;
    const int t0 = ci * kChunk;
    const bool active = ci < n_chunks;
    if (active) {
      // Stage V rows: 32 rows x D bf16, 16 bytes per lane per step.
      for (int e = lane; e < kChunk * (D / 8); e += 64) {
        const int tt = e / (D / 8), part = e % (D / 8);
        v4i x = {0, 0, 0, 0};
        if (t0 + tt < n_total) x = *reinterpret_cast<const v4i*>(row_v(t0 + tt) + part * 8);
        *reinterpret_cast<v4i*>(vr + tt * kVRow + part * 16) = x;
      }
    }
    __syncthreads();
    if (active) {
      v4f sc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = t0 + h * 16 + j;
        const bool ok = i < n_total;
        const uint16_t* kr = ok ? row_k(i) : nullptr;
        v4f acc = {0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          if (kk * 32 >= D) break;
          const v4i aop = ok ? *reinterpret_cast<const v4i*>(kr + kk * 32 + 8 * g) : v4i{0, 0, 0, 0};
          acc = mfma16_bf16(aop, qop[kk], acc);
        }
        sc[h] = acc;
      }
      float s[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int tk = chunk_tok(g, i);
        const float x = i < 4 ? sc[0][i] : sc[1][i - 4];
        s[i] = (valid(t0 + tk) && j < G) ? x : -__builtin_huge_valf();
      }
      v4i bhi, blo;
      float alpha;
      softmax_chunk(st, s, a.c, bhi, blo, alpha);
      pv_chunk(st, vr, lane, bhi, blo, alpha, D);
    }
    __syncthreads();
  }

  combine_store<D>(vstage, st, a, b, hk, a.n_split, n_slot);
}

// ---------------------------------------------------------------------------
// Bitmap of the selected tokens that the bf16 set holds (idx < ctx-window),
// one workgroup per (batch, KV head); built in LDS, written whole.
__global__ __launch_bounds__(256) void hybrid_mask_kernel(DecodeArgs a) {
  extern __shared__ uint32_t bits[];
  const int hk = blockIdx.x, b = blockIdx.y;
  const int words = (a.Tcap + 31) / 32;
  const int64_t bh = static_cast<int64_t>(b) * a.Hkv + hk;
  for (int w = threadIdx.x; w < words; w += blockDim.x) bits[w] = 0u;
  __syncthreads();
  int ctx = a.ctx_len[b];
  ctx = ctx < 1 ? 1 : (ctx > a.Tcap ? a.Tcap : ctx);
  const int win = a.window < ctx ? a.window : ctx;
  int nsel = a.max_sel > 0 ? a.n_sel[bh] : 0;
  nsel = nsel < 0 ? 0 : (nsel > a.max_sel ? a.max_sel : nsel);
  for (int i = threadIdx.x; i < nsel; i += blockDim.x) {
    const int t = a.idx[bh * a.max_sel + i];
    if (t >= 0 && t < ctx - win) atomicOr(&bits[t >> 5], 1u << (t & 31));
  }
  __syncthreads();
  uint32_t* dst = a.mask + bh * words;
  for (int w = threadIdx.x; w < words; w += blockDim.x) dst[w] = bits[w];
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the split partials, in split order.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a) {
  const int hq = blockIdx.x, b = blockIdx.y;
  const int d = threadIdx.x;
  const int n_slot = a.n_split + (a.hybrid ? 1 : 0);
  const float* p = a.part + (static_cast<int64_t>(b) * a.Hq + hq) * n_slot * (D + 2);
  float M = -__builtin_huge_valf();
  for (int s = 0; s < n_slot; ++s) M = fmaxf(M, p[s * (D + 2) + D]);
  float num = 0.0f, den = 0.0f;
  for (int s = 0; s < n_slot; ++s) {
    const float ms = p[s * (D + 2) + D];
    if (ms == -__builtin_huge_valf()) continue;
    const float f = fast_exp2((ms - M) * a.c);
    num += f * p[s * (D + 2) + d];
    den += f * p[s * (D + 2) + D + 1];
  }
  const int64_t row = static_cast<int64_t>(b) * a.Hq + hq;
  a.out[row * D + d] = num / den;
  if (a.lse != nullptr && d == 0) a.lse[row] = M * a.softmax_scale + logf(den);
}

hipError_t launch_decode(const DecodeArgs& a, int D, hipStream_t stream) {
  if (a.hybrid) {
    const size_t words = (a.Tcap + 31) / 32;
    hipLaunchKernelGGL(hybrid_mask_kernel, dim3(a.Hkv, a.B), dim3(256), words * sizeof(uint32_t), stream, a);
  }
  const dim3 grid(a.n_split, a.Hkv, a.B);
  if (D == 128) {
    hipLaunchKernelGGL(decode_fp4_kernel<128>, grid, dim3(kDecThreads), 0, stream, a);
    if (a.hybrid) hipLaunchKernelGGL(decode_bf16_kernel<128>, dim3(1, a.Hkv, a.B), dim3(kDecThreads), 0, stream, a);
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(a.Hq, a.B), dim3(128), 0, stream, a);
  } else {
    hipLaunchKernelGGL(decode_fp4_kernel<64>, grid, dim3(kDecThreads), 0, stream, a);
    if (a.hybrid) hipLaunchKernelGGL(decode_bf16_kernel<64>, dim3(1, a.Hkv, a.B), dim3(kDecThreads), 0, stream, a);
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(a.Hq, a.B), dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mxattn

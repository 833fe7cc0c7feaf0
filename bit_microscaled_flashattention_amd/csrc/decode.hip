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
//   * The next chunks' K and V bytes are loaded (non-temporal: the cache is
//     streamed once) while the current one is computed.  Partial (O, m, l) per split go to the workspace and a merge
//     kernel combines them in a fixed order (deterministic).
#include <mutex>

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
                                              float& alpha, bool& moved) {
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, s[i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m, mx);
  // m_new = -inf only while nothing has been seen: keep the state at zero.
  const bool none = m_new == -__builtin_huge_valf();
  alpha = none ? 1.0f : fast_exp2((st.m - m_new) * c);
  moved = __builtin_amdgcn_ballot_w64(m_new > st.m) != 0;
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
                                         bool moved, int D) {
  const int dl = lane & 15, g = lane >> 4;
  if (moved) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      if (dt * 16 < D) st.O[dt] *= alpha;
  }
  // The A operand of lane (channel dl, group g) is the bf16 of tokens
  // chunk_tok(g, 0..7) in channel 16 dt + dl, read with the LDS transpose
  // load: in each 16-lane group, lane 4a + b receives element b of the
  // 8-byte reads of lanes a, a + 4, a + 8, a + 12.  So lane s reads channels
  // [16 dt + 4 (s % 4), +4) of token 4g + s / 4 (then 16 more tokens on).
  const int s16 = lane & 15;
  const uint8_t* vsrc = vr + (4 * g + (s16 >> 2)) * kVRow + 8 * (s16 & 3);
  (void)dl;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    if (dt * 16 >= D) break;
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef int v2i_t __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    lds_v4s* p0 = (lds_v4s*)(vsrc + 32 * dt);
    lds_v4s* p1 = (lds_v4s*)(vsrc + 32 * dt + 16 * kVRow);
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0);
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p1);
    const v2i_t l2 = __builtin_bit_cast(v2i_t, lo), h2 = __builtin_bit_cast(v2i_t, hi);
    const v4i aop = {l2[0], l2[1], h2[0], h2[1]};
    const v4f o = mfma16_bf16(aop, bhi, st.O[dt]);
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
// Per-lane bytes of one 32-token chunk: the K operands of the two 16-key
// logit tiles and two (token, 32-channel) V blocks for the bf16 staging.
struct ChunkRegs {
  v4i k[2];
  int ks[2];
  v4i v[2];
  int vs[2];
};

// Make this wave's LDS writes visible to its own later reads (LDS requests of
// one wave execute in order; the wait also keeps the compiler from moving
// the reads above it).
__device__ __forceinline__ void wave_lds_sync() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Convert the chunk's V blocks to bf16 rows (exact: code x 2^e) in the wave's
// staging rows.
template <int D>
__device__ __forceinline__ void stage_v(const ChunkRegs& r, uint8_t* vr, int lane) {
  constexpr int nblk_d = D / 32;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int bi = lane + 64 * h;
    const int tt = bi / nblk_d, db = bi % nblk_d;
    if (tt < kChunk) {
      const float scl = r.vs[h] > 0 ? scale_of_byte(r.vs[h]) : 0.0f;
      uint32_t w[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t src = static_cast<uint32_t>(r.v[h][q]);
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

// Buffer resource over [base, base + bytes): loads at offsets past the end
// return zero and fetch nothing, so tail and padding lanes need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}
constexpr uint32_t kOutOfRange = 0x80000000u;   // any offset past every buffer
constexpr int kAuxStream = 2;                   // non-temporal: the cache is read once

// Bitmap of the selected tokens of one split held in LDS (bit t - t_begin).
constexpr int kMaxSplitWords = 8192 / 32;

// FP4 cache scan of one split.  Each wave streams its own chunks (wave w
// takes chunks w, w+4, ...) with two chunks of loads in flight, through its
// own LDS staging rows, so the waves never wait for each other until the
// final combine.  Every load is unconditional (range-checked by the buffer
// resource), which keeps the wait counts exact: the scan of one chunk waits
// only for that chunk's bytes.
// DUAL: the query is a dual-residual pair (a.q, a.q2); each logit MFMA is
// followed by one against the residual query, accumulating into it.
// PAGED: the cache is a pool of pages of page_size tokens (BitDecoding-FP4,
// "System-Level Optimization": paged KV cache with a block table).  A split
// starts on a page boundary and spans at most 64 pages; each lane holds the
// physical page of one of them, and a chunk (32 tokens, inside one page)
// takes its page with a lane read and addresses it through resources built
// on that page, so a bad table entry reads zeros instead of stray memory.
template <int D, bool DUAL, bool PAGED>
__device__ __forceinline__ void fp4_split(const DecodeArgs& a, uint8_t* vstage, uint32_t* selbits, int split,
                                          int hk, int b) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int G = a.Hq / a.Hkv;
  int ctx = a.ctx_len[b];
  ctx = ctx < 1 ? 1 : (ctx > a.Tcap ? a.Tcap : ctx);
  const int win = a.hybrid ? (a.window < ctx ? a.window : ctx) : 0;
  const int end4 = ctx - win;                    // 4-bit tokens are [0, end4)
  const int t_begin = split * a.split_len;
  const int t_end = max(t_begin, min(t_begin + a.split_len, end4));

  // Query operand: column j (query head hk*G + j), channels [32g, 32g+32).
  v4i qop = {0, 0, 0, 0}, qop2 = {0, 0, 0, 0};
  int qsc = 0, qsc2 = 0;
  // Encoded in the scan (q_fused): the lane's 32 bf16 query values are
  // loaded here, before the first chunks' loads.  One 32-channel block per
  // lane, the quantiser's rule (OCP) and encoder: the codes mxattn_quantize
  // writes.  The contiguous scan encodes after its first chunk loads are
  // issued, so their wait covers the query load alone; the paged scan
  // encodes here, which measured faster there (its first loads wait on the
  // block table anyway).
  v4i qraw[4] = {};
  const bool q_lane = j < G && g < D / 32;
  auto encode_q = [&]() {
    float y[32];
    uint32_t amax = 0;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = static_cast<uint32_t>(qraw[c4][e]);
        y[8 * c4 + 2 * e] = __uint_as_float(u << 16);
        y[8 * c4 + 2 * e + 1] = __uint_as_float(u & 0xFFFF0000u);
      }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t mg = __float_as_uint(y[i]) & 0x7FFFFFFFu;
      amax = mg > amax ? mg : amax;
    }
    qsc = e8m0_byte(amax, false, 0.0f);
    qop = v4i{(int)encode8(y, qsc), (int)encode8(y + 8, qsc), (int)encode8(y + 16, qsc), (int)encode8(y + 24, qsc)};
  };
  if (q_lane && a.q_fused) {
    const uint16_t* src = a.q_bf16 + (static_cast<int64_t>(b) * a.Hq + hk * G + j) * D + g * 32;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) qraw[c4] = *reinterpret_cast<const v4i*>(src + 8 * c4);
    if constexpr (PAGED) encode_q();
  } else if (j < G && g < D / 32) {
    const int hq = hk * G + j;
    const uint8_t* qc = a.q.codes + b * a.q.cs[0] + hq * a.q.cs[1];
    const uint8_t* qs = a.q.scales + b * a.q.ss[0] + hq * a.q.ss[1];
    qop = *reinterpret_cast<const v4i*>(qc + g * 16);
    qsc = qs[g];
    if constexpr (DUAL) {
      const uint8_t* qc2 = a.q2.codes + b * a.q2.cs[0] + hq * a.q2.cs[1];
      const uint8_t* qs2 = a.q2.scales + b * a.q2.ss[0] + hq * a.q2.ss[1];
      qop2 = *reinterpret_cast<const v4i*>(qc2 + g * 16);
      qsc2 = qs2[g];
    }
  }
  const int64_t kcs = a.k.cs[2], kss = a.k.ss[2], vcs = a.v.cs[2], vss = a.v.ss[2];
  // Contiguous cache: one resource per operand over the split's (batch, KV
  // head).  Paged: rebuilt per chunk from its page.
  const int64_t bsel = PAGED ? 0 : b;
  const __amdgpu_buffer_rsrc_t rkc0 = make_rsrc(a.k.codes + bsel * a.k.cs[0] + hk * a.k.cs[1], uint32_t(t_end * kcs));
  const __amdgpu_buffer_rsrc_t rks0 = make_rsrc(a.k.scales + bsel * a.k.ss[0] + hk * a.k.ss[1], uint32_t(t_end * kss));
  const __amdgpu_buffer_rsrc_t rvc0 = make_rsrc(a.v.codes + bsel * a.v.cs[0] + hk * a.v.cs[1], uint32_t(t_end * vcs));
  const __amdgpu_buffer_rsrc_t rvs0 = make_rsrc(a.v.scales + bsel * a.v.ss[0] + hk * a.v.ss[1], uint32_t(t_end * vss));
  int pg = -1;  // PAGED: physical page of the split's page `lane` (-1: none)
  if constexpr (PAGED) {
    const int np = a.split_len / a.page_size;
    const int lp = t_begin / a.page_size + lane;
    if (lane < np && lp < a.max_pages) {
      const int e = a.block_table[static_cast<int64_t>(b) * a.max_pages + lp];
      pg = (e >= 0 && e < a.n_pages) ? e : -1;
    }
  }
  uint8_t* vr = vstage + wave * kChunk * kVRow;

  DecState st;
  st.m = -__builtin_huge_valf();
  st.l = 0.0f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.O[dt] = v4f{0, 0, 0, 0};

  constexpr int nblk_d = D / 32;
  auto load = [&](ChunkRegs& r, int t0) {
    __amdgpu_buffer_rsrc_t rkc = rkc0, rks = rks0, rvc = rvc0, rvs = rvs0;
    int tb = 0;  // token at offset 0 of the resources
    if constexpr (PAGED) {
      const int P = a.page_size;
      int pi = (t0 - t_begin) / P;  // chunks past the split only meet out-of-range offsets
      pi = pi < 63 ? pi : 63;
      const int page = __builtin_amdgcn_readlane(pg, pi);
      const int64_t pp = page >= 0 ? page : 0;
      const uint32_t rec = page >= 0 ? 1u : 0u;
      rkc = make_rsrc(a.k.codes + pp * a.k.cs[0] + hk * a.k.cs[1], rec * uint32_t(P * kcs));
      rks = make_rsrc(a.k.scales + pp * a.k.ss[0] + hk * a.k.ss[1], rec * uint32_t(P * kss));
      rvc = make_rsrc(a.v.codes + pp * a.v.cs[0] + hk * a.v.cs[1], rec * uint32_t(P * vcs));
      rvs = make_rsrc(a.v.scales + pp * a.v.ss[0] + hk * a.v.ss[1], rec * uint32_t(P * vss));
      tb = t_begin + pi * P;
    }
    // Hybrid: tokens held in bf16 are not fetched from the 4-bit cache (their
    // codes read as zeros; their logits are masked in `process`).
    uint32_t selw = 0u;
    if (a.hybrid && t0 < t_end) selw = selbits[(t0 - t_begin) >> 5];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = t0 + h * 16 + j;
      const bool ok = t < t_end && g < nblk_d && !((selw >> (h * 16 + j)) & 1u);
      const uint32_t oc = ok ? uint32_t((t - tb) * kcs + g * 16) : kOutOfRange;
      const uint32_t os = ok ? uint32_t((t - tb) * kss + g) : kOutOfRange;
      r.k[h] = __builtin_amdgcn_raw_buffer_load_b128(rkc, oc, 0, kAuxStream);
      r.ks[h] = __builtin_amdgcn_raw_buffer_load_b8(rks, os, 0, 0);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int bi = lane + 64 * h;
      const int tt = bi / nblk_d, db = bi % nblk_d;
      const int t = t0 + tt;
      const bool ok = tt < kChunk && t < t_end && !((selw >> (tt & 31)) & 1u);
      const uint32_t oc = ok ? uint32_t((t - tb) * vcs + db * 16) : kOutOfRange;
      const uint32_t os = ok ? uint32_t((t - tb) * vss + db) : kOutOfRange;
      r.v[h] = __builtin_amdgcn_raw_buffer_load_b128(rvc, oc, 0, kAuxStream);
      r.vs[h] = __builtin_amdgcn_raw_buffer_load_b8(rvs, os, 0, 0);
    }
  };

  if (a.hybrid) {
    // Selected tokens of this split (they are scored in the bf16 set).
    const int64_t bh = static_cast<int64_t>(b) * a.Hkv + hk;
    int nsel = a.max_sel > 0 ? a.n_sel[bh] : 0;
    nsel = nsel < 0 ? 0 : (nsel > a.max_sel ? a.max_sel : nsel);
    for (int w = threadIdx.x; w < kMaxSplitWords; w += kDecThreads) selbits[w] = 0u;
    __syncthreads();
    const int32_t* idx = a.idx + bh * a.max_sel;
    for (int i = threadIdx.x; i < nsel; i += kDecThreads) {
      const int t = idx[i];
      if (t >= t_begin && t < t_end) atomicOr(&selbits[(t - t_begin) >> 5], 1u << (t & 31));
    }
    __syncthreads();
  }

  auto process = [&](const ChunkRegs& r, int t0) {
    stage_v<D>(r, vr, lane);
    v4f s0 = mfma16_fp4(r.k[0], qop, v4f{0, 0, 0, 0}, r.ks[0], qsc);
    v4f s1 = mfma16_fp4(r.k[1], qop, v4f{0, 0, 0, 0}, r.ks[1], qsc);
    if constexpr (DUAL) {
      s0 = mfma16_fp4(r.k[0], qop2, s0, r.ks[0], qsc2);
      s1 = mfma16_fp4(r.k[1], qop2, s1, r.ks[1], qsc2);
    }
    float sv[8];
    const uint32_t mw = a.hybrid ? selbits[(t0 - t_begin) >> 5] : 0u;   // chunks are 32-aligned
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tk = chunk_tok(g, i);
      const float x = i < 4 ? s0[i] : s1[i - 4];
      const bool absent = (t0 + tk >= t_end) || ((mw >> tk) & 1u) || j >= G;
      sv[i] = absent ? -__builtin_huge_valf() : x;
    }
    v4i bhi, blo;
    float alpha;
    bool moved;
    softmax_chunk(st, sv, a.c, bhi, blo, alpha, moved);
    wave_lds_sync();
    pv_chunk(st, vr, lane, bhi, blo, alpha, moved, D);
  };

  const int n_chunks = (t_end - t_begin + kChunk - 1) / kChunk;
  const int mine = n_chunks > wave ? (n_chunks - wave + 3) / 4 : 0;   // chunks of this wave
  ChunkRegs A, B;
  auto chunk_t0 = [&](int i) { return t_begin + (wave + 4 * i) * kChunk; };
  // The scheduling barriers keep each chunk's loads together and in issue
  // order, so a chunk's wait never covers the loads of the chunk after it.
  load(A, chunk_t0(0));
  __builtin_amdgcn_sched_barrier(0);
  load(B, chunk_t0(1));
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!PAGED) {
    if (q_lane && a.q_fused) encode_q();
  }
  for (int i = 0; i < mine; i += 2) {
    process(A, chunk_t0(i));
    __builtin_amdgcn_sched_barrier(0);
    load(A, chunk_t0(i + 2));
    __builtin_amdgcn_sched_barrier(0);
    if (i + 1 < mine) process(B, chunk_t0(i + 1));
    __builtin_amdgcn_sched_barrier(0);
    load(B, chunk_t0(i + 3));
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  combine_store<D>(vstage, st, a, b, hk, split, a.n_split + a.n_bf16);
}

// ---------------------------------------------------------------------------
// bf16 hybrid set: the selected rows (those below ctx - window) followed by
// the window rows, kBf16Rows rows per workgroup, each result in its own
// partial slot after the 4-bit splits.
template <int D>
__device__ __forceinline__ void bf16_part(const DecodeArgs& a, uint8_t* vstage, int part_id, int hk, int b) {
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
  const int woff = a.window - win;   // window rows before token 0 are unused
  const int r_begin = part_id * kBf16Rows;
  const int r_end = min(r_begin + kBf16Rows, n_total);
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

  DecState st;
  st.m = -__builtin_huge_valf();
  st.l = 0.0f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.O[dt] = v4f{0, 0, 0, 0};

  // Wave w takes the chunks r_begin + 32 (w + 4 i).  A chunk's row loads are
  // all issued together, and the next chunk's are issued as soon as this
  // chunk's rows have gone to LDS and into its QK^T products, so they land
  // during this chunk's softmax and PV.  Rows past r_end read row r_end - 1
  // (finite values that only meet P = 0 or a masked score).
  constexpr int kParts = D / 8;                     // 16-byte pieces per bf16 row
  constexpr int kVIter = kChunk * kParts / 64;      // V pieces per lane
  v4i vx[kVIter];
  v4i kx[2][4];
  bool ok_row = false;
  auto load_chunk = [&](int t0) {
    ok_row = false;
    if (lane < kChunk && t0 + lane < r_end) ok_row = t0 + lane >= nsel || idx[t0 + lane] < limit;
#pragma unroll
    for (int it = 0; it < kVIter; ++it) {
      const int e = lane + 64 * it;
      const int tt = e / kParts, part = e % kParts;
      const int i = min(t0 + tt, r_end - 1);
      vx[it] = *reinterpret_cast<const v4i*>(row_v(i) + part * 8);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = min(t0 + h * 16 + j, r_end - 1);
      const uint16_t* kr = row_k(i);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        kx[h][kk] = kk * 32 < D ? *reinterpret_cast<const v4i*>(kr + kk * 32 + 8 * g) : v4i{0, 0, 0, 0};
    }
  };
  int t0 = r_begin + wave * kChunk;
  if (t0 < r_end) load_chunk(t0);
  for (; t0 < r_end; t0 += 4 * kChunk) {
    // Validity of the chunk's rows as a bit mask: lane i < 32 tested row t0 + i.
    const uint32_t vmask = static_cast<uint32_t>(__builtin_amdgcn_ballot_w64(ok_row));
#pragma unroll
    for (int it = 0; it < kVIter; ++it) {
      const int e = lane + 64 * it;
      const int tt = e / kParts, part = e % kParts;
      *reinterpret_cast<v4i*>(vr + tt * kVRow + part * 16) = vx[it];
    }
    v4f sc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v4f acc = {0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk * 32 >= D) break;
        acc = mfma16_bf16(kx[h][kk], qop[kk], acc);
      }
      sc[h] = acc;
    }
    if (t0 + 4 * kChunk < r_end) load_chunk(t0 + 4 * kChunk);
    float sv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tk = chunk_tok(g, i);
      const float x = i < 4 ? sc[0][i] : sc[1][i - 4];
      sv[i] = (((vmask >> tk) & 1u) && j < G) ? x : -__builtin_huge_valf();
    }
    v4i bhi, blo;
    float alpha;
    bool moved;
    softmax_chunk(st, sv, a.c, bhi, blo, alpha, moved);
    wave_lds_sync();
    pv_chunk(st, vr, lane, bhi, blo, alpha, moved, D);
    // The next chunk's rows overwrite this wave's staging rows.
    wave_lds_sync();
  }
  __syncthreads();
  combine_store<D>(vstage, st, a, b, hk, a.n_split + part_id, a.n_split + a.n_bf16);
}

// One launch for the whole scan, longest work first: the first
// n_split x Hkv x B workgroups are the 4-bit splits (split fastest), the
// rest the shorter bf16 hybrid parts, which fill the slots the splits free
// at the end.
template <int D, bool DUAL, bool PAGED>
__global__ __launch_bounds__(kDecThreads, 3) void decode_scan_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t vstage[kStageBytes];
  __shared__ uint32_t selbits[kMaxSplitWords];
  const int bid = static_cast<int>(blockIdx.x);
  const int n4 = a.n_split * a.Hkv * a.B;
  if (bid < n4) {
    const int bh = bid / a.n_split;
    fp4_split<D, DUAL, PAGED>(a, vstage, selbits, bid % a.n_split, bh % a.Hkv, bh / a.Hkv);
  } else {
    const int r = bid - n4;
    const int bh = r / a.n_bf16;
    bf16_part<D>(a, vstage, r % a.n_bf16, bh % a.Hkv, bh / a.Hkv);
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the partial slots, in slot order.  One workgroup per
// (batch, query head): the slots' (m, l) go through LDS once, then every
// channel sums its weighted partials with independent loads.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecodeArgs a) {
  __shared__ float wgt[kMaxSlots];
  __shared__ float s_den, s_m;
  const int hq = blockIdx.x, b = blockIdx.y;
  const int d = threadIdx.x;
  const int n_slot = a.n_split + a.n_bf16;
  const float* p = a.part + (static_cast<int64_t>(b) * a.Hq + hq) * n_slot * (D + 2);
  if (d < 64) {
    // One wave: maximum and weights of all slots.
    float M = -__builtin_huge_valf();
    for (int s = d; s < n_slot; s += 64) M = fmaxf(M, p[s * (D + 2) + D]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float den = 0.0f;
    for (int s = d; s < n_slot; s += 64) {
      const float ms = p[s * (D + 2) + D];
      const float w = ms == -__builtin_huge_valf() ? 0.0f : fast_exp2((ms - M) * a.c);
      wgt[s] = w;
      den += w * p[s * (D + 2) + D + 1];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
    if (d == 0) {
      s_den = den;
      s_m = M;
    }
  }
  __syncthreads();
  float num = 0.0f;
  int s = 0;
  for (; s + 4 <= n_slot; s += 4) {
    const float x0 = p[(s + 0) * (D + 2) + d], x1 = p[(s + 1) * (D + 2) + d];
    const float x2 = p[(s + 2) * (D + 2) + d], x3 = p[(s + 3) * (D + 2) + d];
    num += wgt[s] * x0;
    num += wgt[s + 1] * x1;
    num += wgt[s + 2] * x2;
    num += wgt[s + 3] * x3;
  }
  for (; s < n_slot; ++s) num += wgt[s] * p[s * (D + 2) + d];
  const int64_t row = static_cast<int64_t>(b) * a.Hq + hq;
  a.out[row * D + d] = num / s_den;
  if (a.lse != nullptr && d == 0) a.lse[row] = s_m * a.softmax_scale + logf(s_den);
}

template <int D, bool DUAL>
static void launch_scan(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
  if (a.paged)
    hipLaunchKernelGGL((decode_scan_kernel<D, DUAL, true>), grid, dim3(kDecThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_scan_kernel<D, DUAL, false>), grid, dim3(kDecThreads), 0, stream, a);
}

// ---------------------------------------------------------------------------
// Scratch of mxattn_decode_noalloc: the partial slots in a file-scope device
// array instead of a caller's workspace, for callers that cannot allocate.
// Every device the library runs on holds its own copy until the process
// ends.  In host code the array's name is only a stand-in: its address on the
// current device comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, int D, hipStream_t stream) {
  const dim3 grid((a.n_split + (a.hybrid ? a.n_bf16 : 0)) * a.Hkv * a.B);
  if (D == 128) {
    if (a.dual) launch_scan<128, true>(a, grid, stream);
    else launch_scan<128, false>(a, grid, stream);
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(a.Hq, a.B), dim3(128), 0, stream, a);
  } else {
    if (a.dual) launch_scan<64, true>(a, grid, stream);
    else launch_scan<64, false>(a, grid, stream);
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(a.Hq, a.B), dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace mxattn

// Vertical-line selection for hybrid-precision decode.
//
// Method: HyQuant page (method paragraphs).  A key's score is the attention
// probability it has received from the queries decoded since the last call,
// summed into a per-key total; a call adds to that total and returns the
// rho fraction of highest-scoring keys before the recent window.
//
// Kernels
//   stats    -- per (context chunk, batch x KV head): every recent
//               query's partial row max and row sum of the logits (S^T =
//               K_hat q_hat^T on the scaled FP4 MFMA, queries staged in
//               LDS), merged per query in chunk order by `finalize`.
//   colmass  -- per key block: the normalised probabilities of every
//               recent query of the KV head's group, summed per key (in-lane
//               over 16 queries, a permlane32 swap for the other 16) and added
//               to col_mass.  Each key belongs to exactly one lane: no atomics.
//   topk     -- per (batch, KV head), one 1024-thread workgroup holding the
//               masses in registers: the k-th largest fp32 bit pattern found
//               by a radix select over 12-, 10- and 10-bit digits (bit
//               patterns of non-negative values order like the values), then
//               one ordered compaction, a single prefix scan, that emits the
//               indices ascending, ties at the threshold going to the lower
//               indices.
#include <type_traits>

#include "mx_device.h"
#include "kernels.h"

namespace mxattn {

constexpr int kSelThreads = 256;

__device__ __forceinline__ int clamp_ctx(const SelectArgs& a, int b) {
  int ctx = a.ctx_len[b];
  return ctx < 1 ? 1 : (ctx > a.Tcap ? a.Tcap : ctx);
}

// Recent query qi of a KV head's group: query head g = qi / R, token r = qi % R.
__device__ __forceinline__ void query_operand(const SelectArgs& a, int b, int hk, int qi, int hh, int dc, v4i& op,
                                              int& sc) {
  const int G = a.Hq / a.Hkv;
  op = v4i{0, 0, 0, 0};
  sc = 0;
  if (qi < G * a.R) {
    const int hq = hk * G + qi / a.R, r = qi % a.R;
    const uint8_t* c = a.q.codes + b * a.q.cs[0] + hq * a.q.cs[1] + static_cast<int64_t>(r) * a.q.cs[2];
    const uint8_t* s = a.q.scales + b * a.q.ss[0] + hq * a.q.ss[1] + static_cast<int64_t>(r) * a.q.ss[2];
    op = *reinterpret_cast<const v4i*>(c + dc * 32 + hh * 16);
    sc = s[2 * dc + hh];
  }
}

__device__ __forceinline__ float* stat_slot(const SelectArgs& a, int b, int hk, int qi, int slot) {
  const int G = a.Hq / a.Hkv;
  const int nchunk = (a.Tcap + a.chunk - 1) / a.chunk;
  const int hq = hk * G + qi / a.R, r = qi % a.R;
  return a.stats + ((((static_cast<int64_t>(b) * a.Hq + hq) * a.R + r) * (nchunk + 1)) + slot) * 2;
}

// ---------------------------------------------------------------------------
constexpr int kMaxRecent = 512;    // recent queries x group size held in LDS
constexpr int kMaxChunks = 32;     // context chunks (the host sizes chunks to stay within it)

// The group's recent queries in LDS: codes [nq][D/2] and scales [nq][D/32].
// Queries past nq up to the next multiple of 32 are zero codes with scale
// byte 0, so a whole group of 32 can be read without guards (their logits
// are 0 and they are never reported).
template <int D>
__device__ __forceinline__ void stage_queries(const SelectArgs& a, int b, int hk, uint8_t* q_lds, uint8_t* qs_lds) {
  const int G = a.Hq / a.Hkv;
  const int nq = G * a.R, nq32 = (nq + 31) / 32 * 32;
  for (int e = threadIdx.x; e < nq32 * (D / 32); e += kSelThreads) {
    const int qi = e / (D / 32), part = e % (D / 32);
    v4i code = {0, 0, 0, 0};
    uint8_t sc = 0;
    if (qi < nq) {
      const int hq = hk * G + qi / a.R, r = qi % a.R;
      const uint8_t* c = a.q.codes + b * a.q.cs[0] + hq * a.q.cs[1] + static_cast<int64_t>(r) * a.q.cs[2];
      const uint8_t* s = a.q.scales + b * a.q.ss[0] + hq * a.q.ss[1] + static_cast<int64_t>(r) * a.q.ss[2];
      code = *reinterpret_cast<const v4i*>(c + part * 16);
      sc = s[part];
    }
    *reinterpret_cast<v4i*>(q_lds + qi * (D / 2) + part * 16) = code;
    qs_lds[qi * (D / 32) + part] = sc;
  }
}

// One 32-key block of K codes/scales for the MFMA (rows = keys, lane j:
// key t0 + j, half hh), read through a buffer resource: keys past `t_hi`
// read as zeros.
template <int D>
struct KBlock {
  v4i op[D / 64];
  int sc[D / 64];
};

template <int D>
__device__ __forceinline__ KBlock<D> load_kblock(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, int kcs,
                                                 int kss, int t, int t_hi, int hh) {
  KBlock<D> k;
  const bool ok = t < t_hi;
#pragma unroll
  for (int dc = 0; dc < D / 64; ++dc) {
    k.op[dc] = __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? static_cast<uint32_t>(t * kcs + dc * 32 + hh * 16)
                                                            : 0x80000000u, 0, 0);
    k.sc[dc] = __builtin_amdgcn_raw_buffer_load_b8(rs, ok ? static_cast<uint32_t>(t * kss + 2 * dc + hh)
                                                          : 0x80000000u, 0, 0);
  }
  return k;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sel_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// Per (context chunk, batch x KV head): every recent query's partial row max
// and row sum over the chunk.  The queries sit in LDS; wave w takes the
// chunk's 32-key blocks w, w+4, ... for all query groups (K read once), and
// the four waves' (max, sum) are merged in LDS at the end.
//
// NG is the largest number of 32-query groups the instance holds (8 or 16):
// the per-query state and the LDS are sized by it, so the common case of 256
// recent queries x group size keeps four workgroups per CU.
template <int D, int NG>
__global__ __launch_bounds__(kSelThreads, 2) void select_stats_kernel(SelectArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[NG * 32 * (D / 2)];
  __shared__ uint8_t qs_lds[NG * 32 * (D / 32)];
  // The waves' (max, sum) per query reuse the query codes' LDS after the scan.
  static_assert(4 * NG * 32 * 2 * sizeof(float) <= sizeof(q_lds), "reduction does not fit");
  float (*red)[NG * 32][2] = reinterpret_cast<float (*)[NG * 32][2]>(q_lds);
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, j = lane & 31, hh = lane >> 5;
  const int G = a.Hq / a.Hkv;
  const int nq = G * a.R, ng = (nq + 31) / 32;
  const int ctx = clamp_ctx(a, b);
  const int t_lo = chunk * a.chunk;
  const int t_hi = min(t_lo + a.chunk, ctx);
  stage_queries<D>(a, b, hk, q_lds, qs_lds);
  __syncthreads();
  const __amdgpu_buffer_rsrc_t rc = sel_rsrc(a.k.codes + b * a.k.cs[0] + hk * a.k.cs[1], int64_t(ctx) * a.k.cs[2]);
  const __amdgpu_buffer_rsrc_t rs = sel_rsrc(a.k.scales + b * a.k.ss[0] + hk * a.k.ss[1], int64_t(ctx) * a.k.ss[2]);
  const int kcs = static_cast<int>(a.k.cs[2]), kss = static_cast<int>(a.k.ss[2]);
  float m[NG], l[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    m[g] = -__builtin_huge_valf();
    l[g] = 0.0f;
  }
  // Up to 16 query operands (8 groups at D = 128) stay in registers for the
  // whole chunk instead of being read from LDS for every key block: 92 ->
  // 89 us on the 32K batch-8 selection; 16 groups at D = 128 would spill.
  constexpr bool kQReg = NG * (D / 64) <= 16;
  v4i qreg[kQReg ? NG : 1][D / 64];
  int qsreg[kQReg ? NG : 1][D / 64];
  if constexpr (kQReg) {
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int dc = 0; dc < D / 64; ++dc) {
        const int qi = g * 32 + j;
        qreg[g][dc] = *reinterpret_cast<const v4i*>(q_lds + qi * (D / 2) + dc * 32 + hh * 16);
        qsreg[g][dc] = qs_lds[qi * (D / 32) + 2 * dc + hh];
      }
  }
  int t0 = t_lo + wave * 32;
  KBlock<D> kn = load_kblock<D>(rc, rs, kcs, kss, t0 + j, t_hi, hh);
  for (; t0 < t_hi; t0 += 128) {
    const KBlock<D> kb = kn;
    kn = load_kblock<D>(rc, rs, kcs, kss, t0 + 128 + j, t_hi, hh);
    // All query groups against this block; the key mask is compiled only
    // into the form for a chunk's partial last block.
    auto groups = [&](auto tail_tag) {
      constexpr bool TAIL = decltype(tail_tag)::value;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (g >= ng) continue;   // uniform; the loop stays unrolled, m[g]/l[g] in fixed registers
        // B operand: query g*32 + j, from registers or LDS.
        const int qi = g * 32 + j;
        v16f s = v16f{};
#pragma unroll
        for (int dc = 0; dc < D / 64; ++dc) {
          if constexpr (kQReg) {
            s = mfma32_fp4(kb.op[dc], qreg[g][dc], s, kb.sc[dc], qsreg[g][dc]);
          } else {
            const v4i qop = *reinterpret_cast<const v4i*>(q_lds + qi * (D / 2) + dc * 32 + hh * 16);
            const int qsc = qs_lds[qi * (D / 32) + 2 * dc + hh];
            s = mfma32_fp4(kb.op[dc], qop, s, kb.sc[dc], qsc);
          }
        }
        // Lane (query j, half hh) holds keys t0 + 8(r/4) + 4hh + r%4.
        if constexpr (TAIL) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (t0 + 8 * (r >> 2) + 4 * hh + (r & 3) >= t_hi) s[r] = -__builtin_huge_valf();
        }
        const float m0 = fmaxf(fmaxf(s[0], s[1]), s[2]), m1 = fmaxf(fmaxf(s[3], s[4]), s[5]);
        const float m2 = fmaxf(fmaxf(s[6], s[7]), s[8]), m3 = fmaxf(fmaxf(s[9], s[10]), s[11]);
        const float m4 = fmaxf(fmaxf(s[12], s[13]), s[14]);
        float x = fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), s[15]));
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        const float m_new = fmaxf(m[g], x);
        const float alpha = m[g] == -__builtin_huge_valf() ? 0.0f : fast_exp2((m[g] - m_new) * a.c);
        const float mc = m_new * a.c;
        float sum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += fast_exp2(__builtin_fmaf(s[r], a.c, -mc));
        l[g] = l[g] * alpha + sum;
        m[g] = m_new;
      }
    };
    if (t0 + 32 > t_hi) groups(std::true_type{});
    else groups(std::false_type{});
  }
  // This wave's (max, sum) per query (the two lane halves hold halves of the
  // sum), then the ordered merge of the four waves.
  __syncthreads();   // every wave is done reading q_lds
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (g >= ng) continue;
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l[g]), __float_as_uint(l[g]), false, false);
    const float lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (hh == 0) {
      red[wave][g * 32 + j][0] = m[g];
      red[wave][g * 32 + j][1] = lt;
    }
  }
  __syncthreads();
  for (int qi = threadIdx.x; qi < nq; qi += kSelThreads) {
    float M = -__builtin_huge_valf();
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red[w][qi][0]);
    float L = 0.0f;
    for (int w = 0; w < 4; ++w)
      if (red[w][qi][0] != -__builtin_huge_valf()) L += fast_exp2((red[w][qi][0] - M) * a.c) * red[w][qi][1];
    float* st = stat_slot(a, b, hk, qi, chunk);
    st[0] = M;
    st[1] = L;
  }
}

// Ordered merge of the chunk partials of every recent query into the slot
// after them.  Every partial is read at once (at most kMaxChunks of them):
// a loop of dependent reads cost one memory latency per chunk.
__global__ __launch_bounds__(kSelThreads) void select_finalize_kernel(SelectArgs a) {
  const int G = a.Hq / a.Hkv;
  const int nq = a.B * a.Hkv * G * a.R;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nq) return;
  const int qi = i % (G * a.R);
  const int bh = i / (G * a.R);
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int nchunk = (a.Tcap + a.chunk - 1) / a.chunk;
  const int used = (clamp_ctx(a, b) + a.chunk - 1) / a.chunk;
  float2 st[kMaxChunks];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c)
    st[c] = c < used ? *reinterpret_cast<const float2*>(stat_slot(a, b, hk, qi, c))
                     : make_float2(-__builtin_huge_valf(), 0.0f);
  float M = -__builtin_huge_valf();
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) M = fmaxf(M, st[c].x);
  float L = 0.0f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c)
    if (st[c].x != -__builtin_huge_valf()) L += fast_exp2((st[c].x - M) * a.c) * st[c].y;
  float* out = stat_slot(a, b, hk, qi, nchunk);
  out[0] = M;
  out[1] = 1.0f / L;
}

// ---------------------------------------------------------------------------
// Per (block of cm_keys keys, batch x KV head): the normalised
// probabilities of every recent query of the group, summed per key and added
// to col_mass.  Lane (key j, half hh) of a 32x32 product holds 16 queries, in
// four runs of four consecutive ones, so their offsets w = m c + log2 l come
// from LDS as float4s (exp2(s c - w) = exp2(s c - m c) / l: one LDS word per
// query instead of two).  Each key belongs to one lane pair: no atomics.

template <int D, int NG>
__global__ __launch_bounds__(kSelThreads) void select_colmass_kernel(SelectArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[NG * 32 * (D / 2)];
  __shared__ uint8_t qs_lds[NG * 32 * (D / 32)];
  __shared__ __attribute__((aligned(16))) float w_lds[NG * 32];
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int nq = G * a.R, ng = (nq + 31) / 32;
  const int nchunk = (a.Tcap + a.chunk - 1) / a.chunk;
  const int ctx = clamp_ctx(a, b);
  const int k_lo = blk * a.cm_keys;
  if (k_lo >= ctx) return;
  const int k_hi = min(k_lo + a.cm_keys, ctx);
  stage_queries<D>(a, b, hk, q_lds, qs_lds);
  for (int qi = threadIdx.x; qi < ng * 32; qi += kSelThreads) {
    float w = __builtin_huge_valf();   // padding queries contribute exp2(-inf) = 0
    if (qi < nq) {
      const float* st = stat_slot(a, b, hk, qi, nchunk);
      w = st[0] * a.c - log2f(st[1]);   // st[1] = 1 / l
    }
    w_lds[qi] = w;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, j = lane & 31, hh = lane >> 5;
  const __amdgpu_buffer_rsrc_t rc = sel_rsrc(a.k.codes + b * a.k.cs[0] + hk * a.k.cs[1], int64_t(ctx) * a.k.cs[2]);
  const __amdgpu_buffer_rsrc_t rs = sel_rsrc(a.k.scales + b * a.k.ss[0] + hk * a.k.ss[1], int64_t(ctx) * a.k.ss[2]);
  const int kcs = static_cast<int>(a.k.cs[2]), kss = static_cast<int>(a.k.ss[2]);
  float* cm = a.col_mass + (static_cast<int64_t>(b) * a.Hkv + hk) * a.Tcap;
  int t0 = k_lo + wave * 32;
  KBlock<D> kn = load_kblock<D>(rc, rs, kcs, kss, t0 + j, k_hi, hh);
  for (; t0 < k_hi; t0 += 128) {
    const KBlock<D> kb = kn;
    kn = load_kblock<D>(rc, rs, kcs, kss, t0 + 128 + j, k_hi, hh);
    float colsum = 0.0f;
    // Unrolled over the largest group count with a uniform skip, so the next
    // group's MFMAs can issue while this group's exponentials run.
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g >= ng) continue;
      // A operand: queries g*32 + (lane % 32) from LDS.
      const int qa = g * 32 + j;
      v16f s = v16f{};
#pragma unroll
      for (int dc = 0; dc < D / 64; ++dc) {
        const v4i qop = *reinterpret_cast<const v4i*>(q_lds + qa * (D / 2) + dc * 32 + hh * 16);
        const int qsc = qs_lds[qa * (D / 32) + 2 * dc + hh];
        s = mfma32_fp4(qop, kb.op[dc], s, qsc, kb.sc[dc]);
      }
      // Lane (key j, half hh) holds queries g*32 + 8(r/4) + 4hh + r%4.
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int qb = g * 32 + 8 * q4 + 4 * hh;
        const v4f wv = *reinterpret_cast<const v4f*>(w_lds + qb);
#pragma unroll
        for (int r = 0; r < 4; ++r) colsum += fast_exp2(__builtin_fmaf(s[4 * q4 + r], a.c, -wv[r]));
      }
    }
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(colsum), __float_as_uint(colsum), false, false);
    colsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const int t = t0 + j;
    if (hh == 0 && t < k_hi) cm[t] += colsum;
  }
}

// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
// Radix digits from the top of the fp32 bit pattern: 12 bits (sign, exponent
// and three mantissa bits, so the masses of one binade fall on 8 counters),
// then 10 and 10.  The counters have eight copies, lane l adding to copy
// l % 8; the copies are 4 words out of bank step, so lanes of one atomic
// instruction that meet the same digit hit up to eight different banks.
constexpr int kTkBits0 = 12, kTkBits1 = 10;
constexpr int kTkCopies = 8;
constexpr int kTkStride = (1 << kTkBits0) + 4;            // words per copy
constexpr int kTopkStage = kTkCopies * (1 << kTkBits0);   // indices staged in the counters' LDS

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8
// inside each row of 16 lanes (DPP row_shr; a source outside the row reads
// as the 0 passed for `old`), then the totals of the lower rows, read from
// lanes 15, 31 and 47.
__device__ __forceinline__ int wave_scan_incl(int x, int lane) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
  const int r0 = __builtin_amdgcn_readlane(x, 15);
  const int r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane >> 4;
  return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Inclusive prefix sum over the 1024 threads of the workgroup (wave scans
// with shuffles, then the 16 wave totals through LDS).
__device__ __forceinline__ int block_scan_incl(int x, int* wtot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_scan_incl(x, lane);
  if (lane == 63) wtot[wave] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wtot[w];
  __syncthreads();
  return x + base;
}

// Per (batch, KV head): the k largest masses of the non-window prefix,
// indices ascending, ties at the threshold to the lower indices.  One
// workgroup of 1024 threads holds the masses in registers.
template <int kTopkChunks>   // register capacity: kTopkChunks x 4096 keys
__global__ __launch_bounds__(kTopkThreads) void select_topk_kernel(SelectArgs a) {
  constexpr int kSlots = kTopkChunks * kTopkWaves;   // (chunk, wave) pairs in index order
  __shared__ __attribute__((aligned(16))) uint32_t hist[kTkCopies * kTkStride];
  __shared__ int wtot[kTopkWaves];
  __shared__ int wsum[2][kSlots];
  __shared__ int s_digit, s_above, s_eq;
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv;
  const int ctx = clamp_ctx(a, b);
  const int n = ctx > a.window ? ctx - a.window : 0;
  int k = static_cast<int>((static_cast<int64_t>(n) * a.rho_num + a.rho_den - 1) / a.rho_den);
  k = k > a.max_sel ? a.max_sel : k;
  const uint32_t* v = reinterpret_cast<const uint32_t*>(a.col_mass + static_cast<int64_t>(bh) * a.Tcap);
  int32_t* out = a.idx_out + static_cast<int64_t>(bh) * a.max_sel;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) a.n_out[bh] = k;
  // The masses stay in registers for all passes: entry c*4096 + 4*tid + u
  // in x[c][u], read as one 16-byte load per lane for whole chunks.  Entries
  // at or past n hold 0, the smallest pattern: with k <= n they never change
  // the k-th largest, never exceed it, and come after every real entry in
  // index order, so no pass or the compaction needs to test the index.
  uint32_t x[kTopkChunks][4];
  const int nch = (n + kTopkThreads * 4 - 1) / (kTopkThreads * 4);
  const bool vec = (reinterpret_cast<uintptr_t>(v) & 15u) == 0;
#pragma unroll
  for (int c = 0; c < kTopkChunks; ++c) {
    const int i0 = c * kTopkThreads * 4 + tid * 4;
    if (vec && (c + 1) * kTopkThreads * 4 <= n) {   // uniform
      const uint4 w = *reinterpret_cast<const uint4*>(v + i0);
      x[c][0] = w.x;
      x[c][1] = w.y;
      x[c][2] = w.z;
      x[c][3] = w.w;
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) x[c][u] = (c < nch && i0 + u < n) ? v[i0 + u] : 0u;
    }
  }
  // Threshold: the k-th largest fp32 bit pattern tau (bit patterns of
  // non-negative values order like the values; any other pattern is ordered
  // as an unsigned integer, so exactly k entries are always taken).  Radix
  // select from the top: each pass counts, among the entries whose higher
  // digits equal tau's, how many take each value of the next digit, then
  // takes the digit at which the count from the top reaches k.  `above`
  // counts the entries already known to exceed tau.
  uint32_t tau = 0;
  int above = 0;
  if (k > 0) {
    uint32_t pmask = 0;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int bits = pass == 0 ? kTkBits0 : kTkBits1;
      const int shift = pass == 0 ? 32 - kTkBits0 : (pass == 1 ? 32 - kTkBits0 - kTkBits1 : 0);
      const uint32_t dmask = (1u << bits) - 1u;
      const int nb = 1 << bits;
      // Clear the nb counters of every copy (16-byte words; kTkStride is a
      // multiple of 4).
      static_assert(kTkStride % 4 == 0, "counters are cleared as 16-byte words");
      for (int e = tid; e < kTkCopies * nb / 4; e += kTopkThreads) {
        const int cp = e / (nb / 4), w4 = e % (nb / 4);
        reinterpret_cast<uint4*>(hist + cp * kTkStride)[w4] = uint4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
      uint32_t* h = hist + (lane & (kTkCopies - 1)) * kTkStride;
      if (pass == 0) {   // every entry counts
#pragma unroll
        for (int c = 0; c < kTopkChunks; ++c) {
          if (c >= nch) continue;   // uniform: every later chunk is empty too
#pragma unroll
          for (int u = 0; u < 4; ++u) atomicAdd(&h[x[c][u] >> shift], 1u);
        }
      } else {
#pragma unroll
        for (int c = 0; c < kTopkChunks; ++c) {
          if (c >= nch) continue;
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if ((x[c][u] & pmask) == tau) atomicAdd(&h[(x[c][u] >> shift) & dmask], 1u);
        }
      }
      __syncthreads();
      // Thread t owns the digits of descending rank t*bpt .. t*bpt + bpt - 1
      // (digit nb - 1 - rank), so its inclusive scan counts the entries at
      // or above its lowest digit.
      const int bpt = nb / kTopkThreads;
      int cnt = 0;
      for (int j = 0; j < bpt; ++j) {
        const int dg = nb - 1 - (tid * bpt + j);
#pragma unroll
        for (int cp = 0; cp < kTkCopies; ++cp) cnt += static_cast<int>(hist[cp * kTkStride + dg]);
      }
      const int incl = block_scan_incl(cnt, wtot);
      int acc = above + incl - cnt;
      if (acc < k && above + incl >= k) {
        for (int j = 0; j < bpt; ++j) {
          const int dg = nb - 1 - (tid * bpt + j);
          int cj = 0;
#pragma unroll
          for (int cp = 0; cp < kTkCopies; ++cp) cj += static_cast<int>(hist[cp * kTkStride + dg]);
          if (acc + cj >= k) {
            s_digit = dg;
            s_above = acc;
            s_eq = cj;   // after the last pass: the entries equal to tau
            break;
          }
          acc += cj;
        }
      }
      __syncthreads();
      tau |= static_cast<uint32_t>(s_digit) << shift;
      pmask |= dmask << shift;
      above = s_above;
    }
  }
  // Ordered compaction in one scan.  Entries above tau are all taken; of the
  // entries equal to tau the first take_eq in index order.  Index order is
  // (chunk, wave, lane, u): in-wave prefixes by DPP scans, then the (chunk,
  // wave) totals scanned by wave 0.  The indices go through LDS (the
  // counters' space, free now) when they fit, so the global writes are whole
  // rows instead of scattered words; entries not taken write to spare words
  // past the staged indices.  Positions of taken entries are below k by
  // construction; the test keeps every write inside the k-entry output all
  // the same.
  const int take_eq = k - above;
  auto scan_slots = [&](int s) __attribute__((always_inline)) {
    constexpr int F = kSlots / 64;   // slots per lane of wave 0
    int val[F], tot = 0;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      val[f] = wsum[s][lane * F + f];
      tot += val[f];
    }
    int run = wave_scan_incl(tot, lane) - tot;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      wsum[s][lane * F + f] = run;
      run += val[f];
    }
  };
  int* stage = reinterpret_cast<int*>(hist);
  static_assert(kTopkStage + 32 <= kTkCopies * kTkStride, "no spare words after the staged indices");
  const int spare = kTopkStage + (lane & 31);
  const bool staged = k <= kTopkStage;
  if (k > 0 && s_eq == take_eq) {
    // Every entry equal to tau is taken (no tie is cut): the taken entries
    // are those at or above tau, one count per (chunk, thread).
    int pre[kTopkChunks];
#pragma unroll
    for (int c = 0; c < kTopkChunks; ++c) {
      int t = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) t += x[c][u] >= tau ? 1 : 0;
      const int incl = wave_scan_incl(t, lane);
      pre[c] = incl - t;
      if (lane == 63) wsum[0][c * kTopkWaves + wave] = incl;
    }
    __syncthreads();
    if (wave == 0) scan_slots(0);
    __syncthreads();
    auto emit = [&](auto&& put) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < kTopkChunks; ++c) {
        if (c >= nch) continue;   // uniform: every later chunk is empty too
        int pos = wsum[0][c * kTopkWaves + wave] + pre[c];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bool keep = x[c][u] >= tau;
          put(keep, pos, c * kTopkThreads * 4 + tid * 4 + u);
          pos += keep ? 1 : 0;
        }
      }
    };
    if (staged) emit([&](bool keep, int pos, int i) { stage[keep && pos < k ? pos : spare] = i; });
    else emit([&](bool keep, int pos, int i) { if (keep && pos < k) out[pos] = i; });
  } else if (k > 0) {
    // Ties at tau are cut: an entry's position is (entries above tau before
    // it) + min(entries equal to tau before it, take_eq), the two counts
    // packed in one word for the in-wave scan (each at most 256 per wave and
    // chunk).
    int pre[kTopkChunks];
#pragma unroll
    for (int c = 0; c < kTopkChunks; ++c) {
      int g = 0, e = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        g += x[c][u] > tau ? 1 : 0;
        e += x[c][u] == tau ? 1 : 0;
      }
      const int own = g | (e << 16);
      const int incl = wave_scan_incl(own, lane);
      pre[c] = incl - own;
      if (lane == 63) {
        wsum[0][c * kTopkWaves + wave] = incl & 0xFFFF;
        wsum[1][c * kTopkWaves + wave] = incl >> 16;
      }
    }
    __syncthreads();
    if (wave == 0) {
      scan_slots(0);
      scan_slots(1);
    }
    __syncthreads();
    auto emit = [&](auto&& put) __attribute__((always_inline)) {
#pragma unroll
      for (int c = 0; c < kTopkChunks; ++c) {
        if (c >= nch) continue;   // uniform: every later chunk is empty too
        int g = wsum[0][c * kTopkWaves + wave] + (pre[c] & 0xFFFF);
        int e = wsum[1][c * kTopkWaves + wave] + (pre[c] >> 16);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bool gt = x[c][u] > tau, eq = x[c][u] == tau;
          const int ecl = e < take_eq ? e : take_eq;
          put(gt || (eq && e < take_eq), g + (gt ? ecl : e), c * kTopkThreads * 4 + tid * 4 + u);
          g += gt ? 1 : 0;
          e += eq ? 1 : 0;
        }
      }
    };
    if (staged) emit([&](bool keep, int pos, int i) { stage[keep && pos < k ? pos : spare] = i; });
    else emit([&](bool keep, int pos, int i) { if (keep && pos < k) out[pos] = i; });
  }
  if (k > 0 && staged) {
    __syncthreads();
    for (int i = tid; i < k; i += kTopkThreads) out[i] = stage[i];
  }
  for (int i = k + tid; i < a.max_sel; i += kTopkThreads) out[i] = -1;
}

hipError_t launch_select(const SelectArgs& a, int D, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  if (a.R > 0) {
    const int nchunk = (a.Tcap + a.chunk - 1) / a.chunk;
    const dim3 g1(nchunk, a.B * a.Hkv);
    const int nq = a.B * a.Hkv * G * a.R;
    const dim3 g3((a.Tcap + a.cm_keys - 1) / a.cm_keys, a.B * a.Hkv);
    // Up to 256 recent queries x group size: the 8-group instances; the
    // host caps the count at kMaxRecent, which the 16-group ones hold.
    static_assert(kMaxRecent <= 16 * 32, "recent queries beyond the largest instance");
    const bool small = G * a.R <= 8 * 32;
    void (*stats)(SelectArgs) = nullptr;
    void (*colmass)(SelectArgs) = nullptr;
    if (D == 128) {
      stats = small ? select_stats_kernel<128, 8> : select_stats_kernel<128, 16>;
      colmass = small ? select_colmass_kernel<128, 8> : select_colmass_kernel<128, 16>;
    } else {
      stats = small ? select_stats_kernel<64, 8> : select_stats_kernel<64, 16>;
      colmass = small ? select_colmass_kernel<64, 8> : select_colmass_kernel<64, 16>;
    }
    hipLaunchKernelGGL(stats, g1, dim3(kSelThreads), 0, stream, a);
    hipLaunchKernelGGL(select_finalize_kernel, dim3((nq + kSelThreads - 1) / kSelThreads), dim3(kSelThreads), 0,
                       stream, a);
    hipLaunchKernelGGL(colmass, g3, dim3(kSelThreads), 0, stream, a);
  }
  // Contexts up to 32K keep 32 masses per thread in registers; longer ones
  // (up to 64K) hold 64, part of them spilled.
  if (a.Tcap <= 8 * kTopkThreads * 4)
    hipLaunchKernelGGL(select_topk_kernel<8>, dim3(a.B * a.Hkv), dim3(kTopkThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(select_topk_kernel<16>, dim3(a.B * a.Hkv), dim3(kTopkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mxattn

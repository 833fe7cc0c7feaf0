// Vertical-line selection for hybrid-precision decode.
//
// Method: HyQuant page (method paragraphs).  A key's score is the attention
// probability it has received from the queries decoded since the last call,
// summed into a per-key total; a call adds to that total and returns the
// rho fraction of highest-scoring keys before the recent window.
//
// Kernels
//   stats    -- per (2048-key context chunk, batch x KV head): every recent
//               query's partial row max and row sum of the logits (S^T =
//               K_hat q_hat^T on the scaled FP4 MFMA, queries staged in
//               LDS), merged per query in chunk order by `finalize`.
//   colmass  -- per 512-key block: the normalised probabilities of every
//               recent query of the KV head's group, summed per key (in-lane
//               over 16 queries, a permlane32 swap for the other 16) and added
//               to col_mass.  Each key belongs to exactly one lane: no atomics.
//   topk     -- per (batch, KV head), one 1024-thread workgroup holding the
//               masses in registers: the k-th largest fp32 bit pattern found
//               by a radix select over 8-bit digits (bit patterns of
//               non-negative values order like the values), then one ordered
//               compaction that emits the indices ascending, ties at the
//               threshold going to the lower indices.
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
constexpr int kStatGroups = kMaxRecent / 32;

template <int D>
__global__ __launch_bounds__(kSelThreads, 2) void select_stats_kernel(SelectArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[kMaxRecent * (D / 2)];
  __shared__ uint8_t qs_lds[kMaxRecent * (D / 32)];
  __shared__ float red[4][kMaxRecent][2];
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
  float m[kStatGroups], l[kStatGroups];
#pragma unroll
  for (int g = 0; g < kStatGroups; ++g) {
    m[g] = -__builtin_huge_valf();
    l[g] = 0.0f;
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
      for (int g = 0; g < kStatGroups; ++g) {
        if (g >= ng) continue;   // uniform; the loop stays unrolled, m[g]/l[g] in fixed registers
        // B operand: query g*32 + j from LDS.
        const int qi = g * 32 + j;
        v16f s = v16f{};
#pragma unroll
        for (int dc = 0; dc < D / 64; ++dc) {
          const v4i qop = *reinterpret_cast<const v4i*>(q_lds + qi * (D / 2) + dc * 32 + hh * 16);
          const int qsc = qs_lds[qi * (D / 32) + 2 * dc + hh];
          s = mfma32_fp4(kb.op[dc], qop, s, kb.sc[dc], qsc);
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
#pragma unroll
  for (int g = 0; g < kStatGroups; ++g) {
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

// Ordered merge of the chunk partials of every recent query.
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
  float M = -__builtin_huge_valf();
  for (int c = 0; c < used; ++c) M = fmaxf(M, stat_slot(a, b, hk, qi, c)[0]);
  float L = 0.0f;
  for (int c = 0; c < used; ++c) {
    const float* st = stat_slot(a, b, hk, qi, c);
    if (st[0] != -__builtin_huge_valf()) L += fast_exp2((st[0] - M) * a.c) * st[1];
  }
  float* out = stat_slot(a, b, hk, qi, nchunk);
  out[0] = M;
  out[1] = 1.0f / L;
}

// ---------------------------------------------------------------------------
// Per (512-key block, batch x KV head): the normalised probabilities of
// every recent query of the group, summed per key and added to col_mass.
// Lane (key j, half hh) of a 32x32 product holds 16 queries, in four runs of
// four consecutive ones, so their (m c, 1/l) come from LDS as float4s.  Each
// key belongs to one lane pair: no atomics.
constexpr int kCmKeys = 512;

template <int D>
__global__ __launch_bounds__(kSelThreads) void select_colmass_kernel(SelectArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[kMaxRecent * (D / 2)];
  __shared__ uint8_t qs_lds[kMaxRecent * (D / 32)];
  __shared__ __attribute__((aligned(16))) float mc_lds[kMaxRecent + 32], il_lds[kMaxRecent + 32];
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int nq = G * a.R, ng = (nq + 31) / 32;
  const int nchunk = (a.Tcap + a.chunk - 1) / a.chunk;
  const int ctx = clamp_ctx(a, b);
  const int k_lo = blk * kCmKeys;
  if (k_lo >= ctx) return;
  const int k_hi = min(k_lo + kCmKeys, ctx);
  stage_queries<D>(a, b, hk, q_lds, qs_lds);
  for (int qi = threadIdx.x; qi < ng * 32; qi += kSelThreads) {
    float mcv = 0.0f, il = 0.0f;   // padding queries contribute 0
    if (qi < nq) {
      const float* st = stat_slot(a, b, hk, qi, nchunk);
      mcv = st[0] * a.c;
      il = st[1];
    }
    mc_lds[qi] = mcv;
    il_lds[qi] = il;
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
    for (int g = 0; g < kStatGroups; ++g) {
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
        const v4f mcv = *reinterpret_cast<const v4f*>(mc_lds + qb);
        const v4f ilv = *reinterpret_cast<const v4f*>(il_lds + qb);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          colsum = __builtin_fmaf(fast_exp2(__builtin_fmaf(s[4 * q4 + r], a.c, -mcv[r])), ilv[r], colsum);
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


// Inclusive prefix sum over the 1024 threads of the workgroup (wave scans
// with shuffles, then the 16 wave totals through LDS).
__device__ __forceinline__ int block_scan_incl(int x, int* wtot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
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
  __shared__ int wtot[kTopkWaves];
  __shared__ uint32_t hist[kTopkWaves][256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_krem, s_digit, s_above;
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv;
  const int ctx = clamp_ctx(a, b);
  const int n = ctx > a.window ? ctx - a.window : 0;
  int k = static_cast<int>((static_cast<int64_t>(n) * a.rho_num + a.rho_den - 1) / a.rho_den);
  k = k > a.max_sel ? a.max_sel : k;
  const uint32_t* v = reinterpret_cast<const uint32_t*>(a.col_mass + static_cast<int64_t>(bh) * a.Tcap);
  int32_t* out = a.idx_out + static_cast<int64_t>(bh) * a.max_sel;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) {
    s_prefix = 0;
    s_krem = k;
    a.n_out[bh] = k;
  }
  __syncthreads();
  // The masses stay in registers for all passes: entry c*4096 + 4*tid + u
  // in x[c][u].
  uint32_t x[kTopkChunks][4];
  const int nch = (n + kTopkThreads * 4 - 1) / (kTopkThreads * 4);
#pragma unroll
  for (int c = 0; c < kTopkChunks; ++c)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = c * kTopkThreads * 4 + tid * 4 + u;
      x[c][u] = (c < nch && i < n) ? v[i] : 0u;
    }
  // Threshold: the k-th largest fp32 bit pattern tau (bit patterns of
  // non-negative values order like the values; any other pattern is ordered
  // as an unsigned integer, so exactly k entries are always taken).  Radix
  // select, 8 bits per pass from the top: each pass counts, among the
  // entries whose higher digits equal tau's, how many take each value of the
  // next digit (wave-private LDS histograms), then takes the digit at which
  // the count from the top reaches k.  `above` counts the entries already
  // known to exceed tau.
  uint32_t tau_bits = 0;
  int above = 0;
  if (k > 0) {
    uint32_t pmask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int e = tid; e < kTopkWaves * 256; e += kTopkThreads) hist[e >> 8][e & 255] = 0u;
      __syncthreads();
#pragma unroll
      for (int cc = 0; cc < kTopkChunks; ++cc) {
        if (cc >= nch) break;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = cc * kTopkThreads * 4 + tid * 4 + u;
          const bool on = i < n && (x[cc][u] & pmask) == tau_bits;
          const uint32_t dg = (x[cc][u] >> shift) & 255u;
          if (shift == 24) {
            // The top digit (sign and high exponent bits) takes few distinct
            // values, so most lanes of a wave would add to the same counter
            // at once.  Lanes with equal digits are counted by ballot and one
            // of them adds the count.
            uint64_t act = __ballot(on);
            while (act != 0ull) {
              const int leader = __builtin_ctzll(act);
              const uint32_t dl = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(dg), leader));
              const uint64_t same = __ballot(on && dg == dl);
              if (lane == leader) atomicAdd(&hist[wave][dl], static_cast<uint32_t>(__popcll(same)));
              act &= ~same;
            }
          } else if (on) {
            atomicAdd(&hist[wave][dg], 1u);
          }
        }
      }
      __syncthreads();
      // Thread t < 256 owns digit 255 - t, so its inclusive scan is the
      // count of entries at or above that digit.
      int cnt = 0;
      if (tid < 256) {
        for (int w = 0; w < kTopkWaves; ++w) cnt += static_cast<int>(hist[w][255 - tid]);
      }
      const int incl = block_scan_incl(cnt, wtot);
      if (tid < 256 && above + incl - cnt < k && above + incl >= k) {
        s_digit = 255 - tid;
        s_above = above + incl - cnt;
      }
      __syncthreads();
      tau_bits |= static_cast<uint32_t>(s_digit) << shift;
      pmask |= 255u << shift;
      above = s_above;
      __syncthreads();
    }
    if (tid == 0) {
      s_prefix = tau_bits;
      s_krem = k - above;
    }
  }
  __syncthreads();
  const uint32_t tau = s_prefix;
  const int take_eq = s_krem;  // entries equal to the threshold to keep, lowest indices first
  // Ordered compaction, chunk by chunk; ranks within a wave from ballots,
  // across waves from the wave totals.
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int base_sel = 0, base_eq = 0;
#pragma unroll
  for (int c = 0; c < kTopkChunks; ++c) {
    if (c >= nch || k == 0) break;
    const int c0 = c * kTopkThreads * 4;
    bool gt[4], eq[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = c0 + tid * 4 + u;
      gt[u] = i < n && x[c][u] > tau;
      eq[u] = i < n && x[c][u] == tau;
    }
    // Rank of each equal entry among the equal entries (index order).
    int eq_before = 0, eq_mine = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      eq_before += __popcll(__ballot(eq[u]) & lt);
      eq_mine += eq[u] ? 1 : 0;
    }
    if (lane == 63) wtot[wave] = eq_before + eq_mine;
    __syncthreads();
    int eq_base = base_eq, eq_total = 0;
    for (int w = 0; w < kTopkWaves; ++w) {
      if (w < wave) eq_base += wtot[w];
      eq_total += wtot[w];
    }
    __syncthreads();
    bool sel[4];
    int r_eq = eq_base + eq_before;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sel[u] = gt[u];
      if (eq[u]) {
        sel[u] = r_eq < take_eq;
        ++r_eq;
      }
    }
    int sel_before = 0, sel_mine = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sel_before += __popcll(__ballot(sel[u]) & lt);
      sel_mine += sel[u] ? 1 : 0;
    }
    if (lane == 63) wtot[wave] = sel_before + sel_mine;
    __syncthreads();
    int pos = base_sel + sel_before, sel_total = 0;
    for (int w = 0; w < kTopkWaves; ++w) {
      if (w < wave) pos += wtot[w];
      sel_total += wtot[w];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (sel[u]) out[pos++] = c0 + tid * 4 + u;
    base_sel += sel_total;
    base_eq += eq_total;
  }
  for (int i = k + tid; i < a.max_sel; i += kTopkThreads) out[i] = -1;
}

hipError_t launch_select(const SelectArgs& a, int D, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  if (a.R > 0) {
    const int nchunk = (a.Tcap + a.chunk - 1) / a.chunk;
    const dim3 g1(nchunk, a.B * a.Hkv);
    const int nq = a.B * a.Hkv * G * a.R;
    const dim3 g3((a.Tcap + kCmKeys - 1) / kCmKeys, a.B * a.Hkv);
    if (D == 128) {
      hipLaunchKernelGGL(select_stats_kernel<128>, g1, dim3(kSelThreads), 0, stream, a);
      hipLaunchKernelGGL(select_finalize_kernel, dim3((nq + kSelThreads - 1) / kSelThreads), dim3(kSelThreads), 0,
                         stream, a);
      hipLaunchKernelGGL(select_colmass_kernel<128>, g3, dim3(kSelThreads), 0, stream, a);
    } else {
      hipLaunchKernelGGL(select_stats_kernel<64>, g1, dim3(kSelThreads), 0, stream, a);
      hipLaunchKernelGGL(select_finalize_kernel, dim3((nq + kSelThreads - 1) / kSelThreads), dim3(kSelThreads), 0,
                         stream, a);
      hipLaunchKernelGGL(select_colmass_kernel<64>, g3, dim3(kSelThreads), 0, stream, a);
    }
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

// Vertical-line selection for hybrid-precision decode.
//
// Method: HyQuant page (method paragraphs) -- the vertical-line score of a key
// is its accumulated column mass; the top-rho fraction of the non-window
// prefix is kept in full precision; identification is a light reduction run
// every 64 tokens.
//
// Kernels
//   stats    -- per (context chunk, 128 recent queries): partial row max and
//               row sum of the logits (S^T = K_hat q_hat^T on the scaled FP4
//               MFMA), merged per query in chunk order by `finalize`.
//   colmass  -- per 256-key block: the normalised probabilities of every
//               recent query of the KV head's group, summed per key (in-lane
//               over 16 queries, a permlane32 swap for the other 16) and added
//               to col_mass.  Each key belongs to exactly one lane: no atomics.
//   topk     -- per (batch, KV head): exact radix select of the k-th largest
//               mass (4 passes of 8 bits over the fp32 bit patterns, which
//               order like the non-negative values), then one ordered
//               compaction that emits the indices ascending, ties at the
//               threshold going to the lower indices.
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
template <int D>
__global__ __launch_bounds__(kSelThreads) void select_stats_kernel(SelectArgs a) {
  const int chunk = blockIdx.x, qgrp = blockIdx.y, bh = blockIdx.z;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, j = lane & 31, hh = lane >> 5;
  const int qi = (qgrp * 4 + wave) * 32 + j;
  const int G = a.Hq / a.Hkv;
  const int ctx = clamp_ctx(a, b);
  const int t_lo = chunk * a.chunk;
  const int t_hi = min(t_lo + a.chunk, ctx);
  if ((qgrp * 4 + wave) * 32 >= G * a.R) return;  // whole wave past the queries
  v4i qop[D / 64];
  int qsc[D / 64];
#pragma unroll
  for (int dc = 0; dc < D / 64; ++dc) query_operand(a, b, hk, qi, hh, dc, qop[dc], qsc[dc]);
  const uint8_t* kc = a.k.codes + b * a.k.cs[0] + hk * a.k.cs[1];
  const uint8_t* ks = a.k.scales + b * a.k.ss[0] + hk * a.k.ss[1];
  float m = -__builtin_huge_valf(), l = 0.0f;
  for (int t0 = t_lo; t0 < t_hi; t0 += 32) {
    const int t = t0 + j;
    v16f s = v16f{};
#pragma unroll
    for (int dc = 0; dc < D / 64; ++dc) {
      const bool ok = t < t_hi;
      const v4i kop = ok ? *reinterpret_cast<const v4i*>(kc + static_cast<int64_t>(t) * a.k.cs[2] + dc * 32 + hh * 16)
                         : v4i{0, 0, 0, 0};
      const int ksc = ok ? ks[static_cast<int64_t>(t) * a.k.ss[2] + 2 * dc + hh] : 0;
      s = mfma32_fp4(kop, qop[dc], s, ksc, qsc[dc]);
    }
    // Lane (query j, half hh) holds keys 8(r/4) + 4hh + r%4 of the block.
    float x = -__builtin_huge_valf();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = t0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (key >= t_hi) s[r] = -__builtin_huge_valf();
      x = fmaxf(x, s[r]);
    }
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    const float m_new = fmaxf(m, x);
    const float alpha = m == -__builtin_huge_valf() ? 0.0f : fast_exp2((m - m_new) * a.c);
    const float mc = m_new * a.c;
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += fast_exp2(__builtin_fmaf(s[r], a.c, -mc));
    l = l * alpha + sum;
    m = m_new;
  }
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
  l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  if (hh == 0 && qi < G * a.R) {
    float* st = stat_slot(a, b, hk, qi, chunk);
    st[0] = m;
    st[1] = l;
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
constexpr int kCmKeys = 256;       // keys per colmass workgroup (4 waves x 2 blocks)
constexpr int kMaxRecent = 512;    // recent queries x group size held in LDS

template <int D>
__global__ __launch_bounds__(kSelThreads) void select_colmass_kernel(SelectArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[kMaxRecent * (D / 2)];
  __shared__ uint8_t qs_lds[kMaxRecent * (D / 32)];
  __shared__ float mst[kMaxRecent], inv_l[kMaxRecent];
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.Hkv, hk = bh % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int nq = G * a.R;
  const int nchunk = (a.Tcap + a.chunk - 1) / a.chunk;
  const int ctx = clamp_ctx(a, b);
  const int k_lo = blk * kCmKeys;
  if (k_lo >= ctx) return;
  // Stage the group's recent queries (codes, scales, max, 1/sum).
  for (int e = threadIdx.x; e < nq * (D / 32); e += kSelThreads) {
    const int qi = e / (D / 32), part = e % (D / 32);
    const int hq = hk * G + qi / a.R, r = qi % a.R;
    const uint8_t* c = a.q.codes + b * a.q.cs[0] + hq * a.q.cs[1] + static_cast<int64_t>(r) * a.q.cs[2];
    const uint8_t* s = a.q.scales + b * a.q.ss[0] + hq * a.q.ss[1] + static_cast<int64_t>(r) * a.q.ss[2];
    *reinterpret_cast<v4i*>(q_lds + qi * (D / 2) + part * 16) = *reinterpret_cast<const v4i*>(c + part * 16);
    qs_lds[qi * (D / 32) + part] = s[part];
  }
  for (int qi = threadIdx.x; qi < nq; qi += kSelThreads) {
    const float* st = stat_slot(a, b, hk, qi, nchunk);
    mst[qi] = st[0];
    inv_l[qi] = st[1];
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, j = lane & 31, hh = lane >> 5;
  const uint8_t* kc = a.k.codes + b * a.k.cs[0] + hk * a.k.cs[1];
  const uint8_t* ks = a.k.scales + b * a.k.ss[0] + hk * a.k.ss[1];
  float* cm = a.col_mass + (static_cast<int64_t>(b) * a.Hkv + hk) * a.Tcap;
  for (int kb = 0; kb < kCmKeys / 128; ++kb) {
    const int t0 = k_lo + (kb * 4 + wave) * 32;
    const int t = t0 + j;
    if (t0 >= ctx) break;
    const bool ok = t < ctx;
    // B operand: key column j.
    v4i kop[D / 64];
    int ksc[D / 64];
#pragma unroll
    for (int dc = 0; dc < D / 64; ++dc) {
      kop[dc] = ok ? *reinterpret_cast<const v4i*>(kc + static_cast<int64_t>(t) * a.k.cs[2] + dc * 32 + hh * 16)
                   : v4i{0, 0, 0, 0};
      ksc[dc] = ok ? ks[static_cast<int64_t>(t) * a.k.ss[2] + 2 * dc + hh] : 0;
    }
    float colsum = 0.0f;
    for (int q0 = 0; q0 < nq; q0 += 32) {
      // A operand: queries q0 + (lane % 32).
      const int qa = q0 + j;
      v16f s = v16f{};
#pragma unroll
      for (int dc = 0; dc < D / 64; ++dc) {
        v4i qop = {0, 0, 0, 0};
        int qsc = 0;
        if (qa < nq) {
          qop = *reinterpret_cast<const v4i*>(q_lds + qa * (D / 2) + dc * 32 + hh * 16);
          qsc = qs_lds[qa * (D / 32) + 2 * dc + hh];
        }
        s = mfma32_fp4(qop, kop[dc], s, qsc, ksc[dc]);
      }
      // Lane (key j, half hh) holds queries q0 + 8(r/4) + 4hh + r%4.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = q0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (qr < nq) colsum += fast_exp2(__builtin_fmaf(s[r], a.c, -mst[qr] * a.c)) * inv_l[qr];
      }
    }
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(colsum), __float_as_uint(colsum), false, false);
    colsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if (hh == 0 && ok) cm[t] += colsum;
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(SelectArgs a) {
  __shared__ int hist[256];
  __shared__ int scan_sel[kSelThreads], scan_eq[kSelThreads];
  __shared__ uint32_t s_prefix;
  __shared__ int s_krem;
  const int bh = blockIdx.x;
  const int b = bh / a.Hkv;
  const int ctx = clamp_ctx(a, b);
  const int n = ctx > a.window ? ctx - a.window : 0;
  int k = static_cast<int>((static_cast<int64_t>(n) * a.rho_num + a.rho_den - 1) / a.rho_den);
  k = k > a.max_sel ? a.max_sel : k;
  const uint32_t* v = reinterpret_cast<const uint32_t*>(a.col_mass + static_cast<int64_t>(bh) * a.Tcap);
  int32_t* out = a.idx_out + static_cast<int64_t>(bh) * a.max_sel;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_prefix = 0;
    s_krem = k;
    a.n_out[bh] = k;
  }
  __syncthreads();
  uint32_t mask = 0;
  if (k > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      const uint32_t prefix = s_prefix;
      for (int i = tid; i < n; i += kSelThreads) {
        const uint32_t x = v[i];
        if ((x & mask) == prefix) atomicAdd(&hist[(x >> shift) & 0xFF], 1);
      }
      __syncthreads();
      if (tid == 0) {
        int krem = s_krem, above = 0, bin = 255;
        for (; bin > 0; --bin) {
          if (above + hist[bin] >= krem) break;
          above += hist[bin];
        }
        s_krem = krem - above;
        s_prefix = prefix | (static_cast<uint32_t>(bin) << shift);
      }
      mask |= 0xFFu << shift;
      __syncthreads();
    }
  }
  const uint32_t tau = s_prefix;
  const int take_eq = s_krem;  // equal-to-threshold entries to keep, lowest indices first
  int base_sel = 0, base_eq = 0;
  for (int c0 = 0; c0 < n && k > 0; c0 += kSelThreads * 4) {
    int fsel[4], feq[4], lsel = 0, leq = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = c0 + tid * 4 + u;
      const uint32_t x = i < n ? v[i] : 0u;
      feq[u] = (i < n && x == tau) ? 1 : 0;
      fsel[u] = (i < n && x > tau) ? 1 : 0;
      leq += feq[u];
    }
    scan_eq[tid] = leq;
    __syncthreads();
    for (int off = 1; off < kSelThreads; off <<= 1) {  // inclusive scan of equal counts
      const int add = tid >= off ? scan_eq[tid - off] : 0;
      __syncthreads();
      scan_eq[tid] += add;
      __syncthreads();
    }
    int eq_rank = base_eq + scan_eq[tid] - leq;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (feq[u]) {
        fsel[u] = eq_rank < take_eq ? 1 : 0;
        ++eq_rank;
      }
      lsel += fsel[u];
    }
    scan_sel[tid] = lsel;
    __syncthreads();
    for (int off = 1; off < kSelThreads; off <<= 1) {
      const int add = tid >= off ? scan_sel[tid - off] : 0;
      __syncthreads();
      scan_sel[tid] += add;
      __syncthreads();
    }
    int pos = base_sel + scan_sel[tid] - lsel;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (fsel[u]) out[pos++] = c0 + tid * 4 + u;
    base_sel += scan_sel[kSelThreads - 1];
    base_eq += scan_eq[kSelThreads - 1];
    __syncthreads();
  }
  for (int i = k + tid; i < a.max_sel; i += kSelThreads) out[i] = -1;
}

hipError_t launch_select(const SelectArgs& a, int D, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  if (a.R > 0) {
    const int nchunk = (a.Tcap + a.chunk - 1) / a.chunk;
    const int qgroups = (G * a.R + 127) / 128;
    const dim3 g1(nchunk, qgroups, a.B * a.Hkv);
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
  hipLaunchKernelGGL(select_topk_kernel, dim3(a.B * a.Hkv), dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mxattn

// MXFP4 FlashAttention forward with pre-normalisation P quantisation.
//
// Method: HiFA4 page (Abstract) -- QK^T and PV both run as 4-bit GEMMs, the
// online-softmax state stays in higher precision (fp32 here), and the
// normaliser is accumulated from the same quantised weights P_hat that feed
// the PV product ("P-Reordering"), which also lets the normaliser ride inside
// the PV GEMM.  MXAttention page (Abstract) -- PNQ quantises the unnormalised
// exponentials before the row sum; UOS bounds the block scale at Qmax = 7.25.
// BitDecoding-FP4 page ("System-Level Optimization") -- transposed softmax:
// the normalisation runs along the GEMM accumulation direction so P is
// quantised in place and never written to memory.
//
// gfx950 design (one workgroup = 4 waves = 128 query rows of one head):
//   * S^T = K_hat Q_hat^T with v_mfma_scale_f32_32x32x64_f8f6f4 (E2M1 x E2M1,
//     E8M0 scales per lane).  The K rows fed to the MFMA are permuted so that
//     lane (query j, half h) receives keys 16h..16h+15 of each 32-key block:
//     the row max, block maxima and the P quantisation are in-lane work plus
//     one permlane32 swap.
//   * P~ = exp2(S*c - m*c) (c = softmax_scale*log2 e), quantised per
//     (query, 32 keys) by v_cvt_scalef32_pk_fp4_f32, whose rounding is the
//     format's round-to-nearest-even.  The block exponent comes from
//     exp2((blockmax - m)*c), exact (= 1) for the block holding the maximum.
//   * One permlane32 swap per code dword turns the codes into the B operand
//     of O^T += V_hat^T P_hat^T (32 consecutive keys per lane, scale = the P
//     block scale); V is stored key-blocked so its A operand and scales load
//     straight from LDS.
//   * The normaliser l = sum P_hat comes out of the same MFMA stream: an A
//     operand with two rows of E2M1 ones (the fused normaliser of HiFA4).
//   * K/V tiles are double-buffered in LDS (rows padded to avoid bank
//     conflicts); the grid is ordered longest-first for causal masks and
//     mapped so that each XCD works on whole KV heads.
#include "mx_device.h"
#include "kernels.h"

namespace mxattn {

constexpr int kBR = 128;      // query rows per workgroup
constexpr int kThreads = 256;

template <int D, int BC>
struct Cfg {
  static constexpr int KB = BC / 32;        // 32-key blocks per tile
  static constexpr int DC = D / 64;         // 64-deep chunks of the QK^T contraction
  static constexpr int DT = D / 32;         // 32-channel tiles of O^T
  static constexpr int KRB = D / 2;         // bytes per K row (one key)
  static constexpr int VRB = BC / 2;        // bytes per V row (one channel, BC keys)
  static constexpr int KSROW = D / 32;
  static constexpr int VSROW = BC / 32;
  static constexpr int OFF_V = BC * KRB;
  static constexpr int OFF_KS = OFF_V + D * VRB;
  static constexpr int OFF_VS = OFF_KS + BC * KSROW;
  static constexpr int STAGE = ((OFF_VS + D * VSROW) + 15) / 16 * 16;
  static constexpr int K_LOADS = BC * KRB / 1024;  // 1 KB direct-to-LDS wave loads per tile
  static constexpr int V_LOADS = D * VRB / 1024;
  static constexpr int NKS = BC * D / 32;          // K scale bytes per tile
  static constexpr int NVS = D * BC / 32;          // V scale bytes per tile
  static constexpr int IKS = (NKS + kThreads - 1) / kThreads;
  static constexpr int IVS = (NVS + kThreads - 1) / kThreads;
};

// MFMA row i of the S^T product holds key sigma(i) of the 32-key block, so
// that C row 8(r/4) + 4h + r%4 (lane half h, register r) is key 16h + r.
__device__ __forceinline__ int sigma(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

// LDS rows of RB bytes hold their 16-byte chunks XOR-swizzled by the row's
// position inside a 256-byte bank period, so 16 lanes reading the same chunk
// of 16 consecutive rows hit 16 different bank groups.
template <int RB>
__device__ __forceinline__ int swz(int row, int chunk) {
  constexpr int rows_per_period = 256 / RB;
  constexpr int chunks = RB / 16;
  return chunk ^ ((row / rows_per_period) % chunks);
}

template <int D, int BC>
struct ScaleRegs {
  uint8_t ks[Cfg<D, BC>::IKS];
  uint8_t vs[Cfg<D, BC>::IVS];
};

// Issue the direct HBM->LDS loads of a tile's K and V codes (this wave's
// share of the 1 KB loads) and fetch its share of the scale bytes into
// registers.  Rows past the sequence read a clamped valid row; their logits
// are masked and their P is 0, so the bytes never matter.
template <int D, int BC>
__device__ __forceinline__ void issue_tile(const PrefillArgs& a, int b, int hk, int t0, uint8_t* stage,
                                           ScaleRegs<D, BC>& sr, int tid) {
  using C = Cfg<D, BC>;
  const int wave = tid >> 6, lane = tid & 63;
  const uint8_t* kc = a.k.codes + b * a.k.cs[0] + hk * a.k.cs[1];
  const uint8_t* ks = a.k.scales + b * a.k.ss[0] + hk * a.k.ss[1];
  const uint8_t* vc = a.v.codes + b * a.v.cs[0] + hk * a.v.cs[1];
  const uint8_t* vs = a.v.scales + b * a.v.ss[0] + hk * a.v.ss[1];
  const int nblk = (a.Sk + 31) / 32;
#pragma unroll
  for (int i = wave; i < C::K_LOADS; i += 4) {
    const int o = i * 1024 + 16 * lane;
    const int r = o / C::KRB, pos = (o % C::KRB) / 16;
    const int chunk = pos ^ ((r / (256 / C::KRB)) % (C::KRB / 16));
    int t = t0 + (r & ~31) + sigma(r & 31);
    t = t < a.Sk ? t : a.Sk - 1;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(kc + t * a.k.cs[2] + chunk * 16),
                                     (__attribute__((address_space(3))) void*)(stage + i * 1024),
                                     16, 0, 0);
  }
#pragma unroll
  for (int i = wave; i < C::V_LOADS; i += 4) {
    const int o = i * 1024 + 16 * lane;
    const int d = o / C::VRB, pos = (o % C::VRB) / 16;
    const int chunk = pos ^ ((d / (256 / C::VRB)) % (C::VRB / 16));
    int blk = t0 / 32 + chunk;
    blk = blk < nblk ? blk : nblk - 1;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(vc + d * a.v.cs[2] + blk * 16),
                                     (__attribute__((address_space(3))) void*)(stage + C::OFF_V + i * 1024),
                                     16, 0, 0);
  }
  // Scale bytes: indices are clamped instead of branched on; a clamped key
  // is masked and a clamped V block only meets P = 0, and both read real
  // (finite) scale bytes.
#pragma unroll
  for (int i = 0; i < C::IKS; ++i) {
    const int e = (tid + kThreads * i) % C::NKS;
    const int r = e / C::KSROW, part = e % C::KSROW;
    int t = t0 + (r & ~31) + sigma(r & 31);
    t = t < a.Sk ? t : a.Sk - 1;
    sr.ks[i] = ks[t * a.k.ss[2] + part];
  }
#pragma unroll
  for (int i = 0; i < C::IVS; ++i) {
    const int e = (tid + kThreads * i) % C::NVS;
    const int d = e / C::VSROW, part = e % C::VSROW;
    int blk = t0 / 32 + part;
    blk = blk < nblk ? blk : nblk - 1;
    sr.vs[i] = vs[d * a.v.ss[2] + blk];
  }
}

// The scale bytes of one LDS scale row (2, 4 or 8 bytes) as a 64-bit word.
template <int ROWBYTES>
__device__ __forceinline__ uint64_t scale_row(const uint8_t* base, int row) {
  if constexpr (ROWBYTES == 8) return *reinterpret_cast<const uint64_t*>(base + row * 8);
  if constexpr (ROWBYTES == 4) return *reinterpret_cast<const uint32_t*>(base + row * 4);
  return *reinterpret_cast<const uint16_t*>(base + row * 2);
}

__device__ __forceinline__ int scale_byte(uint64_t w, int i) { return static_cast<int>((w >> (8 * i)) & 0xFF); }

template <int D, int BC>
__device__ __forceinline__ void store_scales(const ScaleRegs<D, BC>& sr, uint8_t* stage, int tid) {
  using C = Cfg<D, BC>;
#pragma unroll
  for (int i = 0; i < C::IKS; ++i) {
    const int e = tid + kThreads * i;
    if (e < C::NKS) stage[C::OFF_KS + e] = sr.ks[i];
  }
#pragma unroll
  for (int i = 0; i < C::IVS; ++i) {
    const int e = tid + kThreads * i;
    if (e < C::NVS) stage[C::OFF_VS + e] = sr.vs[i];
  }
}

// Workgroup -> (query block, batch, query head).  Consecutive workgroups go
// to different XCDs (round robin over 8); the mapping gives each XCD whole
// (batch, KV head) pairs so their K/V stay in that XCD's L2, and issues the
// longest causal query blocks first.
__device__ __forceinline__ void map_block(const PrefillArgs& a, bool causal, int& qb, int& b, int& hq) {
  const int G = a.Hq / a.Hkv;
  const int pairs = a.B * a.Hkv;
  const int bid = blockIdx.x;
  int qi, pair, g;
  if (pairs % 8 == 0) {
    const int slot = bid % 8, rank = bid / 8;
    const int per = pairs / 8;
    qi = rank / (per * G);
    const int rem = rank % (per * G);
    pair = slot * per + rem / G;
    g = rem % G;
  } else {
    qi = bid / (pairs * G);
    const int rem = bid % (pairs * G);
    pair = rem / G;
    g = rem % G;
  }
  qb = causal ? (a.n_qblk - 1 - qi) : qi;
  b = pair / a.Hkv;
  hq = (pair % a.Hkv) * G + g;
}

template <int D, int BC, bool CAUSAL>
__global__ __launch_bounds__(kThreads, (BC == 256 ? 1 : 2)) void prefill_kernel(PrefillArgs a) {
  using C = Cfg<D, BC>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, j = lane & 31, hh = lane >> 5;

  int qb, b, hq;
  map_block(a, CAUSAL, qb, b, hq);
  const int hk = hq / (a.Hq / a.Hkv);
  const int q0 = qb * kBR;
  const int my_q = q0 + wave * 32 + j;
  const int qrow = my_q < a.Sq ? my_q : a.Sq - 1;  // padding rows recompute the last row

  // B operand of S^T: query qrow, channels [64 dc + 32 hh, +32).
  v4i qop[C::DC];
  int qsc[C::DC];
  {
    const uint8_t* qc = a.q.codes + b * a.q.cs[0] + hq * a.q.cs[1] + static_cast<int64_t>(qrow) * a.q.cs[2];
    const uint8_t* qs = a.q.scales + b * a.q.ss[0] + hq * a.q.ss[1] + static_cast<int64_t>(qrow) * a.q.ss[2];
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) {
      qop[dc] = *reinterpret_cast<const v4i*>(qc + dc * 32 + hh * 16);
      qsc[dc] = qs[2 * dc + hh];
    }
  }

  const int last_q = (q0 + kBR - 1 < a.Sq - 1) ? q0 + kBR - 1 : a.Sq - 1;
  const int nt = CAUSAL ? last_q / BC + 1 : (a.Sk + BC - 1) / BC;
  const int wave_last_q = (q0 + wave * 32 + 31 < a.Sq - 1) ? q0 + wave * 32 + 31 : a.Sq - 1;
  const int my_nt = CAUSAL ? wave_last_q / BC + 1 : nt;
  const int wave_first_q = q0 + wave * 32;

  // E2M1 ones for the normaliser: a 16x16x128 A operand whose rows 0-7 sum
  // the k-groups of lanes 0-15 and 32-47 (queries 0-15 of both key blocks)
  // and rows 8-15 those of lanes 16-31 and 48-63 (queries 16-31).
  const int one_r = lane & 15, one_kg = lane >> 4;
  const bool one_on = (one_r < 8) ? (one_kg == 0 || one_kg == 2) : (one_kg == 1 || one_kg == 3);
  const int onev = one_on ? 0x22222222 : 0;
  const v4i ones = {onev, onev, onev, onev};
  const int l_query = (lane & 15) + 16 * (lane >> 5);

  float m = -__builtin_huge_valf();
  float lsum = 0.0f;  // baseline normaliser (sum of unquantised P~)
  v16f O[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) O[dt] = v16f{};
  v4f L = v4f{0, 0, 0, 0};

  ScaleRegs<D, BC> sr;
  issue_tile<D, BC>(a, b, hk, 0, smem, sr, tid);
  store_scales<D, BC>(sr, smem, tid);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int jt = 0; jt < nt; ++jt) {
    const int t0 = jt * BC;
    uint8_t* next = smem + ((jt + 1) & 1) * C::STAGE;
    if (jt + 1 < nt) issue_tile<D, BC>(a, b, hk, t0 + BC, next, sr, tid);
    if (jt < my_nt) {
      const uint8_t* base = smem + (jt & 1) * C::STAGE;
      const uint8_t* Kc = base;
      const uint8_t* Vc = base + C::OFF_V;
      const uint8_t* Ks = base + C::OFF_KS;
      const uint8_t* Vs = base + C::OFF_VS;

      // ---- S^T = K_hat Q_hat^T (each block's operands are read into their
      // own registers before its MFMAs, so LDS latency overlaps the MFMAs)
      v16f S[C::KB];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const int r = kb * 32 + j;
        v4i aop[C::DC];
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc)
          aop[dc] = *reinterpret_cast<const v4i*>(Kc + r * C::KRB + 16 * swz<C::KRB>(r, 2 * dc + hh));
        const uint64_t ksw = scale_row<C::KSROW>(Ks, r);
        v16f acc = v16f{};
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc) acc = mfma32_fp4(aop[dc], qop[dc], acc, scale_byte(ksw, 2 * dc + hh), qsc[dc]);
        S[kb] = acc;
      }

      // ---- masks: causal (key > query) and keys past the end
      const bool tail = t0 + BC > a.Sk;
      const bool diag = CAUSAL && (t0 + BC - 1 > wave_first_q);
      if (tail || diag) {
        const int qlim = CAUSAL ? qrow : 0x7FFFFFFF;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int t = t0 + kb * 32 + 16 * hh + r;
            if (t > qlim || t >= a.Sk) S[kb][r] = -__builtin_huge_valf();
          }
      }

      // ---- block maxima (raw logits), running maximum
      float bm[C::KB];
      float tmax = -__builtin_huge_valf();
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        float x = S[kb][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) x = fmaxf(x, S[kb][r]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        bm[kb] = x;
        tmax = fmaxf(tmax, x);
      }
      const float m_new = fmaxf(m, tmax);
      const float alpha = fast_exp2((m - m_new) * a.c);
      const float mc = m_new * a.c;

      // ---- P~ (in place of S), its MXFP4 codes, the PV B operands
      uint32_t code[C::KB][2];
      int eb[C::KB];
      float tile_sum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        const float pmax = fast_exp2((bm[kb] - m_new) * a.c);
        int byte = e8m0_byte(__float_as_uint(pmax), a.p_uos != 0, a.p_qmax_quarter);
        byte = byte < 1 ? 1 : byte;  // keep the convert's scale a normal float
        eb[kb] = byte;
        const float scl = scale_of_byte(byte);
#pragma unroll
        for (int r = 0; r < 16; ++r) S[kb][r] = fast_exp2(__builtin_fmaf(S[kb][r], a.c, -mc));
        if (!a.l_from_quantized) {
#pragma unroll
          for (int r = 0; r < 16; ++r) tile_sum += S[kb][r];
        }
        const v16f& p = S[kb];
        uint32_t w0 = 0, w1 = 0;
        w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, p[0], p[1], scl, 0);
        w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, p[2], p[3], scl, 1);
        w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, p[4], p[5], scl, 2);
        w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, p[6], p[7], scl, 3);
        w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, p[8], p[9], scl, 0);
        w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, p[10], p[11], scl, 1);
        w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, p[12], p[13], scl, 2);
        w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, p[14], p[15], scl, 3);
        code[kb][0] = w0;
        code[kb][1] = w1;
      }
      if (!a.l_from_quantized) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tile_sum), __float_as_uint(tile_sum), false, false);
        lsum = alpha * lsum + (__uint_as_float(sw[0]) + __uint_as_float(sw[1]));
      }

      // ---- rescale the accumulators (skipped when no row's maximum moved)
      if (__builtin_amdgcn_ballot_w64(m_new > m) != 0) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) O[dt] *= alpha;
        // L[0] of this lane is the normaliser of query l%16 + 16*(l/32),
        // whose factor lives in that query's lane.
        L[0] *= __shfl(alpha, l_query);
      }
      m = m_new;

      // ---- O^T += V_hat^T P_hat^T, and l += ones^T P_hat^T
#pragma unroll
      for (int pp = 0; pp < C::KB / 2; ++pp) {
        const auto r0 = __builtin_amdgcn_permlane32_swap(code[2 * pp][0], code[2 * pp + 1][0], false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(code[2 * pp][1], code[2 * pp + 1][1], false, false);
        const v4i bop = {(int)r0[0], (int)r1[0], (int)r0[1], (int)r1[1]};
        const int bsc = hh ? eb[2 * pp + 1] : eb[2 * pp];
        v4i aop[C::DT];
        int sa[C::DT];
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          const int vrow = dt * 32 + j;
          aop[dt] = *reinterpret_cast<const v4i*>(Vc + vrow * C::VRB + 16 * swz<C::VRB>(vrow, 2 * pp + hh));
          sa[dt] = scale_byte(scale_row<C::VSROW>(Vs, vrow), 2 * pp + hh);
        }
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) O[dt] = mfma32_fp4(aop[dt], bop, O[dt], sa[dt], bsc);
        L = mfma16_fp4(ones, bop, L, a.one_scale, bsc);
      }
    }
    if (jt + 1 < nt) store_scales<D, BC>(sr, next, tid);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- finalise: out = O / l, lse = m * softmax_scale + ln l
  // The normaliser of query j sits in lane j (j < 16) or j + 16 (j >= 16).
  const float lq = __shfl(L[0], j < 16 ? j : j + 16);
  if (my_q >= a.Sq) return;
  const float l = a.l_from_quantized ? lq : lsum;
  const float inv = 1.0f / l;
  const int64_t orow = (static_cast<int64_t>(b) * a.Hq + hq) * a.Sq + my_q;
  if (a.lse != nullptr && hh == 0) a.lse[orow] = m * a.softmax_scale + logf(l);
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = dt * 32 + 8 * g4 + 4 * hh;
      const float o0 = O[dt][4 * g4 + 0] * inv, o1 = O[dt][4 * g4 + 1] * inv;
      const float o2 = O[dt][4 * g4 + 2] * inv, o3 = O[dt][4 * g4 + 3] * inv;
      if (a.out_dtype == 0) {
        *reinterpret_cast<v4f*>(reinterpret_cast<float*>(a.out) + orow * D + d) = v4f{o0, o1, o2, o3};
      } else if (a.out_dtype == 2) {
        const __bf16 h0 = static_cast<__bf16>(o0), h1 = static_cast<__bf16>(o1);
        const __bf16 h2 = static_cast<__bf16>(o2), h3 = static_cast<__bf16>(o3);
        const uint32_t lo = __builtin_bit_cast(uint16_t, h0) | (uint32_t(__builtin_bit_cast(uint16_t, h1)) << 16);
        const uint32_t hi = __builtin_bit_cast(uint16_t, h2) | (uint32_t(__builtin_bit_cast(uint16_t, h3)) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + orow * D + d) = uint2{lo, hi};
      } else {
        const _Float16 h0 = static_cast<_Float16>(o0), h1 = static_cast<_Float16>(o1);
        const _Float16 h2 = static_cast<_Float16>(o2), h3 = static_cast<_Float16>(o3);
        const uint32_t lo = __builtin_bit_cast(uint16_t, h0) | (uint32_t(__builtin_bit_cast(uint16_t, h1)) << 16);
        const uint32_t hi = __builtin_bit_cast(uint16_t, h2) | (uint32_t(__builtin_bit_cast(uint16_t, h3)) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + orow * D + d) = uint2{lo, hi};
      }
    }
}

template <int D, int BC>
static void launch_t(const PrefillArgs& a, int causal, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(a.n_qblk) * a.B * a.Hq;
  if (causal)
    hipLaunchKernelGGL((prefill_kernel<D, BC, true>), dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, BC, false>), dim3(grid), dim3(kThreads), 0, stream, a);
}

hipError_t launch_prefill(const PrefillArgs& a, int D, int kv_tile, int causal, hipStream_t stream) {
  if (a.n_qblk == 0) return hipSuccess;
  if (D == 128) {
    if (kv_tile == 64) launch_t<128, 64>(a, causal, stream);
    else if (kv_tile == 128) launch_t<128, 128>(a, causal, stream);
    else launch_t<128, 256>(a, causal, stream);
  } else {
    if (kv_tile == 64) launch_t<64, 64>(a, causal, stream);
    else if (kv_tile == 128) launch_t<64, 128>(a, causal, stream);
    else launch_t<64, 256>(a, causal, stream);
  }
  return hipGetLastError();
}

}  // namespace mxattn

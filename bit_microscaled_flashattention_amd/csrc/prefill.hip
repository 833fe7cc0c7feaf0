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
//
// Hybrid variant (HyQuant page, prefill paragraph: the 4-bit tiles and the
// full-precision vertical-line and window keys share one kernel and one
// online softmax).  Query i keeps its `window` most recent keys and the
// selected keys in bf16.  The 4-bit tiles run first with those keys masked
// out (the window as a causal limit shifted by `window`, the selected keys
// through a bitmap in LDS), so every P quantisation decision is that of the
// plain kernel on the remaining keys.  Then the workgroup walks the bf16 keys
// in chunks of 32 (its window range, then the selected list): S^T and
// O^T += V^T P^T on the bf16 MFMA, P unquantised as hi + lo bf16 parts.
#include <type_traits>

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
  static constexpr int KSROW = D / 32;        // K scale bytes per key
  static constexpr int VSROW = BC / 32;       // V scale bytes per channel in a tile
  // Scale bytes sit in LDS so that lane (row i, half hh) finds every byte
  // one MFMA needs at a fixed position of one 32-bit word: word group g,
  // half hh, row i is at g*256 + hh*128 + 4i.  K: group = kb / KPD, byte
  // (kb % KPD)*DC + dc.  V: group = dt / DPD, byte (dt % DPD)*(KB/2) + pp.
  static constexpr int KPD = 4 / DC;          // key blocks per K scale word
  static constexpr int DPD = (KB / 2) >= 4 ? 1 : 4 / (KB / 2);  // channel tiles per V scale word
  static constexpr int KS_BYTES = ((KB + KPD - 1) / KPD) * 256;
  static constexpr int VS_BYTES = ((DT + DPD - 1) / DPD) * 256;
  static constexpr int OFF_V = BC * KRB;
  static constexpr int OFF_KS = OFF_V + D * VRB;
  static constexpr int OFF_VS = OFF_KS + KS_BYTES;
  static constexpr int STAGE = ((OFF_VS + VS_BYTES) + 15) / 16 * 16;
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

// Buffer resources over one (batch, KV head) of the K and V operands.  K
// rows past the sequence lie past the K resources' end: their loads return
// zeros without fetching (those keys are masked).  V rows are channels, so a
// block index past the sequence is clamped to the last block instead (those
// keys only meet P = 0).
struct TileSrc {
  __amdgpu_buffer_rsrc_t kc, ks, vc, vs;
  int kcs, kss, vcs, vss;  // row strides in bytes
  int nblk;                // 32-key blocks of the sequence
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

template <int D>
__device__ __forceinline__ TileSrc make_tile_src(const PrefillArgs& a, int b, int hk) {
  TileSrc t;
  t.kcs = static_cast<int>(a.k.cs[2]);
  t.kss = static_cast<int>(a.k.ss[2]);
  t.vcs = static_cast<int>(a.v.cs[2]);
  t.vss = static_cast<int>(a.v.ss[2]);
  t.nblk = (a.Sk + 31) / 32;
  t.kc = rsrc_of(a.k.codes + b * a.k.cs[0] + hk * a.k.cs[1], static_cast<int64_t>(a.Sk) * t.kcs);
  t.ks = rsrc_of(a.k.scales + b * a.k.ss[0] + hk * a.k.ss[1], static_cast<int64_t>(a.Sk) * t.kss);
  t.vc = rsrc_of(a.v.codes + b * a.v.cs[0] + hk * a.v.cs[1], static_cast<int64_t>(D) * t.vcs);
  t.vs = rsrc_of(a.v.scales + b * a.v.ss[0] + hk * a.v.ss[1], static_cast<int64_t>(D) * t.vss);
  return t;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Issue the direct HBM->LDS loads of a tile's K and V codes (this wave's
// share of the 1 KB loads) and fetch its share of the scale bytes into
// registers.  `wave` is wave-uniform (a scalar), so the LDS destinations are
// scalars and the trip counts static.  Whole offsets go in the per-lane
// operand, which is what the resource's range check covers.  V code blocks past the sequence read whatever lies
// next in the V resource (another channel's finite codes, or zeros past its
// end): those keys only meet P = 0.  V scale blocks are clamped to the last
// real block, so the scale applied to them is a real, finite one.
template <int D, int BC>
__device__ __forceinline__ void issue_tile(const TileSrc& src, int t0, uint8_t* stage, ScaleRegs<D, BC>& sr,
                                           int tid, int wave) {
  using C = Cfg<D, BC>;
  const int lane = tid & 63;
#pragma unroll
  for (int k = 0; k < (C::K_LOADS + 3) / 4; ++k) {
    const int i = wave + 4 * k;
    if (C::K_LOADS % 4 != 0 && i >= C::K_LOADS) break;
    const int o = i * 1024 + 16 * lane;
    const int r = o / C::KRB, pos = (o % C::KRB) / 16;
    const int chunk = pos ^ ((r / (256 / C::KRB)) % (C::KRB / 16));
    const int rt = (r & ~31) + sigma(r & 31);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.kc, (lds_ptr_t)(stage + i * 1024), 16,
                                             static_cast<uint32_t>((t0 + rt) * src.kcs + chunk * 16), 0, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < (C::V_LOADS + 3) / 4; ++k) {
    const int i = wave + 4 * k;
    if (C::V_LOADS % 4 != 0 && i >= C::V_LOADS) break;
    const int o = i * 1024 + 16 * lane;
    const int d = o / C::VRB, pos = (o % C::VRB) / 16;
    const int chunk = pos ^ ((d / (256 / C::VRB)) % (C::VRB / 16));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.vc, (lds_ptr_t)(stage + C::OFF_V + i * 1024), 16,
                                             static_cast<uint32_t>(d * src.vcs + (t0 / 32 + chunk) * 16), 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < C::IKS; ++i) {
    const int e = (tid + kThreads * i) % C::NKS;
    const int r = e / C::KSROW, part = e % C::KSROW;
    const int rt = (r & ~31) + sigma(r & 31);
    sr.ks[i] = __builtin_amdgcn_raw_buffer_load_b8(src.ks, static_cast<uint32_t>((t0 + rt) * src.kss + part), 0, 0);
  }
#pragma unroll
  for (int i = 0; i < C::IVS; ++i) {
    const int e = (tid + kThreads * i) % C::NVS;
    const int d = e / C::VSROW, part = e % C::VSROW;
    int blk = t0 / 32 + part;
    blk = blk < src.nblk ? blk : src.nblk - 1;
    sr.vs[i] = __builtin_amdgcn_raw_buffer_load_b8(src.vs, static_cast<uint32_t>(d * src.vss + blk), 0, 0);
  }
}

// LDS positions (inside a stage) of the scale bytes a thread fetched: K
// byte e is (tile row r = e / KSROW, chunk c = e % KSROW), used by lane
// (row r % 32, half c % 2) in the MFMA of key block r / 32 and 64-deep chunk
// c / 2.  V byte e is (channel d = e / VSROW, key block k = e % VSROW), used
// by lane (row d % 32, half k % 2) in the MFMA of channel tile d / 32 and
// key-block pair k / 2.
template <int D, int BC>
__device__ __forceinline__ int ks_pos(int e) {
  using C = Cfg<D, BC>;
  const int r = e / C::KSROW, c = e % C::KSROW, kb = r / 32;
  return C::OFF_KS + (kb / C::KPD) * 256 + (c % 2) * 128 + (r % 32) * 4 + (kb % C::KPD) * C::DC + c / 2;
}
template <int D, int BC>
__device__ __forceinline__ int vs_pos(int e) {
  using C = Cfg<D, BC>;
  const int d = e / C::VSROW, k = e % C::VSROW, dt = d / 32;
  return C::OFF_VS + (dt / C::DPD) * 256 + (k % 2) * 128 + (d % 32) * 4 + (dt % C::DPD) * (C::KB / 2) + k / 2;
}

template <int D, int BC>
__device__ __forceinline__ void store_scales(const ScaleRegs<D, BC>& sr, uint8_t* stage, int tid) {
  using C = Cfg<D, BC>;
#pragma unroll
  for (int i = 0; i < C::IKS; ++i) {
    const int e = tid + kThreads * i;
    if (e < C::NKS) stage[ks_pos<D, BC>(e)] = sr.ks[i];
  }
#pragma unroll
  for (int i = 0; i < C::IVS; ++i) {
    const int e = tid + kThreads * i;
    if (e < C::NVS) stage[vs_pos<D, BC>(e)] = sr.vs[i];
  }
}

// E8M0 scale of a P block maximum pmax in [0, 1], as the float 2^(b-127):
// b = floor(log2 pmax) - 2 (OCP), one more when the significand exceeds
// thr (UOS), clamped below at 1 so the convert's scale stays a normal float
// (zero and tiny maxima take byte 1; their codes are 0 either way).  In
// floats: the power of two at or below pmax, times 1/4, times 2 under the
// UOS condition, at least 2^-126.  Subnormal intermediates are kept (the
// code is built without denormal flushing), so this equals the integer
// rule exactly.  pmax <= 1 keeps the byte below 126.
__device__ __forceinline__ float p_block_scale(float pmax, bool uos, int thr) {
  const uint32_t bits = __float_as_uint(pmax);
  float s = __uint_as_float(bits & 0x7F800000u) * 0.25f;
  if (uos) s = static_cast<int>(bits & 0x7FFFFFu) > thr ? s * 2.0f : s;
  return fmaxf(s, 0x1p-126f);
}

// Workgroup -> (query block, batch, query head).  Consecutive workgroups go
// to different XCDs (round robin over 8); the mapping gives each XCD whole
// (batch, KV head) pairs so their K/V stay in that XCD's L2, and issues the
// longest causal query blocks first.  Without a causal mask every block is
// equally long, and an XCD runs the blocks of one (batch, KV head) pair
// after another (query block fastest): its resident workgroups then share
// one pair's K/V in L2, where with the pairs interleaved each block read
// its pair's K/V again from beyond the L2 once the XCD's pairs together
// outgrew it.
__device__ __forceinline__ void map_block(const PrefillArgs& a, bool causal, int& qb, int& b, int& hq) {
  const int G = a.Hq / a.Hkv;
  const int pairs = a.B * a.Hkv;
  const int bid = blockIdx.x;
  int qi, pair, g;
  if (pairs % 8 == 0) {
    const int slot = bid % 8, rank = bid / 8;
    const int per = pairs / 8;
    if (causal) {
      qi = rank / (per * G);
      const int rem = rank % (per * G);
      pair = slot * per + rem / G;
      g = rem % G;
    } else {
      qi = rank % a.n_qblk;
      const int rem = rank / a.n_qblk;
      pair = slot * per + rem / G;
      g = rem % G;
    }
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

// LDS of one bf16 chunk of the hybrid pass (two of them, alternating): 32 K
// rows, 32 V rows (row stride padded by 16 bytes) and the 32 key positions.
template <int D>
struct HybCfg {
  static constexpr int ROW = 2 * D + 16;
  static constexpr int V_OFF = 32 * ROW;
  static constexpr int POS_OFF = 64 * ROW;
  static constexpr int BYTES = POS_OFF + 32 * 4;
  static constexpr int PB = 2 * D / 8;  // bytes of a row staged by each of 8 threads
};

// Key of the 32-key chunk held by MFMA row i of the bf16 S^T product: bits 2
// and 3 of i swapped, so that lane half h, register r of the result is key
// 16 (r / 8) + 8 h + r % 8 -- the B operand layout of the PV k-steps.
__device__ __forceinline__ int hyb_key(int i) { return (i & 0x13) | ((i & 4) << 1) | ((i & 8) >> 1); }

__device__ __forceinline__ v16f mfma32_bf16(v4i a, v4i b, v16f c) {
  typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0,
                                                  0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 x = static_cast<__bf16>(lo), y = static_cast<__bf16>(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, x)) | (uint32_t(__builtin_bit_cast(uint16_t, y)) << 16);
}

// Paired causal schedule (a.paired): one round of workgroups, each running
// two query blocks of one query head in turn.  On this GPU the workgroups
// of a CU are issued oldest first: the one dispatched first (the lower
// half of the grid when the grid fills every CU twice) runs about 1.8x
// faster than its neighbour.  So the first half takes the heavier pairs and
// the second half the rest, and the two on a CU finish together instead of
// one running alone at the end.  With N query blocks per head (N % 4 == 0)
// and c = a.pair_c, the heavy pairs are (N-1-i, c+i), i < N/4; the light
// pairs take the remaining blocks smallest with largest.  At c = N/4 every
// heavy pair holds 5N/4 + 1 tiles and every light pair 3N/4 + 1.  Each XCD
// (bid % 8) works on whole KV heads, as in map_block.  qb2 = -1: no second
// block.
__device__ __forceinline__ void map_pair(const PrefillArgs& a, int& qb1, int& qb2, int& b, int& hq) {
  const int G = a.Hq / a.Hkv;
  const int N = a.n_qblk, N4 = N / 4;
  const int per = (a.B * a.Hkv) / 8;          // (batch, KV head) pairs per XCD
  const int slot = blockIdx.x % 8, local = blockIdx.x / 8;
  const int heavy = per * G * N4;             // heavy workgroups per XCD
  const bool is_heavy = local < heavy;
  const int l2 = is_heavy ? local : local - heavy;
  const int head = l2 / N4, m = l2 % N4;      // query head of the XCD's range, pair index
  const int pair = slot * per + head / G;
  b = pair / a.Hkv;
  hq = (pair % a.Hkv) * G + head % G;
  if (is_heavy) {
    qb1 = N - 1 - m;
    qb2 = a.pair_c + m;
  } else {
    // The remaining blocks {0..c-1} and {c+N/4 .. 3N/4-1}, r-th in order.
    auto rest = [&](int r) { return r < a.pair_c ? r : r + N4; };
    qb1 = rest(N / 2 - 1 - m);
    qb2 = rest(m);
  }
}

template <int D, int BC, bool CAUSAL, bool LQ, bool PUOS, bool HYB>
__device__ __forceinline__ void prefill_item(const PrefillArgs& a, const int qb, const int b, const int hq,
                                             uint8_t* __restrict__ smem, uint32_t* __restrict__ selmap) {
  using C = Cfg<D, BC>;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, j = lane & 31, hh = lane >> 5;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int hk = hq / (a.Hq / a.Hkv);
  const int q0 = qb * kBR;
  const int my_q = q0 + wave_s * 32 + j;
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

  // The 4-bit path sees key t of query row i iff t <= i - shift (causal);
  // the hybrid kernel shifts the limit by its window.
  const int shift = HYB ? a.window : 0;
  const int last_q = (q0 + kBR - 1 < a.Sq - 1) ? q0 + kBR - 1 : a.Sq - 1;
  const int nt = HYB ? (last_q - shift < 0 ? 0 : (last_q - shift) / BC + 1)
                     : (CAUSAL ? last_q / BC + 1 : (a.Sk + BC - 1) / BC);
  const int wave_last_q = (q0 + wave_s * 32 + 31 < a.Sq - 1) ? q0 + wave_s * 32 + 31 : a.Sq - 1;
  const int my_nt = HYB ? (wave_last_q - shift < 0 ? 0 : (wave_last_q - shift) / BC + 1)
                        : (CAUSAL ? wave_last_q / BC + 1 : nt);
  const int wave_first_q = q0 + wave_s * 32;
  // Smallest and largest query row of this wave (padding rows repeat Sq - 1),
  // moved down by the shift.
  const int lo_q = (wave_first_q < a.Sq - 1 ? wave_first_q : a.Sq - 1) - shift;
  const int hi_q = wave_last_q - shift;

  // E2M1 ones for the normaliser: a 16x16x128 A operand whose rows 0-7 sum
  // the k-groups of lanes 0-15 and 32-47 (queries 0-15 of both key blocks)
  // and rows 8-15 those of lanes 16-31 and 48-63 (queries 16-31).
  const int one_r = lane & 15, one_kg = lane >> 4;
  const bool one_on = (one_r < 8) ? (one_kg == 0 || one_kg == 2) : (one_kg == 1 || one_kg == 3);
  const int onev = one_on ? 0x22222222 : 0;
  const v4i ones = {onev, onev, onev, onev};
  const int l_query = (lane & 15) + 16 * (lane >> 5);

  // Per-lane LDS byte offsets inside a stage.  The XOR swizzle of a row
  // depends only on the row's position within its 32-row group, so key block
  // kb / channel tile dt add the compile-time offsets kb*32*KRB / dt*32*VRB.
  int koff[C::DC], voff[C::KB / 2];
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) koff[dc] = j * C::KRB + 16 * swz<C::KRB>(j, 2 * dc + hh);
#pragma unroll
  for (int pp = 0; pp < C::KB / 2; ++pp) voff[pp] = C::OFF_V + j * C::VRB + 16 * swz<C::VRB>(j, 2 * pp + hh);
  const int ksoff = C::OFF_KS + hh * 128 + j * 4, vsoff = C::OFF_VS + hh * 128 + j * 4;
  // UOS (read only when PUOS): a P block maximum whose significand 1.m
  // exceeds qmax/4, a value in (1, 2), takes the next scale up.
  const int p_thr = static_cast<int>(__float_as_uint(a.p_qmax_quarter) & 0x7FFFFFu);

  float m = -__builtin_huge_valf();
  float lsum = 0.0f;  // baseline normaliser (sum of unquantised P~)
  v16f O[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) O[dt] = v16f{};
  v4f L = v4f{0, 0, 0, 0};

  if constexpr (HYB) {
    // Bitmap of the selected keys below the workgroup's last row (the 4-bit
    // tiles never reach further).
    const int nw = (last_q + 1 + 31) >> 5;
    for (int w = tid; w < nw; w += kThreads) selmap[w] = 0u;
    __syncthreads();
    const int pair = b * a.Hkv + hk;
    int ns = a.max_sel > 0 ? a.sel_n[pair] : 0;
    ns = ns < 0 ? 0 : (ns > a.max_sel ? a.max_sel : ns);
    const int32_t* ix = a.sel_idx + static_cast<int64_t>(pair) * a.max_sel;
    for (int i = tid; i < ns; i += kThreads) {
      const int t = ix[i];
      if (t >= 0 && t <= last_q) atomicOr(&selmap[t >> 5], 1u << (t & 31));
    }
  }

  const TileSrc src = make_tile_src<D>(a, b, hk);
  ScaleRegs<D, BC> sr;
  if (!HYB || nt > 0) {
    issue_tile<D, BC>(src, 0, smem, sr, tid, wave_s);
    store_scales<D, BC>(sr, smem, tid);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // One tile step (prefetch the next tile, this tile's body, hand over the
  // stage), compiled twice: FULL, for the leading tiles whose key blocks are
  // all visible to every row of the workgroup (no per-block tests or
  // branches), and the general form for the rest (the diagonal and tail
  // tiles).  The two run as consecutive loops.
  auto step = [&](const int jt, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int t0 = jt * BC;
    uint8_t* next = smem + ((jt + 1) & 1) * C::STAGE;
    if (jt + 1 < nt) issue_tile<D, BC>(src, t0 + BC, next, sr, tid, wave_s);
    auto tile = [&]() {
      const uint8_t* base = smem + (jt & 1) * C::STAGE;
      // Selected-key bitmap words of the tile's key blocks, read with the
      // operands and made scalar after them, so the wait for them leaves
      // those loads in flight.
      uint32_t selw[C::KB];
      if constexpr (HYB) {
        if constexpr (C::KB >= 4) {
#pragma unroll
          for (int q4 = 0; q4 < C::KB / 4; ++q4) {
            const v4i w4 = *reinterpret_cast<const v4i*>(selmap + (t0 >> 5) + 4 * q4);
#pragma unroll
            for (int e = 0; e < 4; ++e) selw[4 * q4 + e] = static_cast<uint32_t>(w4[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < C::KB; ++e) selw[e] = selmap[(t0 >> 5) + e];
        }
      }

      // Key block kb of this tile is [tb, tb + 32), tb = t0 + 32 kb.  Against
      // this wave's 32 query rows it is fully visible, empty (skipped) or
      // needs the per-element mask (the diagonal block, or keys past Sk).
      auto blk_empty = [&](int kb) {
        const int tb = t0 + kb * 32;
        return !FULL && (tb >= a.Sk || (CAUSAL && tb > hi_q));
      };
      auto blk_masked = [&](int kb) {
        const int tb = t0 + kb * 32;
        return !FULL && (tb + 32 > a.Sk || (CAUSAL && tb + 31 > lo_q));
      };
      // Logits of block kb: S^T = K_hat Q_hat^T over the D/64 chunks.
      // Every K operand and scale word of the tile is read before the first
      // logit MFMA (the scheduling barrier keeps the reads together), so the
      // tile pays the LDS latency once instead of once per key block.
      v4i kop[C::KB][C::DC];
      int ksws[(C::KB + C::KPD - 1) / C::KPD];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        if (blk_empty(kb)) continue;
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc)
          kop[kb][dc] = *reinterpret_cast<const v4i*>(base + koff[dc] + kb * 32 * C::KRB);
      }
#pragma unroll
      for (int g = 0; g < (C::KB + C::KPD - 1) / C::KPD; ++g)
        ksws[g] = *reinterpret_cast<const int*>(base + ksoff + g * 256);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (HYB) {
#pragma unroll
        for (int e = 0; e < C::KB; ++e) selw[e] = __builtin_amdgcn_readfirstlane(selw[e]);
      }
      auto logits = [&](int kb) -> v16f {
        const v4i* aop = kop[kb];
        const int ksw = ksws[kb / C::KPD];
        v16f acc = v16f{};
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc)
          acc = mfma32_fp4_sel(aop[dc], qop[dc], acc, ksw, (kb % C::KPD) * C::DC + dc, qsc[dc]);
        if (blk_masked(kb)) {
          const int qlim = CAUSAL ? qrow - shift : 0x7FFFFFFF;
#pragma unroll
          for (int r2 = 0; r2 < 16; ++r2) {
            const int t = t0 + kb * 32 + 16 * hh + r2;
            if (t > qlim || t >= a.Sk) acc[r2] = -__builtin_huge_valf();
          }
        }
        if constexpr (HYB) {
          // Selected keys go to the bf16 pass.  Lane half hh holds keys
          // 16 hh + r2 of the block, so the select of register r2 takes its
          // lane mask from bits r2 (lanes 0-31) and 16 + r2 (lanes 32-63) of
          // the block's bitmap word, built in scalar registers.
          const uint32_t w = selw[kb];
          if (w != 0u) {
            const float ninf = -__builtin_huge_valf();
#pragma unroll
            for (int r2 = 0; r2 < 16; ++r2) {
              const uint32_t lo = static_cast<uint32_t>(static_cast<int32_t>(w << (31 - r2)) >> 31);
              const uint32_t hi = static_cast<uint32_t>(static_cast<int32_t>(w << (15 - r2)) >> 31);
              const uint64_t lm = static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
              acc[r2] = __builtin_amdgcn_inverse_ballot_w64(lm) ? ninf : acc[r2];
            }
          }
        }
        return acc;
      };

      // ---- logits of the tile, their block maxima, the running maximum.
      // The logits stay in registers (64 per lane) for the exponentials.
      v16f S[C::KB];
      float bm[C::KB];
      float tmax = -__builtin_huge_valf();
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        bm[kb] = -__builtin_huge_valf();
        if (blk_empty(kb)) continue;
        S[kb] = logits(kb);
        const v16f& x16 = S[kb];
        // Max of the 16 values as a depth-3 tree of max3 (no serial chain).
        const float m0 = fmaxf(fmaxf(x16[0], x16[1]), x16[2]), m1 = fmaxf(fmaxf(x16[3], x16[4]), x16[5]);
        const float m2 = fmaxf(fmaxf(x16[6], x16[7]), x16[8]), m3 = fmaxf(fmaxf(x16[9], x16[10]), x16[11]);
        const float m4 = fmaxf(fmaxf(x16[12], x16[13]), x16[14]);
        float x = fmaxf(fmaxf(fmaxf(m0, m1), m2), fmaxf(fmaxf(m3, m4), x16[15]));
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        bm[kb] = x;
        tmax = fmaxf(tmax, x);
      }
      const float m_new = fmaxf(m, tmax);
      // The hybrid kernel can meet rows with no 4-bit key yet (m_new = -inf):
      // their state stays zero.
      const bool none = HYB && m_new == -__builtin_huge_valf();
      const float mref = none ? 0.0f : m_new;
      const float alpha = none ? 1.0f : fast_exp2((m - m_new) * a.c);
      const float mc = mref * a.c;

      // ---- rescale the accumulators (skipped when no row's maximum moved)
      if (__builtin_amdgcn_ballot_w64(m_new > m) != 0) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) O[dt] *= alpha;
        // L[0] of this lane is the normaliser of query l%16 + 16*(l/32),
        // whose factor lives in that query's lane.
        L[0] *= __shfl(alpha, l_query);
        if (!LQ) lsum *= alpha;
      }
      m = m_new;

      // ---- per pair of key blocks: P~ in place of the logits, its MXFP4
      // codes, then O^T += V_hat^T P_hat^T and l += ones^T P_hat^T.
#pragma unroll
      for (int pp = 0; pp < C::KB / 2; ++pp) {
        uint32_t code[2][2];
        int eb[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int kb = 2 * pp + h2;
          code[h2][0] = code[h2][1] = 0u;
          eb[h2] = 1;
          if (blk_empty(kb)) continue;
          v16f& p = S[kb];
          const float scl = p_block_scale(fast_exp2((bm[kb] - mref) * a.c), PUOS, p_thr);
          eb[h2] = static_cast<int>(__float_as_uint(scl) >> 23);
#pragma unroll
          for (int r = 0; r < 16; ++r) p[r] = fast_exp2(__builtin_fmaf(p[r], a.c, -mc));
          if constexpr (!LQ) {
            float ts = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) ts += p[r];
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ts), __float_as_uint(ts), false, false);
            lsum += __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
          }
          // Each word's chain of converts starts from the register of its
          // first input, which is dead after that convert (every byte is
          // overwritten), so no placeholder value has to be copied in.
          uint32_t w0 = __float_as_uint(p[0]), w1 = __float_as_uint(p[8]);
          w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, p[0], p[1], scl, 0);
          w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, p[8], p[9], scl, 0);
          w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, p[2], p[3], scl, 1);
          w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, p[10], p[11], scl, 1);
          w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, p[4], p[5], scl, 2);
          w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, p[12], p[13], scl, 2);
          w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, p[6], p[7], scl, 3);
          w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, p[14], p[15], scl, 3);
          code[h2][0] = w0;
          code[h2][1] = w1;
        }
        if (blk_empty(2 * pp) && blk_empty(2 * pp + 1)) continue;
        const auto r0 = __builtin_amdgcn_permlane32_swap(code[0][0], code[1][0], false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(code[0][1], code[1][1], false, false);
        const v4i bop = {(int)r0[0], (int)r1[0], (int)r0[1], (int)r1[1]};
        const int bsc = hh ? eb[1] : eb[0];
        v4i aop[C::DT];
        int sa[C::DT];
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
          aop[dt] = *reinterpret_cast<const v4i*>(base + voff[pp] + dt * 32 * C::VRB);
          sa[dt] = *reinterpret_cast<const int*>(base + vsoff + (dt / C::DPD) * 256);
        }
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
          O[dt] = mfma32_fp4_sel(aop[dt], bop, O[dt], sa[dt], (dt % C::DPD) * (C::KB / 2) + pp, bsc);
        L = mfma16_fp4(ones, bop, L, a.one_scale, bsc);
      }
    };
    if (FULL || jt < my_nt) tile();
    if (jt + 1 < nt) store_scales<D, BC>(sr, next, tid);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // Leading tiles fully visible to every row of the workgroup: keys below
  // the first query row (causal) and below Sk.
  const int full_keys = HYB ? (q0 + 1 - shift < 0 ? 0 : q0 + 1 - shift)
                            : (CAUSAL ? (q0 + 1 < a.Sk ? q0 + 1 : a.Sk) : a.Sk);
  const int n_full = full_keys / BC < nt ? full_keys / BC : nt;
  int jt = 0;
  for (; jt < n_full; ++jt) step(jt, std::true_type{});
  for (; jt < nt; ++jt) step(jt, std::false_type{});

  // ---- hybrid: the bf16 keys, after every 4-bit tile, in chunks of 32.
  float lb = 0.0f;  // their share of the normaliser (unquantised P)
  if constexpr (HYB) {
    using H = HybCfg<D>;
    const int W = a.window;
    const int pair = b * a.Hkv + hk;
    // Chunks: the workgroup's window keys [w_lo, last_q], then the selected
    // list up to the last entry some row uses (entries are ascending).
    const int w_lo = q0 - W + 1 > 0 ? q0 - W + 1 : 0;
    const int n_wc = W > 0 ? (last_q - w_lo + 32) / 32 : 0;
    int ns = a.max_sel > 0 ? a.sel_n[pair] : 0;
    ns = ns < 0 ? 0 : (ns > a.max_sel ? a.max_sel : ns);
    const int32_t* ix = a.sel_idx + static_cast<int64_t>(pair) * a.max_sel;
    const int sel_lim = last_q - W;  // a selected key above this is in the window of every row
    // Chunks of the list whose first entry some row uses: a prefix, since
    // the entries ascend, counted 64 chunks per ballot.
    const int nct = (ns + 31) / 32;
    int n_sc = 0;
    for (int base = 0; base < nct; base += 64) {
      const int l = base + lane;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(l < nct && ix[32 * l] <= sel_lim);
      n_sc += __builtin_popcountll(bal);
      if (bal != ~0ull) break;
    }
    const int n_ch = n_wc + n_sc;
    // B operand of S^T: bf16 query row qrow, channels 16 st + 8 hh .. +7.
    v4i qb[D / 16];
    if (n_ch > 0) {
      const uint16_t* qsrc = a.qf + ((static_cast<int64_t>(b) * a.Hq + hq) * a.Sq + qrow) * D + 8 * hh;
#pragma unroll
      for (int st = 0; st < D / 16; ++st) qb[st] = *reinterpret_cast<const v4i*>(qsrc + 16 * st);
    }
    const int slot = tid >> 3, part = tid & 7;
    const uint16_t* kbase = a.kf + static_cast<int64_t>(pair) * a.Sk * D;
    const uint16_t* vbase = a.vf + static_cast<int64_t>(pair) * a.Sk * D;
    const int g16 = lane >> 4, s16 = lane & 15;
    // This wave's rows (unshifted): a chunk none of them uses is skipped.
    const int wq0 = lo_q + shift, wq1 = wave_last_q;

    // Key position of this thread's slot in chunk ch (-1: empty slot).  A
    // selected chunk's list entry is loaded one chunk ahead (sel_raw) and
    // checked only when used, so the load stays in flight meanwhile.
    auto sel_raw = [&](int ch) {
      const int i = 32 * (ch - n_wc) + slot;
      return i < ns ? ix[i] : -1;
    };
    auto slot_pos = [&](int ch, int raw) {
      if (ch < n_wc) {
        const int t = w_lo + 32 * ch + slot;
        return t > last_q ? -1 : t;
      }
      return (raw < 0 || raw > sel_lim) ? -1 : raw;
    };
    // Rows of the next chunk travel in registers while the current one is
    // computed (two LDS buffers, one barrier per chunk); the positions of the
    // chunk after that are loaded one step earlier still.
    v4i kv[H::PB / 16], vv[H::PB / 16];
    int tpos = -1, tnext = -1;
    auto fetch = [&]() {
#pragma unroll
      for (int u = 0; u < H::PB / 16; ++u) {
        kv[u] = v4i{0, 0, 0, 0};
        vv[u] = v4i{0, 0, 0, 0};
      }
      if (tpos >= 0) {
        const uint8_t* ks = reinterpret_cast<const uint8_t*>(kbase + static_cast<int64_t>(tpos) * D) + part * H::PB;
        const uint8_t* vs = reinterpret_cast<const uint8_t*>(vbase + static_cast<int64_t>(tpos) * D) + part * H::PB;
#pragma unroll
        for (int u = 0; u < H::PB / 16; ++u) {
          kv[u] = *reinterpret_cast<const v4i*>(ks + 16 * u);
          vv[u] = *reinterpret_cast<const v4i*>(vs + 16 * u);
        }
      }
    };
    if (n_ch > 0) {
      tpos = slot_pos(0, n_wc == 0 ? sel_raw(0) : -1);
      fetch();
    }
    if (n_ch > 1 && n_wc <= 1) tnext = sel_raw(1);
    for (int ch = 0; ch < n_ch; ++ch) {
      uint8_t* kl = smem + (ch & 1) * H::BYTES;
      uint8_t* vl = kl + H::V_OFF;
      int* pos = reinterpret_cast<int*>(kl + H::POS_OFF);
#pragma unroll
      for (int u = 0; u < H::PB / 16; ++u) {
        *reinterpret_cast<v4i*>(kl + slot * H::ROW + part * H::PB + 16 * u) = kv[u];
        *reinterpret_cast<v4i*>(vl + slot * H::ROW + part * H::PB + 16 * u) = vv[u];
      }
      if (part == 0) pos[slot] = tpos;
      __syncthreads();
      if (ch + 1 < n_ch) {
        tpos = slot_pos(ch + 1, tnext);
        fetch();
      }
      if (ch + 2 < n_ch && ch + 2 >= n_wc) tnext = sel_raw(ch + 2);

      // Skip a chunk no row of this wave uses; drop the per-element mask
      // when every row uses every key of it.
      const bool win_chunk = ch < n_wc;
      bool used, every;
      if (win_chunk) {
        const int c0 = w_lo + 32 * ch;
        used = c0 <= wq1 && c0 + 31 > wq0 - W;
        every = c0 > wq1 - W && c0 + 31 <= wq0;
      } else {
        // Slot 0 holds the smallest entry, slot 31 the largest (-1: empty).
        const int f = pos[0], lst = pos[31];
        used = f < 0 || f <= wq1 - W;
        every = f >= 0 && lst >= 0 && lst <= wq0 - W;
      }
      if (!used) continue;

      // S^T = K Q^T: lane (query j, half hh), register r is key 16(r/8) + 8hh + r%8.
      const uint8_t* krow = kl + hyb_key(j) * H::ROW + 16 * hh;
      v16f sc = v16f{};
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
        sc = mfma32_bf16(*reinterpret_cast<const v4i*>(krow + 32 * st), qb[st], sc);
      const v4i pa = *reinterpret_cast<const v4i*>(pos + 8 * hh);
      const v4i pb = *reinterpret_cast<const v4i*>(pos + 8 * hh + 4);
      const v4i pc = *reinterpret_cast<const v4i*>(pos + 16 + 8 * hh);
      const v4i pd = *reinterpret_cast<const v4i*>(pos + 16 + 8 * hh + 4);
      const int tk[16] = {pa[0], pa[1], pa[2], pa[3], pb[0], pb[1], pb[2], pb[3],
                          pc[0], pc[1], pc[2], pc[3], pd[0], pd[1], pd[2], pd[3]};
      if (!every) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tt = tk[r];
          const bool ok = tt >= 0 && tt <= qrow && (win_chunk ? tt > qrow - W : tt <= qrow - W);
          if (!ok) sc[r] = -__builtin_huge_valf();
        }
      }
      float mx = -__builtin_huge_valf();
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float m_new = fmaxf(m, mx);
      const bool none = m_new == -__builtin_huge_valf();
      const float alpha = none ? 1.0f : fast_exp2((m - m_new) * a.c);
      const float mc = none ? 0.0f : m_new * a.c;
      float pv[16];
      float ps = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pv[r] = fast_exp2(__builtin_fmaf(sc[r], a.c, -mc));
        ps += pv[r];
      }
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps), __float_as_uint(ps), false, false);
        ps = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      if (__builtin_amdgcn_ballot_w64(m_new > m) != 0) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) O[dt] *= alpha;
        L[0] *= __shfl(alpha, l_query);
        if (!LQ) lsum *= alpha;
      }
      lb = lb * alpha + ps;
      m = m_new;

      // P^T as hi + lo bf16 B operands, k-step st = keys 16 st + 8 hh .. +7.
      v4i bhi[2], blo[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        uint32_t h4[4], l4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = pv[8 * st + 2 * i], x1 = pv[8 * st + 2 * i + 1];
          h4[i] = pack_bf16x2(x0, x1);
          l4[i] = pack_bf16x2(x0 - __uint_as_float(h4[i] << 16), x1 - __uint_as_float(h4[i] & 0xFFFF0000u));
        }
        bhi[st] = v4i{(int)h4[0], (int)h4[1], (int)h4[2], (int)h4[3]};
        blo[st] = v4i{(int)l4[0], (int)l4[1], (int)l4[2], (int)l4[3]};
      }
      // O^T += V^T P^T.  The A operand of lane (channel 32 dt + lane % 32,
      // half hh) is V[16 st + 8 hh + 0..7][channel], read with the LDS
      // transpose load: in each 16-lane group, lane 4a + b receives element
      // b of the 8-byte reads of lanes a, a + 4, a + 8, a + 12, so lane s16
      // reads channels 4 (s16 % 4) .. +3 of its group's 16 at key row
      // s16 / 4 (then 4 rows on).
      typedef short v4s __attribute__((ext_vector_type(4)));
      typedef int v2i_t __attribute__((ext_vector_type(2)));
      typedef __attribute__((address_space(3))) v4s lds_v4s;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const uint8_t* src = vl + (16 * st + 8 * hh + (s16 >> 2)) * H::ROW +
                               2 * (32 * dt + 16 * (g16 & 1) + 4 * (s16 & 3));
          const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(src));
          const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(src + 4 * H::ROW));
          const v2i_t l2 = __builtin_bit_cast(v2i_t, lo), h2 = __builtin_bit_cast(v2i_t, hi);
          const v4i aop = {l2[0], l2[1], h2[0], h2[1]};
          O[dt] = mfma32_bf16(aop, bhi[st], O[dt]);
          O[dt] = mfma32_bf16(aop, blo[st], O[dt]);
        }
    }
  }

  // ---- finalise: out = O / l, lse = m * softmax_scale + ln l
  // The normaliser of query j sits in lane j (j < 16) or j + 16 (j >= 16).
  const float lq = __shfl(L[0], j < 16 ? j : j + 16);
  if (my_q >= a.Sq) return;
  const float l = (LQ ? lq : lsum) + (HYB ? lb : 0.0f);
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

template <int D, int BC, bool CAUSAL, bool LQ, bool PUOS, bool HYB>
__global__ __launch_bounds__(kThreads, (BC == 256 ? 1 : 2)) void prefill_kernel(PrefillArgs a) {
  using C = Cfg<D, BC>;
  static_assert(!HYB || CAUSAL, "the hybrid kernel is causal");
  constexpr int SMEM = (HYB && 2 * HybCfg<D>::BYTES > 2 * C::STAGE) ? 2 * HybCfg<D>::BYTES : 2 * C::STAGE;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  // Padded by 8 words: a tile reads the words of all its blocks at once
  // (those past the last row belong to empty blocks and are never used).
  __shared__ __attribute__((aligned(16))) uint32_t selmap[HYB ? kHybSelWords + 8 : 1];
  int qb1, qb2 = -1, b, hq;
  if (CAUSAL && a.paired) map_pair(a, qb1, qb2, b, hq);
  else map_block(a, CAUSAL, qb1, b, hq);
  prefill_item<D, BC, CAUSAL, LQ, PUOS, HYB>(a, qb1, b, hq, smem, selmap);
  if (qb2 >= 0) {
    // The first block's last tile step ended with a barrier; this one keeps
    // its output epilogue clear of the next block's LDS writes as well.
    __syncthreads();
    prefill_item<D, BC, CAUSAL, LQ, PUOS, HYB>(a, qb2, b, hq, smem, selmap);
  }
}

template <int D, int BC, bool PUOS>
static void launch_tp(const PrefillArgs& a, int causal, bool hyb, hipStream_t stream) {
  unsigned grid = static_cast<unsigned>(a.n_qblk) * a.B * a.Hq;
  if (a.paired) grid /= 2;
  const bool lq = a.l_from_quantized != 0;
  if (hyb && lq)
    hipLaunchKernelGGL((prefill_kernel<D, BC, true, true, PUOS, true>), dim3(grid), dim3(kThreads), 0, stream, a);
  else if (hyb)
    hipLaunchKernelGGL((prefill_kernel<D, BC, true, false, PUOS, true>), dim3(grid), dim3(kThreads), 0, stream, a);
  else if (causal && lq)
    hipLaunchKernelGGL((prefill_kernel<D, BC, true, true, PUOS, false>), dim3(grid), dim3(kThreads), 0, stream, a);
  else if (causal)
    hipLaunchKernelGGL((prefill_kernel<D, BC, true, false, PUOS, false>), dim3(grid), dim3(kThreads), 0, stream, a);
  else if (lq)
    hipLaunchKernelGGL((prefill_kernel<D, BC, false, true, PUOS, false>), dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, BC, false, false, PUOS, false>), dim3(grid), dim3(kThreads), 0, stream,
                       a);
}

template <int D, int BC>
static void launch_t(const PrefillArgs& a, int causal, bool hyb, hipStream_t stream) {
  if (a.p_uos) launch_tp<D, BC, true>(a, causal, hyb, stream);
  else launch_tp<D, BC, false>(a, causal, hyb, stream);
}

hipError_t launch_prefill(const PrefillArgs& a, int D, int kv_tile, int causal, hipStream_t stream) {
  if (a.n_qblk == 0) return hipSuccess;
  const bool hyb = a.hybrid != 0;  // the caller checked causal
  if (D == 128) {
    if (kv_tile == 64) launch_t<128, 64>(a, causal, hyb, stream);
    else if (kv_tile == 128) launch_t<128, 128>(a, causal, hyb, stream);
    else launch_t<128, 256>(a, causal, hyb, stream);
  } else {
    if (kv_tile == 64) launch_t<64, 64>(a, causal, hyb, stream);
    else if (kv_tile == 128) launch_t<64, 128>(a, causal, hyb, stream);
    else launch_t<64, 256>(a, causal, hyb, stream);
  }
  return hipGetLastError();
}

}  // namespace mxattn

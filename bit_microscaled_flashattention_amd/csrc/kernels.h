// Kernel argument blocks and launchers shared between the host dispatch
// (api.cpp) and the device sources.  Plain structs passed by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxattn {

struct QuantArgs {
  const void* x;
  int dtype;  // 0 f32, 1 f16, 2 bf16
  int64_t xs[3];
  const float* chan_scale;
  int uos;
  float qmax_quarter;
  int key_layout;
  int hadamard;         // rotate each head-dim row before quantising
  float rot_scale;      // float32(1 / sqrt(D))
  int64_t B, H, S, D;
  uint8_t* codes;
  uint8_t* scales;
  int64_t cs[3];
  int64_t ss[3];
  // Dual residual (head-dim blocks only): codes2/scales2 receive the MXFP4
  // of x - dequant(codes, scales); null when unused.
  uint8_t* codes2;
  uint8_t* scales2;
  int64_t cs2[3];
  int64_t ss2[3];
};

// bf16 hybrid rows per decode workgroup (one partial slot each), and the
// partial slots per (sequence, query head) the decode merge accepts.
constexpr int kBf16Rows = 512;
constexpr int kMaxSlots = 4096;

// Up to kMaxQuantJobs tensors quantised by one launch; start[i] is the first
// workgroup of job i and start[n] the grid size, gx[i] the workgroups along
// the sequence of one (batch, head) of job i.
constexpr int kMaxQuantJobs = 4;
// flat[i]: job i has fewer head-dim blocks per (batch, head) than one
// workgroup covers (a decode query, S = 1), so its workgroups run over the
// rows of all heads and batches in order instead of one head each.
struct QuantBatch {
  QuantArgs job[kMaxQuantJobs];
  int start[kMaxQuantJobs + 1];
  int gx[kMaxQuantJobs];
  int flat[kMaxQuantJobs];
  int n;
};

struct CalibArgs {
  const void* q;
  const void* k;
  int dtype;
  int hq, hkv;
  int64_t tokens;
  int dim;
  float* q_scale;
  float* k_scale;
};

// One MXFP4 operand as the kernels see it: base pointers and byte strides of
// the (batch, head, row) dimensions.
struct MxView {
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t cs[3];
  int64_t ss[3];
};

struct PrefillArgs {
  MxView q, k, v;
  void* out;
  float* lse;
  int out_dtype;
  int B, Hq, Hkv, Sq, Sk;
  float c;              // softmax_scale * log2(e)
  float softmax_scale;
  int p_uos;
  float p_qmax_quarter;
  int l_from_quantized;
  int n_qblk;           // query blocks of 128 rows
  int one_scale;        // 127, kept in a kernel argument so it stays a register value
  // hybrid (causal only): bf16 rows [B][H][S][D] contiguous, selected keys
  int hybrid;
  const uint16_t* qf;
  const uint16_t* kf;
  const uint16_t* vf;
  const int32_t* sel_idx;  // [B][Hkv][max_sel], ascending
  const int32_t* sel_n;    // [B][Hkv]
  int max_sel;
  int window;
  // Paired causal schedule: two query blocks per workgroup, heavier pairs
  // first (see map_pair); pair_c is the first block of the heavy pairs'
  // short halves.
  int paired;
  int pair_c;
};

// Longest sequence of the hybrid prefill: the selected-key bitmap of a
// workgroup lives in LDS (one bit per key).
constexpr int kHybMaxSeq = 65536;
constexpr int kHybSelWords = kHybMaxSeq / 32;

struct DecodeArgs {
  MxView q, k, v;
  MxView q2;            // residual query of a dual-residual split (when dual)
  int dual;
  const int32_t* ctx_len;
  int B, Hq, Hkv, Tcap;
  float c;
  float softmax_scale;
  int split_len, n_split;
  int n_bf16;           // partial slots of the bf16 hybrid set (0 without hybrid)
  float* part;          // [B][Hq][n_split+n_bf16][D+2] partial (O, m, l)
  float* out;
  float* lse;
  // hybrid
  int hybrid;
  const uint16_t* q_bf16;   // bf16 [B][Hq][D]: the hybrid set's query, and the source of q when q_fused
  int q_fused;              // q is encoded from q_bf16 inside the scan (OCP rule)
  const int32_t* idx;
  const int32_t* n_sel;
  int max_sel, window;
  const uint16_t* k_sel;
  const uint16_t* v_sel;
  const uint16_t* k_win;
  const uint16_t* v_win;
  // paged cache: k, v are pools [n_pages][Hkv][page_size][D]
  int paged;
  const int32_t* block_table;  // [B][max_pages]
  int max_pages, page_size, n_pages;
};

struct SelectArgs {
  MxView q, k;
  const int32_t* ctx_len;
  int B, Hq, Hkv, R, Tcap;
  float c;
  int window, rho_num, rho_den, max_sel;
  float* col_mass;
  float* stats;         // [B][Hq][R][nchunk+1][2] partial row max / sum (workspace)
  int chunk;            // keys per context chunk of the stats kernel (multiple of 128)
  int cm_keys;          // keys per column-mass workgroup (multiple of 128)
  int32_t* idx_out;
  int32_t* n_out;
};

struct GatherArgs {
  const uint16_t* k;    // bf16 [B][H][T][D], element strides ks / vs (D contiguous)
  const uint16_t* v;
  int64_t ks[3], vs[3];
  const int32_t* idx;   // [B][H][max_sel]
  const int32_t* n_sel; // [B][H]
  uint16_t* k_out;      // bf16 [B][H][max_sel][D]
  uint16_t* v_out;
  int B, H, T, D, max_sel;
};

hipError_t launch_quantize_batch(const QuantArgs* jobs, int n, hipStream_t stream);
hipError_t launch_smooth_calibrate(const CalibArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, int D, int kv_tile, int causal, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int D, hipStream_t stream);

// Built-in partial-slot scratch of mxattn_decode_noalloc (one copy per device).
constexpr size_t kDecodeScratchBytes = size_t{16} << 20;
// Device address of that scratch on the current device (looked up once per
// device, then cached).
hipError_t decode_scratch(void** ptr);
hipError_t launch_select(const SelectArgs& a, int D, hipStream_t stream);
hipError_t launch_gather_rows(const GatherArgs& a, hipStream_t stream);

}  // namespace mxattn

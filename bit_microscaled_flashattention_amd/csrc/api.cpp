// Host side of libmxattn.so: argument validation, workspace sizing, kernel
// dispatch, status strings.  Every check runs before any launch, so an error
// status leaves all outputs untouched.
//
// Debug environment variables:
//   MXATTN_SYNC=1               synchronise the stream after each launch and
//                               report device errors as MXATTN_ERR_HIP.
//   MXATTN_INJECT=<fn>:<code>   make entry point <fn> (e.g. "prefill") return
//                               status <code> without launching (tests of the
//                               callers' error handling).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/mxattn.h"
#include "kernels.h"

static_assert(MXATTN_MAX_QUANTIZE_JOBS == mxattn::kMaxQuantJobs, "batch size limits differ");
static_assert(MXATTN_DECODE_SCRATCH_BYTES == mxattn::kDecodeScratchBytes, "decode scratch sizes differ");

using namespace mxattn;

namespace {

thread_local std::string g_last_error;

mxattn_status_t fail(mxattn_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

mxattn_status_t ok() {
  g_last_error.clear();
  return MXATTN_OK;
}

bool injected(const char* fn, mxattn_status_t* st) {
  const char* env = getenv("MXATTN_INJECT");
  if (env == nullptr) return false;
  const char* colon = strchr(env, ':');
  if (colon == nullptr) return false;
  if (strncmp(env, fn, colon - env) != 0 || strlen(fn) != static_cast<size_t>(colon - env)) return false;
  *st = static_cast<mxattn_status_t>(atoi(colon + 1));
  g_last_error = std::string("injected failure in ") + fn;
  return true;
}

mxattn_status_t after_launch(hipError_t e, hipStream_t stream, const char* what) {
  if (e != hipSuccess) return fail(MXATTN_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  const char* sync = getenv("MXATTN_SYNC");
  if (sync != nullptr && sync[0] == '1') {
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(MXATTN_ERR_HIP, "%s: device error: %s", what, hipGetErrorString(e));
  }
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t key_blocks(int64_t s) { return (s + 31) / 32; }

// Shape / stride / alignment checks of one MXFP4 descriptor.
mxattn_status_t check_mx(const mxattn_mx_t* t, const char* name, int want_layout) {
  if (t == nullptr) return fail(MXATTN_ERR_INVALID_ARG, "%s: null descriptor", name);
  if (t->codes == nullptr || t->scales == nullptr) return fail(MXATTN_ERR_INVALID_ARG, "%s: null codes/scales", name);
  if (t->layout != MXATTN_LAYOUT_HD && t->layout != MXATTN_LAYOUT_KEY)
    return fail(MXATTN_ERR_INVALID_ARG, "%s: unknown layout %d", name, t->layout);
  if (want_layout >= 0 && t->layout != want_layout)
    return fail(MXATTN_ERR_UNSUPPORTED, "%s: layout must be %s", name, want_layout == 0 ? "HD" : "KEY");
  if (t->batch < 1 || t->heads < 1 || t->seq < 1)
    return fail(MXATTN_ERR_INVALID_ARG, "%s: empty shape [%lld,%lld,%lld,%lld]", name, (long long)t->batch,
                (long long)t->heads, (long long)t->seq, (long long)t->dim);
  if (t->dim != 64 && t->dim != 128) return fail(MXATTN_ERR_UNSUPPORTED, "%s: head_dim %lld not in {64,128}", name, (long long)t->dim);
  // Batch and heads index grid dimensions of some launches (the decode merge,
  // the selection kernels), which allow up to 65535; positions inside one
  // head are 32-bit in the kernels.
  if (t->batch > 65535 || t->heads > 65535 || t->seq > (int64_t{1} << 26))
    return fail(MXATTN_ERR_UNSUPPORTED, "%s: batch/heads above 65535 or seq above 2^26", name);
  if (!aligned16(t->codes)) return fail(MXATTN_ERR_INVALID_ARG, "%s: codes not 16-byte aligned", name);
  for (int i = 0; i < 3; ++i)
    if (t->code_stride[i] < 0 || t->code_stride[i] % 16 != 0 || t->scale_stride[i] < 0)
      return fail(MXATTN_ERR_INVALID_ARG, "%s: code strides must be non-negative multiples of 16", name);
  const int64_t row_codes = t->layout == MXATTN_LAYOUT_HD ? t->dim / 2 : key_blocks(t->seq) * 16;
  const int64_t row_scales = t->layout == MXATTN_LAYOUT_HD ? t->dim / 32 : key_blocks(t->seq);
  if (t->code_stride[2] < row_codes || t->scale_stride[2] < row_scales)
    return fail(MXATTN_ERR_INVALID_ARG, "%s: row stride smaller than a row", name);
  const int64_t rows = t->layout == MXATTN_LAYOUT_HD ? t->seq : t->dim;
  if (t->code_stride[1] < rows * t->code_stride[2] && t->heads > 1)
    return fail(MXATTN_ERR_INVALID_ARG, "%s: head stride overlaps rows", name);
  if (t->code_stride[0] < t->heads * t->code_stride[1] && t->batch > 1 && t->code_stride[1] > 0)
    return fail(MXATTN_ERR_INVALID_ARG, "%s: batch stride overlaps heads", name);
  return MXATTN_OK;
}

MxView view_of(const mxattn_mx_t* t) {
  MxView v;
  v.codes = t->codes;
  v.scales = t->scales;
  for (int i = 0; i < 3; ++i) {
    v.cs[i] = t->code_stride[i];
    v.ss[i] = t->scale_stride[i];
  }
  return v;
}

bool valid_qmax(float q) { return q > 4.0f && q < 8.0f; }

}  // namespace

extern "C" {

const char* mxattn_version(void) { return "mxattn 0.1 (gfx950)"; }

const char* mxattn_last_error(void) { return g_last_error.c_str(); }

const char* mxattn_status_string(mxattn_status_t s) {
  switch (s) {
    case MXATTN_OK: return "ok";
    case MXATTN_ERR_INVALID_ARG: return "invalid argument";
    case MXATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case MXATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case MXATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

// Validates one quantisation request and fills its kernel arguments.
static mxattn_status_t quantize_args(const void* x, mxattn_dtype_t x_dtype, const int64_t x_stride[3],
                                     const float* chan_scale, mxattn_scale_rule_t rule, float qmax,
                                     int32_t flags, const mxattn_mx_t* out, const char* name, QuantArgs* a) {
  mxattn_status_t st;
  if (x == nullptr || x_stride == nullptr) return fail(MXATTN_ERR_INVALID_ARG, "%s: null input", name);
  if (x_dtype != MXATTN_F32 && x_dtype != MXATTN_F16 && x_dtype != MXATTN_BF16)
    return fail(MXATTN_ERR_INVALID_ARG, "%s: unknown dtype %d", name, (int)x_dtype);
  if (rule != MXATTN_SCALE_OCP && rule != MXATTN_SCALE_UOS) return fail(MXATTN_ERR_INVALID_ARG, "%s: unknown rule", name);
  if (rule == MXATTN_SCALE_UOS && !valid_qmax(qmax))
    return fail(MXATTN_ERR_UNSUPPORTED, "%s: UOS qmax must lie in (4, 8)", name);
  if ((st = check_mx(out, name, -1)) != MXATTN_OK) return st;
  if ((flags & ~MXATTN_QUANT_HADAMARD) != 0) return fail(MXATTN_ERR_INVALID_ARG, "%s: unknown flags 0x%x", name, flags);
  if ((flags & MXATTN_QUANT_HADAMARD) && out->layout != MXATTN_LAYOUT_HD)
    return fail(MXATTN_ERR_UNSUPPORTED, "%s: the Hadamard rotation needs the HD layout", name);
  for (int i = 0; i < 3; ++i)
    if (x_stride[i] < 0) return fail(MXATTN_ERR_INVALID_ARG, "%s: negative input stride", name);
  // Rows are read 8 elements (16 or 32 bytes) at a time.
  const int esz = x_dtype == MXATTN_F32 ? 4 : 2;
  if ((reinterpret_cast<uintptr_t>(x) % 16) != 0 || (x_stride[0] * esz) % 16 != 0 || (x_stride[1] * esz) % 16 != 0 ||
      (x_stride[2] * esz) % 16 != 0)
    return fail(MXATTN_ERR_INVALID_ARG, "%s: input and its row strides must be 16-byte aligned", name);
  if (chan_scale != nullptr && (reinterpret_cast<uintptr_t>(chan_scale) % 16) != 0)
    return fail(MXATTN_ERR_INVALID_ARG, "%s: chan_scale must be 16-byte aligned", name);
  *a = QuantArgs{};
  a->x = x;
  a->dtype = x_dtype == MXATTN_F32 ? 0 : (x_dtype == MXATTN_F16 ? 1 : 2);
  for (int i = 0; i < 3; ++i) {
    a->xs[i] = x_stride[i];
    a->cs[i] = out->code_stride[i];
    a->ss[i] = out->scale_stride[i];
  }
  a->chan_scale = chan_scale;
  a->uos = rule == MXATTN_SCALE_UOS;
  a->qmax_quarter = qmax * 0.25f;
  a->key_layout = out->layout == MXATTN_LAYOUT_KEY;
  a->hadamard = (flags & MXATTN_QUANT_HADAMARD) != 0;
  a->rot_scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(out->dim)));
  a->B = out->batch;
  a->H = out->heads;
  a->S = out->seq;
  a->D = out->dim;
  a->codes = out->codes;
  a->scales = out->scales;
  return MXATTN_OK;
}

mxattn_status_t mxattn_quantize(const void* x, mxattn_dtype_t x_dtype, const int64_t x_stride[3],
                                const float* chan_scale, mxattn_scale_rule_t rule, float qmax, int32_t flags,
                                const mxattn_mx_t* out, mxattn_stream_t stream) {
  mxattn_status_t st;
  if (injected("quantize", &st)) return st;
  QuantArgs a;
  if ((st = quantize_args(x, x_dtype, x_stride, chan_scale, rule, qmax, flags, out, "quantize", &a)) != MXATTN_OK)
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(launch_quantize_batch(&a, 1, s), s, "quantize");
}

mxattn_status_t mxattn_quantize_dual(const void* x, mxattn_dtype_t x_dtype, const int64_t x_stride[3],
                                     const float* chan_scale, mxattn_scale_rule_t rule, float qmax, int32_t flags,
                                     const mxattn_mx_t* out, const mxattn_mx_t* out_res, mxattn_stream_t stream) {
  mxattn_status_t st;
  if (injected("quantize_dual", &st)) return st;
  QuantArgs a;
  if ((st = quantize_args(x, x_dtype, x_stride, chan_scale, rule, qmax, flags, out, "quantize_dual", &a)) !=
      MXATTN_OK)
    return st;
  if (out->layout != MXATTN_LAYOUT_HD) return fail(MXATTN_ERR_UNSUPPORTED, "quantize_dual: out must use the HD layout");
  if ((st = check_mx(out_res, "quantize_dual.out_res", MXATTN_LAYOUT_HD)) != MXATTN_OK) return st;
  if (out_res->batch != out->batch || out_res->heads != out->heads || out_res->seq != out->seq ||
      out_res->dim != out->dim)
    return fail(MXATTN_ERR_INVALID_ARG, "quantize_dual: out and out_res shapes differ");
  a.codes2 = out_res->codes;
  a.scales2 = out_res->scales;
  for (int i = 0; i < 3; ++i) {
    a.cs2[i] = out_res->code_stride[i];
    a.ss2[i] = out_res->scale_stride[i];
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(launch_quantize_batch(&a, 1, s), s, "quantize_dual");
}

mxattn_status_t mxattn_quantize_batch(const mxattn_quantize_job_t* jobs, int32_t n_jobs, mxattn_stream_t stream) {
  mxattn_status_t st;
  if (injected("quantize_batch", &st)) return st;
  if (jobs == nullptr) return fail(MXATTN_ERR_INVALID_ARG, "quantize_batch: null job list");
  if (n_jobs < 1 || n_jobs > MXATTN_MAX_QUANTIZE_JOBS)
    return fail(MXATTN_ERR_INVALID_ARG, "quantize_batch: n_jobs %d not in [1, %d]", (int)n_jobs, MXATTN_MAX_QUANTIZE_JOBS);
  QuantArgs a[MXATTN_MAX_QUANTIZE_JOBS];
  for (int i = 0; i < n_jobs; ++i) {
    char name[40];
    snprintf(name, sizeof(name), "quantize_batch.job[%d]", i);
    const mxattn_quantize_job_t& j = jobs[i];
    if ((st = quantize_args(j.x, j.x_dtype, j.x_stride, j.chan_scale, j.rule, j.qmax, j.flags, j.out, name, &a[i])) !=
        MXATTN_OK)
      return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(launch_quantize_batch(a, n_jobs, s), s, "quantize_batch");
}

mxattn_status_t mxattn_smooth_calibrate(const void* q_cal, const void* k_cal, mxattn_dtype_t dtype, int64_t hq,
                                        int64_t hkv, int64_t tokens, int64_t dim, float* q_scale, float* k_scale,
                                        mxattn_stream_t stream) {
  mxattn_status_t st;
  if (injected("smooth_calibrate", &st)) return st;
  if (!q_cal || !k_cal || !q_scale || !k_scale) return fail(MXATTN_ERR_INVALID_ARG, "smooth_calibrate: null pointer");
  if (dtype != MXATTN_F32 && dtype != MXATTN_F16 && dtype != MXATTN_BF16)
    return fail(MXATTN_ERR_INVALID_ARG, "smooth_calibrate: unknown dtype");
  if (hq < 1 || hkv < 1 || tokens < 1 || dim < 1) return fail(MXATTN_ERR_INVALID_ARG, "smooth_calibrate: empty shape");
  if (hq % hkv != 0) return fail(MXATTN_ERR_INVALID_ARG, "smooth_calibrate: Hq %% Hkv != 0");
  if (dim > 256) return fail(MXATTN_ERR_UNSUPPORTED, "smooth_calibrate: dim > 256");
  CalibArgs a{};
  a.q = q_cal;
  a.k = k_cal;
  a.dtype = dtype == MXATTN_F32 ? 0 : (dtype == MXATTN_F16 ? 1 : 2);
  a.hq = static_cast<int>(hq);
  a.hkv = static_cast<int>(hkv);
  a.tokens = tokens;
  a.dim = static_cast<int>(dim);
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(launch_smooth_calibrate(a, s), s, "smooth_calibrate");
}

// Compute units of the current device, read once per device (0 if unknown).
static int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

static mxattn_status_t prefill_common(const mxattn_mx_t* q, const mxattn_mx_t* k, const mxattn_mx_t* v,
                                      const mxattn_prefill_params_t* p, const mxattn_prefill_hybrid_t* hy,
                                      void* out, mxattn_dtype_t out_dtype, float* lse, mxattn_stream_t stream) {
  mxattn_status_t st;
  if ((st = check_mx(q, "prefill.q", MXATTN_LAYOUT_HD)) != MXATTN_OK) return st;
  if ((st = check_mx(k, "prefill.k", MXATTN_LAYOUT_HD)) != MXATTN_OK) return st;
  if ((st = check_mx(v, "prefill.v", MXATTN_LAYOUT_KEY)) != MXATTN_OK) return st;
  if (p == nullptr || out == nullptr) return fail(MXATTN_ERR_INVALID_ARG, "prefill: null params/out");
  if (q->dim != k->dim || k->dim != v->dim) return fail(MXATTN_ERR_INVALID_ARG, "prefill: head_dim mismatch");
  if (q->batch != k->batch || k->batch != v->batch) return fail(MXATTN_ERR_INVALID_ARG, "prefill: batch mismatch");
  if (k->heads != v->heads || k->seq != v->seq) return fail(MXATTN_ERR_INVALID_ARG, "prefill: K/V shape mismatch");
  if (q->heads % k->heads != 0) return fail(MXATTN_ERR_INVALID_ARG, "prefill: Hq %% Hkv != 0");
  if (p->causal && q->seq != k->seq) return fail(MXATTN_ERR_UNSUPPORTED, "prefill: causal needs Sq == Sk");
  const int kv_tile = p->kv_tile == 0 ? 128 : p->kv_tile;
  if (kv_tile != 64 && kv_tile != 128 && kv_tile != 256)
    return fail(MXATTN_ERR_UNSUPPORTED, "prefill: kv_tile %d not in {64,128,256}", kv_tile);
  if (p->p_rule != MXATTN_SCALE_OCP && p->p_rule != MXATTN_SCALE_UOS)
    return fail(MXATTN_ERR_INVALID_ARG, "prefill: unknown p_rule");
  if (p->p_rule == MXATTN_SCALE_UOS && !valid_qmax(p->p_qmax))
    return fail(MXATTN_ERR_UNSUPPORTED, "prefill: UOS p_qmax must lie in (4, 8)");
  if (out_dtype != MXATTN_F32 && out_dtype != MXATTN_F16 && out_dtype != MXATTN_BF16)
    return fail(MXATTN_ERR_INVALID_ARG, "prefill: unknown out dtype");
  if (!(p->softmax_scale >= 0.0f) || !std::isfinite(p->softmax_scale))
    return fail(MXATTN_ERR_INVALID_ARG, "prefill: softmax_scale must be finite and >= 0");
  if (!aligned16(out)) return fail(MXATTN_ERR_INVALID_ARG, "prefill: out not 16-byte aligned");
  if (hy != nullptr) {
    if (!p->causal) return fail(MXATTN_ERR_UNSUPPORTED, "prefill_hybrid: the hybrid prefill is causal");
    if (q->seq > kHybMaxSeq)
      return fail(MXATTN_ERR_UNSUPPORTED, "prefill_hybrid: sequence %lld above %d", (long long)q->seq, kHybMaxSeq);
    if (hy->q == nullptr || hy->k == nullptr || hy->v == nullptr)
      return fail(MXATTN_ERR_INVALID_ARG, "prefill_hybrid: null bf16 q/k/v");
    if (!aligned16(hy->q) || !aligned16(hy->k) || !aligned16(hy->v))
      return fail(MXATTN_ERR_INVALID_ARG, "prefill_hybrid: bf16 q/k/v not 16-byte aligned");
    if (hy->window < 0 || hy->max_sel < 0) return fail(MXATTN_ERR_INVALID_ARG, "prefill_hybrid: negative window/max_sel");
    if (hy->max_sel > 0 && (hy->idx == nullptr || hy->n_sel == nullptr))
      return fail(MXATTN_ERR_INVALID_ARG, "prefill_hybrid: null idx/n_sel with max_sel > 0");
  }
  const int64_t grid = ((q->seq + 127) / 128) * q->batch * q->heads;
  if (grid > 0x7FFFFFFF || q->seq > 0x7FFFFFFF || k->seq > 0x7FFFFFFF)
    return fail(MXATTN_ERR_UNSUPPORTED, "prefill: problem too large for one launch");
  // The kernel reads one (batch, KV head) of K and V through buffer resources
  // with 32-bit sizes and 32-bit offsets: K rows are visited up to the end of
  // the last 256-key tile, V channel rows up to 128 bytes past their last block.
  {
    const int64_t sk_pad = (k->seq + 255) / 256 * 256;
    if (sk_pad * k->code_stride[2] > 0x7FFFFFFF || sk_pad * k->scale_stride[2] > 0x7FFFFFFF ||
        v->dim * v->code_stride[2] + 256 > 0x7FFFFFFF || v->dim * v->scale_stride[2] > 0x7FFFFFFF)
      return fail(MXATTN_ERR_UNSUPPORTED, "prefill: one head of K or V must span less than 2 GiB");
  }
  PrefillArgs a{};
  a.q = view_of(q);
  a.k = view_of(k);
  a.v = view_of(v);
  a.out = out;
  a.lse = lse;
  a.out_dtype = out_dtype == MXATTN_F32 ? 0 : (out_dtype == MXATTN_F16 ? 1 : 2);
  a.B = static_cast<int>(q->batch);
  a.Hq = static_cast<int>(q->heads);
  a.Hkv = static_cast<int>(k->heads);
  a.Sq = static_cast<int>(q->seq);
  a.Sk = static_cast<int>(k->seq);
  const float sm = p->softmax_scale == 0.0f ? 1.0f / std::sqrt(static_cast<float>(q->dim)) : p->softmax_scale;
  a.softmax_scale = sm;
  a.c = sm * 1.4426950408889634f;
  a.p_uos = p->p_rule == MXATTN_SCALE_UOS;
  a.p_qmax_quarter = p->p_qmax * 0.25f;
  a.l_from_quantized = p->l_from_quantized != 0;
  a.n_qblk = static_cast<int>((q->seq + 127) / 128);
  a.one_scale = 127;
  if (hy != nullptr) {
    a.hybrid = 1;
    a.qf = static_cast<const uint16_t*>(hy->q);
    a.kf = static_cast<const uint16_t*>(hy->k);
    a.vf = static_cast<const uint16_t*>(hy->v);
    a.sel_idx = hy->idx;
    a.sel_n = hy->n_sel;
    a.max_sel = hy->max_sel;
    a.window = hy->window;
  }
  // Paired schedule: a causal launch (plain or hybrid) whose query blocks,
  // two per workgroup, make exactly one round of two workgroups per CU
  // (kv_tile 256 holds one workgroup per CU), with whole KV heads per XCD.
  if (p->causal && kv_tile != 256 && a.n_qblk >= 4 && a.n_qblk % 4 == 0 &&
      (a.B * a.Hkv) % 8 == 0) {
    const int n_cu = device_cu_count();
    if (n_cu > 0 && static_cast<int64_t>(a.n_qblk) * a.B * a.Hq == 4LL * n_cu) {
      a.paired = 1;
      a.pair_c = a.n_qblk / 4;   // every light pair then holds 3N/4 + 1 tiles
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(launch_prefill(a, static_cast<int>(q->dim), kv_tile, p->causal != 0, s), s,
                      hy != nullptr ? "prefill_hybrid" : "prefill");
}

mxattn_status_t mxattn_prefill(const mxattn_mx_t* q, const mxattn_mx_t* k, const mxattn_mx_t* v,
                               const mxattn_prefill_params_t* p, void* out, mxattn_dtype_t out_dtype, float* lse,
                               mxattn_stream_t stream) {
  mxattn_status_t st;
  if (injected("prefill", &st)) return st;
  return prefill_common(q, k, v, p, nullptr, out, out_dtype, lse, stream);
}

mxattn_status_t mxattn_prefill_hybrid(const mxattn_mx_t* q, const mxattn_mx_t* k, const mxattn_mx_t* v,
                                      const mxattn_prefill_params_t* p, const mxattn_prefill_hybrid_t* hy,
                                      void* out, mxattn_dtype_t out_dtype, float* lse, mxattn_stream_t stream) {
  mxattn_status_t st;
  if (injected("prefill_hybrid", &st)) return st;
  if (hy == nullptr) return fail(MXATTN_ERR_INVALID_ARG, "prefill_hybrid: null hybrid set");
  return prefill_common(q, k, v, p, hy, out, out_dtype, lse, stream);
}

static int64_t bf16_slots(int64_t hybrid_rows) { return hybrid_rows > 0 ? (hybrid_rows + kBf16Rows - 1) / kBf16Rows : 0; }

size_t mxattn_decode_workspace_bytes(int64_t batch, int64_t hq, int64_t hkv, int64_t dim, int64_t tcap,
                                     int32_t split_len, int32_t hybrid_rows) {
  if (batch < 1 || hq < 1 || hkv < 1 || dim < 1 || tcap < 1 || split_len < 1 || hybrid_rows < 0) return 0;
  const int64_t n_slot = (tcap + split_len - 1) / split_len + bf16_slots(hybrid_rows);
  size_t bytes = static_cast<size_t>(batch * hq * n_slot * (dim + 2)) * sizeof(float);
  bytes = (bytes + 255) / 256 * 256;
  return bytes;
}

static mxattn_status_t decode_common(const mxattn_mx_t* q, const mxattn_mx_t* q_res, const void* q_bf16,
                                     const mxattn_mx_t* kc, const mxattn_mx_t* vc, const mxattn_paging_t* pg,
                                     const int32_t* ctx_len, const mxattn_hybrid_t* hy, float softmax_scale,
                                     int32_t split_len, void* workspace, size_t workspace_bytes, float* out,
                                     float* lse, mxattn_stream_t stream, bool use_scratch = false) {
  mxattn_status_t st;
  // A query descriptor without codes and scales gives only the shape: the
  // scan encodes q_bf16 itself.
  const bool q_fused = q != nullptr && q->codes == nullptr && q->scales == nullptr;
  if (q_fused) {
    if (q_bf16 == nullptr) return fail(MXATTN_ERR_INVALID_ARG, "decode: q without codes needs q_bf16 to encode");
    if (q_res != nullptr) return fail(MXATTN_ERR_UNSUPPORTED, "decode: a dual-residual query must come encoded");
    if (!aligned16(q_bf16)) return fail(MXATTN_ERR_INVALID_ARG, "decode: q_bf16 not 16-byte aligned");
    if (q->layout != MXATTN_LAYOUT_HD) return fail(MXATTN_ERR_UNSUPPORTED, "decode.q: layout must be HD");
    if (q->batch < 1 || q->heads < 1 || q->seq < 1) return fail(MXATTN_ERR_INVALID_ARG, "decode.q: empty shape");
    if (q->dim != 64 && q->dim != 128) return fail(MXATTN_ERR_UNSUPPORTED, "decode.q: head_dim not in {64,128}");
    if (q->batch > 65535 || q->heads > 65535) return fail(MXATTN_ERR_UNSUPPORTED, "decode.q: batch/heads above 65535");
  } else if ((st = check_mx(q, "decode.q", MXATTN_LAYOUT_HD)) != MXATTN_OK) {
    return st;
  }
  if ((st = check_mx(kc, "decode.k_cache", MXATTN_LAYOUT_HD)) != MXATTN_OK) return st;
  if ((st = check_mx(vc, "decode.v_cache", MXATTN_LAYOUT_HD)) != MXATTN_OK) return st;
  if (ctx_len == nullptr || out == nullptr) return fail(MXATTN_ERR_INVALID_ARG, "decode: null ctx_len/out");
  if (q->seq != 1) return fail(MXATTN_ERR_UNSUPPORTED, "decode: one query token per sequence");
  if (q_res != nullptr) {
    if ((st = check_mx(q_res, "decode.q_res", MXATTN_LAYOUT_HD)) != MXATTN_OK) return st;
    if (q_res->batch != q->batch || q_res->heads != q->heads || q_res->seq != q->seq || q_res->dim != q->dim)
      return fail(MXATTN_ERR_INVALID_ARG, "decode: q_res shape differs from q");
  }
  if (q->dim != kc->dim || kc->dim != vc->dim) return fail(MXATTN_ERR_INVALID_ARG, "decode: head_dim mismatch");
  if (pg == nullptr && (q->batch != kc->batch || kc->batch != vc->batch))
    return fail(MXATTN_ERR_INVALID_ARG, "decode: batch mismatch");
  if (kc->heads != vc->heads || kc->seq != vc->seq) return fail(MXATTN_ERR_INVALID_ARG, "decode: K/V cache shape mismatch");
  // Token capacity per sequence: the cache length, or the block table's.
  int64_t tcap = kc->seq;
  if (pg != nullptr) {
    if (kc->batch != vc->batch) return fail(MXATTN_ERR_INVALID_ARG, "decode_paged: K/V pools differ in pages");
    if (pg->block_table == nullptr) return fail(MXATTN_ERR_INVALID_ARG, "decode_paged: null block_table");
    if (pg->max_pages < 1) return fail(MXATTN_ERR_INVALID_ARG, "decode_paged: max_pages must be >= 1");
    const int64_t P = kc->seq;
    if (P < 32 || P % 32 != 0) return fail(MXATTN_ERR_UNSUPPORTED, "decode_paged: page_size must be a multiple of 32");
    if (split_len % P != 0 || split_len / P > 64)
      return fail(MXATTN_ERR_UNSUPPORTED, "decode_paged: split_len must be a multiple of page_size, at most 64 pages");
    if (kc->batch > 0x7FFFFFFF) return fail(MXATTN_ERR_UNSUPPORTED, "decode_paged: too many pages");
    tcap = static_cast<int64_t>(pg->max_pages) * P;
    if (tcap > 0x7FFFFFFF) return fail(MXATTN_ERR_UNSUPPORTED, "decode_paged: max_pages x page_size too large");
  }
  if (q->heads % kc->heads != 0) return fail(MXATTN_ERR_INVALID_ARG, "decode: Hq %% Hkv != 0");
  const int64_t g = q->heads / kc->heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return fail(MXATTN_ERR_UNSUPPORTED, "decode: group size %lld", (long long)g);
  if (split_len < 64 || split_len % 64 != 0) return fail(MXATTN_ERR_UNSUPPORTED, "decode: split_len must be a positive multiple of 64");
  if (!(softmax_scale >= 0.0f) || !std::isfinite(softmax_scale))
    return fail(MXATTN_ERR_INVALID_ARG, "decode: softmax_scale must be finite and >= 0");
  // The scan addresses one (batch, KV head) of the cache with 32-bit offsets.
  for (const mxattn_mx_t* c : {kc, vc})
    if (c->seq * c->code_stride[2] > 0x7FFFFFFF || c->seq * c->scale_stride[2] > 0x7FFFFFFF)
      return fail(MXATTN_ERR_UNSUPPORTED, "decode: one head of the cache must span less than 2 GiB");
  const int hybrid = hy != nullptr;
  if (hybrid) {
    if (q_bf16 == nullptr) return fail(MXATTN_ERR_INVALID_ARG, "decode: hybrid needs q_bf16");
    if (hy->window < 0 || hy->max_sel < 0) return fail(MXATTN_ERR_INVALID_ARG, "decode: negative window/max_sel");
    if (hy->max_sel > 0 && (!hy->idx || !hy->n_sel || !hy->k_sel || !hy->v_sel))
      return fail(MXATTN_ERR_INVALID_ARG, "decode: hybrid selected set pointers missing");
    if (hy->window > 0 && (!hy->k_win || !hy->v_win)) return fail(MXATTN_ERR_INVALID_ARG, "decode: hybrid window pointers missing");
    if (split_len > 8192) return fail(MXATTN_ERR_UNSUPPORTED, "decode: hybrid needs split_len <= 8192");
    if (hy->max_sel + static_cast<int64_t>(hy->window) > tcap)
      return fail(MXATTN_ERR_INVALID_ARG, "decode: max_sel + window exceeds the cache");
  }
  const int64_t hybrid_rows = hybrid ? static_cast<int64_t>(hy->max_sel) + hy->window : 0;
  const int64_t n_split = (tcap + split_len - 1) / split_len;
  if (n_split + bf16_slots(hybrid_rows) > kMaxSlots)
    return fail(MXATTN_ERR_UNSUPPORTED, "decode: more than %lld partial slots; use a longer split_len", (long long)kMaxSlots);
  if ((n_split + bf16_slots(hybrid_rows)) * q->batch * kc->heads > 0x7FFFFFFF)
    return fail(MXATTN_ERR_UNSUPPORTED, "decode: problem too large for one launch");
  const size_t need = mxattn_decode_workspace_bytes(q->batch, q->heads, kc->heads, q->dim, tcap, split_len,
                                                    static_cast<int32_t>(hybrid_rows));
  if (use_scratch) {
    // The built-in scratch: sized once, looked up (not allocated) per device.
    if (need > kDecodeScratchBytes)
      return fail(MXATTN_ERR_UNSUPPORTED, "decode_noalloc: %zu bytes of partial slots needed, the built-in scratch "
                  "holds %zu; use mxattn_decode with a workspace or a longer split_len", need, kDecodeScratchBytes);
    const hipError_t e = decode_scratch(&workspace);
    if (e != hipSuccess) return fail(MXATTN_ERR_HIP, "decode_noalloc: scratch address: %s", hipGetErrorString(e));
    workspace_bytes = kDecodeScratchBytes;
  }
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MXATTN_ERR_WORKSPACE, "decode: workspace of %zu bytes needed", need);
  if (!aligned16(workspace)) return fail(MXATTN_ERR_INVALID_ARG, "decode: workspace not 16-byte aligned");
  DecodeArgs a{};
  a.q = view_of(q);
  a.dual = q_res != nullptr;
  if (a.dual) a.q2 = view_of(q_res);
  a.k = view_of(kc);
  a.v = view_of(vc);
  a.ctx_len = ctx_len;
  a.B = static_cast<int>(q->batch);
  a.Hq = static_cast<int>(q->heads);
  a.Hkv = static_cast<int>(kc->heads);
  a.Tcap = static_cast<int>(tcap);
  if (pg != nullptr) {
    a.paged = 1;
    a.block_table = pg->block_table;
    a.max_pages = pg->max_pages;
    a.page_size = static_cast<int>(kc->seq);
    a.n_pages = static_cast<int>(kc->batch);
  }
  const float sm = softmax_scale == 0.0f ? 1.0f / std::sqrt(static_cast<float>(q->dim)) : softmax_scale;
  a.softmax_scale = sm;
  a.c = sm * 1.4426950408889634f;
  a.split_len = split_len;
  a.n_split = static_cast<int>(n_split);
  a.n_bf16 = static_cast<int>(bf16_slots(hybrid_rows));
  a.part = static_cast<float*>(workspace);
  a.out = out;
  a.lse = lse;
  a.hybrid = hybrid;
  a.q_fused = q_fused;
  if (hybrid || q_fused) a.q_bf16 = static_cast<const uint16_t*>(q_bf16);
  if (hybrid) {
    a.idx = hy->idx;
    a.n_sel = hy->n_sel;
    a.max_sel = hy->max_sel;
    a.window = hy->window;
    a.k_sel = static_cast<const uint16_t*>(hy->k_sel);
    a.v_sel = static_cast<const uint16_t*>(hy->v_sel);
    a.k_win = static_cast<const uint16_t*>(hy->k_win);
    a.v_win = static_cast<const uint16_t*>(hy->v_win);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(launch_decode(a, static_cast<int>(q->dim), s), s, pg != nullptr ? "decode_paged" : "decode");
}

mxattn_status_t mxattn_decode(const mxattn_mx_t* q, const mxattn_mx_t* q_res, const void* q_bf16, const mxattn_mx_t* kc,
                              const mxattn_mx_t* vc, const int32_t* ctx_len, const mxattn_hybrid_t* hy,
                              float softmax_scale, int32_t split_len, void* workspace, size_t workspace_bytes,
                              float* out, float* lse, mxattn_stream_t stream) {
  mxattn_status_t st;
  if (injected("decode", &st)) return st;
  return decode_common(q, q_res, q_bf16, kc, vc, nullptr, ctx_len, hy, softmax_scale, split_len, workspace,
                       workspace_bytes, out, lse, stream);
}

mxattn_status_t mxattn_decode_noalloc(const mxattn_mx_t* q, const mxattn_mx_t* q_res, const void* q_bf16,
                                      const mxattn_mx_t* kc, const mxattn_mx_t* vc, const int32_t* ctx_len,
                                      const mxattn_hybrid_t* hy, float softmax_scale, int32_t split_len, float* out,
                                      float* lse, mxattn_stream_t stream) {
  mxattn_status_t st;
  if (injected("decode_noalloc", &st)) return st;
  return decode_common(q, q_res, q_bf16, kc, vc, nullptr, ctx_len, hy, softmax_scale, split_len, nullptr, 0, out,
                       lse, stream, true);
}

mxattn_status_t mxattn_decode_paged(const mxattn_mx_t* q, const mxattn_mx_t* q_res, const void* q_bf16,
                                    const mxattn_mx_t* k_pool, const mxattn_mx_t* v_pool,
                                    const mxattn_paging_t* paging, const int32_t* ctx_len,
                                    const mxattn_hybrid_t* hybrid, float softmax_scale, int32_t split_len,
                                    void* workspace, size_t workspace_bytes, float* out, float* lse,
                                    mxattn_stream_t stream) {
  mxattn_status_t st;
  if (injected("decode_paged", &st)) return st;
  if (paging == nullptr) return fail(MXATTN_ERR_INVALID_ARG, "decode_paged: null paging");
  return decode_common(q, q_res, q_bf16, k_pool, v_pool, paging, ctx_len, hybrid, softmax_scale, split_len,
                       workspace, workspace_bytes, out, lse, stream);
}

// Per (batch, query head, recent query, context chunk): partial (max, sum)
// of the logits, then one slot for their merge.  Chunks are 2048 keys when
// the batch gives the stats kernel at least 128 chunks per KV head, shorter
// (down to 256) for short contexts so that their few workgroups still spread
// over the CUs; never more than 32 chunks (the merge reads that many at once).
static int64_t select_chunk(int64_t batch, int64_t tcap) {
  int64_t chunk = 2048;
  while (chunk > 256 && batch * ((tcap + chunk - 1) / chunk) < 128) chunk /= 2;
  while ((tcap + chunk - 1) / chunk > 32) chunk *= 2;
  return chunk;
}

// Keys per column-mass workgroup: 512, down to 128 for short contexts.
static int select_cm_keys(int64_t batch, int64_t tcap) {
  int keys = 512;
  while (keys > 128 && batch * ((tcap + keys - 1) / keys) < 256) keys /= 2;
  return keys;
}

size_t mxattn_select_workspace_bytes(int64_t batch, int64_t hq, int64_t recent, int64_t tcap) {
  if (batch < 1 || hq < 1 || recent < 0 || tcap < 1) return 0;
  const int64_t chunk = select_chunk(batch, tcap);
  const int64_t nchunk = (tcap + chunk - 1) / chunk;
  const int64_t n = batch * hq * (recent > 0 ? recent : 1) * (nchunk + 1) * 2;
  return static_cast<size_t>(n) * sizeof(float);
}

mxattn_status_t mxattn_select_vertical(const mxattn_mx_t* q, const mxattn_mx_t* kc, const int32_t* ctx_len,
                                       float softmax_scale, int32_t window, int32_t rho_num, int32_t rho_den,
                                       float* col_mass, int32_t* idx_out, int32_t* n_out, int32_t max_sel,
                                       void* workspace, size_t workspace_bytes, mxattn_stream_t stream) {
  mxattn_status_t st;
  if (injected("select_vertical", &st)) return st;
  if ((st = check_mx(kc, "select.k_cache", MXATTN_LAYOUT_HD)) != MXATTN_OK) return st;
  if (q != nullptr && (st = check_mx(q, "select.q_recent", MXATTN_LAYOUT_HD)) != MXATTN_OK) return st;
  if (!ctx_len || !col_mass || !idx_out || !n_out) return fail(MXATTN_ERR_INVALID_ARG, "select: null pointer");
  if (window < 0 || rho_num < 0 || rho_den < 1 || rho_num > rho_den || max_sel < 0)
    return fail(MXATTN_ERR_INVALID_ARG, "select: bad window / rho / max_sel");
  const int R = q ? static_cast<int>(q->seq) : 0;
  if (q) {
    if (q->dim != kc->dim || q->batch != kc->batch) return fail(MXATTN_ERR_INVALID_ARG, "select: shape mismatch");
    if (q->heads % kc->heads != 0) return fail(MXATTN_ERR_INVALID_ARG, "select: Hq %% Hkv != 0");
    if (R > 64) return fail(MXATTN_ERR_UNSUPPORTED, "select: more than 64 recent queries");
    if ((q->heads / kc->heads) * R > 512)
      return fail(MXATTN_ERR_UNSUPPORTED, "select: recent queries x group size above 512");
  }
  if (kc->seq > 65536) return fail(MXATTN_ERR_UNSUPPORTED, "select: cache longer than 65536");
  if (kc->seq * kc->code_stride[2] > 0x7FFFFFFF || kc->seq * kc->scale_stride[2] > 0x7FFFFFFF)
    return fail(MXATTN_ERR_UNSUPPORTED, "select: one head of the cache must span less than 2 GiB");
  const int64_t worst = kc->seq > window ? ((kc->seq - window) * rho_num + rho_den - 1) / rho_den : 0;
  if (worst > max_sel) return fail(MXATTN_ERR_INVALID_ARG, "select: max_sel %d below the worst-case count %lld", max_sel, (long long)worst);
  const size_t need = mxattn_select_workspace_bytes(kc->batch, q ? q->heads : kc->heads, R, kc->seq);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(MXATTN_ERR_WORKSPACE, "select: workspace of %zu bytes needed", need);
  if (!aligned16(workspace)) return fail(MXATTN_ERR_INVALID_ARG, "select: workspace not 16-byte aligned");
  SelectArgs a{};
  a.stats = static_cast<float*>(workspace);
  a.chunk = static_cast<int>(select_chunk(kc->batch, kc->seq));
  a.cm_keys = select_cm_keys(kc->batch, kc->seq);
  if (q) a.q = view_of(q);
  a.k = view_of(kc);
  a.ctx_len = ctx_len;
  a.B = static_cast<int>(kc->batch);
  a.Hq = q ? static_cast<int>(q->heads) : static_cast<int>(kc->heads);
  a.Hkv = static_cast<int>(kc->heads);
  a.R = R;
  a.Tcap = static_cast<int>(kc->seq);
  const float sm = softmax_scale == 0.0f ? 1.0f / std::sqrt(static_cast<float>(kc->dim)) : softmax_scale;
  a.c = sm * 1.4426950408889634f;
  a.window = window;
  a.rho_num = rho_num;
  a.rho_den = rho_den;
  a.max_sel = max_sel;
  a.col_mass = col_mass;
  a.idx_out = idx_out;
  a.n_out = n_out;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(launch_select(a, static_cast<int>(kc->dim), s), s, "select_vertical");
}

mxattn_status_t mxattn_gather_rows(const void* k, const void* v, const int64_t shape[4], const int64_t k_stride[3],
                                   const int64_t v_stride[3], const int32_t* idx, const int32_t* n_sel,
                                   int32_t max_sel, void* k_out, void* v_out, mxattn_stream_t stream) {
  mxattn_status_t st;
  if (injected("gather_rows", &st)) return st;
  if (!shape || !k_stride || !v_stride) return fail(MXATTN_ERR_INVALID_ARG, "gather_rows: null shape/strides");
  if (max_sel < 0) return fail(MXATTN_ERR_INVALID_ARG, "gather_rows: negative max_sel");
  const int64_t B = shape[0], H = shape[1], T = shape[2], D = shape[3];
  if (B < 1 || H < 1 || T < 1) return fail(MXATTN_ERR_INVALID_ARG, "gather_rows: empty shape");
  if (D != 64 && D != 128) return fail(MXATTN_ERR_UNSUPPORTED, "gather_rows: head_dim %lld not in {64,128}", (long long)D);
  if (B * H > 65535 || T > 0x7FFFFFFF) return fail(MXATTN_ERR_UNSUPPORTED, "gather_rows: batch x heads above 65535");
  if (max_sel == 0) return ok();
  if (!k || !v || !idx || !n_sel || !k_out || !v_out) return fail(MXATTN_ERR_INVALID_ARG, "gather_rows: null pointer");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_out) || !aligned16(v_out))
    return fail(MXATTN_ERR_INVALID_ARG, "gather_rows: rows must be 16-byte aligned");
  for (int i = 0; i < 3; ++i)
    if (k_stride[i] < 0 || v_stride[i] < 0 || (k_stride[i] * 2) % 16 != 0 || (v_stride[i] * 2) % 16 != 0)
      return fail(MXATTN_ERR_INVALID_ARG, "gather_rows: strides must be non-negative multiples of 8 elements");
  if (k_stride[2] < D || v_stride[2] < D) return fail(MXATTN_ERR_INVALID_ARG, "gather_rows: row stride below D");
  GatherArgs a{};
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  for (int i = 0; i < 3; ++i) {
    a.ks[i] = k_stride[i];
    a.vs[i] = v_stride[i];
  }
  a.idx = idx;
  a.n_sel = n_sel;
  a.k_out = static_cast<uint16_t*>(k_out);
  a.v_out = static_cast<uint16_t*>(v_out);
  a.B = static_cast<int>(B);
  a.H = static_cast<int>(H);
  a.T = static_cast<int>(T);
  a.D = static_cast<int>(D);
  a.max_sel = max_sel;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return after_launch(launch_gather_rows(a, s), s, "gather_rows");
}

}  // extern "C"

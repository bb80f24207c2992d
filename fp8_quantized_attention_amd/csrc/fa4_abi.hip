// Host side of the C ABI: argument validation, error reporting and dispatch to the kernel launchers.
// Every check runs before anything is enqueued; a failed check returns its status and records a
// thread-local message for fa4_last_error().
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "fa4_internal.h"

namespace {

thread_local std::string g_last_error;

fa4_status fail(fa4_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fa4_status ok() {
  g_last_error.clear();
  return FA4_OK;
}

fa4_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(FA4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQUIRE(cond, st, ...) \
  do {                         \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

// The attention kernel stages tiles in up to ~70 KB of LDS; kernels above the default dynamic limit
// are opted in once per process.
}  // namespace

extern "C" {

const char *fa4_status_string(int s) {
  switch (s) {
    case FA4_OK: return "ok";
    case FA4_ERR_NULL: return "null pointer";
    case FA4_ERR_SHAPE: return "invalid shape";
    case FA4_ERR_UNSUPPORTED: return "unsupported combination";
    case FA4_ERR_ALIGN: return "misaligned pointer";
    case FA4_ERR_WORKSPACE: return "workspace too small";
    case FA4_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *fa4_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace {

// The checks of one quantization; *empty is set when there is nothing to enqueue.
fa4_status check_quantize(const fa4_qinput *in, uint32_t flags, const fa4_qoutput *out, const fa4_qoutput *residual,
                          float *row_norm2, bool *empty) {
  *empty = false;
  REQUIRE(in && out, FA4_ERR_NULL, "quantize: input or output descriptor is NULL");
  REQUIRE(in->dtype == FA4_F32 || in->dtype == FA4_BF16, FA4_ERR_UNSUPPORTED, "quantize: dtype %d", in->dtype);
  REQUIRE(in->d == 64 || in->d == 128, FA4_ERR_UNSUPPORTED, "quantize: d=%d (64 or 128)", in->d);
  REQUIRE(out->fmt == FA4_MXFP4 || out->fmt == FA4_NVFP4 || out->fmt == FA4_FP8_TOKEN || out->fmt == FA4_MXFP8 ||
              out->fmt == FA4_MXFP4_KEYS,
          FA4_ERR_UNSUPPORTED, "quantize: format %d", out->fmt);
  if (out->fmt == FA4_MXFP4_KEYS) {
    REQUIRE(flags == 0 && !residual && !row_norm2 && !in->page_table && !in->row_counts && !in->channel_scale &&
                !out->fold_w && !out->fold_scale,
            FA4_ERR_UNSUPPORTED, "quantize: MXFP4_KEYS takes no flags, residual, row norms, paging, ragged rows, "
                                 "smoothing or fold outputs");
    REQUIRE(in->rows % 32 == 0, FA4_ERR_SHAPE, "quantize: MXFP4_KEYS needs rows in multiples of 32 (rows=%lld)",
            (long long)in->rows);
    REQUIRE(in->rows / 32 <= 0x7fffffff, FA4_ERR_SHAPE, "quantize: MXFP4_KEYS grid too large");
  }
  REQUIRE((flags & ~(uint32_t)(FA4_HADAMARD128 | FA4_DUAL_RESIDUAL | FA4_SCALE_SEARCH)) == 0, FA4_ERR_UNSUPPORTED,
          "quantize: unknown flags 0x%x", flags);
  if (flags & FA4_SCALE_SEARCH) {
    REQUIRE(out->fmt == FA4_MXFP4 || out->fmt == FA4_NVFP4, FA4_ERR_UNSUPPORTED,
            "quantize: scale search needs MXFP4 or NVFP4");
    REQUIRE(!(flags & FA4_DUAL_RESIDUAL), FA4_ERR_UNSUPPORTED, "quantize: scale search with the dual residual");
  }
  REQUIRE(aligned(in->channel_scale, 4), FA4_ERR_ALIGN, "quantize: channel_scale must be 4-byte aligned");
  REQUIRE(in->outer >= 0 && in->heads >= 1 && in->rows >= 0, FA4_ERR_SHAPE,
          "quantize: outer=%lld heads=%d rows=%lld", (long long)in->outer, in->heads, (long long)in->rows);
  const int64_t groups = in->outer * in->heads;
  REQUIRE(groups <= 65535, FA4_ERR_SHAPE, "quantize: %lld groups (at most 65535)", (long long)groups);
  REQUIRE(in->rows <= (int64_t)1 << 31, FA4_ERR_SHAPE, "quantize: rows=%lld", (long long)in->rows);
  if (groups == 0 || (in->rows == 0 && out->fmt != FA4_NVFP4)) {
    *empty = true;
    return ok();
  }
  REQUIRE(in->rows == 0 || in->x, FA4_ERR_NULL, "quantize: x is NULL");
  REQUIRE(out->codes || in->rows == 0, FA4_ERR_NULL, "quantize: codes is NULL");
  if (out->fmt != FA4_FP8_TOKEN && in->rows > 0)
    REQUIRE(out->block_scales, FA4_ERR_NULL, "quantize: block_scales is NULL");
  if (out->fmt == FA4_NVFP4) REQUIRE(out->scales, FA4_ERR_NULL, "quantize: NVFP4 tensor scales are NULL");
  if (out->fmt == FA4_FP8_TOKEN) REQUIRE(out->scales, FA4_ERR_NULL, "quantize: FP8 per-token scales NULL");
  if (flags & FA4_HADAMARD128) {
    REQUIRE(in->d == 128, FA4_ERR_UNSUPPORTED, "quantize: Hadamard rotation needs d=128");
    REQUIRE(out->fmt != FA4_FP8_TOKEN, FA4_ERR_UNSUPPORTED, "quantize: Hadamard rotation with FP8 output");
  }
  if (flags & FA4_DUAL_RESIDUAL) {
    REQUIRE(out->fmt == FA4_NVFP4 || out->fmt == FA4_MXFP4, FA4_ERR_UNSUPPORTED,
            "quantize: dual residual needs NVFP4 or MXFP4");
    const bool nv = out->fmt == FA4_NVFP4;
    REQUIRE(residual && (!nv || residual->scales) && (in->rows == 0 || (residual->codes && residual->block_scales)),
            FA4_ERR_NULL, "quantize: dual residual output missing");
    REQUIRE(residual->fmt == out->fmt, FA4_ERR_UNSUPPORTED, "quantize: residual format must match the output's");
    REQUIRE(aligned(residual->codes, 16) && aligned(residual->block_scales, 4) && aligned(residual->scales, 4),
            FA4_ERR_ALIGN, "quantize: residual codes must be 16-byte aligned, scales 4-byte aligned");
  }
  // every lane reads one 16-byte run of a row (8 bf16 or 4 float values)
  const int64_t epl = in->dtype == FA4_F32 ? 4 : 8;
  REQUIRE(in->rows == 0 || aligned(in->x, 16), FA4_ERR_ALIGN, "quantize: x must be 16-byte aligned");
  REQUIRE(in->stride_outer % epl == 0 && in->stride_head % epl == 0 && in->stride_row % epl == 0, FA4_ERR_ALIGN,
          "quantize: strides must be multiples of %lld elements (16 bytes)", (long long)epl);
  REQUIRE(in->stride_outer >= 0 && in->stride_head >= 0 && in->stride_row >= in->d, FA4_ERR_SHAPE,
          "quantize: strides must be non-negative and stride_row >= d");
  REQUIRE(aligned(out->codes, 16) && aligned(out->block_scales, 4) && aligned(out->scales, 4), FA4_ERR_ALIGN,
          "quantize: codes must be 16-byte aligned, scales 4-byte aligned");
  if (in->page_table) {
    REQUIRE(in->page_size > 0 && in->max_pages > 0 && in->num_pages > 0, FA4_ERR_SHAPE,
            "quantize: paged output needs page_size, max_pages and num_pages > 0");
    REQUIRE(in->rows <= (int64_t)in->page_size * in->max_pages, FA4_ERR_SHAPE,
            "quantize: rows=%lld exceed max_pages*page_size", (long long)in->rows);
    REQUIRE(row_norm2 == nullptr, FA4_ERR_UNSUPPORTED, "quantize: row norms need unpaged output");
  }
  REQUIRE(aligned(row_norm2, 4), FA4_ERR_ALIGN, "quantize: row_norm2 must be 4-byte aligned");
  if (out->fold_w || out->fold_scale) {
    REQUIRE(out->fmt == FA4_FP8_TOKEN, FA4_ERR_UNSUPPORTED, "quantize: fold outputs need FP8_TOKEN");
    REQUIRE(out->fold_w && out->fold_scale, FA4_ERR_NULL, "quantize: fold_w and fold_scale go together");
    REQUIRE(in->rows % 128 == 0 && !in->page_table && !in->row_counts, FA4_ERR_UNSUPPORTED,
            "quantize: fold outputs need unpaged, non-ragged rows in multiples of 128");
    REQUIRE(aligned(out->fold_w, 4) && aligned(out->fold_scale, 4), FA4_ERR_ALIGN, "quantize: fold alignment");
  }
  return ok();
}

}  // namespace

extern "C" {

fa4_status fa4_quantize_blockscaled(const fa4_qinput *in, uint32_t flags, const fa4_qoutput *out,
                                    const fa4_qoutput *residual, float *row_norm2, void *stream) {
  bool empty;
  const fa4_status st = check_quantize(in, flags, out, residual, row_norm2, &empty);
  if (st != FA4_OK || empty) return st;
  return hip_status(fa4::launch_quantize(in, flags, out, residual, row_norm2, (hipStream_t)stream),
                    "quantize launch");
}

fa4_status fa4_quantize_prefill(const fa4_qinput *q, const fa4_qinput *k, const fa4_qinput *v,
                                const fa4_qoutput *q_out, const fa4_qoutput *k_out, const fa4_qoutput *v_out,
                                float *q_norm2, float *k_norm2, void *stream) {
  REQUIRE(q && k && v && q_out && k_out && v_out, FA4_ERR_NULL, "quantize_prefill: a descriptor is NULL");
  REQUIRE((q_out->fmt == FA4_MXFP4 || q_out->fmt == FA4_MXFP8) && k_out->fmt == q_out->fmt, FA4_ERR_UNSUPPORTED,
          "quantize_prefill: Q and K must both be MXFP4 or both MXFP8 (formats %d, %d)", q_out->fmt, k_out->fmt);
  const bool v4 = v_out->fmt == FA4_MXFP4_KEYS;
  REQUIRE((v_out->fmt == FA4_FP8_TOKEN && v_out->fold_w && v_out->fold_scale) ||
              (v4 && q_out->fmt == FA4_MXFP4 && q->d == 128),
          FA4_ERR_UNSUPPORTED,
          "quantize_prefill: V must be FP8 per token with its fold outputs, or 4-bit V (MXFP4_KEYS) with MXFP4 Q/K "
          "and d = 128");
  REQUIRE(q->dtype == k->dtype && k->dtype == v->dtype && q->d == k->d && k->d == v->d, FA4_ERR_UNSUPPORTED,
          "quantize_prefill: Q, K and V must share dtype and d");
  REQUIRE(!q->page_table && !k->page_table && !v->page_table && !q->row_counts && !k->row_counts && !v->row_counts,
          FA4_ERR_UNSUPPORTED, "quantize_prefill: paged or ragged rows need fa4_quantize_blockscaled");
  REQUIRE((q_norm2 == nullptr) == (k_norm2 == nullptr), FA4_ERR_UNSUPPORTED,
          "quantize_prefill: row norms of both Q and K, or of neither");
  bool eq, ek, ev;
  fa4_status st;
  if ((st = check_quantize(q, 0, q_out, nullptr, q_norm2, &eq)) != FA4_OK) return st;
  if ((st = check_quantize(k, 0, k_out, nullptr, k_norm2, &ek)) != FA4_OK) return st;
  if ((st = check_quantize(v, 0, v_out, nullptr, nullptr, &ev)) != FA4_OK) return st;
  REQUIRE(fa4::prefill_quant_blocks(q, k, v, v4) < ((int64_t)1 << 31), FA4_ERR_SHAPE, "quantize_prefill: grid too large");
  if (eq && ek && ev) return ok();
  return hip_status(fa4::launch_quantize_prefill(q, k, v, q_out, k_out, v_out, q_norm2, k_norm2, (hipStream_t)stream),
                    "quantize_prefill launch");
}

fa4_status fa4_select_tiles(const float *q_norm2, const float *k_norm2, int32_t B, int32_t Hq, int32_t Hkv,
                            int32_t Lq, int32_t Lk, int32_t causal, int32_t num, int32_t den,
                            uint8_t *bitmap, int32_t *counts, void *stream) {
  REQUIRE(B >= 0 && Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, FA4_ERR_SHAPE,
          "select: B=%d Hq=%d Hkv=%d (Hq must be a multiple of Hkv)", B, Hq, Hkv);
  REQUIRE(Lq > 0 && Lk > 0 && Lq % 128 == 0 && Lk % 128 == 0, FA4_ERR_SHAPE,
          "select: Lq=%d Lk=%d must be positive multiples of 128", Lq, Lk);
  REQUIRE(Lq / 128 <= 1024 && Lk / 128 <= 4096, FA4_ERR_SHAPE, "select: at most 1024 x 4096 tiles");
  REQUIRE(!causal || Lq <= Lk, FA4_ERR_SHAPE, "select: causal needs Lq <= Lk");
  REQUIRE(den > 0 && num >= 0 && num <= den, FA4_ERR_SHAPE, "select: fraction %d/%d", num, den);
  REQUIRE(B <= 65535 && Hq <= 65535, FA4_ERR_SHAPE, "select: grid too large");
  if (B == 0) return ok();
  REQUIRE(q_norm2 && k_norm2 && bitmap, FA4_ERR_NULL, "select: q_norm2, k_norm2 and bitmap are required");
  REQUIRE(aligned(q_norm2, 4) && aligned(k_norm2, 4) && aligned(counts, 4), FA4_ERR_ALIGN, "select: alignment");
  return hip_status(fa4::launch_select(q_norm2, k_norm2, B, Hq, Hkv, Lq, Lk, causal != 0, num, den, bitmap,
                                       counts, (hipStream_t)stream),
                    "select launch");
}

fa4_status fa4_attn_fwd(const fa4_attn_args *a, void *stream) {
  REQUIRE(a, FA4_ERR_NULL, "attn: args is NULL");
  REQUIRE(a->fmt == FA4_MXFP4 || a->fmt == FA4_NVFP4 || a->fmt == FA4_MXFP8, FA4_ERR_UNSUPPORTED,
          "attn: Q/K format %d", a->fmt);
  REQUIRE(a->B >= 0 && a->Hq >= 1 && a->Hkv >= 1 && a->Hq % a->Hkv == 0, FA4_ERR_SHAPE,
          "attn: B=%d Hq=%d Hkv=%d", a->B, a->Hq, a->Hkv);
  REQUIRE(a->Lq >= 0 && a->Lk > 0 && a->Lq % 128 == 0 && a->Lk % 128 == 0, FA4_ERR_SHAPE,
          "attn: Lq=%d Lk=%d must be multiples of 128 (Lk > 0)", a->Lq, a->Lk);
  REQUIRE(!a->causal || a->Lq <= a->Lk, FA4_ERR_SHAPE, "attn: causal needs Lq <= Lk");
  REQUIRE((int64_t)(a->Lq / 128) * a->Hq * a->B < ((int64_t)1 << 31), FA4_ERR_SHAPE, "attn: grid too large");
  if (a->fmt == FA4_MXFP4)
    REQUIRE(a->d == 128 || (a->d == 64 && !a->bitmap), FA4_ERR_UNSUPPORTED,
            "attn: MXFP4 supports d=128, or d=64 without tile selection (d=%d)", a->d);
  else
    REQUIRE(a->d == 128, FA4_ERR_UNSUPPORTED, "attn: NVFP4 and MXFP8 need d=128 (d=%d)", a->d);
  const bool v4 = a->v_fmt == FA4_MXFP4_KEYS;
  REQUIRE(v4 || a->v_fmt == 0 || a->v_fmt == FA4_FP8_TOKEN, FA4_ERR_UNSUPPORTED, "attn: V format %d", a->v_fmt);
  if (v4)
    REQUIRE(a->fmt == FA4_MXFP4 && a->d == 128, FA4_ERR_UNSUPPORTED, "attn: 4-bit V needs MXFP4 Q/K and d=128");
  REQUIRE(a->p_fmt == FA4_P_FP8 || a->p_fmt == FA4_P_MXFP4, FA4_ERR_UNSUPPORTED, "attn: probability format %d",
          a->p_fmt);
  if (a->p_fmt == FA4_P_MXFP4)
    REQUIRE(a->fmt == FA4_MXFP4 && a->d == 128, FA4_ERR_UNSUPPORTED, "attn: MXFP4 probabilities need MXFP4 Q/K and d=128");
  if (a->B == 0 || a->Lq == 0) return ok();
  if (v4)
    REQUIRE(a->q_codes && a->q_scales && a->k_codes && a->k_scales && a->v_codes && a->v_block_scales && a->o,
            FA4_ERR_NULL, "attn: a required pointer is NULL");
  else
    REQUIRE(a->q_codes && a->q_scales && a->k_codes && a->k_scales && a->v_codes && a->v_scales && a->o &&
                a->v_fold_w && a->v_fold_scale,
            FA4_ERR_NULL, "attn: a required pointer is NULL");
  REQUIRE(aligned(a->v_block_scales, 16), FA4_ERR_ALIGN, "attn: every pointer must be 16-byte aligned");
  if (a->fmt == FA4_NVFP4) REQUIRE(a->q_tscale && a->k_tscale, FA4_ERR_NULL, "attn: NVFP4 tensor scales NULL");
  if (a->bitmap) REQUIRE(a->q_bf16 && a->k_bf16 && a->v_bf16, FA4_ERR_NULL, "attn: bf16 originals needed with a bitmap");
  const void *ptrs[] = {a->q_codes, a->q_scales, a->k_codes, a->k_scales, a->v_codes, a->v_scales, a->o,
                        a->lse, a->q_bf16, a->k_bf16, a->v_bf16, a->q_tscale, a->k_tscale, a->v_fold_w,
                        a->v_fold_scale};
  for (const void *p : ptrs) REQUIRE(aligned(p, 16), FA4_ERR_ALIGN, "attn: every pointer must be 16-byte aligned");
  REQUIRE(a->softmax_scale > 0.0f, FA4_ERR_SHAPE, "attn: softmax_scale must be positive");
  return hip_status(fa4::launch_attn(a, (hipStream_t)stream), "attention launch");
}

fa4_status fa4_smoothing_factors(const fa4_qinput *q, const fa4_qinput *k, float *q_scale, float *k_scale,
                                 void *stream) {
  REQUIRE(q && k && q_scale && k_scale, FA4_ERR_NULL, "smoothing: a required pointer is NULL");
  for (const fa4_qinput *in : {q, k}) {
    REQUIRE(in->dtype == FA4_F32 || in->dtype == FA4_BF16, FA4_ERR_UNSUPPORTED, "smoothing: dtype %d", in->dtype);
    REQUIRE(in->d == 64 || in->d == 128, FA4_ERR_UNSUPPORTED, "smoothing: d=%d (64 or 128)", in->d);
    REQUIRE(in->outer >= 0 && in->heads >= 1 && in->rows >= 0, FA4_ERR_SHAPE, "smoothing: bad shape");
    REQUIRE(in->outer * in->heads <= 65535, FA4_ERR_SHAPE, "smoothing: too many groups");
    REQUIRE(in->rows <= (int64_t)1 << 31, FA4_ERR_SHAPE, "smoothing: rows=%lld", (long long)in->rows);
    REQUIRE(in->page_table == nullptr, FA4_ERR_UNSUPPORTED, "smoothing: calibration input must be unpaged");
    REQUIRE(in->rows == 0 || in->outer == 0 || in->x, FA4_ERR_NULL, "smoothing: x is NULL");
    const int64_t epl = in->dtype == FA4_F32 ? 4 : 8;
    REQUIRE(aligned(in->x, 16), FA4_ERR_ALIGN, "smoothing: x must be 16-byte aligned");
    REQUIRE(in->stride_outer % epl == 0 && in->stride_head % epl == 0 && in->stride_row % epl == 0,
            FA4_ERR_ALIGN, "smoothing: strides must be multiples of 16 bytes");
    REQUIRE(in->stride_outer >= 0 && in->stride_head >= 0 && in->stride_row >= in->d, FA4_ERR_SHAPE,
            "smoothing: strides must be non-negative and stride_row >= d");
  }
  REQUIRE(q->d == k->d, FA4_ERR_SHAPE, "smoothing: d differs (%d, %d)", q->d, k->d);
  REQUIRE(q->heads % k->heads == 0, FA4_ERR_SHAPE, "smoothing: Hq=%d is not a multiple of Hkv=%d", q->heads,
          k->heads);
  REQUIRE(aligned(q_scale, 4) && aligned(k_scale, 4), FA4_ERR_ALIGN, "smoothing: outputs must be 4-byte aligned");
  return hip_status(fa4::launch_smoothing(q, k, q_scale, k_scale, (hipStream_t)stream), "smoothing launch");
}

// ---- decode without a caller workspace. The split partials live in `scratch`, a device global of
// FA4_DECODE_SCRATCH_BYTES per GPU. In host code `scratch` names a host-side stand-in, not device memory:
// its device address on each GPU comes from hipGetSymbolAddress, called once per device with that device
// current, and only that address is handed to the kernels.
}  // extern "C"
namespace {
__device__ __align__(256) uint8_t scratch[FA4_DECODE_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];          // device address of `scratch` per device, once looked up
}  // namespace
extern "C" {

fa4_status fa4_decode_paged_noalloc(const fa4_decode_args *a, void *stream) {
  REQUIRE(a, FA4_ERR_NULL, "decode (no allocation): args is NULL");
  const size_t need = fa4_decode_workspace_bytes(a);
  REQUIRE(need <= FA4_DECODE_SCRATCH_BYTES, FA4_ERR_WORKSPACE,
          "decode (no allocation): these shapes need %zu bytes of scratch, more than the %zu the library holds; "
          "use fa4_decode_paged with a workspace",
          need, (size_t)FA4_DECODE_SCRATCH_BYTES);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "decode (no allocation): hipGetDevice");
  REQUIRE(dev >= 0 && dev < kMaxDevices, FA4_ERR_UNSUPPORTED, "decode (no allocation): device %d", dev);
  void *ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
      void *p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e, "decode (no allocation): hipGetSymbolAddress(scratch)");
      REQUIRE(p != nullptr, FA4_ERR_HIP, "decode (no allocation): no device address for the scratch array");
      g_scratch_ptr[dev] = p;
    }
    ptr = g_scratch_ptr[dev];
  }
  return fa4_decode_paged(a, ptr, FA4_DECODE_SCRATCH_BYTES, stream);
}

size_t fa4_decode_workspace_bytes(const fa4_decode_args *a) {
  if (!a || a->B <= 0 || a->Hkv <= 0 || a->max_pages <= 0) return 0;
  return a->d_v != 0 ? fa4::decode_mla_workspace_bytes(a) : fa4::decode_workspace_bytes(a);
}

static fa4_status decode_mla(const fa4_decode_args *a, void *ws, size_t ws_bytes, void *stream) {
  REQUIRE(a->d_v == fa4::MLA_DV && a->d == fa4::MLA_D, FA4_ERR_UNSUPPORTED, "decode (MLA): d=%d d_v=%d (576, 512)",
          a->d, a->d_v);
  REQUIRE(a->fmt == FA4_MXFP4 && a->p_fmt == FA4_P_FP8, FA4_ERR_UNSUPPORTED,
          "decode (MLA): needs an MXFP4 cache and FP8 probabilities (fmt=%d p_fmt=%d)", a->fmt, a->p_fmt);
  REQUIRE(a->Hq == fa4::MLA_H && a->Hkv == 1, FA4_ERR_UNSUPPORTED, "decode (MLA): needs Hq=16, Hkv=1 (Hq=%d Hkv=%d)",
          a->Hq, a->Hkv);
  REQUIRE(a->page_size == 64, FA4_ERR_UNSUPPORTED, "decode (MLA): page_size=%d (64)", a->page_size);
  REQUIRE(a->B >= 0 && a->B <= 65535, FA4_ERR_SHAPE, "decode (MLA): B=%d", a->B);
  REQUIRE(a->max_pages >= 1 && a->num_pages >= 1, FA4_ERR_SHAPE, "decode (MLA): max_pages and num_pages >= 1");
  REQUIRE((int64_t)a->max_pages * 64 <= ((int64_t)1 << 30), FA4_ERR_SHAPE, "decode (MLA): context too long");
  REQUIRE(((int64_t)a->max_pages + fa4::MLA_PAGES - 1) / fa4::MLA_PAGES * a->B < ((int64_t)1 << 31), FA4_ERR_SHAPE, "decode (MLA): grid too large");
  if (a->B == 0) return ok();
  REQUIRE(a->q1_codes && a->q1_scales && a->q2_codes && a->q2_scales && a->k_codes && a->k_scales &&
              a->page_table && a->ctx_len && a->o,
          FA4_ERR_NULL, "decode (MLA): a required pointer is NULL");
  const void *ptrs16[] = {a->q1_codes, a->q2_codes, a->k_codes, a->k_scales};
  for (const void *p : ptrs16)
    REQUIRE(aligned(p, 16), FA4_ERR_ALIGN, "decode (MLA): code and cache scale arrays must be 16-byte aligned");
  const size_t need = fa4::decode_mla_workspace_bytes(a);
  REQUIRE(ws && ws_bytes >= need, FA4_ERR_WORKSPACE, "decode (MLA): workspace %zu bytes, %zu needed", ws_bytes, need);
  REQUIRE(aligned(ws, 256), FA4_ERR_ALIGN, "decode (MLA): workspace must be 256-byte aligned");
  return hip_status(fa4::launch_decode_mla(a, ws, (hipStream_t)stream), "decode (MLA) launch");
}

fa4_status fa4_decode_paged(const fa4_decode_args *a, void *ws, size_t ws_bytes, void *stream) {
  REQUIRE(a, FA4_ERR_NULL, "decode: args is NULL");
  if (a->d_v != 0) return decode_mla(a, ws, ws_bytes, stream);
  REQUIRE(a->fmt == FA4_NVFP4 || a->fmt == FA4_MXFP4, FA4_ERR_UNSUPPORTED, "decode: format %d", a->fmt);
  REQUIRE(a->p_fmt == FA4_P_FP8 || a->p_fmt == FA4_P_NVFP4, FA4_ERR_UNSUPPORTED, "decode: probability format %d",
          a->p_fmt);
  REQUIRE(a->d == 128, FA4_ERR_UNSUPPORTED, "decode: d=%d (128)", a->d);
  REQUIRE(a->page_size == 64, FA4_ERR_UNSUPPORTED, "decode: page_size=%d (64)", a->page_size);
  REQUIRE(a->B >= 0 && a->Hkv >= 1 && a->Hq >= a->Hkv && a->Hq % a->Hkv == 0 && a->Hq / a->Hkv <= 64,
          FA4_ERR_UNSUPPORTED, "decode: needs Hq a multiple of Hkv, at most 64 Hkv (Hq=%d Hkv=%d)", a->Hq, a->Hkv);
  REQUIRE(a->max_pages >= 1 && a->num_pages >= 1, FA4_ERR_SHAPE, "decode: max_pages and num_pages >= 1");
  REQUIRE(a->B <= 65535 && a->Hkv <= 65535 && a->Hq <= 65535, FA4_ERR_SHAPE, "decode: grid too large");
  REQUIRE(((int64_t)a->max_pages * 64 + fa4::DEC_SPLIT_KEYS - 1) / fa4::DEC_SPLIT_KEYS * a->B * a->Hkv *
                  ((a->Hq / a->Hkv + 3) / 4) <
              ((int64_t)1 << 31),
          FA4_ERR_SHAPE,
          "decode: grid too large");
  REQUIRE((int64_t)a->max_pages * 64 <= ((int64_t)1 << 30), FA4_ERR_SHAPE, "decode: context too long");
  if (a->B == 0) return ok();
  REQUIRE(a->q1_codes && a->q1_scales && a->q2_codes && a->q2_scales && a->k_codes && a->k_scales &&
              a->v_codes && a->v_scales && a->page_table && a->ctx_len && a->o,
          FA4_ERR_NULL, "decode: a required pointer is NULL");
  if (a->fmt == FA4_NVFP4)
    REQUIRE(a->q1_tscale && a->q2_tscale && a->k_tscale && a->v_tscale, FA4_ERR_NULL,
            "decode: NVFP4 tensor scales are NULL");
  const void *ptrs16[] = {a->q1_codes, a->q2_codes, a->k_codes, a->v_codes};
  for (const void *p : ptrs16) REQUIRE(aligned(p, 16), FA4_ERR_ALIGN, "decode: code arrays must be 16-byte aligned");
  // block scales: 8 (NVFP4) or 4 (MXFP4) bytes per row, read in whole rows
  const size_t sal = a->fmt == FA4_NVFP4 ? 8 : 4;
  const void *ptrs8[] = {a->q1_scales, a->q2_scales, a->k_scales, a->v_scales};
  for (const void *p : ptrs8)
    REQUIRE(aligned(p, sal), FA4_ERR_ALIGN, "decode: scale arrays must be %zu-byte aligned", sal);
  const size_t need = fa4::decode_workspace_bytes(a);
  REQUIRE(ws && ws_bytes >= need, FA4_ERR_WORKSPACE, "decode: workspace %zu bytes, %zu needed", ws_bytes, need);
  REQUIRE(aligned(ws, 256), FA4_ERR_ALIGN, "decode: workspace must be 256-byte aligned");
  return hip_status(fa4::launch_decode(a, ws, (hipStream_t)stream), "decode launch");
}

}  // extern "C"

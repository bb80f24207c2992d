// Internal declarations shared by the host-side C ABI and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include "../../include/fa4.h"

namespace fa4 {

// Each launcher enqueues its kernels on `s` and returns the first launch error (hipSuccess if none).
// Arguments have been validated by the caller.
hipError_t launch_quantize(const fa4_qinput *in, uint32_t flags, const fa4_qoutput *out,
                           const fa4_qoutput *residual, float *row_norm2, hipStream_t s);
hipError_t launch_quantize_prefill(const fa4_qinput *q, const fa4_qinput *k, const fa4_qinput *v,
                                   const fa4_qoutput *qo, const fa4_qoutput *ko, const fa4_qoutput *vo,
                                   float *q_norm2, float *k_norm2, hipStream_t s);
int64_t prefill_quant_blocks(const fa4_qinput *q, const fa4_qinput *k, const fa4_qinput *v, bool v4);
hipError_t launch_smoothing(const fa4_qinput *q, const fa4_qinput *k, float *q_scale, float *k_scale,
                            hipStream_t s);
hipError_t launch_select(const float *qn, const float *kn, int B, int Hq, int Hkv, int Lq, int Lk,
                         int causal, int num, int den, uint8_t *bitmap, int32_t *counts, hipStream_t s);
hipError_t launch_attn(const fa4_attn_args *a, hipStream_t s);
size_t decode_workspace_bytes(const fa4_decode_args *a);
hipError_t launch_decode(const fa4_decode_args *a, void *ws, hipStream_t s);

// MLA geometry of fa4_decode_paged: latent row width (key), value width, query heads.
constexpr int MLA_D = 576, MLA_DV = 512, MLA_H = 16;
constexpr int DEC_SPLIT_KEYS = 2048;   // keys per workgroup of the GQA decode (one split)
constexpr int MLA_PAGES = 40;          // pages (64-key tiles) per workgroup of the MLA decode
size_t decode_mla_workspace_bytes(const fa4_decode_args *a);
hipError_t launch_decode_mla(const fa4_decode_args *a, void *ws, hipStream_t s);

}  // namespace fa4

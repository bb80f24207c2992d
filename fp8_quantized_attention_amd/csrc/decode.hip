// Decode attention over a paged NVFP4 KV cache for gfx950, with a dual-residual NVFP4 query.
//
// Source: "BitDecoding-FP4" (sns.style digest): native FP4 KV-cache decoding over pages, the query
// split into two FP4 tensors (the second carries the first one's residual), probabilities quantized
// under a scale that cannot underflow, and the query heads of a GQA group stacked into one
// matrix-core tile. "MpFA QK4V8" section 3.3: the softmax statistics stay in FP32.
//
// Work decomposition: the keys of each (sequence, key head) are cut into splits of 512 keys; a
// workgroup owns one split and each of its 4 waves one 128-key tile (the probability tile). The 8
// query rows of a GQA group (4 heads x {Q1, Q2}) form the columns of a 16x16x32 fp16 MFMA whose rows
// are 16 keys: NVFP4 values code * s_b are exact in fp16 (at most 6 significant bits), so K and Q
// codes are expanded in registers (hardware fp4->fp16 conversion, then one packed multiply by the
// block scale) and the tensor scales are applied to the fp32 scores. The d axis of the QK product is
// permuted so that each lane's operand is one 16-byte run of a key's codes. V is expanded into LDS
// (fp16) and read back transposed (ds_read_b64_tr_b16) as the A operand of O^T = V^T P^T; P^ = E4M3
// (448 P') is exact in fp16. A tile's (max, sum, P^V) is merged over the 4 waves in LDS and written
// as the split's partial; a second kernel merges the splits of each (sequence, head).
#include "fa4_device.h"
#include "fa4_internal.h"

namespace fa4 {

constexpr int DEC_THREADS = 256;
constexpr int DEC_SPLIT = 512;            // keys per workgroup (4 tiles of 128)
constexpr int DEC_PART = 130;             // floats per (split, head) partial: m, l, O[128]
constexpr int V16_RS = 272;               // LDS row stride (bytes) of fp16 V rows
constexpr float DEC_LOG2E = 1.4426950408889634f;

struct DecArgs {
  const uint8_t *q1c, *q1s, *q2c, *q2s;
  const float *q1t, *q2t;
  const uint8_t *kc, *ks, *vc, *vs;
  const float *kt, *vt;
  const int32_t *pt, *ctx;
  int B, Hq, Hkv, max_pages, nsplit;
  int64_t num_pages;
  float scale;
  float *ws, *o;
};

typedef __attribute__((address_space(3))) v4s lds_v4s_d;

// 8 E2M1 codes (4 bytes) times an fp16 block scale, as exact fp16 values.
__device__ __forceinline__ v8h expand8(uint32_t w, _Float16 sb) {
  const v2h s2 = {sb, sb};
  const v2h t0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const v2h t1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const v2h t2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const v2h t3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return (v8h){t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
}

__device__ __forceinline__ _Float16 e4m3_f16(uint32_t code) { return (_Float16)e4m3_value(code); }

__global__ void __launch_bounds__(DEC_THREADS) decode_split_kernel(DecArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t vl[4][32 * V16_RS];   // fp16 V, 32 keys per wave
  __shared__ float part[4][4][DEC_PART];
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int L = min(a.ctx[b], a.max_pages * 64);
  if (split * DEC_SPLIT >= L) return;                      // uniform per workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;                  // MFMA column (query row) / lane group
  const int t0 = split * DEC_SPLIT + wave * 128;           // this wave's first key
  const bool has_tile = t0 < L;
  const int32_t *pt = a.pt + (int64_t)b * a.max_pages;

  float mt = -INFINITY, lsum = 0.0f;
  v4f acc[8];
#pragma unroll
  for (int i = 0; i < 8; i++) acc[i] = (v4f){0.f, 0.f, 0.f, 0.f};

  if (has_tile) {
    // ---- query operand: column n = residual (n / 4) of head 4 kvh + n % 4; columns 8..15 are zero.
    // Physical d of (lane group g, step s, element j) = 32 g + 8 s + j.
    v8h qop[4];
    const int hq = kvh * 4 + (n & 3);
    const bool realq = n < 8;
    {
      const uint8_t *qc = (n < 4 ? a.q1c : a.q2c) + ((int64_t)b * a.Hq + hq) * 64 + 16 * g;
      const uint8_t *qs = (n < 4 ? a.q1s : a.q2s) + ((int64_t)b * a.Hq + hq) * 8 + 2 * g;
      const v4i w = realq ? *reinterpret_cast<const v4i *>(qc) : (v4i){0, 0, 0, 0};
      const uint32_t sw = realq ? *reinterpret_cast<const uint16_t *>(qs) : 0u;
#pragma unroll
      for (int s = 0; s < 4; s++) qop[s] = expand8((uint32_t)w[s], e4m3_f16((sw >> (8 * (s >> 1))) & 0xffu));
    }
    // ---- S^T = K Q^T for 8 blocks of 16 keys
    v4f S[8];
#pragma unroll
    for (int kb = 0; kb < 8; kb++) {
      const int key = t0 + 16 * kb + n;
      v4i w = {0, 0, 0, 0};
      uint32_t sw = 0;
      if (key < L) {
        const int pg = pt[key >> 6];
        if (pg >= 0 && (int64_t)pg < a.num_pages) {
          const int64_t row = ((int64_t)pg * a.Hkv + kvh) * 64 + (key & 63);
          w = *reinterpret_cast<const v4i *>(a.kc + row * 64 + 16 * g);
          sw = *reinterpret_cast<const uint16_t *>(a.ks + row * 8 + 2 * g);
        }
      }
      S[kb] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; s++) {
        const v8h kop = expand8((uint32_t)w[s], e4m3_f16((sw >> (8 * (s >> 1))) & 0xffu));
        S[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[s], S[kb], 0, 0, 0);
      }
    }
    // ---- scores of head n (lanes n < 4): x = log2e * scale * s_tK * (s_t1 D[n] + s_t2 D[n+4])
    const int64_t bq = (int64_t)b * a.Hq + kvh * 4 + (n & 3);
    const float ck = DEC_LOG2E * a.scale * a.kt[(int64_t)b * a.Hkv + kvh];
    const float c1 = ck * a.q1t[bq], c2 = ck * a.q2t[bq];
#pragma unroll
    for (int kb = 0; kb < 8; kb++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float d2 = __shfl_down(S[kb][i], 4, 16);
        const int key = t0 + 16 * kb + 4 * g + i;
        const float x = c1 * S[kb][i] + c2 * d2;
        S[kb][i] = (n < 4 && key < L) ? x : -INFINITY;
        mt = fmaxf(mt, S[kb][i]);
      }
    mt = fmaxf(mt, shfl_xor_f(mt, 16));
    mt = fmaxf(mt, shfl_xor_f(mt, 32));
    // ---- P' = 2^(x - m~), P^ = E4M3(448 P') (exact in fp16); columns >= 4 get zeros
    v8h pop[4];
#pragma unroll
    for (int kb = 0; kb < 8; kb++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float p = (n < 4) ? __builtin_amdgcn_exp2f(S[kb][i] - mt) : 0.0f;
        lsum += p;
        pop[kb >> 1][4 * (kb & 1) + i] = e4m3_f16(e4m3_encode(448.0f * p));
      }
    // ---- O^T += V^T P^T, 32 keys at a time through this wave's LDS region
    uint8_t *vw = vl[wave];
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      {
        const int r = lane & 31, dh = lane >> 5;              // key row r, d half dh (64 elements)
        const int key = t0 + 32 * ks + r;
        v4i w[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
        uint32_t sw = 0;
        if (key < L) {
          const int pg = pt[key >> 6];
          if (pg >= 0 && (int64_t)pg < a.num_pages) {
            const int64_t row = ((int64_t)pg * a.Hkv + kvh) * 64 + (key & 63);
            w[0] = *reinterpret_cast<const v4i *>(a.vc + row * 64 + 32 * dh);
            w[1] = *reinterpret_cast<const v4i *>(a.vc + row * 64 + 32 * dh + 16);
            sw = *reinterpret_cast<const uint32_t *>(a.vs + row * 8 + 4 * dh);
          }
        }
#pragma unroll
        for (int c = 0; c < 2; c++)
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const int blk = 2 * c + (e >> 1);                   // 16-element block within the half
            const v8h vv = expand8((uint32_t)w[c][e], e4m3_f16((sw >> (8 * blk)) & 0xffu));
            *reinterpret_cast<v8h *>(vw + r * V16_RS + 2 * (64 * dh + 32 * c + 8 * e)) = vv;
          }
      }
      // the region is private to this wave and LDS requests of a wave complete in order; the fence
      // only stops the compiler from moving the transposed reads above the writes
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const v8h pb = pop[ks];
#pragma unroll
      for (int db = 0; db < 8; db++) {
        // A operand: row d = 16 db + n, keys {4g + t, 16 + 4g + t}; tr16 source lane 16g + aa + 4t
        const int aa = lane & 3, t = (lane >> 2) & 3;
        v4s rr[2];
#pragma unroll
        for (int v = 0; v < 2; v++) {
          const int key = 16 * v + 4 * g + t;
          rr[v] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_d *)(vw + key * V16_RS + 2 * (16 * db + 4 * aa)));
        }
        // whole-vector reinterpretation (inserting bit-cast elements one at a time miscompiles)
        const v8h vop = __builtin_bit_cast(v8h, (v8s)__builtin_shufflevector(rr[0], rr[1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pb, acc[db], 0, 0, 0);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    lsum += shfl_xor_f(lsum, 16);
    lsum += shfl_xor_f(lsum, 32);
  }
  // ---- per-wave partial -> LDS (lanes n < 4 hold head n; d = 16 db + 4 g + i)
  if (n < 4) {
    if (g == 0) { part[wave][n][0] = mt; part[wave][n][1] = lsum; }
#pragma unroll
    for (int db = 0; db < 8; db++)
#pragma unroll
      for (int i = 0; i < 4; i++) part[wave][n][2 + 16 * db + 4 * g + i] = acc[db][i];
  }
  __syncthreads();
  // ---- merge the 4 tiles: thread -> (head, two d values)
  {
    const int hd = tid >> 6, d0 = 2 * (tid & 63);
    float mm = -INFINITY;
    for (int w = 0; w < 4; w++) mm = fmaxf(mm, part[w][hd][0]);
    float l = 0.f, o0 = 0.f, o1 = 0.f;
    for (int w = 0; w < 4; w++) {
      const float mw = part[w][hd][0];
      if (mw == -INFINITY) continue;
      const float f = __builtin_amdgcn_exp2f(mw - mm);
      l += f * part[w][hd][1];
      o0 += f * part[w][hd][2 + d0];
      o1 += f * part[w][hd][3 + d0];
    }
    float *dst = a.ws + ((((int64_t)b * a.Hkv + kvh) * a.nsplit + split) * 4 + hd) * DEC_PART;
    if (d0 == 0) { dst[0] = mm; dst[1] = l; }
    dst[2 + d0] = o0;
    dst[3 + d0] = o1;
  }
}

// Merge the splits of each (sequence, head): O = sum e^(m_s - m) O_s / sum e^(m_s - m) l_s, times
// the V tensor scale / 448 (P^ carried a factor 448).
__global__ void __launch_bounds__(128) decode_combine_kernel(DecArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int kvh = h / 4, hd = h & 3;
  const int L = min(a.ctx[b], a.max_pages * 64);
  const int ns = (L + DEC_SPLIT - 1) / DEC_SPLIT;
  const float *base = a.ws + (((int64_t)b * a.Hkv + kvh) * a.nsplit * 4 + hd) * DEC_PART;
  float mm = -INFINITY;
  for (int s = 0; s < ns; s++) mm = fmaxf(mm, base[(int64_t)s * 4 * DEC_PART]);
  float l = 0.f, o = 0.f;
  for (int s = 0; s < ns; s++) {
    const float *p = base + (int64_t)s * 4 * DEC_PART;
    const float f = __builtin_amdgcn_exp2f(p[0] - mm);
    l += f * p[1];
    o += f * p[2 + d];
  }
  const float vts = a.vt[(int64_t)b * a.Hkv + kvh] * (1.0f / 448.0f);
  a.o[((int64_t)b * a.Hq + h) * 128 + d] = o / l * vts;
}

static DecArgs make_dec(const fa4_decode_args *p, void *ws) {
  DecArgs x;
  x.q1c = p->q1_codes; x.q1s = p->q1_scales; x.q2c = p->q2_codes; x.q2s = p->q2_scales;
  x.q1t = p->q1_tscale; x.q2t = p->q2_tscale;
  x.kc = p->k_codes; x.ks = p->k_scales; x.vc = p->v_codes; x.vs = p->v_scales;
  x.kt = p->k_tscale; x.vt = p->v_tscale;
  x.pt = p->page_table; x.ctx = p->ctx_len;
  x.B = p->B; x.Hq = p->Hq; x.Hkv = p->Hkv; x.max_pages = p->max_pages;
  x.nsplit = (p->max_pages * 64 + DEC_SPLIT - 1) / DEC_SPLIT;
  x.num_pages = p->num_pages;
  x.scale = p->softmax_scale;
  x.ws = static_cast<float *>(ws); x.o = p->o;
  return x;
}

size_t decode_workspace_bytes(const fa4_decode_args *p) {
  const int64_t nsplit = ((int64_t)p->max_pages * 64 + DEC_SPLIT - 1) / DEC_SPLIT;
  return (size_t)p->B * p->Hkv * nsplit * 4 * DEC_PART * sizeof(float);
}

hipError_t launch_decode(const fa4_decode_args *p, void *ws, hipStream_t s) {
  if (p->B == 0) return hipSuccess;
  const DecArgs x = make_dec(p, ws);
  hipLaunchKernelGGL(decode_split_kernel, dim3(x.nsplit, x.Hkv, x.B), dim3(DEC_THREADS), 0, s, x);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(x.Hq, x.B), dim3(128), 0, s, x);
  return hipGetLastError();
}

}  // namespace fa4

// Decode in the MLA geometry over a paged MXFP4 latent cache for gfx950.
//
// Source: "BitDecoding-FP4" (sns.style digest): FP4 KV-cache decode with a dual-residual FP4 query,
// reported for GQA and for MLA attention. In the MLA geometry every query head of a sequence attends
// to one shared latent row per token: its 512 latent values and 64 rotary values are the key, the
// latent values alone the value, and each head's query is its absorbed form (576 values). "MpFA
// QK4V8" section 3.3: the softmax statistics stay in FP32.
//
// Cache: MXFP4 rows (E8M0 scale per 32 values) in column-sliced pages. Page p holds slice j (columns
// 64 j .. 64 j + 63) of its 64 tokens as codes [9][64][32 B] and E8M0 scales [9][64][2]: the paged
// quantizer's output for the rows cut into nine 64-wide heads. A page is one probability tile.
//
// A workgroup owns MLA_PAGES consecutive pages of one sequence and brings each page into LDS by
// direct global->LDS loads one page ahead. Wave w scores keys 16 w .. 16 w + 15 of the page against
// the 16 heads with 16x16x128 scaled FP4 MFMAs: the key codes and their scale bytes are the A operand,
// the head's [Q1 | Q2] codes (1152 values, so the dual-residual sum forms in the accumulator) the B
// operand. The page maximum and sum of each head are exchanged through LDS and P^ = E4M3(448 P')
// (exact in bf16) is written to LDS as [head][key]. For PV wave w owns the values d = 128 w ..
// 128 w + 127: each key's 4-byte run of 8 values is converted to bf16 with the key's block scale (code
// * 2^e has at most 2 significant bits), an 8x8 transpose of 16-bit values gives the key-contiguous A
// operand of O^T = V^T P^T, and a 16x16x32 bf16 MFMA adds a 32-key quarter. Each wave keeps the
// running maximum, sum and its part of O; a second kernel merges the workgroups of a sequence.
#include "fa4_device.h"
#include "fa4_internal.h"

namespace fa4 {

constexpr int MLA_THREADS = 256;
constexpr int MLA_PAGES = 32;                     // pages (64-key tiles) per workgroup
constexpr int MLA_NS = MLA_D / 64;                // column slices per page
constexpr int MLA_TC = MLA_NS * 64 * 32;          // code bytes per page
constexpr int MLA_TS = MLA_NS * 64 * 2;           // scale bytes per page
constexpr int MLA_PART = 2 + MLA_DV;              // floats per (split, head) partial: m, l, O
constexpr int MLA_PP = 72;                        // bf16 pitch of a head's row of P^ in LDS
constexpr float MLA_LOG2E = 1.4426950408889634f;

struct MlaArgs {
  const uint8_t *q1c, *q1s, *q2c, *q2s;           // [B*16][288] codes, [B*16][18] E8M0
  const uint8_t *kc, *ks;                         // [num_pages][9][64][32], [num_pages][9][64][2]
  const int32_t *pt, *ctx;
  int B, max_pages, nsplit;
  int64_t num_pages;
  float scale;
  float *ws, *o;
};

typedef __attribute__((address_space(3))) void mla_lds_t;
__device__ __forceinline__ void mla_dma16(const void *g, uint8_t *l) {
  __builtin_amdgcn_global_load_lds(g, (mla_lds_t *)l, 16, 0, 0);
}

__global__ void __launch_bounds__(MLA_THREADS) decode_mla_kernel(MlaArgs a) {
  __shared__ __align__(16) uint8_t tile[2][MLA_TC + MLA_TS];
  __shared__ __align__(16) uint16_t pT[MLA_H * MLA_PP];
  __shared__ float red_m[4][MLA_H], red_l[4][MLA_H];
  // Workgroup order: sequence fastest, split slowest (every XCD gets the same mix of sequences and
  // the mostly empty trailing splits come last).
  const int split = (int)(blockIdx.x / (unsigned)a.B), b = (int)(blockIdx.x - (unsigned)split * a.B);
  const int L = min(a.ctx[b], a.max_pages * 64);
  const int p0 = split * MLA_PAGES;
  if (p0 * 64 >= L) return;                                   // uniform per workgroup
  const int np = min(MLA_PAGES, (L + 63) / 64 - p0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;                     // MFMA row/column, lane group
  const int32_t *pt = a.pt + (int64_t)b * a.max_pages;

  // ---- B operand of QK: head n; chunk s, lane group g holds values 128 s + 32 g .. + 31 of the
  // concatenated [Q1 | Q2] (a 32-block never straddles the two) with its E8M0 scale
  v8i qop[9];
  int qsc[9];
  {
    const int64_t bh = (int64_t)b * MLA_H + n;
#pragma unroll
    for (int s = 0; s < 9; s++) {
      const int c = 128 * s + 32 * g;
      const bool r2 = c >= MLA_D;
      const int d0 = r2 ? c - MLA_D : c;
      const v4i w = *reinterpret_cast<const v4i *>((r2 ? a.q2c : a.q1c) + bh * (MLA_D / 2) + d0 / 2);
      qop[s] = (v8i){w[0], w[1], w[2], w[3], 0, 0, 0, 0};
      qsc[s] = (r2 ? a.q2s : a.q1s)[bh * (MLA_D / 32) + d0 / 32];
    }
  }

  // physical page of the split's page i (wave-uniform); an id outside the cache reads page 0 and
  // masks every key of the tile
  auto page_id = [&](int i) -> int {
    return __builtin_amdgcn_readfirstlane(((const __attribute__((address_space(4))) int32_t *)pt)[p0 + i]);
  };
  auto page_ok = [&](int pg) -> bool { return pg >= 0 && (int64_t)pg < a.num_pages; };
  // page -> LDS: codes in 18 wave-loads of 1 KB, scales in 1 KB + 128 B
  auto issue = [&](int i, int buf) {
    const int pg0 = page_id(i);
    const int64_t pg = page_ok(pg0) ? pg0 : 0;
    const uint8_t *gc = a.kc + pg * MLA_TC, *gs = a.ks + pg * MLA_TS;
    uint8_t *lc = tile[buf];
    for (int k = wave; k < MLA_TC / 1024; k += 4) mla_dma16(gc + 1024 * k + 16 * lane, lc + 1024 * k);
    if (wave == 2) mla_dma16(gs + 16 * lane, lc + MLA_TC);
    if (wave == 3 && lane < (MLA_TS - 1024) / 16) mla_dma16(gs + 1024 + 16 * lane, lc + MLA_TC + 1024);
  };

  const float cs = a.scale * MLA_LOG2E;
  float m_run = -INFINITY, l_run = 0.0f;
  v4f acc[8];
#pragma unroll
  for (int e = 0; e < 8; e++) acc[e] = (v4f){0.f, 0.f, 0.f, 0.f};
  issue(0, 0);
  for (int i = 0; i < np; i++) {
    const int buf = i & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();                                           // page i landed; page i - 1 consumed
    if (i + 1 < np) issue(i + 1, buf ^ 1);                      // in flight during this page's work
    const int kval = page_ok(page_id(i)) ? min(64, L - 64 * (p0 + i)) : 0;   // valid keys (uniform)
    if (kval == 0) continue;
    const uint8_t *lc = tile[buf];

    // ---- S^T = K Q^T for keys 16 wave .. + 15 (rows) and the 16 heads (columns)
    v4f S = (v4f){0.f, 0.f, 0.f, 0.f};
    {
      const int krow = 16 * wave + n;
#pragma unroll
      for (int s = 0; s < 9; s++) {
        const int c = 128 * s + 32 * g;
        const int d0 = c >= MLA_D ? c - MLA_D : c;
        const int sl = d0 >> 6, hf = (d0 >> 5) & 1;
        const v4i t = *reinterpret_cast<const v4i *>(lc + sl * 2048 + krow * 32 + hf * 16);
        const int ksc = lc[MLA_TC + sl * 128 + krow * 2 + hf];
        S = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4((v8i){t[0], t[1], t[2], t[3], 0, 0, 0, 0}, qop[s],
                                                             S, 4, 4, 0, ksc, 0, qsc[s]);
      }
    }
    // ---- this lane: head n, keys 16 wave + 4 g + t
    float x[4], mw = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; t++) {
      x[t] = 16 * wave + 4 * g + t < kval ? S[t] * cs : -INFINITY;
      mw = fmaxf(mw, x[t]);
    }
    mw = fmaxf(mw, shfl_xor_f(mw, 16));
    mw = fmaxf(mw, shfl_xor_f(mw, 32));
    if (g == 0) red_m[wave][n] = mw;
    __syncthreads();
    const float mt = fmaxf(fmaxf(red_m[0][n], red_m[1][n]), fmaxf(red_m[2][n], red_m[3][n]));
    float ls = 0.0f;
    {
      float p[4];
#pragma unroll
      for (int t = 0; t < 4; t++) {
        p[t] = __builtin_amdgcn_exp2f(x[t] - mt);
        ls += p[t];
      }
      // P^ = E4M3(448 P'), as bf16 (exact)
      const uint32_t c01 = e4m3_encode2(448.0f * p[0], 448.0f * p[1]);
      const uint32_t c23 = e4m3_encode2(448.0f * p[2], 448.0f * p[3]);
      const uint32_t u0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c01, 1.0f, false));
      const uint32_t u1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c23, 1.0f, false));
      *reinterpret_cast<uint2 *>(&pT[n * MLA_PP + 16 * wave + 4 * g]) = make_uint2(u0, u1);
    }
    ls += shfl_xor_f(ls, 16);
    ls += shfl_xor_f(ls, 32);
    if (g == 0) red_l[wave][n] = ls;
    __syncthreads();
    const float lt = (red_l[0][n] + red_l[1][n]) + (red_l[2][n] + red_l[3][n]);
    // running merge: O and l stay relative to the running maximum
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);    // 0 on the first tile
    const float f = __builtin_amdgcn_exp2f(mt - m_new);
    l_run = l_run * alpha + lt * f;
    m_run = m_new;

    // ---- O^T += V^T P^T for values d = 128 wave + 8 n + e (A row n of accumulator e), two quarters
    v4f tmp[8];
#pragma unroll
    for (int e = 0; e < 8; e++) tmp[e] = (v4f){0.f, 0.f, 0.f, 0.f};
    const int sl = 2 * wave + (n >> 3);                        // slice of this lane's 8 values
#pragma unroll
    for (int q = 0; q < 2; q++) {
      // B: head n, keys 32 q + 8 g .. + 7
      const v8bf pb = *reinterpret_cast<const v8bf *>(&pT[n * MLA_PP + 32 * q + 8 * g]);
      // A: key 32 q + 8 g + j's run of 8 values -> bf16 with its block scale 2^(code - 127); scale code 0
      // (blocks below 6 * 2^-127) is taken as 2^-126 so that the conversion's scale stays a normal
      // float; keys past the context take 2^0 (their P^ is 0)
      uint32_t kw[8][4];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int key = 32 * q + 8 * g + j;
        const uint32_t wd = *reinterpret_cast<const uint32_t *>(lc + sl * 2048 + key * 32 + 4 * (n & 7));
        uint32_t code = lc[MLA_TC + sl * 128 + key * 2 + ((n & 7) >> 2)];
        code = key < kval ? code : 127u;
        const float sc = __uint_as_float((code > 1u ? code : 1u) << 23);
        kw[j][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 0));
        kw[j][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 1));
        kw[j][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 2));
        kw[j][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, sc, 3));
      }
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        v4i av;
#pragma unroll
        for (int jp = 0; jp < 4; jp++)
          av[jp] = (int)__builtin_amdgcn_perm(kw[2 * jp + 1][e >> 1], kw[2 * jp][e >> 1], sel);
        tmp[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av), pb, tmp[e], 0, 0, 0);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; e++) acc[e] = acc[e] * alpha + tmp[e] * f;
  }
  // ---- partial of this split: lane (head n, group g) holds d = 128 wave + 32 g + 8 t + e in acc[e][t]
  float *dst = a.ws + (((int64_t)b * a.nsplit + split) * MLA_H + n) * MLA_PART;
  if (wave == 0 && g == 0) {
    dst[0] = m_run;
    dst[1] = l_run;
  }
#pragma unroll
  for (int e = 0; e < 8; e++)
#pragma unroll
    for (int t = 0; t < 4; t++) dst[2 + 128 * wave + 32 * g + 8 * t + e] = acc[e][t];
}

// Merge the splits of each (sequence, head): O = sum e^(m_s - m) O_s / sum e^(m_s - m) l_s / 448 (P^
// carried a factor 448). Thread: values tid and tid + 256.
__global__ void __launch_bounds__(256) decode_mla_combine_kernel(MlaArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int L = min(a.ctx[b], a.max_pages * 64);
  const int ns = ((L + 63) / 64 + MLA_PAGES - 1) / MLA_PAGES;
  const float *base = a.ws + ((int64_t)b * a.nsplit * MLA_H + h) * MLA_PART;
  constexpr int SS = MLA_H * MLA_PART;                       // floats between splits
  float mm = -INFINITY;
  for (int s = 0; s < ns; s++) mm = fmaxf(mm, base[(int64_t)s * SS]);
  float l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s = 0; s < ns; s++) {
    const float *p = base + (int64_t)s * SS;
    if (p[0] == -INFINITY) continue;
    const float f = __builtin_amdgcn_exp2f(p[0] - mm);
    l += f * p[1];
    o0 += f * p[2 + tid];
    o1 += f * p[2 + 256 + tid];
  }
  float *o = a.o + ((int64_t)b * MLA_H + h) * MLA_DV;
  const float r = 1.0f / (448.0f * l);
  o[tid] = o0 * r;
  o[tid + 256] = o1 * r;
}

static MlaArgs make_mla(const fa4_decode_args *p, void *ws) {
  MlaArgs x;
  x.q1c = p->q1_codes; x.q1s = p->q1_scales; x.q2c = p->q2_codes; x.q2s = p->q2_scales;
  x.kc = p->k_codes; x.ks = p->k_scales;
  x.pt = p->page_table; x.ctx = p->ctx_len;
  x.B = p->B; x.max_pages = p->max_pages;
  x.nsplit = (p->max_pages + MLA_PAGES - 1) / MLA_PAGES;
  x.num_pages = p->num_pages;
  x.scale = p->softmax_scale;
  x.ws = static_cast<float *>(ws); x.o = p->o;
  return x;
}

size_t decode_mla_workspace_bytes(const fa4_decode_args *p) {
  const int64_t nsplit = ((int64_t)p->max_pages + MLA_PAGES - 1) / MLA_PAGES;
  return (size_t)p->B * nsplit * MLA_H * MLA_PART * sizeof(float);
}

hipError_t launch_decode_mla(const fa4_decode_args *p, void *ws, hipStream_t s) {
  if (p->B == 0) return hipSuccess;
  const MlaArgs x = make_mla(p, ws);
  hipLaunchKernelGGL(decode_mla_kernel, dim3((unsigned)((int64_t)x.nsplit * x.B)), dim3(MLA_THREADS), 0, s, x);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_mla_combine_kernel, dim3(MLA_H, x.B), dim3(256), 0, s, x);
  return hipGetLastError();
}

}  // namespace fa4

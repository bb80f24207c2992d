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
// operand. The page maximum and sum of each head are exchanged through LDS. The page's reference is a
// power of two 2^r (r the smallest integer >= its largest score in log2 units, the prefill's rule), so
// P' = 2^(x - r) and the page's weight against the running reference, 2^(r - R), is exact: it rides
// on P^ = E4M3(448 P') * 2^(r - R) (exact in bf16), written to LDS as [head][key]. For PV wave w owns
// the values d = 128 w .. 128 w + 127: each key's 4-byte run of 8 values is converted to bf16 with the
// key's block scale (code * 2^e has at most 2 significant bits), an 8x8 transpose of 16-bit values
// gives the key-contiguous A operand of O^T = V^T P^T, and a 16x16x32 bf16 MFMA adds a 32-key quarter
// straight into the accumulator. A second kernel merges the workgroups of a sequence.
#include "fa4_device.h"
#include "fa4_internal.h"

namespace fa4 {

constexpr int MLA_THREADS = 256;
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

constexpr int MLA_NB = 2;                         // LDS page buffers: pages are loaded MLA_NB - 1 ahead
constexpr float MLA_HEADROOM = 32.0f;             // largest page weight 2^k before the reference is raised
constexpr int MLA_DMA = 5;                        // direct loads per wave per page (each wave alike)

// Direct global->LDS load of 16 bytes per lane to l + 16 * lane (l wave-uniform). Written as inline asm
// so that the compiler, which cannot tell which LDS bytes such a load writes, does not wait for it
// before every later LDS read; the kernel waits for these loads itself (vmcnt) before the barrier
// that publishes a page. M0 takes the LDS address and needs one wait state before the load; no other
// instruction of these kernels reads M0 (the compiler warns that it does not preserve a clobbered M0).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void mla_dma16(const void *g, uint8_t *l) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t *)l);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}
#pragma clang diagnostic pop
// Wait until at most n of this wave's direct loads are in flight (n: 0, MLA_DMA or 2 MLA_DMA).
__device__ __forceinline__ void mla_wait(int n) {
  if (n >= 2 * MLA_DMA) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
  else if (n >= MLA_DMA) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// max / sum over the four lanes n, n + 16, n + 32, n + 48 (lane swaps on the VALU, no LDS)
__device__ __forceinline__ float quad_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Three workgroups per CU (LDS 50 KB each): at most 168 VGPRs.
__global__ void __launch_bounds__(MLA_THREADS) __attribute__((amdgpu_waves_per_eu(3))) decode_mla_kernel(MlaArgs a) {
  __shared__ __align__(16) uint8_t tile[MLA_NB][MLA_TC + MLA_TS];
  __shared__ __align__(16) uint8_t qlds[2][MLA_H][MLA_D / 2];     // Q1, Q2 codes of the 16 heads
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
  // concatenated [Q1 | Q2] (a 32-block never straddles the two). The codes go to LDS (read once per
  // page); the E8M0 scales stay in registers, four per register, picked by the MFMA's byte select.
  for (int idx = tid; idx < 2 * MLA_H * (MLA_D / 32); idx += MLA_THREADS) {
    const int r = idx / (MLA_H * (MLA_D / 32)), hc = idx - r * (MLA_H * (MLA_D / 32));
    const int h = hc / (MLA_D / 32), c16 = hc - h * (MLA_D / 32);
    *reinterpret_cast<v4i *>(&qlds[r][h][16 * c16]) =
        *reinterpret_cast<const v4i *>((r ? a.q2c : a.q1c) + ((int64_t)b * MLA_H + h) * (MLA_D / 2) + 16 * c16);
  }
  uint32_t qsc[3] = {0u, 0u, 0u};
  {
    const int64_t bh = (int64_t)b * MLA_H + n;
#pragma unroll
    for (int s = 0; s < 9; s++) {
      const int c = 128 * s + 32 * g;
      const bool r2 = c >= MLA_D;
      const int d0 = r2 ? c - MLA_D : c;
      qsc[s >> 2] |= (uint32_t)(r2 ? a.q2s : a.q1s)[bh * (MLA_D / 32) + d0 / 32] << (8 * (s & 3));
    }
    // use the scales here, so that the compiler waits for their loads before the page loop
    // (inside it the count would also cover page loads in flight)
    asm volatile("" ::"v"(qsc[0]), "v"(qsc[1]), "v"(qsc[2]));
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

  // Running state of head n: the reference R (an integer, log2 units), the sum and this wave's part
  // of O, both relative to 2^R. A page with reference r enters with the exact weight 2^(r - R), carried
  // by P^ into the MFMA; R is raised only when a page's r exceeds it by more than MLA_HEADROOM.
  const float cs = a.scale * MLA_LOG2E;
  float R = -INFINITY, l_run = 0.0f;
  v4f acc[8];
#pragma unroll
  for (int e = 0; e < 8; e++) acc[e] = (v4f){0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < MLA_NB - 1 && i < np; i++) issue(i, i);
  int buf = 0;
  for (int i = 0; i < np; i++) {
    mla_wait(MLA_DMA * min(MLA_NB - 2, np - 1 - i));           // this wave's loads of page i are done
    __syncthreads();                                           // page i landed; page i - 1 consumed
    if (i + MLA_NB - 1 < np) issue(i + MLA_NB - 1, buf == 0 ? MLA_NB - 1 : buf - 1);   // page i - 1's buffer
    const int cur = buf;
    buf = buf + 1 == MLA_NB ? 0 : buf + 1;
    const int kval = page_ok(page_id(i)) ? min(64, L - 64 * (p0 + i)) : 0;   // valid keys (uniform)
    if (kval == 0) continue;
    const uint8_t *lc = tile[cur];

    // ---- S^T = K Q^T for keys 16 wave .. + 15 (rows) and the 16 heads (columns)
    v4f S = (v4f){0.f, 0.f, 0.f, 0.f};
    {
      const int krow = 16 * wave + n;
#pragma unroll
      for (int s = 0; s < 9; s++) {
        const int c = 128 * s + 32 * g;
        const bool r2 = c >= MLA_D;
        const int d0 = r2 ? c - MLA_D : c;
        const int sl = d0 >> 6, hf = (d0 >> 5) & 1;
        const v4i t = *reinterpret_cast<const v4i *>(lc + sl * 2048 + krow * 32 + hf * 16);
        const int ksc = lc[MLA_TC + sl * 128 + krow * 2 + hf];
        const v4i qw = *reinterpret_cast<const v4i *>(&qlds[r2][n][d0 / 2]);
        const v8i ka = (v8i){t[0], t[1], t[2], t[3], 0, 0, 0, 0}, qb = (v8i){qw[0], qw[1], qw[2], qw[3], 0, 0, 0, 0};
        switch (s & 3) {                                       // the byte select must be a constant
          case 0: S = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qb, S, 4, 4, 0, ksc, 0, (int)qsc[s >> 2]); break;
          case 1: S = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qb, S, 4, 4, 0, ksc, 1, (int)qsc[s >> 2]); break;
          case 2: S = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qb, S, 4, 4, 0, ksc, 2, (int)qsc[s >> 2]); break;
          default: S = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qb, S, 4, 4, 0, ksc, 3, (int)qsc[s >> 2]); break;
        }
      }
    }
    // ---- this lane: head n, keys 16 wave + 4 g + t; scores in log2 units
    float x[4], mw = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; t++) {
      x[t] = 16 * wave + 4 * g + t < kval ? S[t] * cs : -INFINITY;
      mw = fmaxf(mw, x[t]);
    }
    mw = quad_max(mw);
    if (g == 0) red_m[wave][n] = mw;
    __syncthreads();
    // the page's reference: the smallest integer r >= its largest score (P' = 2^(x - r) <= 1)
    const float r = ceilf(fmaxf(fmaxf(red_m[0][n], red_m[1][n]), fmaxf(red_m[2][n], red_m[3][n])));
    if (__builtin_amdgcn_ballot_w64(r > R + MLA_HEADROOM) != 0) {  // uniform (always on the first page)
      const float R_new = fmaxf(R, r);
      const float alpha = R == -INFINITY ? 0.0f : __builtin_ldexpf(1.0f, (int)(R - R_new));
#pragma unroll
      for (int e = 0; e < 8; e++) acc[e] *= alpha;
      l_run *= alpha;
      R = R_new;
    }
    const int k = (int)fmaxf(r - R, -255.0f);                  // page weight 2^k, k <= MLA_HEADROOM
    float ls = 0.0f;
    {
      float p[4];
#pragma unroll
      for (int t = 0; t < 4; t++) {
        p[t] = __builtin_amdgcn_exp2f(x[t] - r);
        ls += p[t];
      }
      // P^ = E4M3(448 P') times 2^k, as bf16 (exact; a weight under 2^-126 adds nothing representable)
      const uint32_t c01 = e4m3_encode2(448.0f * p[0], 448.0f * p[1]);
      const uint32_t c23 = e4m3_encode2(448.0f * p[2], 448.0f * p[3]);
      const float w = __uint_as_float((uint32_t)(k + 127) << 23);
      uint32_t u0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c01, w, false));
      uint32_t u1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c23, w, false));
      if (k < -126) u0 = u1 = 0u;
      *reinterpret_cast<uint2 *>(&pT[n * MLA_PP + 16 * wave + 4 * g]) = make_uint2(u0, u1);
    }
    ls = quad_sum(ls);
    if (g == 0) red_l[wave][n] = ls;
    __syncthreads();
    l_run += ((red_l[0][n] + red_l[1][n]) + (red_l[2][n] + red_l[3][n])) * __builtin_ldexpf(1.0f, k);

    // ---- O^T += V^T P^T for values d = 128 wave + 8 n + e (A row n of accumulator e), two quarters
    const int sl = 2 * wave + (n >> 3);                        // slice of this lane's 8 values
#pragma unroll
    for (int q = 0; q < 2; q++) {
      // B: head n, keys 32 q + 8 g .. + 7
      const v8bf pb = *reinterpret_cast<const v8bf *>(&pT[n * MLA_PP + 32 * q + 8 * g]);
      // A: key 32 q + 8 g + j's run of 8 values -> bf16 with its block scale 2^(code - 127) (the
      // conversion reads the exponent field of its float scale as an E8M0 code, so code 0 acts as
      // 2^-127, exact in bf16); keys past the context take 2^0 (their P^ is 0)
      uint32_t kw[8][4];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int key = 32 * q + 8 * g + j;
        const uint32_t wd = *reinterpret_cast<const uint32_t *>(lc + sl * 2048 + key * 32 + 4 * (n & 7));
        uint32_t code = lc[MLA_TC + sl * 128 + key * 2 + ((n & 7) >> 2)];
        code = key < kval ? code : 127u;
        const float sc = __uint_as_float(code << 23);
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
        acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av), pb, acc[e], 0, 0, 0);
      }
    }
  }
  // ---- partial of this split, relative to 2^R: lane (head n, group g) holds d = 128 wave + 32 g + 8 t
  // + e in acc[e][t]
  float *dst = a.ws + (((int64_t)b * a.nsplit + split) * MLA_H + n) * MLA_PART;
  if (wave == 0 && g == 0) {
    dst[0] = R;
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
  // every split below ns wrote its partial (R = -inf and zeros when none of its pages was valid); the
  // loops are unrolled so that several splits' loads are in flight at once
  float mm = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < ns; s++) mm = fmaxf(mm, base[(int64_t)s * SS]);
  float l = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll 8
  for (int s = 0; s < ns; s++) {
    const float *p = base + (int64_t)s * SS;
    const float f = p[0] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(p[0] - mm);
    l += f * p[1];
    o0 += f * p[2 + tid];
    o1 += f * p[2 + 256 + tid];
  }
  float *o = a.o + ((int64_t)b * MLA_H + h) * MLA_DV;
  const float r = ns > 0 ? 1.0f / (448.0f * l) : 0.0f;      // an empty context (ctx_len <= 0) gives zeros
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

// Block-scaled quantizer kernels for gfx950: MXFP4, NVFP4 (tensor-amax pre-pass), dual-residual
// queries in either format, FP8 per-token V, optional 128-point Hadamard rotation and squared row norms.
//
// Sources: "MXFP vs NVFP4" (tqpw.cn 81738) sections 2.1-2.2 (block structures) and 3.1 (a fused
// quantization kernel computing in registers with coalesced global access); "BitDecoding-FP4"
// (dual-residual query, Hadamard rotation of keys); "General notes on quantization" (X ~ s * Q,
// per-token and per-group scales); "MpFA QK4V8" section 5.1 (zero maxima must not give a zero scale).
//
// Layout of the work: each lane reads one 16-byte run of a row (4 float or 8 bf16 elements), so a row
// spans d/4 (float) or d/8 (bf16) neighbouring lanes, and the packed codes of a row are written as one
// contiguous run, so both directions are coalesced. Block maxima come from xor-shuffles inside the
// lanes of a block (32 or 16 elements). A workgroup owns a chunk of rows of one group, so the NVFP4 tensor maximum is
// reduced in LDS and published with one atomicMax per workgroup (max is order-independent, so the
// result is deterministic).
#include "fa4_device.h"
#include "fa4_internal.h"

namespace fa4 {

constexpr int QUANT_THREADS = 256;
constexpr int QUANT_CHUNK = 64;      // rows per workgroup (one group; NVFP4 maxima reduce per workgroup)
constexpr int PREFILL_QK_CHUNK = 64; // rows per workgroup of Q and K in the one-launch prefill quantization
constexpr int NV_MAX_CHUNK = 256;    // rows per workgroup of NVFP4's tensor-maximum pass

// 1/sqrt(128) as the float64 nearest to 1/fl64(sqrt(128)).
#define FA4_RSQRT128 0x1.6a09e667f3bccp-4

struct QArgs {
  const void *x;
  int64_t outer, rows;
  int heads;
  int64_t so, sh, sr;
  const int32_t *row_counts;
  const int32_t *page_table;
  int page_size, max_pages;
  int64_t num_pages;
  uint8_t *codes, *bscales;
  float *scales;        // NVFP4: running max then tensor scale per group; FP8: per row
  uint8_t *rcodes, *rbscales;
  float *rscales;       // residual (dual) tensor maxima / scales
  float *norm2;
  float *fold_w, *fold_scale;
  const float *cscale;  // optional per-(head, channel) smoothing factors [heads][D]
};

// Elements per lane: one 16-byte load (8 bf16 or 4 float values).
template <int DT>
struct Epl {
  static constexpr int value = DT == 0 ? 4 : 8;
};

template <int DT, int E>
__device__ __forceinline__ void load_lane(const void *x, int64_t off, float v[E]) {
  if (DT == 0) {
    const float4 t = *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + off);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  } else {
    const uint4 t = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + off);
    const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = bf16_bits_to_float(w[i] & 0xffffu);
      v[2 * i + 1] = bf16_bits_to_float(w[i] >> 16);
    }
  }
}

// One lane's 16-byte run of a row, as loaded, and its E values widened to float.
template <int DT>
__device__ __forceinline__ uint4 load_raw(const void *x, int64_t off) {
  return DT == 0 ? *reinterpret_cast<const uint4 *>(static_cast<const float *>(x) + off)
                 : *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(x) + off);
}
template <int DT, int E>
__device__ __forceinline__ void widen_lane(const uint4 t, float v[E]) {
  const uint32_t w[4] = {t.x, t.y, t.z, t.w};
  if (DT == 0) {
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = __uint_as_float(w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = bf16_bits_to_float(w[i] & 0xffffu);
      v[2 * i + 1] = bf16_bits_to_float(w[i] >> 16);
    }
  }
}

// In-place Sylvester Hadamard transform of a 128-element row held E per lane over 128/E lanes,
// float64, then scaled by 1/sqrt(128) and rounded once to float32. Butterflies at distances below E
// run inside the lane; the others pair lanes (the lane whose mask bit is clear holds the lower
// index: a' = a + b there, b' = a - b in its partner).
template <int E>
__device__ __forceinline__ void hadamard128(float v[E]) {
  double a[E];
#pragma unroll
  for (int i = 0; i < E; i++) a[i] = v[i];
#pragma unroll
  for (int dist = 1; dist < E; dist <<= 1)
#pragma unroll
    for (int i = 0; i < E; i++)
      if ((i & dist) == 0) {
        const double u = a[i], w = a[i + dist];
        a[i] = u + w;
        a[i + dist] = u - w;
      }
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int m = 1; m < 128 / E; m <<= 1) {
#pragma unroll
    for (int i = 0; i < E; i++) {
      const double p = shfl_xor_d(a[i], m);
      a[i] = (lane & m) ? p - a[i] : a[i] + p;
    }
  }
#pragma unroll
  for (int i = 0; i < E; i++) v[i] = (float)(a[i] * FA4_RSQRT128);
}

// E2M1 codes of two values, a in bits 3:0 and b in bits 7:4: the gfx950 conversion rounds to nearest
// with ties to the even code, saturates at +-6 and keeps the sign bit (so -0 and tiny negatives give
// the negative-zero code). With a scale of 1 it applies no scaling; callers scale beforehand.
__device__ __forceinline__ uint32_t e2m1_pair(float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xffu;
}

// E2M1 codes of E values (element i in bits 4i+3 .. 4i)
template <int E>
__device__ __forceinline__ uint32_t e2m1_lane(const float q[E]) {
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < E; i += 2) c |= e2m1_pair(q[i], q[i + 1]) << (4 * i);
  return c;
}

// x / b rounded to nearest float32 (the IEEE quotient) for E values sharing b, from one correctly
// rounded reciprocal: with y = RN(1/b) and q = RN(x y) (within 1 ulp of x/b), r = x - b q is exact
// (FMA) and RN(q + r y) is the correctly rounded x/b (Markstein's theorem; binary arithmetic, no
// over/underflow). b is a positive normal scale here; quotients below 2^-126 only occur for values
// whose codes are zeros in every target format, where only the sign matters; the sign is copied from
// x (the correction step would turn -0 into +0). Scales below 2^-100 (1/b would overflow the
// theorem's range) use the division itself.
template <int E>
__device__ __forceinline__ void div_lane(const float x[E], float b, float q[E]) {
  if (b < 0x1p-100f) {
#pragma unroll
    for (int i = 0; i < E; i++) q[i] = x[i] / b;
    return;
  }
  const float y = 1.0f / b;
#pragma unroll
  for (int i = 0; i < E; i++) {
    const float q0 = x[i] * y;
    const float r = __builtin_fmaf(-q0, b, x[i]);
    q[i] = __builtin_copysignf(__builtin_fmaf(r, y, q0), x[i]);   // the quotient has x's sign
  }
}

// max over the lanes of an aligned group of `n` lanes (n a power of two <= 32)
__device__ __forceinline__ float group_max(float v, int n) {
  for (int m = 1; m < n; m <<= 1) v = fmaxf(v, shfl_xor_f(v, m));
  return v;
}

template <int E>
__device__ __forceinline__ float lane_amax(const float v[E]) {
  float m = fabsf(v[0]);
#pragma unroll
  for (int i = 1; i < E; i++) m = fmaxf(m, fabsf(v[i]));
  return m;
}

// NVFP4 codes of the lane's E elements (one 16-element block spans 16/E lanes) given the tensor
// scale; also returns the dequantized values (float64).
template <int E>
__device__ __forceinline__ uint32_t nv_codes(const float v[E], float st, uint32_t *sb_out, double xh[E]) {
  const float am = group_max(lane_amax<E>(v), 16 / E);
  const float six_st = 6.0f * st;
  const uint32_t sb = e4m3_encode(am / six_st);
  const float sbv = e4m3_value(sb);
  const float denom = sbv * st;
  uint32_t c;
  if (sb == 0u) {                                           // zero block scale: signed zeros
    c = 0;
#pragma unroll
    for (int i = 0; i < E; i++) c |= ((__float_as_uint(v[i]) >> 28) & 8u) << (4 * i);
  } else {
    float qv[E];
    div_lane<E>(v, denom, qv);
    c = e2m1_lane<E>(qv);
  }
#pragma unroll
  for (int i = 0; i < E; i++) xh[i] = (double)(e2m1_value((c >> (4 * i)) & 15u) * sbv) * (double)st;
  *sb_out = sb;
  return c;
}

// Squared reconstruction error of a block, float64: per element (x - x^)^2, summed as a balanced binary
// tree over the block's elements in index order (in-lane pairs first, then neighbouring lanes of the
// block; a lane holds E consecutive elements). Contraction into FMAs is off, so every operation rounds
// as written.
template <int E>
__device__ __forceinline__ double block_sse(const float v[E], const double xh[E], int lanes) {
#pragma clang fp contract(off)
  double t[E];
#pragma unroll
  for (int i = 0; i < E; i++) {
    const double dlt = (double)v[i] - xh[i];
    t[i] = dlt * dlt;
  }
#pragma unroll
  for (int w = 1; w < E; w <<= 1)
#pragma unroll
    for (int i = 0; i < E; i += 2 * w) t[i] = t[i] + t[i + w];
  double sum = t[0];
  for (int m = 1; m < lanes; m <<= 1) sum = sum + shfl_xor_d(sum, m);
  return sum;
}

// NVFP4 codes with the per-block scale search: E4M3 block-scale codes c0, c0 - 1, c0 + 1, c0 - 2 (those
// in [1, 126]; c0 the round-to-nearest code), the first with the smallest squared error wins. A zero c0
// keeps the zero scale.
template <int E>
__device__ __forceinline__ uint32_t nv_codes_search(const float v[E], float st, uint32_t *sb_out, double xh[E]) {
  uint32_t sb;
  uint32_t c = nv_codes<E>(v, st, &sb, xh);
  if (sb == 0u) {
    *sb_out = sb;
    return c;
  }
  double best = block_sse<E>(v, xh, 16 / E);
  const int cand[3] = {(int)sb - 1, (int)sb + 1, (int)sb - 2};
  uint32_t best_sb = sb;
#pragma unroll
  for (int k = 0; k < 3; k++) {
    const int cc = cand[k];
    if (cc < 1 || cc > 126) continue;                      // uniform over the block's lanes
    const float sbv = e4m3_value((uint32_t)cc);
    const float denom = sbv * st;
    float qv[E];
    div_lane<E>(v, denom, qv);
    const uint32_t c2 = e2m1_lane<E>(qv);
    double xh2[E];
#pragma unroll
    for (int i = 0; i < E; i++) xh2[i] = (double)e2m1_value((c2 >> (4 * i)) & 15u) * (double)sbv * (double)st;
    const double err = block_sse<E>(v, xh2, 16 / E);
    if (err < best) {
      best = err;
      best_sb = (uint32_t)cc;
      c = c2;
#pragma unroll
      for (int i = 0; i < E; i++) xh[i] = xh2[i];
    }
  }
  *sb_out = best_sb;
  return c;
}

__device__ __forceinline__ float tensor_scale_from_max(float amax) {
  const float t = amax / 2688.0f;          // zero also when the quotient underflows (amax < ~2.7e-42)
  return t == 0.0f ? 1.0f : t;
}

// store E/2 bytes of packed 4-bit codes (E = 4: 2 bytes, E = 8: 4 bytes)
template <int E>
__device__ __forceinline__ void store_nibbles(uint8_t *p, uint32_t c) {
  if (E == 8) *reinterpret_cast<uint32_t *>(p) = c;
  else *reinterpret_cast<uint16_t *>(p) = (uint16_t)c;
}

// PASS: 0 = group maxima (NVFP4), 1 = codes (+ residual maxima when DUAL), 2 = residual codes.
// PAGED: rows go to a paged cache through the page table (then NORM is false).
// SEARCH: the per-block scale search (MXFP4, NVFP4 codes pass; not with DUAL).
// Fold data of FP8 per-token V for the attention kernel: per 128-row tile a power-of-two scale 2^e,
// e the smallest integer with 448 * 2^e >= sigma (sigma = max of the tile's row scales), clamped to
// [-127, 127], and per row w = s * 2^-e (exact). With sigma = M 2^E, M in [1, 2): e = E - 8 when
// M <= 1.75 (448 * 2^(E-8) = 1.75 * 2^E) and E - 7 otherwise; a subnormal sigma gives -127.
__device__ __forceinline__ int fold_exponent(float sigma) {
  const uint32_t b = __float_as_uint(sigma);
  const int E = (int)((b >> 23) & 0xffu);
  if (E == 0) return -127;
  const int e = E - 127 - 8 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// 2^e as a float for e in [-127, 127] (2^-127 is the subnormal 0x00400000).
__device__ __forceinline__ float pow2_float(int e) {
  return __uint_as_float(e == -127 ? 0x00400000u : (uint32_t)(e + 127) << 23);
}

// One workgroup's share of a quantization: chunk bx (CHUNK rows) of group g (= o * heads + h).
// FOLD (FP8_TOKEN, CHUNK = 128, rows in whole 128-row tiles): the chunk is one key tile, and its fold
// data are formed here from the per-token scales just computed: e = fold_exponent(max of the tile's
// scales), w_c = s_c 2^-e and the tile scale 2^e.
template <int D, int DT, int FMT, int PASS, bool HAD, bool DUAL, bool NORM, bool PAGED, bool SEARCH,
          int CHUNK = QUANT_CHUNK, bool FOLD = false>
__device__ __forceinline__ void quantize_rows(const QArgs &a, int64_t bx, int g) {
  static_assert(!FOLD || (FMT == FA4_FP8_TOKEN && CHUNK == 128), "fold data need FP8 per token, 128-row chunks");
  constexpr int E = Epl<DT>::value;       // elements per lane
  constexpr int LPR = D / E;              // lanes per row
  constexpr int RPW = 64 / LPR;           // rows per wave
  constexpr int RPB = RPW * (QUANT_THREADS / 64);
  __shared__ float red[QUANT_THREADS / 64];

  const int64_t o = g / a.heads;
  const int h = g - (int)o * a.heads;
  int64_t nrows = a.rows;
  if (a.row_counts) nrows = min<int64_t>(nrows, (int64_t)a.row_counts[o]);
  const int64_t r0 = bx * CHUNK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, li = lane % LPR;

  float st = 1.0f, rst = 1.0f;
  if (FMT == FA4_NVFP4 && PASS >= 1) {
    st = tensor_scale_from_max(a.scales[g]);
    if (PASS == 2) rst = tensor_scale_from_max(a.rscales[g]);
  }
  float gmax = 0.0f;

  // All rows of the chunk are loaded before any is processed, so a wave has its whole share of the
  // chunk in flight at once; they are held as loaded (16 bytes per row and lane, bf16 still packed)
  // and widened to float when processed. Every lane runs every iteration (rows past the end are
  // inactive and read nothing), so the lane-group shuffles below always see all their lanes.
  constexpr int NIT = CHUNK / RPB;
  uint4 vin[NIT];
  float skeep[FOLD ? NIT : 1];            // FOLD: this lane's rows' per-token scales
  // static smoothing: this lane's E channels of head h, multiplied in after the row norms
  float csm[E];
  const bool smooth = a.cscale != nullptr;                // uniform
  if (smooth) {
#pragma unroll
    for (int i = 0; i < E; i++) csm[i] = a.cscale[(int64_t)h * D + li * E + i];
  }
#pragma unroll
  for (int it = 0; it < NIT; it++) {
    const int64_t rr = r0 + it * RPB + wave * RPW + sub;
    vin[it] = make_uint4(0u, 0u, 0u, 0u);                 // widens to zeros
    if (rr < nrows) vin[it] = load_raw<DT>(a.x, o * a.so + h * a.sh + rr * a.sr + li * E);
  }
#pragma unroll
  for (int it = 0; it < NIT; it++) {
    const int64_t rr = r0 + it * RPB + wave * RPW + sub;
    const bool active = rr < nrows;
    float v[E];
    widen_lane<DT, E>(vin[it], v);
    // rows are processed by whole lane groups, so inactive lanes only feed zeros to the shuffles
    if (NORM && PASS <= 1) {
      // balanced pairwise tree over the row: in-lane pairs first, then neighbouring lanes
      double t[E];
#pragma unroll
      for (int i = 0; i < E; i++) t[i] = (double)v[i] * v[i];
#pragma unroll
      for (int w = 1; w < E; w <<= 1)
#pragma unroll
        for (int i = 0; i < E; i += 2 * w) t[i] = t[i] + t[i + w];
      double s = t[0];
      for (int m = 1; m < LPR; m <<= 1) s = s + shfl_xor_d(s, m);
      if (active && li == 0) a.norm2[(int64_t)g * a.rows + rr] = (float)s;
    }
    if (smooth) {
#pragma unroll
      for (int i = 0; i < E; i++) v[i] *= csm[i];
    }
    if (HAD) hadamard128<E>(v);
    int64_t orow = (int64_t)g * a.rows + rr;
    bool store = active;
    if (PAGED) {
      // only rows that exist read the page table; a page id outside the cache drops the row
      const int pg = active ? a.page_table[o * a.max_pages + rr / a.page_size] : 0;
      store = active && pg >= 0 && (int64_t)pg < a.num_pages;
      orow = ((int64_t)(store ? pg : 0) * a.heads + h) * a.page_size + rr % a.page_size;
    }
    if (FMT == FA4_MXFP4) {
      const float am = group_max(lane_amax<E>(v), 32 / E);      // 32-element block = 32/E lanes
      int e = mx_exponent(am);
      const float mul = pow2_neg(e);
      float sv[E];
#pragma unroll
      for (int i = 0; i < E; i++) sv[i] = v[i] * mul;          // exact (a power of two)
      uint32_t c = e2m1_lane<E>(sv);
      if (SEARCH && e > -127) {
        // candidates e (round to nearest) and e - 1 (clips at 6 * 2^(e-1), finer elsewhere)
        double xh0[E], xh1[E];
        float sv1[E];
#pragma unroll
        for (int i = 0; i < E; i++) sv1[i] = sv[i] * 2.0f;     // exact
        const uint32_t c1 = e2m1_lane<E>(sv1);
#pragma unroll
        for (int i = 0; i < E; i++) {
          xh0[i] = __builtin_ldexp((double)e2m1_value((c >> (4 * i)) & 15u), e);
          xh1[i] = __builtin_ldexp((double)e2m1_value((c1 >> (4 * i)) & 15u), e - 1);
        }
        const double err0 = block_sse<E>(v, xh0, 32 / E), err1 = block_sse<E>(v, xh1, 32 / E);
        if (err1 < err0) {                                      // uniform over the block's lanes
          e -= 1;
          c = c1;
#pragma unroll
          for (int i = 0; i < E; i++) sv[i] = sv1[i];
        }
      }
      if (store) {
        store_nibbles<E>(a.codes + orow * (D / 2) + li * (E / 2), c);
        if ((li % (32 / E)) == 0) a.bscales[orow * (D / 32) + li / (32 / E)] = (uint8_t)(e + 127);
      }
      if (DUAL) {
        // residual r = x - code * 2^e, formed as (x 2^-e - code) * 2^e: the difference is exact (the
        // code is x 2^-e rounded to a neighbour on the E2M1 grid, |x 2^-e| <= 6), the power-of-two
        // scaling rounds only a subnormal result, and code * 2^e itself (which can exceed the float
        // range when e = 126) is never formed. Then MXFP4 of r with its own scales.
        float rv[E];
#pragma unroll
        for (int i = 0; i < E; i++) rv[i] = __builtin_ldexpf(sv[i] - e2m1_value((c >> (4 * i)) & 15u), e);
        const int re = mx_exponent(group_max(lane_amax<E>(rv), 32 / E));
        const float rmul = pow2_neg(re);
#pragma unroll
        for (int i = 0; i < E; i++) rv[i] *= rmul;
        const uint32_t rc = e2m1_lane<E>(rv);
        if (store) {
          store_nibbles<E>(a.rcodes + orow * (D / 2) + li * (E / 2), rc);
          if ((li % (32 / E)) == 0) a.rbscales[orow * (D / 32) + li / (32 / E)] = (uint8_t)(re + 127);
        }
      }
    } else if (FMT == FA4_MXFP8) {
      const int e = mx8_exponent(group_max(lane_amax<E>(v), 32 / E));
      const float mul = pow2_neg(e);
      uint32_t c[E / 4];
#pragma unroll
      for (int w = 0; w < E / 4; w++)
        c[w] = e4m3_encode2(v[4 * w] * mul, v[4 * w + 1] * mul) |
               (e4m3_encode2(v[4 * w + 2] * mul, v[4 * w + 3] * mul) << 16);   // exact scaling, then RNE
      if (store) {
        if (E == 8) *reinterpret_cast<uint2 *>(a.codes + orow * D + li * 8) = make_uint2(c[0], c[E / 4 - 1]);
        else *reinterpret_cast<uint32_t *>(a.codes + orow * D + li * 4) = c[0];
        if ((li % (32 / E)) == 0) a.bscales[orow * (D / 32) + li / (32 / E)] = (uint8_t)(e + 127);
      }
    } else if (FMT == FA4_FP8_TOKEN) {
      const float am = group_max(lane_amax<E>(v), LPR);
      const float s = am == 0.0f ? 1.0f : am / 448.0f;
      if (FOLD) skeep[FOLD ? it : 0] = s;
      float qv[E];
      div_lane<E>(v, s, qv);
      uint32_t c[E / 4];
#pragma unroll
      for (int w = 0; w < E / 4; w++)
        c[w] = e4m3_encode2(qv[4 * w], qv[4 * w + 1]) | (e4m3_encode2(qv[4 * w + 2], qv[4 * w + 3]) << 16);
      if (store) {
        if (E == 8) *reinterpret_cast<uint2 *>(a.codes + orow * D + li * 8) = make_uint2(c[0], c[E / 4 - 1]);
        else *reinterpret_cast<uint32_t *>(a.codes + orow * D + li * 4) = c[0];
        if (li == 0) a.scales[orow] = s;
      }
    } else {  // NVFP4
      if (PASS == 0) {
        gmax = fmaxf(gmax, active ? lane_amax<E>(v) : 0.0f);
      } else {
        uint32_t sb;
        double xh[E];
        const uint32_t c = SEARCH ? nv_codes_search<E>(v, st, &sb, xh) : nv_codes<E>(v, st, &sb, xh);
        if (PASS == 1) {
          if (store) {
            store_nibbles<E>(a.codes + orow * (D / 2) + li * (E / 2), c);
            if ((li % (16 / E)) == 0) a.bscales[orow * (D / 16) + li / (16 / E)] = (uint8_t)sb;
          }
          if (DUAL) {
            float am = 0.0f;
#pragma unroll
            for (int i = 0; i < E; i++) am = fmaxf(am, fabsf((float)((double)v[i] - xh[i])));
            gmax = fmaxf(gmax, active ? am : 0.0f);
          }
        } else {  // PASS 2: residual codes
          float rv[E];
#pragma unroll
          for (int i = 0; i < E; i++) rv[i] = (float)((double)v[i] - xh[i]);
          uint32_t rsb;
          double rxh[E];
          const uint32_t rc = nv_codes<E>(rv, rst, &rsb, rxh);
          if (store) {
            store_nibbles<E>(a.rcodes + orow * (D / 2) + li * (E / 2), rc);
            if ((li % (16 / E)) == 0) a.rbscales[orow * (D / 16) + li / (16 / E)] = (uint8_t)rsb;
          }
        }
      }
    }
  }
  if (FMT == FA4_NVFP4 && (PASS == 0 || (PASS == 1 && DUAL))) {
    for (int m = 1; m < 64; m <<= 1) gmax = fmaxf(gmax, shfl_xor_f(gmax, m));
    if (lane == 0) red[wave] = gmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      float m = red[0];
      for (int w = 1; w < QUANT_THREADS / 64; w++) m = fmaxf(m, red[w]);
      float *dst = PASS == 0 ? a.scales : a.rscales;
      // non-negative floats order like their bit patterns
      atomicMax(reinterpret_cast<unsigned int *>(dst + g), __float_as_uint(m));
    }
  }
  if constexpr (FOLD) {
    // every lane of a row's lane group holds that row's scale; the tile maximum over all 128 rows
    float m = skeep[0];
#pragma unroll
    for (int i = 1; i < NIT; i++) m = fmaxf(m, skeep[i]);
    for (int k = 1; k < 64; k <<= 1) m = fmaxf(m, shfl_xor_f(m, k));
    if (lane == 0) red[wave] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < QUANT_THREADS / 64; w++) m = fmaxf(m, red[w]);
    const int e = fold_exponent(m);
#pragma unroll
    for (int i = 0; i < NIT; i++) {
      const int64_t rr = r0 + i * RPB + wave * RPW + sub;
      if (li == 0 && rr < nrows) a.fold_w[(int64_t)g * a.rows + rr] = __builtin_ldexpf(skeep[i], -e);
    }
    if (threadIdx.x == 0) a.fold_scale[(int64_t)g * (a.rows / 128) + bx] = pow2_float(e);
  }
}

template <int D, int DT, int FMT, int PASS, bool HAD, bool DUAL, bool NORM, bool PAGED, bool SEARCH,
          int CHUNK = QUANT_CHUNK, bool FOLD = false>
__global__ void __launch_bounds__(QUANT_THREADS) quantize_kernel(QArgs a) {
  quantize_rows<D, DT, FMT, PASS, HAD, DUAL, NORM, PAGED, SEARCH, CHUNK, FOLD>(a, blockIdx.x, (int)blockIdx.y);
}

// The three operands of a prefill in one launch, so that their ramps and tails overlap: workgroups
// [0, nq) take Q's chunks (MXFP4 or MXFP8), [nq, nq + nk) K's, the rest V's (FP8 per token with the
// fold data, 128-row chunks). Each block's work is exactly that of the separate calls.
template <int DT>
__device__ __forceinline__ void mx_keys_unit(const QArgs &a, int d, int c, int64_t rb, int64_t g);

// VF: FA4_FP8_TOKEN (V per token with its fold data, 128-row chunks) or FA4_MXFP4_KEYS (4-bit V: each
// workgroup takes two 32-key units, a column per thread, as mx_keys_kernel; vchunks = rows / 32).
template <int D, int DT, int QKF, bool NORM, int VF = FA4_FP8_TOKEN>
__global__ void __launch_bounds__(QUANT_THREADS) prefill_quant_kernel(QArgs q, QArgs k, QArgs v, int64_t qchunks,
                                                                      int64_t kchunks, int64_t vchunks, int64_t nq,
                                                                      int64_t nk) {
  const int64_t blk = blockIdx.x;
  if (blk < nq) {
    quantize_rows<D, DT, QKF, 1, false, false, NORM, false, false, PREFILL_QK_CHUNK>(q, blk % qchunks,
                                                                                     (int)(blk / qchunks));
  } else if (blk < nq + nk) {
    const int64_t b = blk - nq;
    quantize_rows<D, DT, QKF, 1, false, false, NORM, false, false, PREFILL_QK_CHUNK>(k, b % kchunks,
                                                                                     (int)(b / kchunks));
  } else if constexpr (VF == FA4_MXFP4_KEYS) {
    const int64_t u = 2 * (blk - nq - nk) + (threadIdx.x >> 7), c = threadIdx.x & 127;   // no barrier follows
    if (u < vchunks * v.outer * v.heads && c < D) mx_keys_unit<DT>(v, D, (int)c, u % vchunks, u / vchunks);
  } else {
    const int64_t b = blk - nq - nk;
    quantize_rows<D, DT, FA4_FP8_TOKEN, 1, false, false, false, false, false, 128, true>(v, b % vchunks,
                                                                                       (int)(b / vchunks));
  }
}

// max over the workgroup (every thread calls it; `red` holds QUANT_THREADS / 64 floats)
__device__ __forceinline__ float block_max(float v, float *red) {
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, shfl_xor_f(v, m));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < QUANT_THREADS / 64; w++) r = fmaxf(r, red[w]);
  return r;
}

// NVFP4 of groups small enough for one workgroup (at most QUANT_CHUNK rows, unpaged): the tensor
// maximum, the codes and, with DUAL, the residual's maximum and codes in one launch (one workgroup per
// group). Same arithmetic as the multi-pass path: the maxima are the same maxima, reduced in LDS.
template <int D, int DT, bool DUAL, bool SEARCH>
__global__ void __launch_bounds__(QUANT_THREADS) nv_group_kernel(QArgs a) {
  constexpr int E = Epl<DT>::value;
  constexpr int LPR = D / E;
  constexpr int RPW = 64 / LPR;
  constexpr int RPB = RPW * (QUANT_THREADS / 64);
  constexpr int NIT = (QUANT_CHUNK + RPB - 1) / RPB;
  __shared__ float red0[QUANT_THREADS / 64], red1[QUANT_THREADS / 64];
  const int g = blockIdx.x;
  const int64_t o = g / a.heads;
  const int h = g - (int)o * a.heads;
  int64_t nrows = a.rows;
  if (a.row_counts) nrows = min<int64_t>(nrows, (int64_t)a.row_counts[o]);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, li = lane % LPR;
  float vin[NIT][E];
  float gmax = 0.0f;
#pragma unroll
  for (int it = 0; it < NIT; it++) {
    const int64_t rr = it * RPB + wave * RPW + sub;
#pragma unroll
    for (int i = 0; i < E; i++) vin[it][i] = 0.0f;
    if (rr < nrows) load_lane<DT, E>(a.x, o * a.so + h * a.sh + rr * a.sr + li * E, vin[it]);
    if (a.cscale) {                                         // static smoothing (uniform)
#pragma unroll
      for (int i = 0; i < E; i++) vin[it][i] *= a.cscale[(int64_t)h * D + li * E + i];
    }
    gmax = fmaxf(gmax, lane_amax<E>(vin[it]));            // inactive rows hold zeros
  }
  const float st = tensor_scale_from_max(block_max(gmax, red0));
  if (threadIdx.x == 0) a.scales[g] = st;
  float rmax = 0.0f;
#pragma unroll
  for (int it = 0; it < NIT; it++) {
    const int64_t rr = it * RPB + wave * RPW + sub;
    const bool active = rr < nrows;
    const int64_t orow = (int64_t)g * a.rows + rr;
    uint32_t sb;
    double xh[E];
    const uint32_t c = SEARCH ? nv_codes_search<E>(vin[it], st, &sb, xh) : nv_codes<E>(vin[it], st, &sb, xh);
    if (active) {
      store_nibbles<E>(a.codes + orow * (D / 2) + li * (E / 2), c);
      if ((li % (16 / E)) == 0) a.bscales[orow * (D / 16) + li / (16 / E)] = (uint8_t)sb;
    }
    if (DUAL) {
#pragma unroll
      for (int i = 0; i < E; i++) vin[it][i] = (float)((double)vin[it][i] - xh[i]);   // the residual
      rmax = fmaxf(rmax, active ? lane_amax<E>(vin[it]) : 0.0f);
    }
  }
  if (DUAL) {
    const float rst = tensor_scale_from_max(block_max(rmax, red1));
    if (threadIdx.x == 0) a.rscales[g] = rst;
#pragma unroll
    for (int it = 0; it < NIT; it++) {
      const int64_t rr = it * RPB + wave * RPW + sub;
      const int64_t orow = (int64_t)g * a.rows + rr;
      uint32_t rsb;
      double rxh[E];
      const uint32_t rc = nv_codes<E>(vin[it], rst, &rsb, rxh);
      if (rr < nrows) {
        store_nibbles<E>(a.rcodes + orow * (D / 2) + li * (E / 2), rc);
        if ((li % (16 / E)) == 0) a.rbscales[orow * (D / 16) + li / (16 / E)] = (uint8_t)rsb;
      }
    }
  }
}

// NVFP4 of one-row groups (the decode query: one row per (sequence, head)), unpaged: each row is
// quantized by its own lane group (D/E lanes), so the tensor maximum and, with DUAL, the residual's
// maximum are lane-group shuffles with no workgroup barrier. Same arithmetic as nv_group_kernel: the
// maxima are the same maxima, the codes the same nv_codes.
template <int D, int DT, bool DUAL, bool SEARCH>
__global__ void __launch_bounds__(QUANT_THREADS) nv_row_kernel(QArgs a, int64_t groups) {
  constexpr int E = Epl<DT>::value;
  constexpr int LPR = D / E;
  constexpr int RPW = 64 / LPR;
  constexpr int RPB = RPW * (QUANT_THREADS / 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, li = lane % LPR;
  const int64_t g = (int64_t)blockIdx.x * RPB + wave * RPW + sub;
  const bool live = g < groups;                             // every lane runs the shuffles below
  const int64_t o = live ? g / a.heads : 0;
  const int h = live ? (int)(g - o * a.heads) : 0;
  bool active = live;
  if (live && a.row_counts) active = a.row_counts[o] >= 1;
  float v[E];
  const uint4 raw = active ? load_raw<DT>(a.x, o * a.so + h * a.sh + li * E) : make_uint4(0u, 0u, 0u, 0u);
  widen_lane<DT, E>(raw, v);
  if (a.cscale && live) {                                   // static smoothing
#pragma unroll
    for (int i = 0; i < E; i++) v[i] *= a.cscale[(int64_t)h * D + li * E + i];
  }
  const float st = tensor_scale_from_max(group_max(lane_amax<E>(v), LPR));
  if (live && li == 0) a.scales[g] = st;
  uint32_t sb;
  double xh[E];
  const uint32_t c = SEARCH ? nv_codes_search<E>(v, st, &sb, xh) : nv_codes<E>(v, st, &sb, xh);
  if (active) {
    store_nibbles<E>(a.codes + g * (D / 2) + li * (E / 2), c);
    if ((li % (16 / E)) == 0) a.bscales[g * (D / 16) + li / (16 / E)] = (uint8_t)sb;
  }
  if (DUAL) {
    float rv[E];
#pragma unroll
    for (int i = 0; i < E; i++) rv[i] = (float)((double)v[i] - xh[i]);                // the residual
    const float rst = tensor_scale_from_max(group_max(active ? lane_amax<E>(rv) : 0.0f, LPR));
    if (live && li == 0) a.rscales[g] = rst;
    uint32_t rsb;
    double rxh[E];
    const uint32_t rc = nv_codes<E>(rv, rst, &rsb, rxh);
    if (active) {
      store_nibbles<E>(a.rcodes + g * (D / 2) + li * (E / 2), rc);
      if ((li % (16 / E)) == 0) a.rbscales[g * (D / 16) + li / (16 / E)] = (uint8_t)rsb;
    }
  }
}

__global__ void fill_zero_kernel(float *p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

__global__ void finalize_tensor_scale_kernel(float *p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = tensor_scale_from_max(p[i]);
}

template <int D, int DT, int FMT, int PASS, bool HAD, bool DUAL, bool SEARCH = false>
static hipError_t launch_q(const QArgs &a, int64_t groups, bool norm, hipStream_t s) {
  if (a.rows == 0 || groups == 0) return hipSuccess;       // nothing to read (NVFP4 scales still finalize)
  // NVFP4's maximum passes end every workgroup with an atomicMax on its group's maximum; larger chunks
  // there keep the number of atomics on one address down (2048 per head of 128K rows at 64 rows)
  // MXFP4 dual residual (the decode query: a few thousand rows, two quantizations per row) in chunks of
  // one row per lane group, so that many small workgroups each finish after one row
  constexpr int CH = (FMT == FA4_NVFP4 && PASS == 0) ? NV_MAX_CHUNK
                     : (FMT == FA4_MXFP4 && DUAL)     ? (64 / (D / Epl<DT>::value)) * (QUANT_THREADS / 64)
                                                      : QUANT_CHUNK;
  dim3 grid((unsigned)((a.rows + CH - 1) / CH), (unsigned)groups);
  if (a.page_table)                                        // row norms are only written unpaged
    hipLaunchKernelGGL((quantize_kernel<D, DT, FMT, PASS, HAD, DUAL, false, true, SEARCH, CH>), grid,
                       dim3(QUANT_THREADS), 0, s, a);
  else if (norm)
    hipLaunchKernelGGL((quantize_kernel<D, DT, FMT, PASS, HAD, DUAL, true, false, SEARCH, CH>), grid,
                       dim3(QUANT_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((quantize_kernel<D, DT, FMT, PASS, HAD, DUAL, false, false, SEARCH, CH>), grid,
                       dim3(QUANT_THREADS), 0, s, a);
  return hipGetLastError();
}

template <int D, int DT>
static hipError_t quantize_dispatch(const QArgs &a, int fmt, bool had, bool dual, bool search, int64_t groups,
                                    bool norm, hipStream_t s) {
  hipError_t e = hipSuccess;
  const unsigned small = (unsigned)((groups + 255) / 256);
  if (fmt == FA4_MXFP4 && search)            // (the scale search is never combined with the dual residual)
    return had ? launch_q<D, DT, FA4_MXFP4, 1, true, false, true>(a, groups, norm, s)
               : launch_q<D, DT, FA4_MXFP4, 1, false, false, true>(a, groups, norm, s);
  if (fmt == FA4_MXFP4) {                    // one pass (the residual needs no tensor scale)
    if (dual) return had ? launch_q<D, DT, FA4_MXFP4, 1, true, true>(a, groups, norm, s)
                         : launch_q<D, DT, FA4_MXFP4, 1, false, true>(a, groups, norm, s);
    if (had) return launch_q<D, DT, FA4_MXFP4, 1, true, false>(a, groups, norm, s);
    return launch_q<D, DT, FA4_MXFP4, 1, false, false>(a, groups, norm, s);
  }
  if (fmt == FA4_MXFP8)
    return had ? launch_q<D, DT, FA4_MXFP8, 1, true, false>(a, groups, norm, s)
               : launch_q<D, DT, FA4_MXFP8, 1, false, false>(a, groups, norm, s);
  if (fmt == FA4_FP8_TOKEN) {
    if (!a.fold_w) return launch_q<D, DT, FA4_FP8_TOKEN, 1, false, false>(a, groups, norm, s);
    if (a.rows == 0 || groups == 0) return hipSuccess;
    // with fold data: one workgroup per 128-row key tile (rows are whole tiles, unpaged, not ragged)
    const dim3 grid((unsigned)(a.rows / 128), (unsigned)groups);
    if (norm)
      hipLaunchKernelGGL((quantize_kernel<D, DT, FA4_FP8_TOKEN, 1, false, false, true, false, false, 128, true>), grid,
                         dim3(QUANT_THREADS), 0, s, a);
    else
      hipLaunchKernelGGL((quantize_kernel<D, DT, FA4_FP8_TOKEN, 1, false, false, false, false, false, 128, true>), grid,
                         dim3(QUANT_THREADS), 0, s, a);
    return hipGetLastError();
  }
  // NVFP4, one-row groups: a lane group per row
  if (!had && !norm && !a.page_table && a.rows == 1) {
    constexpr int RPB = (64 / (D / Epl<DT>::value)) * (QUANT_THREADS / 64);
    const dim3 grid((unsigned)((groups + RPB - 1) / RPB));
    if (dual) hipLaunchKernelGGL((nv_row_kernel<D, DT, true, false>), grid, dim3(QUANT_THREADS), 0, s, a, groups);
    else if (search) hipLaunchKernelGGL((nv_row_kernel<D, DT, false, true>), grid, dim3(QUANT_THREADS), 0, s, a, groups);
    else hipLaunchKernelGGL((nv_row_kernel<D, DT, false, false>), grid, dim3(QUANT_THREADS), 0, s, a, groups);
    return hipGetLastError();
  }
  // NVFP4, groups that fit one workgroup: a single launch
  if (!had && !norm && !a.page_table && a.rows <= QUANT_CHUNK) {
    if (dual) hipLaunchKernelGGL((nv_group_kernel<D, DT, true, false>), dim3((unsigned)groups), dim3(QUANT_THREADS), 0, s, a);
    else if (search) hipLaunchKernelGGL((nv_group_kernel<D, DT, false, true>), dim3((unsigned)groups), dim3(QUANT_THREADS), 0, s, a);
    else hipLaunchKernelGGL((nv_group_kernel<D, DT, false, false>), dim3((unsigned)groups), dim3(QUANT_THREADS), 0, s, a);
    return hipGetLastError();
  }
  // NVFP4: zero the group maxima, reduce them, quantize, turn maxima into tensor scales
  hipLaunchKernelGGL(fill_zero_kernel, dim3(small), dim3(256), 0, s, a.scales, groups);
  if (dual) hipLaunchKernelGGL(fill_zero_kernel, dim3(small), dim3(256), 0, s, a.rscales, groups);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (had) {
    if ((e = launch_q<D, DT, FA4_NVFP4, 0, true, false>(a, groups, norm, s)) != hipSuccess) return e;
    if (dual) {
      if ((e = launch_q<D, DT, FA4_NVFP4, 1, true, true>(a, groups, false, s)) != hipSuccess) return e;
      if ((e = launch_q<D, DT, FA4_NVFP4, 2, true, true>(a, groups, false, s)) != hipSuccess) return e;
    } else if ((e = search ? launch_q<D, DT, FA4_NVFP4, 1, true, false, true>(a, groups, false, s)
                           : launch_q<D, DT, FA4_NVFP4, 1, true, false>(a, groups, false, s)) != hipSuccess) {
      return e;
    }
  } else {
    if ((e = launch_q<D, DT, FA4_NVFP4, 0, false, false>(a, groups, norm, s)) != hipSuccess) return e;
    if (dual) {
      if ((e = launch_q<D, DT, FA4_NVFP4, 1, false, true>(a, groups, false, s)) != hipSuccess) return e;
      if ((e = launch_q<D, DT, FA4_NVFP4, 2, false, true>(a, groups, false, s)) != hipSuccess) return e;
    } else if ((e = search ? launch_q<D, DT, FA4_NVFP4, 1, false, false, true>(a, groups, false, s)
                           : launch_q<D, DT, FA4_NVFP4, 1, false, false>(a, groups, false, s)) != hipSuccess) {
      return e;
    }
  }
  hipLaunchKernelGGL(finalize_tensor_scale_kernel, dim3(small), dim3(256), 0, s, a.scales, groups);
  if (dual) hipLaunchKernelGGL(finalize_tensor_scale_kernel, dim3(small), dim3(256), 0, s, a.rscales, groups);
  return hipGetLastError();
}

// ---- static smoothing factors from calibration tensors

// Per (head, channel) maximum |x| over a tensor's rows, published with atomicMax on the float bits into
// amax [heads][D] (zeroed beforehand; non-negative floats order like their bit patterns).
template <int D, int DT>
__global__ void __launch_bounds__(QUANT_THREADS) channel_amax_kernel(QArgs a, float *amax) {
  constexpr int E = Epl<DT>::value;
  constexpr int LPR = D / E;
  constexpr int RPW = 64 / LPR;
  constexpr int RPB = RPW * (QUANT_THREADS / 64);
  constexpr int NIT = QUANT_CHUNK / RPB;
  const int g = blockIdx.y;
  const int64_t o = g / a.heads;
  const int h = g - (int)o * a.heads;
  int64_t nrows = a.rows;
  if (a.row_counts) nrows = min<int64_t>(nrows, (int64_t)a.row_counts[o]);
  const int64_t r0 = (int64_t)blockIdx.x * QUANT_CHUNK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, li = lane % LPR;
  float m[E];
#pragma unroll
  for (int i = 0; i < E; i++) m[i] = 0.0f;
#pragma unroll
  for (int it = 0; it < NIT; it++) {
    const int64_t rr = r0 + it * RPB + wave * RPW + sub;
    if (rr < nrows) {
      float v[E];
      load_lane<DT, E>(a.x, o * a.so + h * a.sh + rr * a.sr + li * E, v);
#pragma unroll
      for (int i = 0; i < E; i++) m[i] = fmaxf(m[i], fabsf(v[i]));
    }
  }
  // lanes li, li + LPR, ... of a wave hold the same channels
#pragma unroll
  for (int i = 0; i < E; i++)
    for (int msk = LPR; msk < 64; msk <<= 1) m[i] = fmaxf(m[i], shfl_xor_f(m[i], msk));
  if (sub == 0) {
#pragma unroll
    for (int i = 0; i < E; i++)
      atomicMax(reinterpret_cast<unsigned int *>(amax + (int64_t)h * D + li * E + i), __float_as_uint(m[i]));
  }
}

// Smoothing exponent per (key head, channel): k = floor((e_K - e_Q + 1) / 2) with e = floor(log2 amax)
// (amax_Q over the query heads of the group), clamped to [-20, 20], 0 when either maximum is zero.
// Writes k_scale = 2^-k and q_scale = 2^k for every query head of the group, in place of the maxima.
__global__ void smoothing_kernel(float *q_scale, float *k_scale, int Hkv, int group, int d) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= Hkv * d) return;
  const int kvh = i / d, c = i - kvh * d;
  float aq = 0.0f;
  for (int j = 0; j < group; j++) aq = fmaxf(aq, q_scale[(int64_t)(kvh * group + j) * d + c]);
  const float ak = k_scale[i];
  int k = 0;
  if (aq > 0.0f && ak > 0.0f) {
    int eq, ek;
    frexpf(aq, &eq);
    frexpf(ak, &ek);
    k = (ek - eq + 1) >> 1;                // floor division by 2 (arithmetic shift)
    k = k < -20 ? -20 : (k > 20 ? 20 : k);
  }
  k_scale[i] = __builtin_ldexpf(1.0f, -k);
  for (int j = 0; j < group; j++) q_scale[(int64_t)(kvh * group + j) * d + c] = __builtin_ldexpf(1.0f, k);
}

static QArgs input_args(const fa4_qinput *in) {
  QArgs a = {};
  a.x = in->x; a.outer = in->outer; a.rows = in->rows; a.heads = in->heads;
  a.so = in->stride_outer; a.sh = in->stride_head; a.sr = in->stride_row;
  a.row_counts = in->row_counts;
  return a;
}

template <int D, int DT>
static hipError_t launch_amax(const fa4_qinput *in, float *amax, hipStream_t s) {
  const int64_t groups = in->outer * in->heads;
  const unsigned n = (unsigned)(in->heads * D);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, s, amax, (int64_t)n);
  if (in->rows > 0 && groups > 0) {
    dim3 grid((unsigned)((in->rows + QUANT_CHUNK - 1) / QUANT_CHUNK), (unsigned)groups);
    hipLaunchKernelGGL((channel_amax_kernel<D, DT>), grid, dim3(QUANT_THREADS), 0, s, input_args(in), amax);
  }
  return hipGetLastError();
}

hipError_t launch_smoothing(const fa4_qinput *q, const fa4_qinput *k, float *q_scale, float *k_scale,
                            hipStream_t s) {
  hipError_t e;
  for (int t = 0; t < 2; t++) {
    const fa4_qinput *in = t == 0 ? q : k;
    float *out = t == 0 ? q_scale : k_scale;
    if (in->d == 128) e = in->dtype == FA4_F32 ? launch_amax<128, 0>(in, out, s) : launch_amax<128, 1>(in, out, s);
    else e = in->dtype == FA4_F32 ? launch_amax<64, 0>(in, out, s) : launch_amax<64, 1>(in, out, s);
    if (e != hipSuccess) return e;
  }
  const int n = k->heads * k->d;
  hipLaunchKernelGGL(smoothing_kernel, dim3((n + 255) / 256), dim3(256), 0, s, q_scale, k_scale, k->heads,
                     q->heads / k->heads, k->d);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------- MXFP4 along rows
// 4-bit V for prefill: MXFP4 with 32-element blocks along the rows (the keys) of each column. Thread =
// (group, column c, block of 32 rows); the loads of a block's rows are coalesced over the columns. Codes
// of column c: [group][d][rows/2], two per byte, low nibble first; within a block, code position j holds
// row 8 ((j >> 2) & 3) + 4 (j >> 4) + (j & 3) of the block (the key order of the attention's FP8
// probability operand). Scales: [group][d][rows/32] E8M0, the MXFP4 rule of the row quantizer.
template <int DT>
__device__ __forceinline__ void mx_keys_unit(const QArgs &a, int d, int c, int64_t rb, int64_t g) {
  const int64_t r0 = 32 * rb;
  const int64_t o = g / a.heads, h = g - o * a.heads;
  const int64_t base = o * a.so + h * a.sh + (int64_t)r0 * a.sr + c;
  float v[32];
#pragma unroll
  for (int j = 0; j < 32; j++)
    v[j] = DT == 0 ? static_cast<const float *>(a.x)[base + j * a.sr]
                   : bf16_bits_to_float(static_cast<const uint16_t *>(a.x)[base + j * a.sr]);
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; j++) am = fmaxf(am, fabsf(v[j]));
  const int e = mx_exponent(am);
  const float mul = pow2_neg(e);                              // exact scaling (a power of two)
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int jp = 0; jp < 32; jp += 2) {                        // positions jp, jp + 1: rows k0, k0 + 1
    const int k0 = 8 * ((jp >> 2) & 3) + 4 * (jp >> 4) + (jp & 3);
    w[jp >> 3] |= e2m1_pair(v[k0] * mul, v[k0 + 1] * mul) << (4 * (jp & 7));
  }
  const int64_t row = g * d + c;
  *reinterpret_cast<uint4 *>(a.codes + row * (a.rows / 2) + r0 / 2) = make_uint4(w[0], w[1], w[2], w[3]);
  a.bscales[row * (a.rows / 32) + r0 / 32] = (uint8_t)(e + 127);
}

template <int DT>
__global__ void __launch_bounds__(128) mx_keys_kernel(QArgs a, int d) {
  if ((int)threadIdx.x < d) mx_keys_unit<DT>(a, d, threadIdx.x, blockIdx.x, blockIdx.y);
}

static QArgs quant_args(const fa4_qinput *in, const fa4_qoutput *out, const fa4_qoutput *res, float *norm2) {
  QArgs a;
  a.x = in->x; a.outer = in->outer; a.rows = in->rows; a.heads = in->heads;
  a.so = in->stride_outer; a.sh = in->stride_head; a.sr = in->stride_row;
  a.row_counts = in->row_counts; a.page_table = in->page_table;
  a.page_size = in->page_size; a.max_pages = in->max_pages; a.num_pages = in->num_pages;
  a.codes = out->codes; a.bscales = out->block_scales; a.scales = out->scales;
  a.rcodes = res ? res->codes : nullptr; a.rbscales = res ? res->block_scales : nullptr;
  a.rscales = res ? res->scales : nullptr;
  a.norm2 = norm2;
  a.fold_w = out->fold_w; a.fold_scale = out->fold_scale;
  a.cscale = in->channel_scale;
  return a;
}

template <int D, int DT>
static hipError_t launch_prefill_quant(const QArgs &q, const QArgs &k, const QArgs &v, int qkf, bool norm, bool v4,
                                       int64_t qch, int64_t kch, int64_t vch, int64_t nq, int64_t nk, int64_t nv,
                                       hipStream_t s) {
  const dim3 grid((unsigned)(nq + nk + nv));
  // chunk counts divide block indices only inside the branch of a tensor that has blocks
  qch = qch > 0 ? qch : 1; kch = kch > 0 ? kch : 1; vch = vch > 0 ? vch : 1;
  if (v4) {                                      // 4-bit V goes with MXFP4 Q and K
    if (norm) hipLaunchKernelGGL((prefill_quant_kernel<D, DT, FA4_MXFP4, true, FA4_MXFP4_KEYS>), grid,
                                 dim3(QUANT_THREADS), 0, s, q, k, v, qch, kch, vch, nq, nk);
    else hipLaunchKernelGGL((prefill_quant_kernel<D, DT, FA4_MXFP4, false, FA4_MXFP4_KEYS>), grid, dim3(QUANT_THREADS),
                            0, s, q, k, v, qch, kch, vch, nq, nk);
    return hipGetLastError();
  }
  if (qkf == FA4_MXFP4) {
    if (norm) hipLaunchKernelGGL((prefill_quant_kernel<D, DT, FA4_MXFP4, true>), grid, dim3(QUANT_THREADS), 0, s, q, k,
                                 v, qch, kch, vch, nq, nk);
    else hipLaunchKernelGGL((prefill_quant_kernel<D, DT, FA4_MXFP4, false>), grid, dim3(QUANT_THREADS), 0, s, q, k, v,
                            qch, kch, vch, nq, nk);
  } else {
    if (norm) hipLaunchKernelGGL((prefill_quant_kernel<D, DT, FA4_MXFP8, true>), grid, dim3(QUANT_THREADS), 0, s, q, k,
                                 v, qch, kch, vch, nq, nk);
    else hipLaunchKernelGGL((prefill_quant_kernel<D, DT, FA4_MXFP8, false>), grid, dim3(QUANT_THREADS), 0, s, q, k, v,
                            qch, kch, vch, nq, nk);
  }
  return hipGetLastError();
}

// workgroups of V in the one-launch quantization: 128-row tiles (FP8 per token) or pairs of 32-key units
static int64_t v_blocks(const fa4_qinput *v, bool v4) {
  return v4 ? (v->rows / 32 * (v->outer * v->heads) + 1) / 2 : v->rows / 128 * (v->outer * v->heads);
}

int64_t prefill_quant_blocks(const fa4_qinput *q, const fa4_qinput *k, const fa4_qinput *v, bool v4) {
  return (q->rows + PREFILL_QK_CHUNK - 1) / PREFILL_QK_CHUNK * (q->outer * q->heads) +
         (k->rows + PREFILL_QK_CHUNK - 1) / PREFILL_QK_CHUNK * (k->outer * k->heads) + v_blocks(v, v4);
}

hipError_t launch_quantize_prefill(const fa4_qinput *q, const fa4_qinput *k, const fa4_qinput *v,
                                   const fa4_qoutput *qo, const fa4_qoutput *ko, const fa4_qoutput *vo,
                                   float *q_norm2, float *k_norm2, hipStream_t s) {
  const QArgs qa = quant_args(q, qo, nullptr, q_norm2), ka = quant_args(k, ko, nullptr, k_norm2),
              va = quant_args(v, vo, nullptr, nullptr);
  const bool v4 = vo->fmt == FA4_MXFP4_KEYS;
  const int64_t qch = (q->rows + PREFILL_QK_CHUNK - 1) / PREFILL_QK_CHUNK,
                kch = (k->rows + PREFILL_QK_CHUNK - 1) / PREFILL_QK_CHUNK, vch = v->rows / (v4 ? 32 : 128);
  const int64_t nq = qch * (q->outer * q->heads), nk = kch * (k->outer * k->heads), nv = v_blocks(v, v4);
  if (nq + nk + nv == 0) return hipSuccess;
  const bool norm = q_norm2 != nullptr;
  if (q->d == 128)
    return q->dtype == FA4_F32
               ? launch_prefill_quant<128, 0>(qa, ka, va, qo->fmt, norm, v4, qch, kch, vch, nq, nk, nv, s)
               : launch_prefill_quant<128, 1>(qa, ka, va, qo->fmt, norm, v4, qch, kch, vch, nq, nk, nv, s);
  if (v4) return hipErrorInvalidValue;           // the ABI admits 4-bit V here only with d = 128
  return q->dtype == FA4_F32 ? launch_prefill_quant<64, 0>(qa, ka, va, qo->fmt, norm, false, qch, kch, vch, nq, nk, nv, s)
                             : launch_prefill_quant<64, 1>(qa, ka, va, qo->fmt, norm, false, qch, kch, vch, nq, nk, nv, s);
}

hipError_t launch_quantize(const fa4_qinput *in, uint32_t flags, const fa4_qoutput *out,
                           const fa4_qoutput *res, float *norm2, hipStream_t s) {
  const QArgs a = quant_args(in, out, res, norm2);
  const int64_t groups = in->outer * in->heads;
  const bool had = flags & FA4_HADAMARD128, dual = flags & FA4_DUAL_RESIDUAL, norm = norm2 != nullptr;
  const bool search = flags & FA4_SCALE_SEARCH;
  if (out->fmt == FA4_MXFP4_KEYS) {
    const dim3 grid((unsigned)(in->rows / 32), (unsigned)groups);
    if (in->dtype == FA4_F32) hipLaunchKernelGGL(mx_keys_kernel<0>, grid, dim3(128), 0, s, a, in->d);
    else hipLaunchKernelGGL(mx_keys_kernel<1>, grid, dim3(128), 0, s, a, in->d);
    return hipGetLastError();
  }
  if (in->d == 128) {
    return in->dtype == FA4_F32 ? quantize_dispatch<128, 0>(a, out->fmt, had, dual, search, groups, norm, s)
                                : quantize_dispatch<128, 1>(a, out->fmt, had, dual, search, groups, norm, s);
  }
  return in->dtype == FA4_F32 ? quantize_dispatch<64, 0>(a, out->fmt, false, dual, search, groups, norm, s)
                              : quantize_dispatch<64, 1>(a, out->fmt, false, dual, search, groups, norm, s);
}

}  // namespace fa4

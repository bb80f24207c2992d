// Tile-importance selection for gfx950 (ThriftAttention-style).
//
// Source: "ThriftAttention" (ai-feeds.com summary), Method step 2 and Limitations: score 128x128
// query-key tiles cheaply from norms and keep about the top 5% for high precision.
//
// One workgroup of 1024 threads per (batch, query head). The k best valid tiles are the tiles whose
// 64-bit key (float32 score bits << 32 | ~linear index) is >= the k-th largest key: scores are
// non-negative, so their bit patterns order like the values, and the index half makes every key
// unique with ties going to the lower index. The k-th largest key is found exactly in steps:
//   1. tile maxima of the squared row norms into LDS (independent vector loads, wave reductions);
//   2. one histogram over the top 12 bits of every valid tile's score (LDS atomics), and a scan from
//      the top that finds the bucket holding the k-th key and how many keys of that bucket are needed;
//   3. the keys of that bucket are compacted into LDS (wave-aggregated append); when there are
//      more than SEL_CAND keys (say, many equal scores) the remaining passes read all valid tiles
//      instead, filtered by the bucket prefix;
//   4. an MSB-first radix select with 8-bit digits over the remaining 52 bits of those keys.
// Integer counts make every step independent of the order of the atomics. The bitmap is then
// written in one coalesced sweep.
#include "fa4_device.h"
#include "fa4_internal.h"

namespace fa4 {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_MAX_NQ = 1024, SEL_MAX_NK = 4096;
constexpr int SEL_CAND = 8192;            // boundary-bucket keys kept in LDS

__device__ __forceinline__ uint64_t tile_key(float a, float b, int lin) {
  const float s = a * b;
  return ((uint64_t)__float_as_uint(s) << 32) | (uint64_t)(0xffffffffu - (uint32_t)lin);
}

// last valid key tile of query tile i (all tiles when not causal)
__device__ __forceinline__ int last_tile(int i, int nk, int off, int causal) {
  return causal ? min(nk - 1, (off + 128 * i + 127) / 128) : nk - 1;
}

// hist[digit] += 1 for each lane with `match` (LDS atomics; lanes of one instruction that hit the same
// counter are serialized by the hardware, at most 64 deep)
__device__ __forceinline__ void add_digits(int *hist, bool match, int digit) {
  if (match) atomicAdd(&hist[digit], 1);
}

// Wave 0: find the digit (bins nbins-1 .. 0, highest first) where the running count from the top
// reaches `remaining`; writes the digit and how many keys of that digit are still needed.
__device__ __forceinline__ void pick_digit(const int *hist, int nbins, int remaining, int lane, int *s_digit,
                                           int *s_remaining) {
  const int per = nbins / 64;                 // bins per lane, lane l owns the l-th group from the top
  int tot = 0;
  for (int e = 0; e < per; e++) tot += hist[nbins - 1 - per * lane - e];
  int incl = tot;
  for (int m = 1; m < 64; m <<= 1) {
    const int y = __shfl_up(incl, m, 64);
    if (lane >= m) incl += y;
  }
  const int before = incl - tot;
  if (before < remaining && remaining <= incl) {
    int acc = before, e = 0;
    while (acc + hist[nbins - 1 - per * lane - e] < remaining) { acc += hist[nbins - 1 - per * lane - e]; e++; }
    *s_digit = nbins - 1 - per * lane - e;
    *s_remaining = remaining - acc;
  }
}

__global__ void __launch_bounds__(SEL_THREADS) select_kernel(const float *qn, const float *kn, int Hq,
                                                             int Hkv, int Lq, int Lk, int causal,
                                                             int num, int den, uint8_t *bitmap,
                                                             int32_t *counts) {
  __shared__ float amax[SEL_MAX_NQ];
  __shared__ float bmax[SEL_MAX_NK];
  __shared__ int hist[4096];
  __shared__ uint64_t cand[SEL_CAND];
  __shared__ int s_digit, s_remaining, s_ncand;
  const int h = blockIdx.x, b = blockIdx.y;
  const int kvh = h / (Hq / Hkv);
  const int nq = Lq / 128, nk = Lk / 128, off = Lk - Lq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *qrow = qn + ((int64_t)b * Hq + h) * Lq;
  const float *krow = kn + ((int64_t)b * Hkv + kvh) * Lk;

  // ---- 1. tile maxima: 8 threads per tile, 16 floats each
  for (int t0 = 0; t0 < nq + nk; t0 += SEL_THREADS / 8) {
    const int t = t0 + tid / 8, part = tid & 7;
    float v = 0.0f;
    if (t < nq + nk) {
      const float *src = (t < nq ? qrow + (int64_t)t * 128 : krow + (int64_t)(t - nq) * 128) + 16 * part;
      const float4 x0 = reinterpret_cast<const float4 *>(src)[0], x1 = reinterpret_cast<const float4 *>(src)[1];
      const float4 x2 = reinterpret_cast<const float4 *>(src)[2], x3 = reinterpret_cast<const float4 *>(src)[3];
      v = fmaxf(fmaxf(fmaxf(fmaxf(x0.x, x0.y), fmaxf(x0.z, x0.w)), fmaxf(fmaxf(x1.x, x1.y), fmaxf(x1.z, x1.w))),
                fmaxf(fmaxf(fmaxf(x2.x, x2.y), fmaxf(x2.z, x2.w)), fmaxf(fmaxf(x3.x, x3.y), fmaxf(x3.z, x3.w))));
    }
    for (int m = 1; m < 8; m <<= 1) v = fmaxf(v, shfl_xor_f(v, m));
    if (t < nq + nk && part == 0) {
      if (t < nq) amax[t] = v; else bmax[t - nq] = v;
    }
  }
  for (int i = tid; i < 4096; i += SEL_THREADS) hist[i] = 0;
  if (tid == 0) s_ncand = 0;
  // number of valid tiles and k = ceil(num * N / den). Causal: row i holds min(nk, o + i + 1) tiles,
  // o = off / 128 (Lq, Lk are multiples of 128), i.e. o + i + 1 for i < c = nk - o - 1, nk after.
  int64_t nvalid = (int64_t)nq * nk;
  if (causal) {
    const int64_t o = off / 128, c = min<int64_t>(max<int64_t>(nk - o - 1, 0), nq);
    nvalid = c * (o + 1) + c * (c - 1) / 2 + (nq - c) * nk;
  }
  const int64_t k = (num * nvalid + den - 1) / den;
  __syncthreads();

  uint64_t thr = ~(uint64_t)0;                   // k-th largest key (no tile selected when k = 0)
  if (k > 0) {
    // ---- 2. histogram of the top 12 bits (key bits 63..52)
    for (int i = wave; i < nq; i += SEL_WAVES) {
      const float ai = amax[i];
      const int jend = last_tile(i, nk, off, causal);
      for (int j0 = 0; j0 <= jend; j0 += 64) {
        const int j = j0 + lane;
        const bool ok = j <= jend;
        const uint64_t key = ok ? tile_key(ai, bmax[j], i * nk + j) : 0;
        add_digits(hist, ok, (int)(key >> 52));
      }
    }
    __syncthreads();
    if (wave == 0) pick_digit(hist, 4096, (int)k, lane, &s_digit, &s_remaining);
    __syncthreads();
    uint64_t prefix = (uint64_t)s_digit << 52, pmask = (uint64_t)0xfff << 52;
    int remaining = s_remaining;
    // ---- 3. compact the bucket's keys
    for (int i = wave; i < nq; i += SEL_WAVES) {
      const float ai = amax[i];
      const int jend = last_tile(i, nk, off, causal);
      for (int j0 = 0; j0 <= jend; j0 += 64) {
        const int j = j0 + lane;
        const uint64_t key = j <= jend ? tile_key(ai, bmax[j], i * nk + j) : 0;
        const bool in = j <= jend && (key & pmask) == prefix;
        const uint64_t mask = __builtin_amdgcn_ballot_w64(in);
        if (mask) {
          int base = 0;
          if (lane == __builtin_ctzll(mask)) base = atomicAdd(&s_ncand, (int)__builtin_popcountll(mask));
          base = __builtin_amdgcn_readlane(base, __builtin_ctzll(mask));
          const int pos = base + (int)__builtin_popcountll(mask & ((1ull << lane) - 1));
          if (in && pos < SEL_CAND) cand[pos] = key;
        }
      }
    }
    __syncthreads();
    const int ncand = s_ncand;
    const bool in_lds = ncand <= SEL_CAND;        // uniform
    // ---- 4. radix select over key bits 51..0, 8-bit digits (the last digit holds 4 bits)
    for (int shift = 44; shift >= -4; shift -= 8) {
      const int sh = shift < 0 ? 0 : shift;
      const uint64_t dmask = shift < 0 ? 0xf : 0xff;
      for (int i = tid; i < 256; i += SEL_THREADS) hist[i] = 0;
      __syncthreads();
      if (in_lds) {
        for (int c0 = wave * 64; c0 < ncand; c0 += SEL_THREADS) {
          const int c = c0 + lane;
          const uint64_t key = c < ncand ? cand[c] : 0;
          add_digits(hist, c < ncand && (key & pmask) == prefix, (int)((key >> sh) & dmask));
        }
      } else {
        for (int i = wave; i < nq; i += SEL_WAVES) {
          const float ai = amax[i];
          const int jend = last_tile(i, nk, off, causal);
          for (int j0 = 0; j0 <= jend; j0 += 64) {
            const int j = j0 + lane;
            const uint64_t key = j <= jend ? tile_key(ai, bmax[j], i * nk + j) : 0;
            add_digits(hist, j <= jend && (key & pmask) == prefix, (int)((key >> sh) & dmask));
          }
        }
      }
      __syncthreads();
      if (wave == 0) pick_digit(hist, 256, remaining, lane, &s_digit, &s_remaining);
      __syncthreads();
      prefix |= (uint64_t)s_digit << sh;
      pmask |= dmask << sh;
      remaining = s_remaining;
      __syncthreads();
    }
    thr = prefix;
  }
  // ---- bitmap: selected = valid and key >= the k-th largest key
  uint8_t *out = bitmap + ((int64_t)b * Hq + h) * ((int64_t)nq * nk);
  for (int i = wave; i < nq; i += SEL_WAVES) {
    const int jend = last_tile(i, nk, off, causal);
    const float ai = amax[i];
    for (int j = lane; j < nk; j += 64)
      out[(int64_t)i * nk + j] = (k > 0 && j <= jend && tile_key(ai, bmax[j], i * nk + j) >= thr) ? 1 : 0;
  }
  if (counts && tid == 0) counts[(int64_t)b * Hq + h] = (int32_t)k;
}

hipError_t launch_select(const float *qn, const float *kn, int B, int Hq, int Hkv, int Lq, int Lk,
                         int causal, int num, int den, uint8_t *bitmap, int32_t *counts, hipStream_t s) {
  if (B == 0 || Hq == 0) return hipSuccess;
  hipLaunchKernelGGL(select_kernel, dim3(Hq, B), dim3(SEL_THREADS), 0, s, qn, kn, Hq, Hkv, Lq, Lk,
                     causal, num, den, bitmap, counts);
  return hipGetLastError();
}

}  // namespace fa4

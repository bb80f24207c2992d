// Tile-importance selection for gfx950 (ThriftAttention-style).
//
// Source: "ThriftAttention" (ai-feeds.com summary), Method step 2 and Limitations: score 128x128
// query-key tiles cheaply from norms and keep about the top 5% for high precision.
//
// One workgroup per (batch, query head). The tile maxima of the squared row norms are reduced into
// LDS (one wave per tile, coalesced), then the k best valid tiles are found by an exact MSB-first
// radix select over 64-bit keys (float32 score bits << 32 | ~linear index): scores are non-negative,
// so their bit patterns order like the values, and the index half makes every key unique with ties
// going to the lower index. Eight 8-bit passes each histogram the candidates sharing the chosen
// prefix (integer LDS atomics: the counts, hence the result, do not depend on their order) and a
// wave-wide suffix scan picks the digit. The bitmap is then written in one coalesced sweep.
#include "fa4_device.h"
#include "fa4_internal.h"

namespace fa4 {

constexpr int SEL_THREADS = 256;
constexpr int SEL_MAX_NQ = 1024, SEL_MAX_NK = 4096;

__device__ __forceinline__ uint64_t tile_key(float a, float b, int lin) {
  const float s = a * b;
  return ((uint64_t)__float_as_uint(s) << 32) | (uint64_t)(0xffffffffu - (uint32_t)lin);
}

__global__ void __launch_bounds__(SEL_THREADS) select_kernel(const float *qn, const float *kn, int Hq,
                                                             int Hkv, int Lq, int Lk, int causal,
                                                             int num, int den, uint8_t *bitmap,
                                                             int32_t *counts) {
  __shared__ float amax[SEL_MAX_NQ];
  __shared__ float bmax[SEL_MAX_NK];
  __shared__ int hist[256];
  __shared__ uint64_t s_prefix;
  __shared__ int s_remaining;
  const int h = blockIdx.x, b = blockIdx.y;
  const int kvh = h / (Hq / Hkv);
  const int nq = Lq / 128, nk = Lk / 128, off = Lk - Lq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *qrow = qn + ((int64_t)b * Hq + h) * Lq;
  const float *krow = kn + ((int64_t)b * Hkv + kvh) * Lk;

  for (int t = wave; t < nq + nk; t += SEL_THREADS / 64) {
    const float *src = t < nq ? qrow + (int64_t)t * 128 : krow + (int64_t)(t - nq) * 128;
    float v = fmaxf(src[lane], src[lane + 64]);
    for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, shfl_xor_f(v, m));
    if (lane == 0) {
      if (t < nq) amax[t] = v; else bmax[t - nq] = v;
    }
  }
  // number of valid tiles and k = ceil(num * N / den)
  int64_t nvalid = 0;
  for (int i = 0; i < nq; i++) nvalid += causal ? min(nk, (off + 128 * i + 127) / 128 + 1) : nk;
  const int64_t k = (num * nvalid + den - 1) / den;
  __syncthreads();

  const int ntot = nq * nk;
  uint64_t prefix = 0, pmask = 0;
  if (k > 0) {
    int remaining = (int)k;
    for (int pass = 0; pass < 8; pass++) {
      const int shift = 56 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
      for (int lin = tid; lin < ntot; lin += SEL_THREADS) {
        const int i = lin / nk, j = lin - i * nk;
        if (causal && 128 * j > off + 128 * i + 127) continue;
        const uint64_t key = tile_key(amax[i], bmax[j], lin);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
      }
      __syncthreads();
      if (wave == 0) {
        // lane l owns digits 255-4l .. 252-4l (highest first); suffix counts from the top
        int c[4], tot = 0;
        for (int e = 0; e < 4; e++) { c[e] = hist[255 - 4 * lane - e]; tot += c[e]; }
        int incl = tot;                                    // inclusive prefix over lanes 0..l
        for (int m = 1; m < 64; m <<= 1) {
          const int y = __shfl_up(incl, m, 64);
          if (lane >= m) incl += y;
        }
        const int before = incl - tot;                     // keys in higher digits than lane's range
        if (before < remaining && remaining <= incl) {
          int acc = before, e = 0;
          while (acc + c[e] < remaining) { acc += c[e]; e++; }
          s_prefix = prefix | ((uint64_t)(255 - 4 * lane - e) << shift);
          s_remaining = remaining - acc;
        }
      }
      __syncthreads();
      prefix = s_prefix;
      remaining = s_remaining;
      pmask |= (uint64_t)255 << shift;
      __syncthreads();
    }
  }
  // write the bitmap: selected = valid and key >= prefix (the k-th largest key)
  uint8_t *out = bitmap + ((int64_t)b * Hq + h) * ntot;
  for (int lin = tid; lin < ntot; lin += SEL_THREADS) {
    const int i = lin / nk, j = lin - i * nk;
    const bool valid = !causal || 128 * j <= off + 128 * i + 127;
    out[lin] = (k > 0 && valid && tile_key(amax[i], bmax[j], lin) >= prefix) ? 1 : 0;
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

// Decode attention over a paged FP4 KV cache for gfx950 (NVFP4 or MXFP4), with a dual-residual query
// in the cache's format.
//
// Source: "BitDecoding-FP4" (sns.style digest): native FP4 KV-cache decoding over pages (NVFP4 and
// MXFP4 caches), the query split into two FP4 tensors (the second carries the first one's residual),
// probabilities quantized under a scale that cannot underflow, and the query heads of a GQA group
// stacked into one matrix-core tile. "MpFA QK4V8" section 3.3: the softmax statistics stay in FP32.
//
// MXFP4 caches: the E8M0 block scales run along d, the contraction axis of QK^T, so K and Q codes go
// straight into the scaled MFMA (16x16x128, FP4 x FP4, one block scale per lane) with no expansion.
// For PV the scales run along d, which is not the contraction axis (the keys are), so V is expanded
// exactly to bf16 (code * 2^e, at most 2 significant bits; the conversion applies a key's scale to the
// 8 values of its d-run before the 8x8 transpose of 16-bit values) and P^ enters as bf16.
//
// Work decomposition: the keys of each (sequence, key head) are cut into splits of DEC_SPLIT keys; a
// workgroup owns one split for one group of up to 4 of the key head's query heads, and its 4 waves
// take the split's 128-key tiles (the probability tiles) in turn. The 8 query rows of the group
// (4 heads x {Q1, Q2}; a smaller group repeats its last head) form the columns of a 16x16x32 fp16
// MFMA whose rows are 16 keys: NVFP4 values code * s_b are exact in fp16 (at most 5 significant
// bits), so K and Q codes are expanded in registers (hardware fp4->fp16 conversion, then one packed
// multiply by the block scales) and the tensor scales are applied to the fp32 scores. The d axis of
// the QK product is permuted so that each lane's operand is one 16-byte run of a key's codes.
// PV is O^T = V^T P^T, whose A operand needs 8 keys of one d in a lane: each lane gets one 4-byte
// word (8 d values) of 8 key rows (loaded as 8-byte runs, one word of each swapped with the
// neighbour lane) and an 8x8 nibble transpose in registers turns them into 8 words of 8 keys each,
// one per d value, so V never goes through LDS. P^ = E4M3(448 P') is exact in fp16.
// Both pages of a tile are resolved with wave-uniform page-table reads; the next tile's K and V
// loads are issued as soon as the registers holding the current tile's codes are consumed, so every
// wave keeps a tile in flight while it computes. Each tile's (max, sum, P^V) goes to LDS, the tiles
// of the workgroup are merged into the split's partial, and a second kernel merges the splits.
#include "fa4_device.h"
#include "fa4_internal.h"

namespace fa4 {

constexpr int DEC_THREADS = 256;
constexpr int DEC_TPW = 4;                        // tiles per wave
constexpr int DEC_SLOTS = 4 * DEC_TPW;            // tiles per workgroup
constexpr int DEC_SPLIT = 128 * DEC_SLOTS;        // keys per workgroup
static_assert(DEC_SPLIT == DEC_SPLIT_KEYS, "the ABI's grid check uses DEC_SPLIT_KEYS");
constexpr int DEC_PART = 130;                     // floats per (split, head) partial: m, l, O[128]
constexpr float DEC_LOG2E = 1.4426950408889634f;
// cache policy of the KV-cache loads: non-temporal (each cache byte is read once per decode step)
constexpr int DEC_NT = 2;

struct DecArgs {
  const uint8_t *q1c, *q1s, *q2c, *q2s;
  const float *q1t, *q2t;
  const uint8_t *kc, *ks, *vc, *vs;
  const float *kt, *vt;
  const int32_t *pt, *ctx;
  int B, Hq, Hkv, max_pages, nsplit;
  int G, VG;                                      // query heads per key head; groups of up to 4 of them
  int64_t num_pages;
  float scale;
  float pscale;                                   // final factor of P^: 1/448 (FP8) or s_t (NVFP4)
  float *ws, *o;
};

// NVFP4 probabilities: a tile row of P' (largest element exactly 1) is one group, so its tensor scale
// is fl32(1/2688) and the block scales are E4M3(amax_b / fl32(6 s_t)).
constexpr float P4_ST = 1.0f / 2688.0f;
constexpr float P4_SIX_ST = 6.0f * P4_ST;

// 8 E2M1 codes (4 bytes) times an fp16 block scale, as exact fp16 values.
__device__ __forceinline__ v8h expand8(uint32_t w, _Float16 sb) {
  const v2h s2 = {sb, sb};
  const v2h t0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const v2h t1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const v2h t2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const v2h t3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return (v8h){t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
}

// 8 E2M1 codes, element j scaled by its own fp16 scale (pairs (2i, 2i+1) in sp[i]).
__device__ __forceinline__ v8h expand8s(uint32_t w, const v2h sp[4]) {
  const v2h t0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sp[0];
  const v2h t1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sp[1];
  const v2h t2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sp[2];
  const v2h t3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sp[3];
  return (v8h){t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
}

__device__ __forceinline__ _Float16 e4m3_f16(uint32_t code) { return (_Float16)e4m3_value(code); }

// Transpose of an 8x8 matrix of nibbles held as 8 words (word j, nibble e) -> (word e, nibble j):
// swap the off-diagonal 4x4 blocks (16-bit halves), then the 2x2 blocks inside them (bytes), then
// the single nibbles. The first two steps are one byte permute per output word (v_perm_b32: byte k
// of the result is byte sel_k of the pair {hi word: bytes 4..7, lo word: bytes 0..3}); the last one
// is a shift and a bit-field merge per output word: 32 instructions in all.
__device__ __forceinline__ void transpose8x8_nibbles(uint32_t w[8]) {
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint32_t lo = __builtin_amdgcn_perm(w[j + 4], w[j], 0x05040100u);   // halves 0 of j, j + 4
    const uint32_t hi = __builtin_amdgcn_perm(w[j + 4], w[j], 0x07060302u);   // halves 1 of j, j + 4
    w[j] = lo;
    w[j + 4] = hi;
  }
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int r = (k & 1) + 4 * (k >> 1);                   // 0, 1, 4, 5
    const uint32_t x = w[r], y = w[r + 2];
    w[r] = __builtin_amdgcn_perm(y, x, 0x06020400u);        // bytes x0 y0 x2 y2
    w[r + 2] = __builtin_amdgcn_perm(y, x, 0x07030501u);    // bytes x1 y1 x3 y3
  }
#pragma unroll
  for (int r = 0; r < 8; r += 2) {
    const uint32_t x = w[r], y = w[r + 1];
    w[r] = (x & 0x0f0f0f0fu) | ((y << 4) & 0xf0f0f0f0u);   // low nibbles of x and y
    w[r + 1] = ((x >> 4) & 0x0f0f0f0fu) | (y & 0xf0f0f0f0u);  // high nibbles of x and y
  }
}

// The two 64-key pages of a tile as buffer resources over this key head's rows of each page (codes
// 4 KB, scales 512 B (NVFP4) or 256 B (MXFP4) per array). A page without keys (past the context, or an id outside the cache)
// gets a zero-size resource: buffer loads past a resource's size return zeros, so its keys read as
// zeros and no load sits behind a branch. All of it is wave-uniform (scalar registers); the loads
// then carry only a 32-bit per-lane offset.
constexpr int BUF_DWORD3 = 0x00020000;      // raw (untyped) buffer access on gfx9-family targets

struct TilePages {
  __amdgpu_buffer_rsrc_t kc[2], ks[2], vc[2], vs[2];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), 0, bytes, BUF_DWORD3);
}

template <int FMT>
__device__ __forceinline__ TilePages tile_pages(const DecArgs &a, const int32_t *pt, int kvh, int t0, int L) {
  constexpr int SB = FMT == FA4_NVFP4 ? 8 : 4;       // scale bytes per row
  TilePages tp;
#pragma unroll
  for (int p = 0; p < 2; p++) {
    const int pid = min((t0 >> 6) + p, a.max_pages - 1);
    const int pg = __builtin_amdgcn_readfirstlane(pt[pid]);
    const bool ok = t0 + 64 * p < L && pg >= 0 && (int64_t)pg < a.num_pages;
    const int64_t row0 = ((int64_t)(ok ? pg : 0) * a.Hkv + kvh) * 64;
    tp.kc[p] = page_rsrc(a.kc + row0 * 64, ok ? 4096 : 0);
    tp.ks[p] = page_rsrc(a.ks + row0 * SB, ok ? 64 * SB : 0);
    tp.vc[p] = page_rsrc(a.vc + row0 * 64, ok ? 4096 : 0);
    tp.vs[p] = page_rsrc(a.vs + row0 * SB, ok ? 64 * SB : 0);
  }
  return tp;
}

// K of a tile for the QK A operand: block kb (16 keys), lane (g, n) -> key 16 kb + n, codes bytes
// 16 g .. 16 g + 15 (d = 32 g .. 32 g + 31) and the two block scales of those 32 values.
__device__ __forceinline__ void load_k(const TilePages &tp, int n, int g, v4i kc[8], uint32_t ks[8]) {
  const int vo_c = n * 64 + 16 * g, vo_s = n * 8 + 2 * g;   // per-lane offsets; the rest is scalar
#pragma unroll
  for (int kb = 0; kb < 8; kb++) {
    const int p = kb >> 2, r0 = 16 * (kb & 3);
    kc[kb] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(tp.kc[p], vo_c, r0 * 64, DEC_NT));
    ks[kb] = (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(tp.ks[p], vo_s, r0 * 8, DEC_NT);
  }
}

// V codes of a tile for the PV A operand: quarter q (32 keys), element j of lane (g, n) is the key
// 32 q + 16 (j / 4) + 4 g + j % 4, of whose codes the lane needs word n (d = 8 n .. 8 n + 7). The
// words arrive as 8-byte runs: lane (g, 2 m + t) loads words 2 m, 2 m + 1 of the keys of elements
// 2 i + t (i = 0..3), and pair_transpose2 (when the quarter is used) swaps one word of each pair
// with the neighbour lane, so that lane 2 m + t' ends with word 2 m + t' of both keys. Measured
// against one 4-byte word per key (NVFP4 cache 5.22 against 5.08-5.13 TB/s, MXFP4 5.52-5.56 against
// 5.28-5.29, same runs); 16-byte runs with a 4x4 word transpose across each quad of lanes ran at
// 5.12 and 5.47-5.50: their exchange costs twice the instructions per word.
__device__ __forceinline__ void load_v_codes(const TilePages &tp, int n, int g, uint32_t vc[4][8]) {
  const int vo_c = (4 * g + (n & 1)) * 64 + 8 * (n >> 1);   // per-lane offsets; the rest is scalar
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const int p = q >> 1;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r0 = 32 * (q & 1) + 16 * (i >> 1) + 2 * (i & 1);
      const v2i w = __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(tp.vc[p], vo_c, r0 * 64, DEC_NT));
      vc[q][2 * i] = (uint32_t)w[0];
      vc[q][2 * i + 1] = (uint32_t)w[1];
    }
  }
}

// 2x2 transpose of words across a lane pair: lane t holds row t in x[0..1]; afterwards it holds
// column t (x[s] = row s's word t): a neighbour exchange (quad permute 1,0,3,2) and a select per word.
__device__ __forceinline__ void pair_transpose2(uint32_t *x, bool odd) {
  const uint32_t a0 = x[0], a1 = x[1];
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)a0, 0xb1, 0xf, 0xf, true);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)a1, 0xb1, 0xf, 0xf, true);
  x[0] = !odd ? a0 : r1;
  x[1] = odd ? a1 : r0;
}

// V of a tile: codes as load_v_codes; the quarter's 32 scale rows (256 contiguous bytes) are loaded
// one word per lane (lane L: key L / 2, blocks 4 (L % 2) .. 4 (L % 2) + 3) and redistributed with
// lane shuffles when the quarter is used.
__device__ __forceinline__ void load_v(const TilePages &tp, int lane, int n, int g, uint32_t vc[4][8],
                                       uint32_t vs[4]) {
  load_v_codes(tp, n, g, vc);
#pragma unroll
  for (int q = 0; q < 4; q++)
    vs[q] = __builtin_amdgcn_raw_buffer_load_b32(tp.vs[q >> 1], 4 * lane, 256 * (q & 1), DEC_NT);
}

// MXFP4 K: as load_k, with the one E8M0 scale of the lane's 32 values (block g of key 16 kb + n).
__device__ __forceinline__ void load_k_mx(const TilePages &tp, int n, int g, v4i kc[8], uint32_t ks[8]) {
  const int vo_c = n * 64 + 16 * g, vo_s = n * 4 + g;
#pragma unroll
  for (int kb = 0; kb < 8; kb++) {
    const int p = kb >> 2, r0 = 16 * (kb & 3);
    kc[kb] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(tp.kc[p], vo_c, r0 * 64, DEC_NT));
    ks[kb] = __builtin_amdgcn_raw_buffer_load_b8(tp.ks[p], vo_s, r0 * 4, DEC_NT);
  }
}

// MXFP4 V: codes as load_v_codes; the quarter's 32 scale rows (4 bytes each, 128 contiguous bytes)
// are loaded one row per lane (lane L: key L % 32) and fetched by lane shuffles when the quarter is
// used.
__device__ __forceinline__ void load_v_mx(const TilePages &tp, int lane, int n, int g, uint32_t vc[4][8],
                                          uint32_t vs[4]) {
  load_v_codes(tp, n, g, vc);
#pragma unroll
  for (int q = 0; q < 4; q++)
    vs[q] = __builtin_amdgcn_raw_buffer_load_b32(tp.vs[q >> 1], 4 * (lane & 31), 128 * (q & 1), DEC_NT);
}

template <int FMT>
__device__ __forceinline__ void load_k_fmt(const TilePages &tp, int n, int g, v4i kc[8], uint32_t ks[8]) {
  if constexpr (FMT == FA4_NVFP4) load_k(tp, n, g, kc, ks);
  else load_k_mx(tp, n, g, kc, ks);
}
template <int FMT>
__device__ __forceinline__ void load_v_fmt(const TilePages &tp, int lane, int n, int g, uint32_t vc[4][8],
                                           uint32_t vs[4]) {
  if constexpr (FMT == FA4_NVFP4) load_v(tp, lane, n, g, vc, vs);
  else load_v_mx(tp, lane, n, g, vc, vs);
}

// two E4M3 codes (bits 15:0) -> two fp16 values (exact)
__device__ __forceinline__ v2h e4m3x2_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}

// lane n of each 16-lane row reads lane n + k of the row (0 past the row's end)
template <int K>
__device__ __forceinline__ int row_shl(int v) {
  return __builtin_amdgcn_mov_dpp(v, 0x100 + K, 0xf, 0xf, true);
}
template <int K>
__device__ __forceinline__ float row_shl_f(float v) {
  return __int_as_float(row_shl<K>(__float_as_int(v)));
}
template <int K>
__device__ __forceinline__ v8h row_shl_v8h(v8h v) {
  v4i x = __builtin_bit_cast(v4i, v);
  x = (v4i){row_shl<K>(x[0]), row_shl<K>(x[1]), row_shl<K>(x[2]), row_shl<K>(x[3])};
  return __builtin_bit_cast(v8h, x);
}

// the 2 values of nibble pair i (constant after unrolling) of w as bf16 with scale sc
__device__ __forceinline__ uint32_t cvt_bf16_fp4_sel(uint32_t w, float sc, int i) {
  switch (i) {
    case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
    case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
    case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
    default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
  }
}

// Three waves per SIMD (at most 168 VGPRs), with no spills: the V scale shuffles share one address
// register and the MXFP4 path expands V one pair of d values at a time. (A spill in the tile loop
// costs more than the third wave brings.)
template <int FMT, int PF>
__global__ void __launch_bounds__(DEC_THREADS, 3) decode_split_kernel(DecArgs a) {
  __shared__ float part[DEC_SLOTS][4][DEC_PART];
  // A workgroup serves one group of up to 4 query heads of a key head (a key head with G query heads
  // has VG = ceil(G / 4) groups; group sub holds heads 4 sub .. min(G, 4 sub + 4) - 1 of it).
  // Workgroup order: (sequence, key head, group) fastest, split slowest. Workgroups are handed to the
  // 8 XCDs round-robin, so every XCD gets the same mix of sequences (with 8 key heads of one group,
  // one key head each, whose pages then stay in that XCD's L2), and the mostly empty trailing splits
  // come last.
  const int nvk = a.Hkv * a.VG, nbk = a.B * nvk;
  const int split = (int)(blockIdx.x / (unsigned)nbk), bk = (int)(blockIdx.x - (unsigned)split * nbk);
  const int b = bk / nvk, vkh = bk - b * nvk;
  const int kvh = vkh / a.VG, sub = vkh - kvh * a.VG;
  const int nh = min(4, a.G - 4 * sub);                   // heads in this group
  const int h0 = kvh * a.G + 4 * sub;                      // its first query head
  const int L = min(a.ctx[b], a.max_pages * 64);
  if (split * DEC_SPLIT >= L) return;                      // uniform per workgroup
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;                  // MFMA column / lane group
  const int rep = n >> 3;                                  // softmax half: key blocks 4 rep .. 4 rep + 3
  const bool qodd = lane & 1;                              // position in the lane's pair
  const int32_t *pt = a.pt + (int64_t)b * a.max_pages;
  // this wave's tiles: split * DEC_SPLIT + 128 (4 it + wave), it = 0 .. DEC_TPW - 1
  const int tbase = split * DEC_SPLIT + 128 * wave;

  // ---- query operand: column n = residual (n >> 2) & 1 of head h0 + (n & 3) (a group of fewer than 4
  // heads repeats its last head in the spare columns, whose results are not kept); columns 8..15
  // repeat columns 0..7, so that both halves of each row hold every score and split the softmax.
  // NVFP4: physical d of (lane group g, step s, element j) = 32 g + 8 s + j. MXFP4: lane group g holds
  // d = 32 g .. 32 g + 31 (one E8M0 block) as FP4 codes with its scale byte.
  v8h qop[4];
  v8i qmx = {};
  int qsc = 0;
  {
    const int hq = h0 + min(n & 3, nh - 1);
    const bool r2 = n & 4;
    const uint8_t *qc = (r2 ? a.q2c : a.q1c) + ((int64_t)b * a.Hq + hq) * 64 + 16 * g;
    const v4i w = *reinterpret_cast<const v4i *>(qc);
    if constexpr (FMT == FA4_NVFP4) {
      const uint8_t *qs = (r2 ? a.q2s : a.q1s) + ((int64_t)b * a.Hq + hq) * 8 + 2 * g;
      const v2h sc = e4m3x2_f16(*reinterpret_cast<const uint16_t *>(qs));
#pragma unroll
      for (int s = 0; s < 4; s++) qop[s] = expand8((uint32_t)w[s], sc[s >> 1]);
    } else {
      qmx = (v8i){w[0], w[1], w[2], w[3], 0, 0, 0, 0};
      qsc = (r2 ? a.q2s : a.q1s)[((int64_t)b * a.Hq + hq) * 4 + g];
    }
  }
  // scores of head n & 3: x = log2e * scale * s_tK * (s_t1 D[Q1 column] + s_t2 D[Q2 column]) (the
  // tensor scales are 1 for MXFP4)
  const int64_t bq = (int64_t)b * a.Hq + h0 + min(n & 3, nh - 1);
  float c1 = DEC_LOG2E * a.scale, c2 = c1;
  if constexpr (FMT == FA4_NVFP4) {
    const float ck = c1 * a.kt[(int64_t)b * a.Hkv + kvh];
    c1 = ck * a.q1t[bq];
    c2 = ck * a.q2t[bq];
  }
  // V scale redistribution: (key j of this lane, block n / 2) sits in lane 2 kk_j + n / 8, byte
  // (n / 2) % 4, kk_j = 16 (j / 4) + 4 g + j % 4 the key's row within its quarter (MXFP4: the key's
  // 4-byte scale row sits in lane kk_j, byte n / 4). The lane shuffle's byte address is one per-lane
  // base plus a constant per j, which goes into the instruction's offset field, so the eight
  // addresses take one register (keeping the NVFP4 kernel within three waves per SIMD without spills).
  const int vs_base = FMT == FA4_NVFP4 ? 4 * (8 * g + (n >> 3)) : 16 * g;
  auto vs_addr = [&](int j) -> int {
    return vs_base + (FMT == FA4_NVFP4 ? 8 * (16 * (j >> 2) + (j & 3)) : 4 * (16 * (j >> 2) + (j & 3)));
  };
  const int vs_sh = FMT == FA4_NVFP4 ? 8 * ((n >> 1) & 3) : 8 * (n >> 2);
  // NVFP4: one byte permute gathers the two keys' scale bytes (byte vs_sh / 8 of each shuffled word)
  // into bits 15:0 (selector 0x0c gives a zero byte)
  const uint32_t vs_sel = 0x0c0c0000u | ((uint32_t)(4 + (vs_sh >> 3)) << 8) | (uint32_t)(vs_sh >> 3);

  // Software pipeline over the wave's tiles: the next tile's K is requested as soon as this tile's
  // QK has consumed the K registers, and its V as soon as this tile's PV has consumed V, so each
  // load overlaps half a tile of compute.
  v4i kc[8];
  uint32_t ks[8], vc[4][8], vs[4];
  if (tbase < L) {
    const TilePages tp = tile_pages<FMT>(a, pt, kvh, tbase, L);
    load_k_fmt<FMT>(tp, n, g, kc, ks);
    load_v_fmt<FMT>(tp, lane, n, g, vc, vs);
  }
#pragma unroll
  for (int it = 0; it < DEC_TPW; it++) {
    const int t0 = tbase + 512 * it;
    const int slot = 4 * it + wave;
    const bool tail = t0 + 128 > L;                        // the tile holds keys past the context
    const bool has_next = it + 1 < DEC_TPW && t0 + 512 < L;
    TilePages tpn;
    if (has_next) tpn = tile_pages<FMT>(a, pt, kvh, t0 + 512, L);
    float mt = -INFINITY, lsum = 0.0f;
    v4f acc[8];
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = (v4f){0.f, 0.f, 0.f, 0.f};
    if (t0 < L) {
      // ---- S^T = K Q^T for 8 blocks of 16 keys
      v4f S[8];
#pragma unroll
      for (int kb = 0; kb < 8; kb++) {
        S[kb] = (v4f){0.f, 0.f, 0.f, 0.f};
        if constexpr (FMT == FA4_NVFP4) {
          const v2h sc = e4m3x2_f16(ks[kb]);
#pragma unroll
          for (int s = 0; s < 4; s++)
            S[kb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(expand8((uint32_t)kc[kb][s], sc[s >> 1]), qop[s],
                                                           S[kb], 0, 0, 0);
        } else {
          const v8i kop = (v8i){kc[kb][0], kc[kb][1], kc[kb][2], kc[kb][3], 0, 0, 0, 0};
          S[kb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kop, qmx, S[kb], 4, 4, 0, (int)ks[kb], 0, qsc);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (has_next) load_k_fmt<FMT>(tpn, n, g, kc, ks);
      // ---- this lane's half: key blocks 4 rep + kk, keys 16 (4 rep + kk) + 4 g + i. Q1 columns
      // (n & 4 == 0) combine with the Q2 column four lanes up; other lanes carry unused values.
      float x[4][4];
#pragma unroll
      for (int kk = 0; kk < 4; kk++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float sv = rep ? S[4 + kk][i] : S[kk][i];
          x[kk][i] = c1 * sv + c2 * row_shl_f<4>(sv);
        }
      if (tail) {
#pragma unroll
        for (int kk = 0; kk < 4; kk++)
#pragma unroll
          for (int i = 0; i < 4; i++)
            if (t0 + 16 * (4 * rep + kk) + 4 * g + i >= L) x[kk][i] = -INFINITY;
#pragma unroll
        for (int q = 0; q < 4; q++)      // scale word of lane L: key 32 q + L / 2 (MXFP4: 32 q + L % 32)
          if (t0 + 32 * q + (FMT == FA4_NVFP4 ? lane >> 1 : lane & 31) >= L) vs[q] = 0u;
      }
#pragma unroll
      for (int kk = 0; kk < 4; kk++)
#pragma unroll
        for (int i = 0; i < 4; i++) mt = fmaxf(mt, x[kk][i]);
      mt = fmaxf(mt, shfl_xor_f(mt, 8));
      mt = fmaxf(mt, shfl_xor_f(mt, 16));
      mt = fmaxf(mt, shfl_xor_f(mt, 32));
      // ---- P' = 2^(x - m~) and P^ in the B layout of quarter 2 rep + kq: element 4 (kk & 1) + i for
      // kk = 2 kq + (kk & 1)
      v8h popl[2];
      if constexpr (PF == FA4_P_NVFP4) {
        // P^ in NVFP4: key block 4 rep + kk (16 keys: i = 0..3 here, the rest in lane groups g ^ 1,
        // g ^ 2, g ^ 3) gets s_b = E4M3(amax_b / (6 s_t)) and codes E2M1(P' / (s_b s_t)) (hardware
        // conversion: nearest even, saturating, sign kept); E2M1 * s_b (at most 6 significant bits,
        // exact in fp16 and bf16) enters the MFMA and s_t is applied with the final normalization.
        v2h pr[2][4];
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; i++) p[i] = __builtin_amdgcn_exp2f(x[kk][i] - mt);
          lsum += (p[0] + p[1]) + (p[2] + p[3]);
          float bm = fmaxf(fmaxf(p[0], p[1]), fmaxf(p[2], p[3]));
          bm = fmaxf(bm, shfl_xor_f(bm, 16));
          bm = fmaxf(bm, shfl_xor_f(bm, 32));
          const float sbv = e4m3_value(e4m3_encode(bm / P4_SIX_ST));
          const float rq = sbv > 0.0f ? 1.0f / (sbv * P4_ST) : 0.0f;
          uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, p[0] * rq, p[1] * rq, 1.0f, 0);
          w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[2] * rq, p[3] * rq, 1.0f, 1);
          v2h r0, r1;
          if constexpr (FMT == FA4_NVFP4) {
            const _Float16 sbh = (_Float16)sbv;
            r0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * (v2h){sbh, sbh};
            r1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * (v2h){sbh, sbh};
          } else {                                            // bf16 bits: the values are exact in bf16
            const auto f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
            const auto f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
            r0 = __builtin_bit_cast(v2h, (__float_as_uint(f0[0] * sbv) >> 16) | (__float_as_uint(f0[1] * sbv) & 0xffff0000u));
            r1 = __builtin_bit_cast(v2h, (__float_as_uint(f1[0] * sbv) >> 16) | (__float_as_uint(f1[1] * sbv) & 0xffff0000u));
          }
          pr[kk >> 1][2 * (kk & 1)] = r0;
          pr[kk >> 1][2 * (kk & 1) + 1] = r1;
        }
#pragma unroll
        for (int kq = 0; kq < 2; kq++)
          popl[kq] = (v8h){pr[kq][0][0], pr[kq][0][1], pr[kq][1][0], pr[kq][1][1],
                           pr[kq][2][0], pr[kq][2][1], pr[kq][3][0], pr[kq][3][1]};
      } else {
        // P^ = E4M3(448 P'), exact in fp16 (bf16 for MXFP4 caches)
#pragma unroll
        for (int kq = 0; kq < 2; kq++) {
          v2h pr[4];
#pragma unroll
          for (int u = 0; u < 4; u++) {
            const int kk = 2 * kq + (u >> 1), i0 = 2 * (u & 1);
            const float p0 = __builtin_amdgcn_exp2f(x[kk][i0] - mt);
            const float p1 = __builtin_amdgcn_exp2f(x[kk][i0 + 1] - mt);
            lsum += p0 + p1;
            const uint32_t pc = e4m3_encode2(448.0f * p0, 448.0f * p1);
            if constexpr (FMT == FA4_NVFP4) {
              pr[u] = e4m3x2_f16(pc);
            } else {                                            // bf16 bits in the same registers
              pr[u] = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pc, 1.0f, false));
            }
          }
          popl[kq] = (v8h){pr[0][0], pr[0][1], pr[1][0], pr[1][1], pr[2][0], pr[2][1], pr[3][0], pr[3][1]};
        }
      }
      lsum += shfl_xor_f(lsum, 8);
      lsum += shfl_xor_f(lsum, 16);
      lsum += shfl_xor_f(lsum, 32);
      // ---- O^T += V^T P^T, one 32-key quarter at a time (columns 0..3 carry the 4 heads)
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const v8h pb = q < 2 ? popl[q] : row_shl_v8h<8>(popl[q - 2]);
#pragma unroll
        for (int i = 0; i < 4; i++) pair_transpose2(&vc[q][2 * i], qodd);   // vc[q][j]: word n of key j
        if constexpr (FMT == FA4_NVFP4) {
          uint32_t w[8];
#pragma unroll
          for (int j = 0; j < 8; j++) w[j] = vc[q][j];
          transpose8x8_nibbles(w);                             // w[e]: keys j = 0..7 at d = 8 n + e
          v2h sp[4];
#pragma unroll
          for (int jp = 0; jp < 4; jp++) {
            const uint32_t s0 = (uint32_t)__builtin_amdgcn_ds_bpermute(vs_addr(2 * jp), (int)vs[q]);
            const uint32_t s1 = (uint32_t)__builtin_amdgcn_ds_bpermute(vs_addr(2 * jp + 1), (int)vs[q]);
            sp[jp] = e4m3x2_f16(__builtin_amdgcn_perm(s1, s0, vs_sel));
          }
#pragma unroll
          for (int e = 0; e < 8; e++)
            acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(expand8s(w[e], sp), pb, acc[e], 0, 0, 0);
        } else {
          // key j's run of 8 d values -> bf16 with its own scale 2^(code - 127). The conversion reads
          // only the exponent field of its float scale, as an E8M0 code, so the code's bits go there
          // directly (code 0 acts as 2^-127: E2M1 * 2^-127 >= 2^-128 is a bf16 subnormal, exact).
          // Converted one pair of d values (i) at a time, right before the two MFMAs (d = 8 n + 2 i,
          // 8 n + 2 i + 1) that take them, so that only 8 converted words are live.
          float sc[8];
#pragma unroll
          for (int j = 0; j < 8; j++) {
            const uint32_t sw = (uint32_t)__builtin_amdgcn_ds_bpermute(vs_addr(j), (int)vs[q]);
            sc[j] = __uint_as_float(__builtin_amdgcn_ubfe(sw, vs_sh, 8) << 23);
          }
#pragma unroll
          for (int i = 0; i < 4; i++) {
            uint32_t kw[8];
#pragma unroll
            for (int j = 0; j < 8; j++)
              kw[j] = cvt_bf16_fp4_sel(vc[q][j], sc[j], i);
            // 8x8 transpose of 16-bit values: A operand of d = 8 n + e holds keys j = 0..7
#pragma unroll
            for (int e = 2 * i; e < 2 * i + 2; e++) {
              const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
              v4i av;
#pragma unroll
              for (int jp = 0; jp < 4; jp++) av[jp] = (int)__builtin_amdgcn_perm(kw[2 * jp + 1], kw[2 * jp], sel);
              acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av),
                                                               __builtin_bit_cast(v8bf, pb), acc[e], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (has_next) load_v_fmt<FMT>(tpn, lane, n, g, vc, vs);
    }
    // ---- tile partial -> LDS (lanes n < 4 hold head n; acc[e][i] is d = 32 g + 8 i + e)
    if (n < 4) {
      if (g == 0) { part[slot][n][0] = mt; part[slot][n][1] = lsum; }
#pragma unroll
      for (int e = 0; e < 8; e++)
#pragma unroll
        for (int i = 0; i < 4; i++) part[slot][n][2 + 32 * g + 8 * i + e] = acc[e][i];
    }
  }
  __syncthreads();
  // ---- merge the workgroup's tiles: thread -> (head, two d values)
  {
    const int hd = tid >> 6, d0 = 2 * (tid & 63);
    float mm = -INFINITY;
    for (int w = 0; w < DEC_SLOTS; w++) mm = fmaxf(mm, part[w][hd][0]);
    float l = 0.f, o0 = 0.f, o1 = 0.f;
    for (int w = 0; w < DEC_SLOTS; w++) {
      const float mw = part[w][hd][0];
      if (mw == -INFINITY) continue;
      const float f = __builtin_amdgcn_exp2f(mw - mm);
      l += f * part[w][hd][1];
      o0 += f * part[w][hd][2 + d0];
      o1 += f * part[w][hd][3 + d0];
    }
    float *dst = a.ws + ((((int64_t)b * nvk + vkh) * a.nsplit + split) * 4 + hd) * DEC_PART;
    if (d0 == 0) { dst[0] = mm; dst[1] = l; }
    dst[2 + d0] = o0;
    dst[3 + d0] = o1;
  }
}

// Merge the splits of each (sequence, head): O = sum e^(m_s - m) O_s / sum e^(m_s - m) l_s, times
// the V tensor scale and P^'s factor (1/448 for FP8 probabilities, s_t for NVFP4 ones); a sequence
// with no key (ctx_len <= 0) gets O = 0. A split's (m, l) are read by all threads of
// the block alike; the loop is unrolled so that the loads of several splits are in flight at once.
__global__ void __launch_bounds__(128) decode_combine_kernel(DecArgs a) {
  __shared__ float red[2];
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int kvh = h / a.G, c = h - kvh * a.G, hd = c & 3;
  const int vkh = kvh * a.VG + (c >> 2);                  // the workgroups of head h's group
  const int L = min(a.ctx[b], a.max_pages * 64);
  const int ns = (L + DEC_SPLIT - 1) / DEC_SPLIT;
  const float *base = a.ws + (((int64_t)b * a.Hkv * a.VG + vkh) * a.nsplit * 4 + hd) * DEC_PART;
  float mm = -INFINITY;
  for (int s = d; s < ns; s += 128) mm = fmaxf(mm, base[(int64_t)s * 4 * DEC_PART]);
  for (int m = 1; m < 64; m <<= 1) mm = fmaxf(mm, shfl_xor_f(mm, m));
  if ((d & 63) == 0) red[d >> 6] = mm;
  __syncthreads();
  mm = fmaxf(red[0], red[1]);
  float l = 0.f, o = 0.f;
#pragma unroll 8
  for (int s = 0; s < ns; s++) {
    const float *p = base + (int64_t)s * 4 * DEC_PART;
    const float f = __builtin_amdgcn_exp2f(p[0] - mm);
    l += f * p[1];
    o += f * p[2 + d];
  }
  const float vts = (a.vt ? a.vt[(int64_t)b * a.Hkv + kvh] : 1.0f) * a.pscale;
  a.o[((int64_t)b * a.Hq + h) * 128 + d] = ns > 0 ? o / l * vts : 0.0f;   // an empty context gives zeros
}

static DecArgs make_dec(const fa4_decode_args *p, void *ws) {
  DecArgs x;
  x.q1c = p->q1_codes; x.q1s = p->q1_scales; x.q2c = p->q2_codes; x.q2s = p->q2_scales;
  x.q1t = p->fmt == FA4_NVFP4 ? p->q1_tscale : nullptr;
  x.q2t = p->fmt == FA4_NVFP4 ? p->q2_tscale : nullptr;
  x.kc = p->k_codes; x.ks = p->k_scales; x.vc = p->v_codes; x.vs = p->v_scales;
  const bool nv = p->fmt == FA4_NVFP4;           // MXFP4 has no tensor scales (the pointers are not read)
  x.kt = nv ? p->k_tscale : nullptr; x.vt = nv ? p->v_tscale : nullptr;
  x.pt = p->page_table; x.ctx = p->ctx_len;
  x.B = p->B; x.Hq = p->Hq; x.Hkv = p->Hkv; x.max_pages = p->max_pages;
  x.G = p->Hq / p->Hkv;
  x.VG = (x.G + 3) / 4;
  x.nsplit = (p->max_pages * 64 + DEC_SPLIT - 1) / DEC_SPLIT;
  x.num_pages = p->num_pages;
  x.scale = p->softmax_scale;
  x.pscale = p->p_fmt == FA4_P_NVFP4 ? P4_ST : 1.0f / 448.0f;
  x.ws = static_cast<float *>(ws); x.o = p->o;
  return x;
}

size_t decode_workspace_bytes(const fa4_decode_args *p) {
  const int64_t nsplit = ((int64_t)p->max_pages * 64 + DEC_SPLIT - 1) / DEC_SPLIT;
  return (size_t)p->B * p->Hkv * ((p->Hq / p->Hkv + 3) / 4) * nsplit * 4 * DEC_PART * sizeof(float);
}

hipError_t launch_decode(const fa4_decode_args *p, void *ws, hipStream_t s) {
  if (p->B == 0) return hipSuccess;
  const DecArgs x = make_dec(p, ws);
  const dim3 grid((unsigned)((int64_t)x.nsplit * x.B * x.Hkv * x.VG));
  const bool p4 = p->p_fmt == FA4_P_NVFP4;
  if (p->fmt == FA4_MXFP4) {
    if (p4) hipLaunchKernelGGL((decode_split_kernel<FA4_MXFP4, FA4_P_NVFP4>), grid, dim3(DEC_THREADS), 0, s, x);
    else hipLaunchKernelGGL((decode_split_kernel<FA4_MXFP4, FA4_P_FP8>), grid, dim3(DEC_THREADS), 0, s, x);
  } else {
    if (p4) hipLaunchKernelGGL((decode_split_kernel<FA4_NVFP4, FA4_P_NVFP4>), grid, dim3(DEC_THREADS), 0, s, x);
    else hipLaunchKernelGGL((decode_split_kernel<FA4_NVFP4, FA4_P_FP8>), grid, dim3(DEC_THREADS), 0, s, x);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(x.Hq, x.B), dim3(128), 0, s, x);
  return hipGetLastError();
}

}  // namespace fa4

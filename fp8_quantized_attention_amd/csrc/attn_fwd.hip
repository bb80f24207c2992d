// Fused prefill attention for gfx950: block-scaled 4-bit QK^T and FP8 PV on the scaled MFMA,
// FP32 online softmax, optional bf16 tiles chosen by the tile selector.
//
// Sources: "MpFA QK4V8" sections 2.1-2.2 and 3.2-3.4 (QK in 4 bits with the per-group scales applied
// inside the product, V in 8 bits, FP32 running max and sum, tiling); "ThriftAttention" Method step 3
// (selected tiles in high precision merged through the same online softmax); "BitDecoding-FP4"
// (probability scales safe from underflow; transposed softmax); "General notes on quantization"
// (a low-precision product rescaled by the merged operand scales).
//
// Work decomposition: one workgroup = one 128-query tile of one (batch, head); 4 waves of 32 queries.
// K/V tiles of 128 keys are staged in LDS and visited in order (tiles above the causal diagonal are
// skipped). Everything is computed transposed, S^T = K Q^T and O^T = V^T P^T, with 32x32 MFMA tiles:
// a lane then owns one query (column l%32) and 64 of a tile's 128 keys, so the row max and sum are
// in-lane plus one exchange with lane l^32, and the per-query rescale of O is a per-lane scalar.
//
// Probabilities: every per-tile scale is a power of two, like the E8M0 scales of the MX formats. A
// tile's row reference is r = ceil(max S) in log2 units and P' = 2^(S - r) <= 1 (no whole-tile
// underflow). For FP8 tiles V's per-token scale is folded into P before rounding:
// P^ = E4M3(P' * w_c), w_c = s_v[c] 2^-e with 2^e the tile's power-of-two V scale (the smallest with
// 448 * 2^e >= max s_v), so V's codes enter the MFMA as-is. The tile then contributes
// 2^(r - m) 2^e (P^ . Vcode) to a running accumulator with reference m: 2^e rides on V^T's E8M0
// operand scale and 2^(r - m) on P^T's, so the MFMA adds each tile exactly and the accumulator is
// rescaled (by a power of two) only when a tile's reference exceeds m by more than ACC_HEADROOM. The
// score transform is one FMA per element, and the denominator uses the unrounded P'.
#include "fa4_device.h"
#include "fa4_internal.h"

namespace fa4 {

constexpr int ATT_THREADS = 256;
constexpr int K4_RS = 80;     // LDS row stride (bytes) of 4-bit K codes (64 B + pad, conflict-free b128 reads)
constexpr int V8_RS = 144;    // LDS row stride of FP8 V rows (128 B + pad)
constexpr int H16_RS = 272;   // LDS row stride of 16-bit rows (256 B + pad)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LOG2_448 = 8.807354922057604f;   // 4-bit V: 448 P' = 2^(x - r + log2 448)
constexpr float ACC_HEADROOM = 32.0f;   // largest tile weight 2^k allowed before the reference is raised

struct AttnArgs {
  const uint8_t *qc, *qs; const float *qt;
  const uint8_t *kc, *ks; const float *kt;
  const uint8_t *vc; const float *vs;
  const float *vw, *vfs;
  const uint8_t *vbs;                 // 4-bit V: E8M0 scales [B][Hkv][d][Lk/32] (codes in vc: [B][Hkv][d][Lk/2])
  const uint16_t *qb, *kb, *vb;
  const uint8_t *bitmap;
  int B, Hq, Hkv, Lq, Lk, causal;
  float scale;
  float *o, *lse;
};

typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) v4s lds_v4s;

__device__ __forceinline__ v2i lds_tr8(const uint8_t *p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i *)(p));
}
__device__ __forceinline__ v4s lds_tr16(const uint8_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(p));
}

// LDS layout (dynamic).
// MXFP4 tiles are double-buffered and filled by direct global->LDS loads (each wave-wide 16-byte load
// writes 1 KB of LDS contiguously, lane L at +16 L). Buffer b starts at b * QBUF and holds
//   [KC: 128 rows x D/2 code bytes | KS: E8M0 scales, D/32 bytes per row (512 B) | VC: 128 rows x D
//    FP8 bytes | W: 128 floats of P-fold factors w_c].
// The 16-byte chunks of a K row are XOR-swizzled by kswz(r) and those of a V row by vswz(r), so the
// QK operand reads (16 rows x one chunk per 16 lanes) and the transposed V reads (16 rows x two
// chunks per instruction) spread over all LDS banks.
// bf16 tiles (and the fp16 values of NVFP4 K, the bf16 values of MXFP8 K) use 16-bit rows with stride H16_RS in a separate
// layout [K16 | V] that overlaps the quantized buffers; those tiles are staged synchronously.
// Q/K formats whose K tiles are expanded to exact 16-bit values in LDS (their block scales are not
// applied by the MFMA): NVFP4 (fp16) and MXFP8 (bf16).
template <int QF>
struct Expanded {
  static constexpr bool value = QF == FA4_NVFP4 || QF == FA4_MXFP8;
};

template <int D, int QF, bool SEL>
struct AttnLds {
  static constexpr int KC = 128 * (D / 2);
  static constexpr int KS = 512;
  static constexpr int VC = 128 * D;
  static constexpr int QBUF = KC + KS + VC + 512;
  static constexpr int QBYTES = QF == FA4_MXFP4 ? 2 * QBUF : 0;
  static constexpr int K16 = 128 * H16_RS;
  static constexpr int V8 = 128 * V8_RS;                 // NVFP4 tiles' FP8 V rows
  static constexpr int V16 = 128 * H16_RS;               // selected tiles' bf16 V rows (overlap V8 onwards)
  // staging of the next tile's raw data (NVFP4, MXFP8): K codes, K scales, V codes, fold factors
  static constexpr int SKC = QF == FA4_MXFP8 ? 128 * D : 128 * (D / 2);
  static constexpr int SKS = QF == FA4_MXFP8 ? 128 * (D / 32) : 128 * (D / 16);
  static constexpr int NVSTAGE = SKC + SKS + 128 * D + 512;
  static constexpr int NBYTES = Expanded<QF>::value ? K16 + V8 + 512 + NVSTAGE : 0;
  static constexpr int SBYTES = SEL ? K16 + V16 : 0;
  static constexpr int HBYTES = NBYTES > SBYTES ? NBYTES : SBYTES;
  static constexpr int BYTES = QBYTES > HBYTES ? QBYTES : HBYTES;
};
template <int D>
__device__ __forceinline__ int kswz(int r) { return D == 128 ? ((r >> 2) & 3) : ((r >> 3) & 1); }
template <int D>
__device__ __forceinline__ int vswz(int r) { return D == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }

typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void dma16(const void *g, uint8_t *l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t *)l, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *g, uint8_t *l) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_t *)l, 4, 0, 0);
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 8 E2M1 codes (4 bytes, low nibble first) times an E4M3 block scale as exact fp16 values (code * s_b
// has at most 6 significant bits): hardware fp4 -> fp16 conversion, then one packed multiply.
__device__ __forceinline__ v8h nv_expand8(uint32_t w, _Float16 sb) {
  const v2h s2 = {sb, sb};
  const v2h t0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const v2h t1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const v2h t2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const v2h t3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return (v8h){t0[0], t0[1], t1[0], t1[1], t2[0], t2[1], t3[0], t3[1]};
}

// MXFP8: an E8M0 scale code as the float 2^(code - 127) for the conversions below (code 0, a block with
// amax below 448 * 2^-127, is taken as 2^-126 so that the scale stays a normal float).
__device__ __forceinline__ float mx8_scale_float(uint32_t code) {
  return __uint_as_float((code > 1u ? code : 1u) << 23);
}
// 8 E4M3 codes (w.x bytes 0-3, w.y bytes 4-7) times 2^e as exact bf16 values (at most 4 significant
// bits; bf16 has the float exponent range), packed two per word in element order.
__device__ __forceinline__ v4i mx8_expand8(uint2 w, float sc) {
  v4i r;
  r[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, sc, false));
  r[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, sc, true));
  r[2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, sc, false));
  r[3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, sc, true));
  return r;
}

// Per-lane LDS byte offsets of every operand read of a tile step. All the XOR swizzles depend only on
// the lane (the tile-varying parts of a key index are multiples of 16 or 32), so each read is
// base + lane offset + a compile-time immediate and only these few registers stay live.
struct LaneOff {
  int k[2];      // MX K codes, per 64-d step s (key = col)
  int ks;        // MX K scales
  int v[4];      // MX V (transposed FP8 reads), per 32-row block mb of d
  int w;         // fold factors
  int k16;       // 16-bit K rows
  int v16;       // bf16 V rows (transposed 16-bit reads)
  int v8;        // NVFP4 tiles' FP8 V rows (stride V8_RS)
};

template <int D>
__device__ __forceinline__ LaneOff lane_offsets(int lane) {
  LaneOff o;
  const int hh = lane >> 5, col = lane & 31, q4 = lane >> 4;
#pragma unroll
  for (int s = 0; s < 2; s++) o.k[s] = col * (D / 2) + 16 * ((2 * s + hh) ^ kswz<D>(col));
  o.ks = col * (D == 128 ? 4 : 2);
  {
    const int aa = lane & 1, tp = (lane >> 1) & 7;
    const int kl = 8 * (tp >> 2) + 4 * (q4 >> 1) + (tp & 3);       // key within its 16-key run
#pragma unroll
    for (int mb = 0; mb < 4; mb++) o.v[mb] = kl * D + 16 * ((2 * mb + (q4 & 1)) ^ vswz<D>(kl)) + 8 * aa;
    o.v8 = kl * V8_RS + 16 * (q4 & 1) + 8 * aa;
  }
  o.w = 16 * hh;
  o.k16 = col * H16_RS + 16 * hh;
  {
    const int aa = lane & 3, t = (lane >> 2) & 3;
    o.v16 = (4 * (q4 >> 1) + t) * H16_RS + 2 * (16 * (q4 & 1) + 4 * aa);
  }
  return o;
}

// ---- pieces of a tile step (this lane: query qrow, keys 32 kb + 8 (i / 4) + 4 hh + i % 4 of S[kb][i])

// S^T for key block kb (32 keys x the wave's 32 queries) from MXFP4 codes in LDS: D/64 scaled FP4 MFMAs,
// the E8M0 scales of K (per key and 32-element block) and of Q applied in-instruction.
template <int D>
__device__ __forceinline__ v16f qk_mx_block(const LaneOff &lo, int kb, int hh, const v8i *qop4, const int *qsc4,
                                            const uint8_t *k4, const uint8_t *ksc) {
  v16f s = (v16f){};
  const uint32_t scw = D == 128 ? *reinterpret_cast<const uint32_t *>(ksc + lo.ks + 128 * kb)
                                : *reinterpret_cast<const uint16_t *>(ksc + lo.ks + 64 * kb);
#pragma unroll
  for (int st = 0; st < D / 64; st++) {
    const int kscl = (int)((scw >> (8 * (2 * st + hh))) & 0xffu);
    const v4i t = *reinterpret_cast<const v4i *>(k4 + lo.k[st] + 32 * kb * (D / 2));
    const v8i kop = (v8i){t[0], t[1], t[2], t[3], 0, 0, 0, 0};
    s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop, qop4[st], s, 4, 4, 0, kscl, 0, qsc4[st]);
  }
  return s;
}

// Keys past the query position get -inf (the tile crossing the causal diagonal).
__device__ __forceinline__ void mask_tile(v16f S[4], int kt, int hh, int qpos) {
#pragma unroll
  for (int kb = 0; kb < 4; kb++)
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int key = kt * 128 + 32 * kb + 8 * (i / 4) + 4 * hh + (i % 4);
      if (key > qpos) S[kb][i] = -INFINITY;
    }
}

// The tile's row reference in log2 units: the smallest integer r >= its largest score, so that
// P' = 2^(S cs - r) <= 1 (its largest value lies in (1/2, 1]). The maximum runs over independent
// partial results, so no long dependent chain forms.
__device__ __forceinline__ float tile_reference(const v16f S[4], float cs) {
  float mp[4];
#pragma unroll
  for (int kb = 0; kb < 4; kb++) {
    mp[kb] = S[kb][0];
#pragma unroll
    for (int i = 1; i < 16; i++) mp[kb] = fmaxf(mp[kb], S[kb][i]);
  }
  float mS = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
  mS = fmaxf(mS, shfl_xor_f(mS, 32));
  return ceilf(mS * cs);
}

// Running reference m (log2 units, an integer): raised only when a tile's reference exceeds it by
// more than ACC_HEADROOM, so the accumulator and the sum (tile weights up to 2^ACC_HEADROOM) stay far
// from overflow; raising rescales both by an exact power of two. Returns the tile weight exponent kB
// (2^kB = 2^(r - m)) and the exponent reference rr0: a weight below 2^-127 (the smallest E8M0 scale)
// adds nothing representable, so those rows take an infinite reference and their probabilities are
// exactly zero (the clamped scale does not inflate them).
template <int NDB>
__device__ __forceinline__ int tile_weight(float r, float &m, float &lsum, v16f *acc, float &rr0) {
  if (__builtin_amdgcn_ballot_w64(r > m + ACC_HEADROOM) != 0) {   // uniform (always on the first tile)
    const float m_new = fmaxf(m, r);
    const float alpha = m == -INFINITY ? 0.0f : __builtin_ldexpf(1.0f, (int)(m - m_new));
#pragma unroll
    for (int i = 0; i < NDB; i++) acc[i] *= alpha;
    lsum *= alpha;
    m = m_new;
  }
  const int kB = (int)fmaxf(r - m, -255.0f);
  rr0 = kB < -127 ? INFINITY : r;
  return kB;
}

// P' = 2^(S cs - r) for key block kb (summed into ts) and P^ = E4M3(P' w_c), w_c = s_v[c] 2^-e
// (exact), packed straight into the PV B operand, so scores and probabilities are never both held.
template <bool V4>
__device__ __forceinline__ void fp8_block(const v16f &Skb, int kb, const float *svs, const LaneOff &lo, float cs,
                                          float rr0, float &ts, v8i pop[2]) {
#pragma unroll
  for (int a4 = 0; a4 < 4; a4++) {
    // 4-bit V has no per-token scale to fold: P^ = E4M3(448 P'), the 448 leaves with the final division
    const float4 w4 = V4 ? make_float4(448.0f, 448.0f, 448.0f, 448.0f)
                         : *reinterpret_cast<const float4 *>(reinterpret_cast<const uint8_t *>(svs) + lo.w +
                                                             4 * (32 * kb + 8 * a4));
    const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
    float pw[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      if (V4) {   // 448 P' straight from the exponent (log2 448 folded into the reference); ts sums 448 P'
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(Skb[4 * a4 + u], cs, -rr0 + LOG2_448));
        ts += p;
        pw[u] = p;
      } else {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(Skb[4 * a4 + u], cs, -rr0));
        ts += p;
        pw[u] = p * wv[u];
      }
    }
    // the first conversion keeps the register's high half, which the second one then writes:
    // starting from the bits of its own (dead) first input avoids materializing a zero
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(pw[0], pw[1], __float_as_int(pw[0]), false);
    x = __builtin_amdgcn_cvt_pk_fp8_f32(pw[2], pw[3], x, true);
    pop[kb >> 1][4 * (kb & 1) + a4] = x;
  }
}

// O^T += V^T P^T for an FP8 tile: the tile's power-of-two V scale 2^e rides on V^T's E8M0 operand scale
// (scA) and the tile weight 2^kBc on P^T's, so the MFMA adds the tile exactly.
template <int D, int QF>
__device__ __forceinline__ void pv_fp8(const v8i pop[2], const uint8_t *vq, const LaneOff &lo, int scA, int kBc,
                                       v16f *acc) {
  constexpr int NDB = D / 32;
#pragma unroll
  for (int t = 0; t < 2; t++) {
#pragma unroll
    for (int mb = 0; mb < NDB; mb++) {
      v8i vop;
#pragma unroll
      for (int u = 0; u < 4; u++) {
        // source lane (16q + a + 2t'): key 64t + 32(u/2) + 16(u%2) + 8(t'/4) + 4g + t'%4,
        //                              d 32mb + 16(q%2) + 8a
        const int krun = 64 * t + 32 * (u >> 1) + 16 * (u & 1);
        const v2i rr = QF == FA4_MXFP4 ? lds_tr8(vq + lo.v[mb] + krun * D)
                                       : lds_tr8(vq + lo.v8 + krun * V8_RS + 32 * mb);
        vop[2 * u] = rr[0];
        vop[2 * u + 1] = rr[1];
      }
      acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop, pop[t], acc[mb], 0, 0, 0, scA, 0, kBc + 127);
    }
  }
}

// O^T += V^T P^T for a tile of 4-bit V (MXFP4, E8M0 scales along the keys): V^T rows (one value of d,
// 128 keys) sit in LDS as 64 code bytes each, 16-byte pieces XOR-swizzled as K's. The A operand of MFMA t
// (keys 64 t .. 64 t + 63) for row 32 mb + (lane % 32) is the piece 2 t + lane / 32, with that
// 32-key block's scale byte: FP4 V^T times FP8 P^T in one scaled MFMA, both scales applied inside.
// Within each 32-key block the codes are stored in the key order of the FP8 operand (P^T's bytes 4 a + u
// of lane half h are keys 8 a + 4 h + u), so no reordering is needed here.
template <int D>
__device__ __forceinline__ void pv_fp4v(const v8i pop[2], const uint8_t *vt, const uint8_t *vts, int lane, int kBc,
                                        v16f *acc) {
  constexpr int NDB = D / 32;
  const int h = lane >> 5;
#pragma unroll
  for (int mb = 0; mb < NDB; mb++) {
    const int row = 32 * mb + (lane & 31);
    const uint32_t sw = *reinterpret_cast<const uint32_t *>(vts + 4 * row);     // the row's 4 block scales
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const v4i c = *reinterpret_cast<const v4i *>(vt + row * 64 + 16 * ((2 * t + h) ^ kswz<128>(row)));
      const int sa = (int)((sw >> (8 * (2 * t + h))) & 0xffu);
      acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4((v8i){c[0], c[1], c[2], c[3], 0, 0, 0, 0}, pop[t],
                                                                acc[mb], 4, 0, 0, sa, 0, kBc + 127);
    }
  }
}

// Wave-uniform reads go through the constant address space, so they become scalar loads (counted
// apart from the vector loads: waiting for one never waits for the tile loads in flight).
template <typename T>
__device__ __forceinline__ T uniform_load(const T *p, int64_t i) {
  return ((const __attribute__((address_space(4))) T *)p)[i];
}

// E8M0 code of tile kt's power-of-two V scale 2^e (stored as a float; 2^-127 is the subnormal whose
// exponent field is 0, matching E8M0 code 0)
__device__ __forceinline__ int v_tile_scale_code(const float *vfs, int64_t bhk, int nk, int kt) {
  return (int)((__float_as_uint(uniform_load(vfs, bhk * nk + kt)) >> 23) & 0xffu);
}

// One 128-key tile for this wave's 32 queries: S^T = K Q^T, softmax step, O^T += V^T P^T.
// MASK: the tile crosses the causal diagonal (keys past the query position get -inf).
// sel: a selected tile, computed from the bf16 originals (QK^T and PV on bf16 MFMA).
template <int D, int QF, bool MASK, bool sel, bool V4 = false>
__device__ __forceinline__ void tile_step(const AttnArgs &a, const LaneOff &lo, int kt, int lane, int hh, int col, int qrow,
                                          int off, int64_t bhq, int64_t bhk, int nk, float cs_q, float cs_b,
                                          const v8i *qop4, const int *qsc4, const v8h *qop16, const uint8_t *k4,
                                          const uint8_t *ksc, const uint8_t *k16, const uint8_t *vq,
                                          const uint8_t *v16, const float *svs, float &m, float &lsum, v16f *acc) {
  constexpr int NDB = D / 32;
  v16f S[4];
  if (sel) {
#pragma unroll
    for (int kb = 0; kb < 4; kb++) S[kb] = (v16f){};
#pragma unroll
    for (int s = 0; s < 8; s++) {
      const v8bf qb = *reinterpret_cast<const v8bf *>(a.qb + (bhq * a.Lq + qrow) * D + 16 * s + 8 * hh);
#pragma unroll
      for (int kb = 0; kb < 4; kb++) {
        const v8bf kop = *reinterpret_cast<const v8bf *>(k16 + lo.k16 + 32 * kb * H16_RS + 32 * s);
        S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qb, S[kb], 0, 0, 0);
      }
    }
  } else if (QF == FA4_MXFP4) {
#pragma unroll
    for (int kb = 0; kb < 4; kb++) S[kb] = qk_mx_block<D>(lo, kb, hh, qop4, qsc4, k4, ksc);
  } else {
    // expanded K (NVFP4: fp16 values; MXFP8: bf16 values, both exact) and the matching Q registers
#pragma unroll
    for (int kb = 0; kb < 4; kb++) S[kb] = (v16f){};
#pragma unroll
    for (int s = 0; s < 8; s++)
#pragma unroll
      for (int kb = 0; kb < 4; kb++) {
        const v8h kop = *reinterpret_cast<const v8h *>(k16 + lo.k16 + 32 * kb * H16_RS + 32 * s);
        if (QF == FA4_MXFP8)
          S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, kop),
                                                          __builtin_bit_cast(v8bf, qop16[s]), S[kb], 0, 0, 0);
        else
          S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop, qop16[s], S[kb], 0, 0, 0);
      }
  }

  const float cs = sel ? cs_b : cs_q;
  if (MASK) mask_tile(S, kt, hh, qrow + off);
  float rr0;
  const int kB = tile_weight<NDB>(tile_reference(S, cs), m, lsum, acc, rr0);
  float ts[4] = {0.0f, 0.0f, 0.0f, 0.0f};        // partial sums, one per 32-key block
  const int kBc = kB < -127 ? -127 : kB;
  if (sel) {
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][i], cs, -rr0));
        ts[kb] += p;
        S[kb][i] = p;
      }
#pragma unroll
    for (int kb = 0; kb < 4; kb++)
#pragma unroll
      for (int p = 0; p < 2; p++) {
        v8s pbs;
#pragma unroll
        for (int j = 0; j < 8; j++) pbs[j] = (short)float_to_bf16_bits(__builtin_ldexpf(S[kb][8 * p + j], kBc));
        const v8bf pb = __builtin_bit_cast(v8bf, pbs);
#pragma unroll
        for (int mb = 0; mb < NDB; mb++) {
          v4s rr[2];
#pragma unroll
          for (int v = 0; v < 2; v++)   // source lane (16q + a + 4t): key 32kb + 16p + 8v + 4g + t, d 32mb + 16(q%2) + 4a
            rr[v] = lds_tr16(v16 + lo.v16 + (32 * kb + 16 * p + 8 * v) * H16_RS + 64 * mb);
          // whole-vector reinterpretation (inserting bit-cast elements one at a time miscompiles)
          const v8bf vop = __builtin_bit_cast(v8bf, (v8s)__builtin_shufflevector(rr[0], rr[1], 0, 1, 2, 3, 4, 5, 6, 7));
          acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb, acc[mb], 0, 0, 0);
        }
      }
  } else {
    v8i pop[2];
#pragma unroll
    for (int kb = 0; kb < 4; kb++) fp8_block<V4>(S[kb], kb, svs, lo, cs, rr0, ts[kb], pop);
    if constexpr (V4)   // vq: V^T codes; svs: V^T block scales (the fold-factor slot of the tile buffer)
      pv_fp4v<D>(pop, vq, reinterpret_cast<const uint8_t *>(svs), lane, kBc, acc);
    else
      pv_fp8<D, QF>(pop, vq, lo, v_tile_scale_code(a.vfs, bhk, nk, kt), kBc, acc);
  }
  const float tsum = (ts[0] + ts[1]) + (ts[2] + ts[3]);
  lsum += __builtin_ldexpf(V4 && !sel ? tsum * (1.0f / 448.0f) : tsum, kB);   // 4-bit V: ts summed 448 P'
}

template <int D, int QF, bool CAUSAL, bool SEL, bool V4 = false>
__global__ void __launch_bounds__(ATT_THREADS, 2) attn_fwd_kernel(AttnArgs a) {
  constexpr int NDB = D / 32;        // 32-row blocks of d in O^T
  typedef AttnLds<D, QF, SEL> L;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t *const k16 = lds;                              // 16-bit K rows, stride H16_RS
  uint8_t *const v16 = lds + L::K16;                     // bf16 V rows (stride H16_RS) / NVFP4 tiles' FP8 V
  float *const hsv = reinterpret_cast<float *>(lds + L::K16 + L::V8);    // w_c of NVFP4 tiles
  uint8_t *const nst = lds + L::K16 + L::V8 + 512;       // NVFP4 staging: [K codes | K scales | V | w]

  const int nq = a.Lq / 128, nk = a.Lk / 128;
  // Work order: one block per (q-tile, batch, head), dispatched longest causal rows first. Blocks are
  // handed to the 8 XCDs round-robin, so when the key-head groups split evenly over the XCDs, all the
  // query heads of one key head land on the same XCD and share its L2 copy of K and V.
  int qt, h, b;
  {
    const int L = blockIdx.x, gq = a.Hq / a.Hkv, nb = a.B * a.Hkv;
    if (nb % 8 == 0) {
      const int x = L & 7, r = L >> 3, per = (nb / 8) * gq;
      const int level = r / per, rem = r - level * per;
      const int bhk = x + 8 * (rem / gq);
      b = bhk / a.Hkv;
      h = (bhk - b * a.Hkv) * gq + rem % gq;
      qt = nq - 1 - level;
    } else {
      const int level = L / (a.B * a.Hq), rem = L - level * (a.B * a.Hq);
      b = rem / a.Hq;
      h = rem - b * a.Hq;
      qt = nq - 1 - level;
    }
  }
  const int kvh = h / (a.Hq / a.Hkv);
  const int off = a.Lk - a.Lq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, col = lane & 31;
  const int qrow = qt * 128 + wave * 32 + col;      // this lane's query (B-operand column)
  const LaneOff lo = lane_offsets<D>(lane);
  const int64_t bhq = (int64_t)b * a.Hq + h, bhk = (int64_t)b * a.Hkv + kvh;

  // ---- query operand, held in registers for the whole key loop
  v8i qop4[D / 64];
  int qsc4[D / 64];
  v8h qop16[8];
  float cs_q = a.scale * LOG2E;           // score -> log2 units, quantized tiles
  const float cs_b = a.scale * LOG2E;     // same for bf16 tiles
  if (QF == FA4_MXFP4) {
#pragma unroll
    for (int s = 0; s < D / 64; s++) {
      const v4i t = *reinterpret_cast<const v4i *>(a.qc + (bhq * a.Lq + qrow) * (D / 2) + 32 * s + 16 * hh);
      qop4[s] = (v8i){t[0], t[1], t[2], t[3], 0, 0, 0, 0};
      qsc4[s] = a.qs[(bhq * a.Lq + qrow) * (D / 32) + 2 * s + hh];
    }
  } else if (QF == FA4_MXFP8) {
    // exact bf16 values code * 2^e (bf16 bits in the fp16-typed registers); lane half hh of step s
    // holds d = 16 s + 8 hh .. + 7 (one E8M0 block)
#pragma unroll
    for (int s = 0; s < 8; s++) {
      const uint2 w = *reinterpret_cast<const uint2 *>(a.qc + (bhq * a.Lq + qrow) * 128 + 16 * s + 8 * hh);
      const float sc = mx8_scale_float(a.qs[(bhq * a.Lq + qrow) * 4 + (s >> 1)]);
      const v4i bf = mx8_expand8(w, sc);
      qop16[s] = __builtin_bit_cast(v8h, bf);
    }
  } else {
    // exact NVFP4 values code * s_b in fp16; the tensor scales move into cs_q
#pragma unroll
    for (int s = 0; s < 8; s++) {
      const uint32_t w = *reinterpret_cast<const uint32_t *>(a.qc + (bhq * a.Lq + qrow) * 64 + 8 * s + 4 * hh);
      const float sb = e4m3_value(a.qs[(bhq * a.Lq + qrow) * 8 + s]);
#pragma unroll
      for (int j = 0; j < 8; j++) qop16[s][j] = (_Float16)(e2m1_value((w >> (4 * j)) & 15u) * sb);
    }
    cs_q *= a.qt[bhq] * a.kt[bhk];
  }

  int kt_end = nk;
  if (CAUSAL) kt_end = min(nk, (off + qt * 128 + 127) / 128 + 1);

  float m = -INFINITY, lsum = 0.0f;
  v16f acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; i++) acc[i] = (v16f){};

  auto is_sel = [&](int kt) -> bool { return SEL && uniform_load(a.bitmap, (bhq * nq + qt) * nk + kt) != 0; };
  auto copy_bf16 = [&](int kt) {
    const int64_t krow0 = bhk * a.Lk + (int64_t)kt * 128;
    for (int c = tid; c < 128 * (D / 8); c += ATT_THREADS) {     // 16-byte chunks of bf16 rows
      const int r = c / (D / 8), j = c % (D / 8);
      const v4i kx = *reinterpret_cast<const v4i *>(a.kb + (krow0 + r) * D + 8 * j);
      const v4i vx = *reinterpret_cast<const v4i *>(a.vb + (krow0 + r) * D + 8 * j);
      *reinterpret_cast<v4i *>(k16 + r * H16_RS + 16 * j) = kx;
      *reinterpret_cast<v4i *>(v16 + r * H16_RS + 16 * j) = vx;
    }
  };
// One tile step; MASKV and SELV must be constants. With Lq and Lk multiples of 128 the only tile that
// crosses the causal diagonal is the last one, so loops run MASKV = false and the diagonal tile is peeled.
#define FA4_TILE_STEP(MASKV, SELV, KT, KC, KS, VC, W)                                                         \
  tile_step<D, QF, MASKV, SELV, V4>(a, lo, KT, lane, hh, col, qrow, off, bhq, bhk, nk, cs_q, cs_b, qop4, qsc4, qop16, \
                                KC, KS, k16, VC, v16, W, m, lsum, acc)

  // Tiles are visited in two passes: first every tile computed from the quantized operands, then the
  // selected (bf16) tiles. The result does not depend on the order (each tile's probabilities use its
  // own row maximum), and each pass then holds one code path only.
  const int last = kt_end - 1;
  auto next_quant = [&](int kt) -> int {        // first non-selected tile >= kt, or kt_end
    if (SEL)
      while (kt < kt_end && is_sel(kt)) kt++;
    return kt;
  };
  if (QF == FA4_MXFP4) {
    // ---- quantized tiles: direct global->LDS loads into a double buffer, one tile ahead
    auto issue = [&](int kt, int b) {
      uint8_t *base = lds + b * L::QBUF;
      const int64_t krow0 = bhk * a.Lk + (int64_t)kt * 128;
      constexpr int KI = L::KC / 1024 / 4, VI = L::VC / 1024 / 4;   // wave-loads per wave
#pragma unroll
      for (int e = 0; e < KI; e++) {
        const int i = wave * KI + e;
        const int r = i * (1024 / (D / 2)) + lane / (D / 32), p = lane % (D / 32);
        dma16(a.kc + (krow0 + r) * (D / 2) + 16 * (p ^ kswz<D>(r)), base + 1024 * i);
      }
      if constexpr (V4) {
        // V^T rows (d = 0 .. 127) of the tile: 64 bytes each at key offset 64 kt, laid out as K's rows
#pragma unroll
        for (int e = 0; e < KI; e++) {
          const int i = wave * KI + e;
          const int r = i * 16 + lane / 4, p = lane % 4;
          dma16(a.vc + (bhk * D + r) * (a.Lk / 2) + (int64_t)kt * 64 + 16 * (p ^ kswz<128>(r)),
                base + L::KC + L::KS + 1024 * i);
        }
      } else {
#pragma unroll
        for (int e = 0; e < VI; e++) {
          const int i = wave * VI + e;
          const int r = i * (1024 / D) + lane / (D / 16), p = lane % (D / 16);
          dma16(a.vc + (krow0 + r) * D + 16 * (p ^ vswz<D>(r)), base + L::KC + L::KS + 1024 * i);
        }
      }
      if (D == 128) {
        if (wave < 2) dma4(a.ks + (krow0 + 64 * wave + lane) * 4, base + L::KC + 256 * wave);
      } else if (wave == 0) {
        dma4(a.ks + krow0 * 2 + 4 * lane, base + L::KC);
      }
      if (V4) {           // the 4 scale bytes of each V^T row into the fold-factor slot
        if (wave >= 2)
          dma4(a.vbs + (bhk * D + 64 * (wave - 2) + lane) * (a.Lk / 32) + (int64_t)kt * 4,
               base + L::KC + L::KS + L::VC + 256 * (wave - 2));
      } else if (wave >= 2) {
        dma4(a.vw + krow0 + 64 * (wave - 2) + lane, base + L::KC + L::KS + L::VC + 256 * (wave - 2));
      }
    };
    int b = 0;
    int kt = next_quant(0);
    if (kt < kt_end) issue(kt, 0);
    const int stop = CAUSAL ? last : kt_end;   // the diagonal tile is peeled below
    while (kt < stop) {
      const int nxt = next_quant(kt + 1);
      wait_vmem();
      __syncthreads();                   // tile kt landed (all waves' loads); the previous tile is consumed
      if (nxt < kt_end) issue(nxt, b ^ 1);   // in flight during this tile's compute
      const uint8_t *base = lds + b * L::QBUF;
      FA4_TILE_STEP(false, false, kt, base, base + L::KC, base + L::KC + L::KS,
                    reinterpret_cast<const float *>(base + L::KC + L::KS + L::VC));
      b ^= 1;
      kt = nxt;
    }
    if (CAUSAL && kt == last) {
      wait_vmem();
      __syncthreads();
      const uint8_t *base = lds + b * L::QBUF;
      FA4_TILE_STEP(true, false, kt, base, base + L::KC, base + L::KC + L::KS,
                    reinterpret_cast<const float *>(base + L::KC + L::KS + L::VC));
    }
  } else {
    // ---- NVFP4 / MXFP8 tiles: the next tile's raw codes, scales, V and fold factors are brought into
    // a staging area by direct global->LDS loads while the current tile is computed; at the start of
    // each tile K is expanded from there to exact 16-bit values (NVFP4: fp16, MXFP8: bf16) and V
    // copied next to it.
    constexpr int SK = 0, SKS = L::SKC, SV = SKS + L::SKS, SW = SV + 128 * D;
    constexpr int KROW = QF == FA4_MXFP8 ? D : D / 2;          // code bytes per K row
    auto issue_nv = [&](int kt) __attribute__((always_inline)) {
      const int64_t krow0 = bhk * a.Lk + (int64_t)kt * 128;
      // K codes (8 or 16 KB), V 16 KB: linear 1 KB chunks spread over the 4 waves
#pragma unroll
      for (int e = 0; e < L::SKC / 4096; e++) {
        const int i = wave * (L::SKC / 4096) + e;
        dma16(a.kc + krow0 * KROW + 1024 * i + 16 * lane, nst + SK + 1024 * i);
      }
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int i = wave * 4 + e;
        dma16(a.vc + krow0 * D + 1024 * i + 16 * lane, nst + SV + 1024 * i);
      }
      if (QF == FA4_MXFP8) {                 // 512 B of E8M0 scales
        if (wave < 2) dma4(a.ks + krow0 * (D / 32) + 256 * wave + 4 * lane, nst + SKS + 256 * wave);
      } else if (wave == 0) {
        dma16(a.ks + krow0 * (D / 16) + 16 * lane, nst + SKS);
      }
      if (wave >= 2) dma4(a.vw + krow0 + 64 * (wave - 2) + lane, nst + SW + 256 * (wave - 2));
    };
    auto expand_nv = [&]() __attribute__((always_inline)) {
      if (QF == FA4_MXFP8) {
        // thread: row tid / 2, d = 64 (tid % 2) .. + 63 (two E8M0 blocks), 8 values per 16-byte store
        const int r = tid >> 1, half = tid & 1;
        const uint8_t *src = nst + SK + r * 128 + 64 * half;
        const uint32_t scw = *reinterpret_cast<const uint16_t *>(nst + SKS + r * 4 + 2 * half);
        const float sc0 = mx8_scale_float(scw & 0xffu), sc1 = mx8_scale_float(scw >> 8);
#pragma unroll
        for (int g = 0; g < 8; g++) {
          const uint2 w = *reinterpret_cast<const uint2 *>(src + 8 * g);
          *reinterpret_cast<v4i *>(k16 + r * H16_RS + 2 * (64 * half + 8 * g)) = mx8_expand8(w, g < 4 ? sc0 : sc1);
        }
      } else {
        const int r = tid >> 1, half = tid & 1;
        const v4i c0 = *reinterpret_cast<const v4i *>(nst + SK + r * 64 + 32 * half);
        const v4i c1 = *reinterpret_cast<const v4i *>(nst + SK + r * 64 + 32 * half + 16);
        const uint32_t sbw = *reinterpret_cast<const uint32_t *>(nst + SKS + r * 8 + 4 * half);
#pragma unroll
        for (int blk = 0; blk < 4; blk++) {
          const v4i &cc = blk < 2 ? c0 : c1;
          const uint32_t w0 = (uint32_t)cc[2 * (blk & 1)], w1 = (uint32_t)cc[2 * (blk & 1) + 1];
          const _Float16 sb = (_Float16)e4m3_value((sbw >> (8 * blk)) & 0xffu);
          *reinterpret_cast<v8h *>(k16 + r * H16_RS + 2 * (64 * half + 16 * blk)) = nv_expand8(w0, sb);
          *reinterpret_cast<v8h *>(k16 + r * H16_RS + 2 * (64 * half + 16 * blk + 8)) = nv_expand8(w1, sb);
        }
      }
#pragma unroll
      for (int c = tid; c < 128 * (D / 16); c += ATT_THREADS) {
        const int rr = c / (D / 16), j = c % (D / 16);
        *reinterpret_cast<v4i *>(v16 + rr * V8_RS + 16 * j) = *reinterpret_cast<const v4i *>(nst + SV + rr * D + 16 * j);
      }
      if (tid < 128) hsv[tid] = reinterpret_cast<const float *>(nst + SW)[tid];
    };
    int kt = next_quant(0);
    if (kt < kt_end) issue_nv(kt);
    const int stop = CAUSAL ? last : kt_end;   // the diagonal tile is peeled below
    while (kt < stop) {
      const int nxt = next_quant(kt + 1);
      wait_vmem();
      __syncthreads();                   // staging holds tile kt; the previous tile's K/V are consumed
      expand_nv();
      __syncthreads();                   // K/V of tile kt ready; the staging area is free
      if (nxt < kt_end) issue_nv(nxt);   // in flight during this tile's compute
      FA4_TILE_STEP(false, false, kt, nullptr, nullptr, v16, hsv);
      kt = nxt;
    }
    if (CAUSAL && kt == last) {
      wait_vmem();
      __syncthreads();
      expand_nv();
      __syncthreads();
      FA4_TILE_STEP(true, false, kt, nullptr, nullptr, v16, hsv);
    }
  }
  if (SEL) {
    // ---- selected tiles from the bf16 originals
    for (int kt = 0; kt < (CAUSAL ? last : kt_end); kt++) {
      if (!is_sel(kt)) continue;          // uniform per workgroup
      __syncthreads();
      copy_bf16(kt);
      __syncthreads();
      FA4_TILE_STEP(false, true, kt, nullptr, nullptr, nullptr, nullptr);
    }
    if (CAUSAL && is_sel(last)) {
      __syncthreads();
      copy_bf16(last);
      __syncthreads();
      FA4_TILE_STEP(true, true, last, nullptr, nullptr, nullptr, nullptr);
    }
  }
#undef FA4_TILE_STEP
  // ---------------- epilogue: O = O_acc / l, LSE = m ln2 + ln l
  const float l = lsum + shfl_xor_f(lsum, 32);
  const float fin = (V4 ? 1.0f / 448.0f : 1.0f) / l;     // 4-bit V: P^ carried a factor 448
  float *orow = a.o + (bhq * a.Lq + qrow) * D;
#pragma unroll
  for (int mb = 0; mb < NDB; mb++)
#pragma unroll
    for (int a4 = 0; a4 < 4; a4++) {
      const float4 v = make_float4(acc[mb][4 * a4] * fin, acc[mb][4 * a4 + 1] * fin,
                                   acc[mb][4 * a4 + 2] * fin, acc[mb][4 * a4 + 3] * fin);
      *reinterpret_cast<float4 *>(orow + 32 * mb + 8 * a4 + 4 * hh) = v;
    }
  if (a.lse && hh == 0) a.lse[bhq * a.Lq + qrow] = m * 0.6931471805599453f + logf(l);
}

// Kernels whose LDS exceeds the default dynamic limit are opted in (idempotent, cheap).
template <int D, int QF, bool CAUSAL, bool SEL, bool V4 = false>
static hipError_t allow_lds() {
  return hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_fwd_kernel<D, QF, CAUSAL, SEL, V4>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, AttnLds<D, QF, SEL>::BYTES);
}

// MXFP4 Q/K with 4-bit V (d = 128, no bitmap)
static hipError_t launch_attn_v4(const AttnArgs &x, bool causal, hipStream_t s) {
  dim3 grid((unsigned)((int64_t)(x.Lq / 128) * x.Hq * x.B));
  hipError_t e = causal ? allow_lds<128, FA4_MXFP4, true, false, true>() : allow_lds<128, FA4_MXFP4, false, false, true>();
  if (e != hipSuccess) return e;
  const size_t l0 = AttnLds<128, FA4_MXFP4, false>::BYTES;
  if (causal) hipLaunchKernelGGL((attn_fwd_kernel<128, FA4_MXFP4, true, false, true>), grid, dim3(ATT_THREADS), l0, s, x);
  else hipLaunchKernelGGL((attn_fwd_kernel<128, FA4_MXFP4, false, false, true>), grid, dim3(ATT_THREADS), l0, s, x);
  return hipGetLastError();
}

template <int D, int QF>
static hipError_t launch_attn_t(const AttnArgs &x, bool causal, bool sel, hipStream_t s) {
  dim3 grid((unsigned)((int64_t)(x.Lq / 128) * x.Hq * x.B));
  hipError_t e = causal ? (sel ? allow_lds<D, QF, true, true>() : allow_lds<D, QF, true, false>())
                        : (sel ? allow_lds<D, QF, false, true>() : allow_lds<D, QF, false, false>());
  if (e != hipSuccess) return e;
  const size_t l1 = AttnLds<D, QF, true>::BYTES, l0 = AttnLds<D, QF, false>::BYTES;
  if (causal) {
    if (sel) hipLaunchKernelGGL((attn_fwd_kernel<D, QF, true, true>), grid, dim3(ATT_THREADS), l1, s, x);
    else hipLaunchKernelGGL((attn_fwd_kernel<D, QF, true, false>), grid, dim3(ATT_THREADS), l0, s, x);
  } else {
    if (sel) hipLaunchKernelGGL((attn_fwd_kernel<D, QF, false, true>), grid, dim3(ATT_THREADS), l1, s, x);
    else hipLaunchKernelGGL((attn_fwd_kernel<D, QF, false, false>), grid, dim3(ATT_THREADS), l0, s, x);
  }
  return hipGetLastError();
}

hipError_t launch_attn(const fa4_attn_args *p, hipStream_t s) {
  AttnArgs x;
  x.qc = p->q_codes; x.qs = p->q_scales; x.qt = p->q_tscale;
  x.kc = p->k_codes; x.ks = p->k_scales; x.kt = p->k_tscale;
  x.vc = p->v_codes; x.vs = p->v_scales;
  x.vw = p->v_fold_w; x.vfs = p->v_fold_scale;
  x.vbs = p->v_block_scales;
  x.qb = p->q_bf16; x.kb = p->k_bf16; x.vb = p->v_bf16;
  x.bitmap = p->bitmap;
  x.B = p->B; x.Hq = p->Hq; x.Hkv = p->Hkv; x.Lq = p->Lq; x.Lk = p->Lk; x.causal = p->causal;
  x.scale = p->softmax_scale;
  x.o = p->o; x.lse = p->lse;
  if (x.B == 0 || x.Hq == 0 || x.Lq == 0) return hipSuccess;
  const bool causal = p->causal != 0, sel = p->bitmap != nullptr;
  if (p->v_fmt == FA4_MXFP4_KEYS) return launch_attn_v4(x, causal, s);
  if (p->fmt == FA4_MXFP4) {
    if (p->d == 64) return launch_attn_t<64, FA4_MXFP4>(x, causal, false, s);
    return launch_attn_t<128, FA4_MXFP4>(x, causal, sel, s);
  }
  if (p->fmt == FA4_MXFP8) return launch_attn_t<128, FA4_MXFP8>(x, causal, sel, s);
  return launch_attn_t<128, FA4_NVFP4>(x, causal, sel, s);
}

}  // namespace fa4

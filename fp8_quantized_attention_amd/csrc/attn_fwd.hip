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
// layout [K16 | V] that overlaps the quantized buffers (the selected tiles' pass runs after the quantized tiles).
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
  // the pipelined d = 128 path: K buffers (codes + E8M0) and V buffers (codes + w_c + the tile's V scale)
  static constexpr int PKBUF = 128 * 64 + 512;
  static constexpr int PVBUF = 128 * 128 + 512 + 16;
  static constexpr int QBYTES = QF != FA4_MXFP4 ? 0 : D == 128 ? 2 * PKBUF + 2 * PVBUF : 2 * QBUF;
  static constexpr int K16 = 128 * H16_RS;
  static constexpr int V16 = 128 * H16_RS;               // selected tiles' bf16 V rows
  // expanded-K formats (NVFP4, MXFP8): [K16 | raw K codes and block scales of the next tile | two V
  // buffers (FP8 rows, XOR-swizzled as the MXFP4 path's, then 128 fold factors)]
  static constexpr int SKC = QF == FA4_MXFP8 ? 128 * D : 128 * (D / 2);
  static constexpr int SKS = QF == FA4_MXFP8 ? 128 * (D / 32) : 128 * (D / 16);
  static constexpr int XVBUF = 128 * D + 512;
  static constexpr int NBYTES = Expanded<QF>::value ? K16 + SKC + SKS + 2 * XVBUF : 0;
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

// The same direct global->LDS loads written as inline asm, for the pipelined MXFP4 loop: the compiler
// cannot tell which LDS bytes such a load writes, so after the builtin it waits for the load before every
// later LDS read, which would put the next tiles' load latency in front of this tile's softmax. These
// loads are waited for explicitly (wait_vmem) before the barrier that publishes their buffers. M0 takes
// the wave-uniform LDS address and needs one wait state before the load; no other code of this kernel
// reads M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Addressing: a wave-uniform 64-bit base (SGPRs) plus a 32-bit per-lane byte offset; the LDS address is
// passed as an integer (the dynamic LDS base taken once from the array, plus an offset).
__device__ __forceinline__ void dma16_nw(const void *sbase, uint32_t voff, uint32_t l) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(l);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_nw(const void *sbase, uint32_t voff, uint32_t l) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(l);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

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

// MXFP8: an E8M0 scale code as the scale operand of the conversions below, which read the exponent
// field of their float scale as an E8M0 code: the code's bits go there unchanged (code 0, a block with
// amax below 448 * 2^-127, acts as 2^-127; its values under bf16's smallest subnormal 2^-133 round).
__device__ __forceinline__ float mx8_scale_float(uint32_t code) { return __uint_as_float(code << 23); }
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

// The same product for d = 128 with the key's scale word read once and shifted by 8 hh, so that the E8M0
// byte of block 2 st + hh is byte 2 st of the operand, picked by the MFMA's scale byte select (no per-MFMA
// extraction).
__device__ __forceinline__ v16f qk_mx128(const LaneOff &lo, int kb, int hh, const v8i *qop4, const int *qsc4,
                                         const uint8_t *k4, const uint8_t *ksc) {
  const int scw = (int)(*reinterpret_cast<const uint32_t *>(ksc + lo.ks + 128 * kb) >> (8 * hh));
  const v4i t0 = *reinterpret_cast<const v4i *>(k4 + lo.k[0] + 32 * kb * 64);
  const v4i t1 = *reinterpret_cast<const v4i *>(k4 + lo.k[1] + 32 * kb * 64);
  v16f s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4((v8i){t0[0], t0[1], t0[2], t0[3], 0, 0, 0, 0}, qop4[0],
                                                          (v16f){}, 4, 4, 0, scw, 0, qsc4[0]);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4((v8i){t1[0], t1[1], t1[2], t1[3], 0, 0, 0, 0}, qop4[1], s,
                                                         4, 4, 2, scw, 0, qsc4[1]);
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

// The same mask for the pipelined loop, where the diagonal tile is met inside the loop. It is written as
// bit arithmetic on an opaque value so that the compiler neither hoists the 64 key comparisons out of the
// loop nor forms them as 64 lane masks in scalar registers: m = -1 exactly when the key lies past the
// query (index > lim), and the score's bits are then replaced by those of -inf.
__device__ __forceinline__ void mask_tile_rt(v16f S[4], int kt, int hh, int qpos) {
  int lim = qpos - kt * 128 - 4 * hh;             // largest unmasked key index within the tile, less 4 hh
  asm volatile("" : "+v"(lim));
#pragma unroll
  for (int kb = 0; kb < 4; kb++)
#pragma unroll
    for (int i = 0; i < 16; i++) {
      int m = lim - (32 * kb + 8 * (i / 4) + (i % 4));
      asm volatile("" : "+v"(m));
      m >>= 31;
      S[kb][i] = __uint_as_float((__float_as_uint(S[kb][i]) & ~(uint32_t)m) | (0xff800000u & (uint32_t)m));
    }
}

// max(a, b, c); the compiler forms one v_max3_f32. (Written as plain code, not inline asm: scores come
// straight from MFMAs, and only for instructions it can see does the compiler insert the wait states that
// a VALU read of an MFMA result needs.)
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// max of this lane's value and lane l ^ 32's, by one lane swap on the VALU (no LDS crossbar round trip)
__device__ __forceinline__ float max_lane32(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}

__device__ __forceinline__ float block_max(const v16f &Skb) {
  // a balanced tree of 3-input maxima (5 + 2 instructions, depth 3)
  const float a = max3f(Skb[0], Skb[1], Skb[2]), b = max3f(Skb[3], Skb[4], Skb[5]);
  const float c = max3f(Skb[6], Skb[7], Skb[8]), d = max3f(Skb[9], Skb[10], Skb[11]);
  const float e = max3f(Skb[12], Skb[13], Skb[14]);
  return max3f(max3f(a, b, c), d, max3f(e, Skb[15], Skb[15]));
}

// fp8_block with the block's fold factors already in registers (w4[a4] = w_c of keys 32 kb + 8 a4 + 4 hh + u).
template <bool V4>
__device__ __forceinline__ void fp8_block_w(const v16f &Skb, const float4 *w4, float cs, float rr0, float &ts,
                                            int &x0, int &x1, int &x2, int &x3) {
  int *xs[4] = {&x0, &x1, &x2, &x3};
#pragma unroll
  for (int a4 = 0; a4 < 4; a4++) {
    const float wv[4] = {w4[a4].x, w4[a4].y, w4[a4].z, w4[a4].w};
    float pw[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      if (V4) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(Skb[4 * a4 + u], cs, -rr0 + LOG2_448));
        ts = (a4 == 0 && u == 0) ? p : ts + p;
        pw[u] = p;
      } else {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(Skb[4 * a4 + u], cs, -rr0));
        ts = (a4 == 0 && u == 0) ? p : ts + p;
        pw[u] = p * wv[u];
      }
    }
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(pw[0], pw[1], __float_as_int(pw[0]), false);
    *xs[a4] = __builtin_amdgcn_cvt_pk_fp8_f32(pw[2], pw[3], x, true);
  }
}

// MXFP4 probabilities: this lane's half of one 32-key block (keys 32 kb + 8 a4 + 4 hh + u, element
// 4 a4 + u of Skb) becomes P' w_c in place (4-bit V: P' itself, nothing to fold); ts sums P' and am
// takes the block's largest value.
template <bool V4>
__device__ __forceinline__ void p4_block_w(v16f &Skb, const float4 *w4, float cs, float rr0, float &ts, float &am) {
#pragma unroll
  for (int a4 = 0; a4 < 4; a4++) {
    const float wv[4] = {w4[a4].x, w4[a4].y, w4[a4].z, w4[a4].w};
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(Skb[4 * a4 + u], cs, -rr0));
      ts = (a4 == 0 && u == 0) ? p : ts + p;
      Skb[4 * a4 + u] = V4 ? p : p * wv[u];
    }
  }
  am = block_max(Skb);
}

// Biased E8M0 code of the MX scale of a block maximum a >= 0: the smallest power of two 2^e with
// 6 * 2^e >= a. With a = 1.f * 2^E, 6 * 2^e >= a holds from e = E - 2 when f <= 0.5 and from e = E - 1
// otherwise; adding 0x3fffff to the bits carries into the exponent field exactly when f > 0.5. Zero and
// subnormal maxima give code 0 (2^-127).
__device__ __forceinline__ int mx_p_code(float a) {
  const int c = (int)((__float_as_uint(a) + 0x3fffffu) >> 23) - 2;
  return c < 0 ? 0 : c;
}

// 16 values (x[8 w + j] into nibble j of word w) as E2M1 codes of x / sc, sc a power of two
// (round to nearest even; the hardware conversion divides by its power-of-two scale).
__device__ __forceinline__ void pack_fp4x16(const v16f &x, float sc, uint32_t &w0, uint32_t &w1) {
  uint32_t a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[0], x[1], sc, 0);
  a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, x[2], x[3], sc, 1);
  a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, x[4], x[5], sc, 2);
  w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, x[6], x[7], sc, 3);
  uint32_t b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[8], x[9], sc, 0);
  b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, x[10], x[11], sc, 1);
  b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, x[12], x[13], sc, 2);
  w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, x[14], x[15], sc, 3);
}

// The FP4 P^T operand of one PV half from the P' w of key blocks 2t (S0) and 2t + 1 (S1). Lane half hh's
// operand holds the 32 keys of block 2t + hh: nibbles 0..15 the keys 8 a + u of that block (held by lane
// half 0), nibbles 16..31 the keys 8 a + 4 + u (held by lane half 1); the FP8 V^T operand pairs its
// k positions with these keys. Each lane quantizes its own halves of both blocks under the block
// scales (block maxima over both lane halves), then swaps one block's words with lane l ^ 32
// (v_permlane32_swap exchanges the upper lanes of its first register with the lower lanes of its second).
// Returns the operand and, in sb, the biased E8M0 B-operand scale: block scale times the tile weight
// 2^kBc; a block below 2^-127 adds nothing representable and is zeroed.
__device__ __forceinline__ v8i p4_operand(const v16f &S0, const v16f &S1, float am0, float am1, int hh, int kBc,
                                          int &sb) {
  const int c0 = mx_p_code(max_lane32(am0)), c1 = mx_p_code(max_lane32(am1));
  uint32_t o0[2], o1[2];
  pack_fp4x16(S0, __uint_as_float((uint32_t)c0 << 23), o0[0], o0[1]);
  pack_fp4x16(S1, __uint_as_float((uint32_t)c1 << 23), o1[0], o1[1]);
  int wv[4];
#pragma unroll
  for (int k = 0; k < 2; k++) {
    const auto x = __builtin_amdgcn_permlane32_swap(o0[k], o1[k], false, false);
    wv[k] = (int)x[0];
    wv[k + 2] = (int)x[1];
  }
  sb = (hh ? c1 : c0) + kBc;
  if (sb < 0) {
    sb = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) wv[k] = 0;
  }
  return (v8i){wv[0], wv[1], wv[2], wv[3], 0, 0, 0, 0};
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
        const v2i rr = lds_tr8(vq + lo.v[mb] + krun * D);
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

// A selected tile from the bf16 originals for this wave's 32 queries, in three steps: S^T = K Q^T on the
// bf16 MFMA (bf16_qk), the online-softmax step with P' = 2^(S cs - r) in fp32 and its rounding to bf16
// after the tile weight 2^kB (bf16_probs), and O^T += V^T P^T on the bf16 MFMA (bf16_pv). qb: this lane's
// bf16 Q operand (d = 16 s + 8 hh .. + 7 for step s); K and V rows in LDS as 16-bit rows of stride H16_RS.
__device__ __forceinline__ void bf16_qk(const v8bf *qb, const uint8_t *k16, const LaneOff &lo, v16f S[4]) {
  // one key block at a time (the scheduling barrier keeps the compiler from holding all 32 K operands)
#pragma unroll
  for (int kb = 0; kb < 4; kb++) {
    v16f sx = (v16f){};
#pragma unroll
    for (int s = 0; s < 8; s++) {
      const v8bf kop = *reinterpret_cast<const v8bf *>(k16 + lo.k16 + 32 * kb * H16_RS + 32 * s);
      sx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qb[s], sx, 0, 0, 0);
    }
    S[kb] = sx;
    __builtin_amdgcn_sched_barrier(0);
  }
}
// The tile weight 2^kB goes into the exponent (2^(S cs - r + kB) = P' 2^kB, the sum then already carries
// it); P' 2^kB is rounded to bf16 by the hardware conversion (nearest even), two values per instruction.
// pb[kb][p]: keys 32 kb + 16 p .. (the PV operand order).
__device__ __forceinline__ void bf16_probs(v16f S[4], float cs, float &m, float &lsum, v16f *acc, v8bf pb[4][2]) {
  float rr0;
  const int kB = tile_weight<4>(tile_reference(S, cs), m, lsum, acc, rr0);
  const float sh = kB < -127 ? -INFINITY : (float)kB - rr0;     // below 2^-127 the tile adds nothing
  float ts[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int kb = 0; kb < 4; kb++)
#pragma unroll
    for (int p = 0; p < 2; p++) {
      float pv[8];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        pv[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][8 * p + j], cs, sh));
        ts[kb] += pv[j];
      }
      pb[kb][p] = (v8bf){(__bf16)pv[0], (__bf16)pv[1], (__bf16)pv[2], (__bf16)pv[3],
                         (__bf16)pv[4], (__bf16)pv[5], (__bf16)pv[6], (__bf16)pv[7]};
    }
  lsum += (ts[0] + ts[1]) + (ts[2] + ts[3]);
}
__device__ __forceinline__ void bf16_pv(const v8bf pb[4][2], const uint8_t *v16, const LaneOff &lo, v16f *acc) {
#pragma unroll
  for (int kb = 0; kb < 4; kb++)
#pragma unroll
    for (int p = 0; p < 2; p++)
#pragma unroll
      for (int mb = 0; mb < 4; mb++) {
        v4s rr[2];
#pragma unroll
        for (int v = 0; v < 2; v++)   // source lane (16q + a + 4t): key 32kb + 16p + 8v + 4g + t, d 32mb + 16(q%2) + 4a
          rr[v] = lds_tr16(v16 + lo.v16 + (32 * kb + 16 * p + 8 * v) * H16_RS + 64 * mb);
        // whole-vector reinterpretation (inserting bit-cast elements one at a time miscompiles)
        const v8bf vop = __builtin_bit_cast(v8bf, (v8s)__builtin_shufflevector(rr[0], rr[1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[kb][p], acc[mb], 0, 0, 0);
      }
}
// One quantized 128-key tile for this wave's 32 queries: S^T = K Q^T, softmax step, O^T += V^T P^T.
// MASK: the tile crosses the causal diagonal (keys past the query position get -inf). sel must be
// false (selected tiles run in a pass of their own, from the bf16 originals).
template <int D, int QF, bool MASK, bool sel, bool V4 = false>
__device__ __forceinline__ void tile_step(const AttnArgs &a, const LaneOff &lo, int kt, int lane, int hh, int col, int qrow,
                                          int off, int64_t bhq, int64_t bhk, int nk, float cs_q, float cs_b,
                                          const v8i *qop4, const int *qsc4, const v8h *qop16, const uint8_t *k4,
                                          const uint8_t *ksc, const uint8_t *k16, const uint8_t *vq,
                                          const uint8_t *v16, const float *svs, float &m, float &lsum, v16f *acc) {
  constexpr int NDB = D / 32;
  static_assert(!sel, "selected tiles take their own pass");
  v16f S[4];
  if (QF == FA4_MXFP4) {
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

  const float cs = cs_q;
  if (MASK) mask_tile(S, kt, hh, qrow + off);
  float rr0;
  const int kB = tile_weight<NDB>(tile_reference(S, cs), m, lsum, acc, rr0);
  float ts[4] = {0.0f, 0.0f, 0.0f, 0.0f};        // partial sums, one per 32-key block
  const int kBc = kB < -127 ? -127 : kB;
  v8i pop[2];
#pragma unroll
  for (int kb = 0; kb < 4; kb++) fp8_block<V4>(S[kb], kb, svs, lo, cs, rr0, ts[kb], pop);
  if constexpr (V4)   // vq: V^T codes; svs: V^T block scales (the fold-factor slot of the tile buffer)
    pv_fp4v<D>(pop, vq, reinterpret_cast<const uint8_t *>(svs), lane, kBc, acc);
  else
    pv_fp8<D, QF>(pop, vq, lo, v_tile_scale_code(a.vfs, bhk, nk, kt), kBc, acc);
  const float tsum = (ts[0] + ts[1]) + (ts[2] + ts[3]);
  lsum += __builtin_ldexpf(V4 ? tsum * (1.0f / 448.0f) : tsum, kB);   // 4-bit V: ts summed 448 P'
}

template <int D, int QF, bool CAUSAL, bool SEL, bool V4 = false, bool P4 = false>
__global__ void __launch_bounds__(ATT_THREADS, 2) attn_fwd_kernel(AttnArgs a) {
  constexpr int NDB = D / 32;        // 32-row blocks of d in O^T
  typedef AttnLds<D, QF, SEL> L;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint8_t *const k16 = lds;                              // 16-bit K rows, stride H16_RS
  uint8_t *const v16 = lds + L::K16;                     // bf16 V rows of the selected tiles (stride H16_RS)

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
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  if constexpr (QF == FA4_MXFP4 && D == 128) {
    // ---- quantized tiles, software-pipelined. K and V have double buffers of their own and K runs one tile
    // ahead of V: iteration i (tile t_i, whose scores S are already in registers with their reference)
    // converts S block by block to FP8 probabilities and, as each block's registers free up, issues the
    // next tile's QK^T MFMAs into them (K(t_{i+1}) in LDS); the two halves of this tile's PV MFMAs go out as
    // soon as their probabilities are packed. The matrix core then works on QK^T(t_{i+1}) and PV(t_i) while
    // the VALU computes the softmax of t_i, and the row maximum of t_{i+1} follows. Loads for K(t_{i+2}) and
    // V(t_{i+1}) are issued at the top of iteration i into the buffers that K(t_i) and V(t_{i-1}) left.
    constexpr int KBUF = L::PKBUF;          // codes (XOR-swizzled rows) + E8M0
    constexpr int VBUF = L::PVBUF;          // V codes + w_c + the tile's V scale (4-bit V: V^T codes + E8M0)
    uint8_t *const vbase = lds + 2 * KBUF;
    const uint32_t lds_addr =
        __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t *)lds);
    // per-lane byte offsets of the loads (loop-invariant; the tile's position goes into the uniform base)
    uint32_t ko[2], vo[4];
#pragma unroll
    for (int e = 0; e < 2; e++) {          // K codes: 16 rows x 64 B per wave-load, two per wave
      const int r = (wave * 2 + e) * 16 + (lane >> 2), p = lane & 3;
      ko[e] = (uint32_t)(r * 64 + 16 * (p ^ kswz<128>(r)));
    }
#pragma unroll
    for (int e = 0; e < 4; e++) {
      if constexpr (V4) {                  // V^T rows (d): 16 rows x 64 B per wave-load, two per wave
        const int r = (wave * 2 + (e & 1)) * 16 + (lane >> 2), p = lane & 3;
        vo[e] = (uint32_t)(r * (a.Lk / 2) + 16 * (p ^ kswz<128>(r)));
      } else {                             // V rows: 8 rows x 128 B per wave-load, four per wave
        const int r = (wave * 4 + e) * 8 + (lane >> 3), p = lane & 7;
        vo[e] = (uint32_t)(r * 128 + 16 * (p ^ vswz<128>(r)));
      }
    }
    const uint32_t so = (uint32_t)(((wave & 1) * 64 + lane) * 4);       // one 4-byte item per row
    const uint32_t vso = V4 ? (uint32_t)(((wave & 1) * 64 + lane) * (a.Lk / 32)) : 0u;   // 4-bit V^T scale rows
    auto issue_k = [&](int kt, int buf) __attribute__((always_inline)) {
      const uint32_t base = lds_addr + buf * KBUF;
      const uint8_t *g = a.kc + (bhk * a.Lk + (int64_t)kt * 128) * 64;
#pragma unroll
      for (int e = 0; e < 2; e++) dma16_nw(g, ko[e], base + 1024 * (wave * 2 + e));
      if (wave < 2) dma4_nw(a.ks + (bhk * a.Lk + (int64_t)kt * 128) * 4, so, base + 8192 + 256 * wave);
    };
    auto issue_v = [&](int kt, int buf) __attribute__((always_inline)) {
      const uint32_t base = lds_addr + 2 * KBUF + buf * VBUF;
      if constexpr (V4) {
        // V^T rows (d = 0 .. 127) of the tile: 64 bytes each at key offset 64 kt, laid out as K's rows
        const uint8_t *g = a.vc + bhk * 128 * (int64_t)(a.Lk / 2) + (int64_t)kt * 64;
#pragma unroll
        for (int e = 0; e < 2; e++) dma16_nw(g, vo[e], base + 1024 * (wave * 2 + e));
        if (wave >= 2) dma4_nw(a.vbs + bhk * 128 * (int64_t)(a.Lk / 32) + (int64_t)kt * 4, vso, base + 8192 + 256 * (wave - 2));
      } else {
        const uint8_t *g = a.vc + (bhk * a.Lk + (int64_t)kt * 128) * 128;
#pragma unroll
        for (int e = 0; e < 4; e++) dma16_nw(g, vo[e], base + 1024 * (wave * 4 + e));
        if (wave >= 2) dma4_nw(a.vw + bhk * a.Lk + (int64_t)kt * 128, so, base + 16384 + 256 * (wave - 2));
        // the tile's power-of-two V scale (4 bytes, one lane): read from LDS in the loop, so that no scalar
        // load (whose wait would also drain the LDS reads in flight) sits on the loop's path
        if (wave == 1 && lane == 0) dma4_nw(a.vfs + bhk * nk + kt, 0u, base + 16384 + 512);
      }
    };
    const float cs = cs_q;
    int tc = next_quant(0);
    if (tc < kt_end) {
      int tn = next_quant(tc + 1);
      issue_k(tc, 0);
      issue_v(tc, 0);
      if (tn < kt_end) issue_k(tn, 1);
      wait_vmem();
      __syncthreads();
      v16f S[4];
#pragma unroll
      for (int kb = 0; kb < 4; kb++) S[kb] = qk_mx128(lo, kb, hh, qop4, qsc4, lds, lds + 8192);
      if (CAUSAL && tc == last) mask_tile_rt(S, tc, hh, qrow + off);
      float rr0;
      int kB = tile_weight<NDB>(tile_reference(S, cs), m, lsum, acc, rr0);
      // The second PV half of each tile is issued in the next iteration's first region (its V operands are
      // read into registers before the barrier that frees the V buffer). Before the first tile the pending
      // half is all zero operands, which add exact zeros.
      v8i vpend[4], ppend = (v8i){};
      int vspend[4];
#pragma unroll
      for (int mb = 0; mb < 4; mb++) {
        vpend[mb] = (v8i){};
        vspend[mb] = 0x7f7f7f7f;                   // E8M0 1.0 in every byte
      }
      int kpend = 0, spend = 127;                  // pending half's P^T weight exponent and V^T scale code
      int ib = 0;                                  // iteration parity: K(t_i) in buffer ib, V(t_i) in buffer ib
      while (true) {
        const bool has_next = tn < kt_end;
        const int tnn = has_next ? next_quant(tn + 1) : kt_end;
        wait_vmem();
        __syncthreads();      // K(t_{i+1}) and V(t_i) landed; every wave is done with K(t_i) and V(t_{i-1})
        if (tnn < kt_end) issue_k(tnn, ib);
        if (has_next) issue_v(tn, ib ^ 1);
        const uint8_t *kq = lds + (ib ^ 1) * KBUF;            // K(t_{i+1})
        const uint8_t *vq = vbase + ib * VBUF;                // V(t_i)
        const float *svs = reinterpret_cast<const float *>(vq + (V4 ? 8192 : 16384));
        const int kBc = kB < -127 ? -127 : kB;
        const int scA = V4 ? 0 : (int)((*reinterpret_cast<const uint32_t *>(vq + 16384 + 512) >> 23) & 0xffu);
        // Five regions, separated by scheduling barriers. Region r < 4 converts block r of this tile to FP8
        // probabilities (VALU) while the matrix core runs: in region 0 the previous tile's second PV half; in
        // region r >= 1 the next tile's QK^T for key block r - 1 (into the registers that block's softmax has
        // just read) and in region 2 this tile's first PV half. Region 4 runs the next tile's QK^T for block 3
        // beside its row maximum over blocks 0-2, and reads this tile's V for the second half. Each region
        // issues its LDS reads first, then spreads its MFMAs through its VALU work. On the last tile the
        // next-tile QK^T reads the other K buffer's stale (in-bounds) bytes and its scores are never used:
        // issuing it unconditionally keeps the score registers in place.
        const bool diag_next = CAUSAL && tn == last;
        float ts[4], mp[3], am[2];
        int psb[2];                  // MXFP4 P: biased E8M0 B-operand scale of each PV half (per lane)
        v8i pop[2];                  // packed FP8 probabilities: the P^T operand of each PV half (keys 64 t ..)
        v8i vop[4];
        int vsw[4];
#pragma unroll
        for (int r = 0; r < 5; r++) {
          // ---- LDS reads
          float4 w4[4];
          if (r < 4 && !V4) {
#pragma unroll
            for (int a4 = 0; a4 < 4; a4++)
              w4[a4] = *reinterpret_cast<const float4 *>(reinterpret_cast<const uint8_t *>(svs) + lo.w + 4 * (32 * r + 8 * a4));
          }
          v4i k0, k1;
          int scw = 0;
          const int qb = r - 1;                            // key block of the next tile's QK^T in this region
          if (r >= 1) {
            k0 = *reinterpret_cast<const v4i *>(kq + lo.k[0] + 2048 * qb);
            k1 = *reinterpret_cast<const v4i *>(kq + lo.k[1] + 2048 * qb);
            scw = (int)(*reinterpret_cast<const uint32_t *>(kq + 8192 + lo.ks + 128 * qb) >> (8 * hh));
          }
          if (r == 2 || r == 4) {                          // V^T operands of half t
            const int t = r == 2 ? 0 : 1;
#pragma unroll
            for (int mb = 0; mb < 4; mb++) {
              if constexpr (V4) {
                const int row = 32 * mb + (lane & 31);
                vsw[mb] = (int)(*reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint8_t *>(svs) + 4 * row) >>
                                (8 * hh));
                const v4i c = *reinterpret_cast<const v4i *>(vq + row * 64 + 16 * ((2 * t + hh) ^ kswz<128>(row)));
                vop[mb] = (v8i){c[0], c[1], c[2], c[3], 0, 0, 0, 0};
              } else {
#pragma unroll
                for (int u = 0; u < 4; u++) {
                  const v2i rr = lds_tr8(vq + lo.v[mb] + (64 * t + 32 * (u >> 1) + 16 * (u & 1)) * 128);
                  vop[mb][2 * u] = rr[0];
                  vop[mb][2 * u + 1] = rr[1];
                }
              }
            }
          }
          // ---- VALU
          if (r < 4) {
            if constexpr (P4) {
              // MXFP4 P: P' w in place; after each pair of blocks, their FP4 operand (the next tile's QK^T
              // into those registers waits for it)
              p4_block_w<V4>(S[r], w4, cs, rr0, ts[r], am[r & 1]);
              if (r & 1) pop[r >> 1] = p4_operand(S[r - 1], S[r], am[0], am[1], hh, kBc, psb[r >> 1]);
            } else {
              int x0, x1, x2, x3;
              fp8_block_w<V4>(S[r], w4, cs, rr0, ts[r], x0, x1, x2, x3);
              pop[r >> 1][4 * (r & 1) + 0] = x0;
              pop[r >> 1][4 * (r & 1) + 1] = x1;
              pop[r >> 1][4 * (r & 1) + 2] = x2;
              pop[r >> 1][4 * (r & 1) + 3] = x3;
            }
          } else {
#pragma unroll
            for (int b = 0; b < 3; b++) {
              mp[b] = block_max(S[b]);                     // (recomputed after masking the diagonal tile)
              asm volatile("" : "+v"(mp[b]));              // computed here, beside block 3's MFMAs
            }
          }
          // ---- MFMA
          if (r == 0) {
#pragma unroll
            for (int mb = 0; mb < 4; mb++) {
              if constexpr (V4)
                acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vpend[mb], ppend, acc[mb], 4, P4 ? 4 : 0, 2, vspend[mb], 0,
                                                                          kpend + 127);
              else
                acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vpend[mb], ppend, acc[mb], 0, P4 ? 4 : 0, 0, spend,
                                                                          0, kpend + 127);
            }
          } else {
            S[qb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4((v8i){k0[0], k0[1], k0[2], k0[3], 0, 0, 0, 0}, qop4[0],
                                                                   (v16f){}, 4, 4, 0, scw, 0, qsc4[0]);
            if (r == 2) {
#pragma unroll
              for (int mb = 0; mb < 4; mb++) {
                if constexpr (V4 && P4)
                  acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[mb], pop[0], acc[mb], 4, 4, 0, vsw[mb], 0,
                                                                            psb[0]);
                else if constexpr (V4)
                  acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[mb], pop[0], acc[mb], 4, 0, 0, vsw[mb], 0,
                                                                            kBc + 127);
                else if constexpr (P4)
                  acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[mb], pop[0], acc[mb], 0, 4, 0, scA, 0,
                                                                            psb[0]);
                else
                  acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[mb], pop[0], acc[mb], 0, 0, 0, scA, 0,
                                                                            kBc + 127);
              }
            }
            S[qb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4((v8i){k1[0], k1[1], k1[2], k1[3], 0, 0, 0, 0}, qop4[1],
                                                                   S[qb], 4, 4, 2, scw, 0, qsc4[1]);
          }
          // ---- schedule: LDS reads first, then the MFMAs spread through the VALU work
          __builtin_amdgcn_sched_group_barrier(0x100, 32, 0);
          if (r == 0) {
#pragma unroll
            for (int g = 0; g < 4; g++) {
              __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
          } else if (r == 2) {
#pragma unroll
            for (int g = 0; g < 6; g++) {
              __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
          } else if (r < 4) {
            __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 30, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          } else {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 24, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // this tile's second PV half goes out in the next region 0
#pragma unroll
        for (int mb = 0; mb < 4; mb++) {
          vpend[mb] = vop[mb];
          vspend[mb] = vsw[mb];
        }
        ppend = pop[1];
        kpend = P4 ? psb[1] - 127 : kBc;
        spend = scA;
        const float tsum = (ts[0] + ts[1]) + (ts[2] + ts[3]);
        lsum += __builtin_ldexpf(V4 && !P4 ? tsum * (1.0f / 448.0f) : tsum, kB);
        if (!has_next) break;
        float mS;
        if (diag_next) {
          mask_tile_rt(S, tn, hh, qrow + off);
          mS = max3f(max3f(block_max(S[0]), block_max(S[1]), block_max(S[2])), block_max(S[3]), block_max(S[3]));
        } else {
          mS = max3f(max3f(mp[0], mp[1], mp[2]), block_max(S[3]), block_max(S[3]));
        }
        mS = max_lane32(mS);
        const float m_old = m;
        kB = tile_weight<NDB>(ceilf(mS * cs), m, lsum, acc, rr0);
        if (m != m_old) {            // the reference was raised: the pending half's weight follows it
          kpend -= (int)(m - m_old);
          if (kpend < -127) {        // below the smallest E8M0 weight: that half adds nothing representable
            kpend = -127;
            ppend = (v8i){};
          }
        }
        tc = tn;
        tn = tnn;
        ib ^= 1;
      }
      // the last tile's second PV half
#pragma unroll
      for (int mb = 0; mb < 4; mb++) {
        if constexpr (V4)
          acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vpend[mb], ppend, acc[mb], 4, P4 ? 4 : 0, 2, vspend[mb], 0,
                                                                    kpend + 127);
        else
          acc[mb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vpend[mb], ppend, acc[mb], 0, P4 ? 4 : 0, 0, spend, 0,
                                                                    kpend + 127);
      }
    }
  } else if (QF == FA4_MXFP4) {
    // ---- quantized tiles (d = 64): direct global->LDS loads into a double buffer, one tile ahead
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
    // ---- NVFP4 / MXFP8 tiles: the next tile's raw K codes and block scales come into a staging area, its
    // V and fold factors straight into the V buffer the previous tile left, by direct global->LDS loads
    // while the current tile is computed; between two barriers at the start of each tile K is expanded
    // from the staging area to exact 16-bit values (NVFP4: fp16 code * s_b, MXFP8: bf16 code * 2^e).
    constexpr int RAWK = L::K16, RAWS = RAWK + L::SKC, VBUF0 = RAWS + L::SKS;
    auto issue_x = [&](int kt, int vb) __attribute__((always_inline)) {
      const int64_t krow0 = bhk * a.Lk + (int64_t)kt * 128;
#pragma unroll
      for (int e = 0; e < L::SKC / 4096; e++) {   // K codes (8 or 16 KB): linear 1 KB chunks
        const int i = wave * (L::SKC / 4096) + e;
        dma16(a.kc + krow0 * (L::SKC / 128) + 1024 * i + 16 * lane, lds + RAWK + 1024 * i);
      }
      if (QF == FA4_MXFP8) {                     // 512 B of E8M0 scales
        if (wave < 2) dma4(a.ks + krow0 * (D / 32) + 256 * wave + 4 * lane, lds + RAWS + 256 * wave);
      } else if (wave == 0) {                    // 1 KB of E4M3 scales
        dma16(a.ks + krow0 * (D / 16) + 16 * lane, lds + RAWS);
      }
      uint8_t *const vbuf = lds + VBUF0 + vb * L::XVBUF;
#pragma unroll
      for (int e = 0; e < 4; e++) {              // V rows: 8 rows x 128 B per wave-load, chunks XOR-swizzled
        const int r = (wave * 4 + e) * 8 + (lane >> 3), p = lane & 7;
        dma16(a.vc + (krow0 + r) * D + 16 * (p ^ vswz<D>(r)), vbuf + 1024 * (wave * 4 + e));
      }
      if (wave >= 2) dma4(a.vw + krow0 + 64 * (wave - 2) + lane, vbuf + 128 * D + 256 * (wave - 2));
    };
    auto expand_k = [&]() __attribute__((always_inline)) {
      const int r = tid >> 1, half = tid & 1;    // thread: row r, d = 64 half .. 64 half + 63
      if (QF == FA4_MXFP8) {
        // two E8M0 blocks, 8 values per 16-byte store
        const uint8_t *src = lds + RAWK + r * 128 + 64 * half;
        const uint32_t scw = *reinterpret_cast<const uint16_t *>(lds + RAWS + r * 4 + 2 * half);
        const float sc0 = mx8_scale_float(scw & 0xffu), sc1 = mx8_scale_float(scw >> 8);
#pragma unroll
        for (int g = 0; g < 8; g++) {
          const uint2 w = *reinterpret_cast<const uint2 *>(src + 8 * g);
          *reinterpret_cast<v4i *>(k16 + r * H16_RS + 2 * (64 * half + 8 * g)) = mx8_expand8(w, g < 4 ? sc0 : sc1);
        }
      } else {
        // four E4M3 blocks of 16 values
        const v4i c0 = *reinterpret_cast<const v4i *>(lds + RAWK + r * 64 + 32 * half);
        const v4i c1 = *reinterpret_cast<const v4i *>(lds + RAWK + r * 64 + 32 * half + 16);
        const uint32_t sbw = *reinterpret_cast<const uint32_t *>(lds + RAWS + r * 8 + 4 * half);
#pragma unroll
        for (int blk = 0; blk < 4; blk++) {
          const v4i &cc = blk < 2 ? c0 : c1;
          const uint32_t w0 = (uint32_t)cc[2 * (blk & 1)], w1 = (uint32_t)cc[2 * (blk & 1) + 1];
          const _Float16 sb = (_Float16)e4m3_value((sbw >> (8 * blk)) & 0xffu);
          *reinterpret_cast<v8h *>(k16 + r * H16_RS + 2 * (64 * half + 16 * blk)) = nv_expand8(w0, sb);
          *reinterpret_cast<v8h *>(k16 + r * H16_RS + 2 * (64 * half + 16 * blk + 8)) = nv_expand8(w1, sb);
        }
      }
    };
    auto vbuf_of = [&](int vb) -> uint8_t * { return lds + VBUF0 + vb * L::XVBUF; };
    auto w_of = [&](int vb) -> const float * { return reinterpret_cast<const float *>(vbuf_of(vb) + 128 * D); };
    int kt = next_quant(0), vb = 0;
    if (kt < kt_end) issue_x(kt, 0);
    const int stop = CAUSAL ? last : kt_end;   // the diagonal tile is peeled below
    while (kt < stop) {
      const int nxt = next_quant(kt + 1);
      wait_vmem();
      __syncthreads();                   // raw K and V of tile kt landed; the previous tile is consumed
      expand_k();
      __syncthreads();                   // K of tile kt ready; the staging area is free
      if (nxt < kt_end) issue_x(nxt, vb ^ 1);   // in flight during this tile's compute
      FA4_TILE_STEP(false, false, kt, nullptr, nullptr, vbuf_of(vb), w_of(vb));
      kt = nxt;
      vb ^= 1;
    }
    if (CAUSAL && kt == last) {
      wait_vmem();
      __syncthreads();
      expand_k();
      __syncthreads();
      FA4_TILE_STEP(true, false, kt, nullptr, nullptr, vbuf_of(vb), w_of(vb));
    }
  }
  if constexpr (V4 && !P4) {
    // 4-bit V: the quantized tiles' P^ carried a factor 448 (their sums did not); bf16 tiles carry none
#pragma unroll
    for (int i = 0; i < NDB; i++) acc[i] *= 1.0f / 448.0f;
  }
  if constexpr (SEL && D == 128) {
    // ---- selected tiles from the bf16 originals. Their K and V rows come by direct global->LDS loads into
    // padded 16-bit rows (a lane whose 16 bytes fall on a row's padding loads the row's first chunk again):
    // the next selected tile's K while this tile's softmax and PV run, its V while the next tile's QK^T
    // runs. The bf16 Q operand is read once (and waited for before the first tile load is issued).
    v8bf qb[8];
#pragma unroll
    for (int s = 0; s < 8; s++) qb[s] = *reinterpret_cast<const v8bf *>(a.qb + (bhq * a.Lq + qrow) * D + 16 * s + 8 * hh);
#pragma unroll
    for (int s = 0; s < 8; s++) {
      v4i t = __builtin_bit_cast(v4i, qb[s]);
      asm volatile("" : "+v"(t));
      qb[s] = __builtin_bit_cast(v8bf, t);
    }
    const uint32_t lds_a =
        __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t *)lds);
    constexpr int NL = L::K16 / 1024;          // 34 wave-loads of 1 KB per tensor: 9 for waves 0, 1, 8 for 2, 3
    auto issue16 = [&](const uint16_t *src, int kt, uint32_t dst) __attribute__((always_inline)) {
      const uint8_t *g = reinterpret_cast<const uint8_t *>(src + (bhk * a.Lk + (int64_t)kt * 128) * 128);
      for (int e = wave; e < NL; e += 4) {
        const uint32_t o = 1024u * e + 16u * lane;
        const uint32_t row = o / H16_RS, c = (o - row * H16_RS) >> 4;
        dma16_nw(g, row * 256 + 16 * (c < 16 ? c : 0), dst + 1024 * e);
      }
    };
    auto wait_all_but_one_tensor = [&]() __attribute__((always_inline)) {   // this wave's older loads
      if (wave < 2)
        asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    };
    auto next_sel = [&](int t) -> int {
      while (t < kt_end && !is_sel(t)) t++;
      return t;
    };
    const uint32_t k_lds = lds_a, v_lds = lds_a + L::K16;
    __syncthreads();                           // the quantized tiles' buffers are free
    int u = next_sel(0);
    if (u < kt_end) {
      issue16(a.kb, u, k_lds);
      issue16(a.vb, u, v_lds);
    }
    while (u < kt_end) {
      const int un = next_sel(u + 1);
      wait_all_but_one_tensor();               // K(u) landed (V(u) may be in flight)
      __syncthreads();
      v16f S[4];
      bf16_qk(qb, k16, lo, S);
      __syncthreads();                         // every wave is done with K(u)
      if (un < kt_end) issue16(a.kb, un, k_lds);
      if (CAUSAL && u == last) mask_tile_rt(S, u, hh, qrow + off);
      v8bf pb[4][2];
      bf16_probs(S, cs_b, m, lsum, acc, pb);
      if (un < kt_end)
        wait_all_but_one_tensor();             // V(u) landed (K(un) may be in flight)
      else
        wait_vmem();
      __syncthreads();
      bf16_pv(pb, v16, lo, acc);
      __syncthreads();                         // every wave is done with V(u)
      if (un < kt_end) issue16(a.vb, un, v_lds);
      u = un;
    }
  }
#undef FA4_TILE_STEP
  // ---------------- epilogue: O = O_acc / l, LSE = m ln2 + ln l
  const float l = lsum + shfl_xor_f(lsum, 32);
  const float fin = 1.0f / l;
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
template <int D, int QF, bool CAUSAL, bool SEL, bool V4 = false, bool P4 = false>
static hipError_t allow_lds() {
  return hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_fwd_kernel<D, QF, CAUSAL, SEL, V4, P4>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, AttnLds<D, QF, SEL>::BYTES);
}

// MXFP4 Q/K with 4-bit V (d = 128)
template <bool CAUSAL, bool SEL>
static hipError_t launch_attn_v4_t(const AttnArgs &x, hipStream_t s) {
  dim3 grid((unsigned)((int64_t)(x.Lq / 128) * x.Hq * x.B));
  hipError_t e = allow_lds<128, FA4_MXFP4, CAUSAL, SEL, true>();
  if (e != hipSuccess) return e;
  constexpr size_t lds_bytes = AttnLds<128, FA4_MXFP4, SEL>::BYTES;
  hipLaunchKernelGGL((attn_fwd_kernel<128, FA4_MXFP4, CAUSAL, SEL, true>), grid, dim3(ATT_THREADS), lds_bytes, s, x);
  return hipGetLastError();
}
static hipError_t launch_attn_v4(const AttnArgs &x, bool causal, bool sel, hipStream_t s) {
  if (causal) return sel ? launch_attn_v4_t<true, true>(x, s) : launch_attn_v4_t<true, false>(x, s);
  return sel ? launch_attn_v4_t<false, true>(x, s) : launch_attn_v4_t<false, false>(x, s);
}
// 4-bit V with MXFP4 probabilities: FP4 V^T x FP4 P^T
template <bool CAUSAL, bool SEL>
static hipError_t launch_attn_v4p4_t(const AttnArgs &x, hipStream_t s) {
  dim3 grid((unsigned)((int64_t)(x.Lq / 128) * x.Hq * x.B));
  hipError_t e = allow_lds<128, FA4_MXFP4, CAUSAL, SEL, true, true>();
  if (e != hipSuccess) return e;
  constexpr size_t lds_bytes = AttnLds<128, FA4_MXFP4, SEL>::BYTES;
  hipLaunchKernelGGL((attn_fwd_kernel<128, FA4_MXFP4, CAUSAL, SEL, true, true>), grid, dim3(ATT_THREADS), lds_bytes,
                     s, x);
  return hipGetLastError();
}
static hipError_t launch_attn_v4p4(const AttnArgs &x, bool causal, bool sel, hipStream_t s) {
  if (causal) return sel ? launch_attn_v4p4_t<true, true>(x, s) : launch_attn_v4p4_t<true, false>(x, s);
  return sel ? launch_attn_v4p4_t<false, true>(x, s) : launch_attn_v4p4_t<false, false>(x, s);
}

// MXFP4 Q/K, FP8 V, MXFP4 probabilities (d = 128)
template <bool CAUSAL, bool SEL>
static hipError_t launch_attn_p4_t(const AttnArgs &x, hipStream_t s) {
  dim3 grid((unsigned)((int64_t)(x.Lq / 128) * x.Hq * x.B));
  hipError_t e = allow_lds<128, FA4_MXFP4, CAUSAL, SEL, false, true>();
  if (e != hipSuccess) return e;
  constexpr size_t lds_bytes = AttnLds<128, FA4_MXFP4, SEL>::BYTES;
  hipLaunchKernelGGL((attn_fwd_kernel<128, FA4_MXFP4, CAUSAL, SEL, false, true>), grid, dim3(ATT_THREADS), lds_bytes,
                     s, x);
  return hipGetLastError();
}
static hipError_t launch_attn_p4(const AttnArgs &x, bool causal, bool sel, hipStream_t s) {
  if (causal) return sel ? launch_attn_p4_t<true, true>(x, s) : launch_attn_p4_t<true, false>(x, s);
  return sel ? launch_attn_p4_t<false, true>(x, s) : launch_attn_p4_t<false, false>(x, s);
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
  if (p->v_fmt == FA4_MXFP4_KEYS)
    return p->p_fmt == FA4_P_MXFP4 ? launch_attn_v4p4(x, causal, sel, s) : launch_attn_v4(x, causal, sel, s);
  if (p->p_fmt == FA4_P_MXFP4) return launch_attn_p4(x, causal, sel, s);
  if (p->fmt == FA4_MXFP4) {
    if (p->d == 64) return launch_attn_t<64, FA4_MXFP4>(x, causal, false, s);
    return launch_attn_t<128, FA4_MXFP4>(x, causal, sel, s);
  }
  // expanded-K formats (NVFP4 -> fp16, MXFP8 -> bf16)
  if (p->fmt == FA4_MXFP8) return launch_attn_t<128, FA4_MXFP8>(x, causal, sel, s);
  return launch_attn_t<128, FA4_NVFP4>(x, causal, sel, s);
}

}  // namespace fa4

// 4-bit FlashAttention forward for gfx950: prefill, split-KV (decode) and merge.
//
// HiFA4 (arXiv 2607.04302), Abstract: QK^T and PV are both 4-bit
// block-scaled GEMMs, the online-softmax state (m, l) is FP16, and with
// P-Reordering the normalizer is summed from the same quantized P_hat that
// feeds the PV GEMM -- which lets it be produced by that GEMM.
//
// Design on CDNA4 (one wavefront = 32 query columns, tiles of KT keys):
//  * Scores are computed transposed, S^T = K_hat Q_hat^T, with the scaled
//    FP4 MFMA 32x32x64: A = 32 keys (16 bytes of one K_hat row per lane),
//    B = the wave's 32 query rows (loop-invariant registers).  The
//    accumulator gives each lane one query column and 16 keys.
//  * Each lane holds 16 keys of every 32-key block for its query; max, exp
//    and the E2M1 conversion run in place on those registers.  The two lanes
//    of a query exchange only each block's partial max and the packed codes
//    (v_permlane32_swap), after which every lane holds one full 32-key block:
//    the B operand of O^T = V_hat^T P_hat^T (A = 32 channels x 64 keys of
//    V_hat, whose tokens are stored in the same in-block order).  The output
//    accumulator is "lane = query" too: alpha, m and l never leave their lane.
//  * P-Reordering: one more (16x16x128) MFMA of the same P_hat registers
//    against E2M1 ones yields rowsum(P_hat) -- the normalizer comes out of the
//    matrix core, as if from [V_hat | 1], instead of a VALU reduction.
//  * Prefill: a workgroup is 4 wavefronts that read the same KV head (the
//    heads of one GQA group, or consecutive row blocks of one head); each
//    K_hat/V_hat tile is loaded once per workgroup with 1 KB-contiguous
//    direct global-to-LDS copies into double-buffered stages in MFMA operand order
//    (a lane reads its operand as one conflict-free 16-byte LDS load).  The
//    grid's fastest dimension is the KV head, so the round-robin dispatch over
//    the 8 XCDs keeps each KV head's tiles in one L2.
//  * Split-KV (decode): one wavefront per (b, KV head, chunk) streams its
//    chunk from HBM with a one-tile register prefetch; an ordered merge
//    kernel combines the FP16 (m, l) partial states.
#include <atomic>

#include "hifa4_device.hpp"
#include "hifa4_internal.hpp"

namespace hifa4 {

namespace {

constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

// Scale word for the S^T MFMA's k-step s: byte 2*(s%2) of word s/2 holds the
// scale of the 32-channel block (2*s + lane/32).  Built from a row's scale
// bytes by shifting out the other half's byte.
template <int D>
__device__ __forceinline__ void row_scales(const uint8_t* row, int hf, uint32_t (&w)[(D / 64 + 1) / 2]) {
  if constexpr (D == 64) {
    w[0] = (uint32_t)(*reinterpret_cast<const uint16_t*>(row)) >> (8 * hf);
  } else if constexpr (D == 128) {
    w[0] = *reinterpret_cast<const uint32_t*>(row) >> (8 * hf);
  } else {
    const uint2 x = *reinterpret_cast<const uint2*>(row);
    w[0] = x.x >> (8 * hf);
    w[1] = x.y >> (8 * hf);
  }
}

// S^T block of a tile: 32 keys x the wave's 32 query columns.
template <int D>
__device__ __forceinline__ v16f score_block(const uint4 (&ka)[D / 64], const uint32_t (&ksw)[(D / 64 + 1) / 2],
                                            const uint4 (&qb)[D / 64], const uint32_t (&qsc)[(D / 64 + 1) / 2]) {
  v16f acc = zero16();
#pragma unroll
  for (int s = 0; s < D / 64; s++) {
    if (s % 2 == 0)
      acc = mfma_fp4<0, 0>(ka[s], (int)ksw[s / 2], qb[s], (int)qsc[s / 2], acc);
    else
      acc = mfma_fp4<2, 2>(ka[s], (int)ksw[s / 2], qb[s], (int)qsc[s / 2], acc);
  }
  return acc;
}

// PV MFMA of 64-key unit u: the V_hat scale of unit u is byte u of the scale word.
__device__ __forceinline__ v16f pv_mfma(int u, const uint4& a, int sa, const uint4& b, int sb, v16f acc) {
  switch (u) {
    case 0: return mfma_fp4<0, 0>(a, sa, b, sb, acc);
    case 1: return mfma_fp4<1, 0>(a, sa, b, sb, acc);
    case 2: return mfma_fp4<2, 0>(a, sa, b, sb, acc);
    default: return mfma_fp4<3, 0>(a, sa, b, sb, acc);
  }
}

// Four E2M1 code bytes (8 values, value i in nibble i) of S^T registers
// r0..r0+7 of one block, RNE(x / sc).
__device__ __forceinline__ uint32_t cvt8(const v16f& x, int r0, float sc) {
  // all four bytes are written: the initial word is a don't-care (a source
  // register, which saves a move)
  uint32_t w = cvt_fp4x2<0>(__float_as_uint(x[r0]), x[r0], x[r0 + 1], sc);
  w = cvt_fp4x2<1>(w, x[r0 + 2], x[r0 + 3], sc);
  w = cvt_fp4x2<2>(w, x[r0 + 4], x[r0 + 5], sc);
  return cvt_fp4x2<3>(w, x[r0 + 6], x[r0 + 7], sc);
}

// The online-softmax step of one tile of KT keys given its S^T blocks:
// running max, P, P_hat, normalizer, O rescale and O^T += V_hat^T P_hat^T
// (softmax_quant, rescale_o and pv_accumulate below, composed by softmax_pv).
// vops.a(u, ct) / vops.sc(ct) supply the V_hat operands (byte u of the scale
// word is unit u's block).  lim: last valid key of this lane's query column.
//
// Lane (query q, half hf) holds, of every 32-key block, the 16 keys with bit 2
// of the key index equal to hf (S^T accumulator register r: key 8(r/4) + 4hf
// + r%4).  All per-element work runs on these registers in place; the lanes of
// a pair (q, 0) / (q, 1) exchange only each block's partial max (one
// permlane32 swap per block) and the packed codes (one swap per two dwords),
// after which lane (q, hf) holds the full 32-code block 2u + hf of unit u --
// the B operand of the PV product -- with its keys in the operand order
// operand_key (the V_hat tiled layout stores tokens in the same order).

// One tile's quantized probabilities, between the softmax and the PV product.
template <int KT>
struct TileP {
  uint4 ph[KT / 64];  // P_hat codes: B operand of unit u (lane: block 2u + hf)
  int psc[KT / 64];   // its E8M0 scale byte
  float alpha;        // 2^(m_old - m_new) of this tile
  float rsp;          // reorder = 0: this row's sum of P over the tile
};

// The softmax half of a tile: running max (m updated), alpha, P = 2^(S c - m),
// the E2M1 codes of P_hat and, for reorder = 0, the row sum of P.
template <int D, int KT, bool REORDER, bool DUMP, bool EXPFREE = false>
__device__ __forceinline__ void softmax_quant(v16f (&s)[KT / 32], int kb0, bool need_mask, int lim,
                                              float c, int noclip, float& m, TileP<KT>& tp,
                                              uint8_t* phat_codes_row, uint8_t* phat_scales_row) {
  constexpr int NB = KT / 32, NU = KT / 64;
  const int hf = (threadIdx.x >> 5) & 1;

  if (need_mask) {
    // key offset o within the tile is valid when o <= room
    const int room = lim - kb0 - 4 * hf;
#pragma unroll
    for (int bb = 0; bb < NB; bb++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int o = 32 * bb + 8 * (r / 4) + (r % 4);
        s[bb][r] = (room < o) ? kNegInf : s[bb][r];
      }
  }

  // block maxima: this lane's 16 keys (a balanced tree of three-input maxima,
  // depth 3 instead of a chain of 8), then the partner lane's 16
  float pm[NB];
#pragma unroll
  for (int bb = 0; bb < NB; bb++) {
    const float a0 = fmaxf(fmaxf(s[bb][0], s[bb][1]), s[bb][2]);
    const float a1 = fmaxf(fmaxf(s[bb][3], s[bb][4]), s[bb][5]);
    const float a2 = fmaxf(fmaxf(s[bb][6], s[bb][7]), s[bb][8]);
    const float a3 = fmaxf(fmaxf(s[bb][9], s[bb][10]), s[bb][11]);
    const float a4 = fmaxf(fmaxf(s[bb][12], s[bb][13]), s[bb][14]);
    pm[bb] = fmaxf(fmaxf(fmaxf(a0, a1), a2), fmaxf(fmaxf(a3, a4), s[bb][15]));
  }
  // full block maxima: a swap of a value with itself hands every lane the
  // partial max of both halves of its query's block
  float bm[NB];
  float rmax = kNegInf;
#pragma unroll
  for (int bb = 0; bb < NB; bb++) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(pm[bb]), __float_as_uint(pm[bb]), false, false);
    bm[bb] = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    rmax = fmaxf(rmax, bm[bb]);
  }

  // running max (log2 domain, FP16 state)
  const float mt = c * rmax;
  const float m_new = round_f16(fmaxf(m, mt));
  const float m_use = (m_new == kNegInf) ? 0.0f : m_new;  // column with no valid key yet
  const float alpha = exp2_hw(m - m_use);

  // per-block exponents from t_max = fma(block max S, c, -m) (the largest t of
  // the block: the map S -> fma(S, c, -m) is monotone), e = fl - 2 with
  //   OCP rule:     fl = floor(t_max),
  //   no clipping:  fl = ceil(fp32(t_max - log2 1.5)) = -floor(fp32(log2 1.5 - t_max)),
  //                 the smallest fl with 2^(t_max - fl + 2) <= 6;
  // the clamp at e >= -127 is applied as fl >= -125 (t_max <= half an FP16 ulp
  // of m, so e never reaches 127).  The rule is a kernel argument (the branch is
  // uniform).  sc[bb] = 2^e scales this lane's elements of block bb; psc[u] is
  // the scale byte of block 2u + hf, the block this lane holds after the code
  // exchange
  float sc[NB];
  int fl[NB];
  int* psc = tp.psc;
  if (noclip) {
    constexpr float kLog2ThreeHalves = 0.584962500721156181453738943947816508759814407692481060455f;
#pragma unroll
    for (int bb = 0; bb < NB; bb++)
      fl[bb] = -(int)floorf(fminf(kLog2ThreeHalves - __builtin_fmaf(bm[bb], c, -m_use), 125.0f));
  } else {
#pragma unroll
    for (int bb = 0; bb < NB; bb++) fl[bb] = (int)floorf(fmaxf(__builtin_fmaf(bm[bb], c, -m_use), -125.0f));
  }
#pragma unroll
  for (int bb = 0; bb < NB; bb++) sc[bb] = __builtin_amdgcn_ldexpf(0.25f, fl[bb]);
  const int hmask = -hf;  // all ones in the upper half-wave
#pragma unroll
  for (int u = 0; u < NU; u++) psc[u] = ((fl[2 * u + 1] & hmask) | (fl[2 * u] & ~hmask)) + 125;

  if constexpr (EXPFREE) {
    // exp-free P_hat: E2M1 of 2^(t - e) straight from the log-domain value
    // u = S c - (m + e) (the block exponent folded into the subtrahend), with
    // the conversion below at scale 1; masked keys (-inf) clamp to 2^-126 -> 0
    static_assert(REORDER, "the exp-free P_hat has no P for a separate row sum");
#pragma unroll
    for (int bb = 0; bb < NB; bb++) {
      const float me = m_use + (float)(fl[bb] - 2);
#pragma unroll
      for (int r = 0; r < 16; r++) s[bb][r] = expcast_e2m1(fmaxf(__builtin_fmaf(s[bb][r], c, -me), -126.0f));
      sc[bb] = 1.0f;
    }
  } else {
    // P = 2^(S c - m)
#pragma unroll
    for (int bb = 0; bb < NB; bb++)
#pragma unroll
      for (int r = 0; r < 16; r++) s[bb][r] = exp2_hw(__builtin_fmaf(s[bb][r], c, -m_use));
  }

  // P_hat codes: this lane's 16 keys of each block as two dwords, then one
  // swap per dword pair hands each lane the partner's half of its block
  uint4* ph = tp.ph;
#pragma unroll
  for (int u = 0; u < NU; u++) {
    const uint32_t a0 = cvt8(s[2 * u], 0, sc[2 * u]), a1 = cvt8(s[2 * u], 8, sc[2 * u]);
    const uint32_t b0 = cvt8(s[2 * u + 1], 0, sc[2 * u + 1]), b1 = cvt8(s[2 * u + 1], 8, sc[2 * u + 1]);
    auto w0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
    auto w1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
    ph[u] = make_uint4(w0[0], w1[0], w0[1], w1[1]);
    if constexpr (DUMP) {
      if (phat_codes_row) {
        // back to ascending key order (operand_key inverted on 16-bit groups)
        const uint4 k = make_uint4((ph[u].x & 0xFFFFu) | (ph[u].z << 16), (ph[u].x >> 16) | (ph[u].z & 0xFFFF0000u),
                                   (ph[u].y & 0xFFFFu) | (ph[u].w << 16), (ph[u].y >> 16) | (ph[u].w & 0xFFFF0000u));
        *reinterpret_cast<uint4*>(phat_codes_row + kb0 / 2 + 32 * u + 16 * hf) = k;
        phat_scales_row[kb0 / 32 + 2 * u + hf] = (uint8_t)psc[u];
      }
    }
  }

  tp.alpha = alpha;
  if constexpr (!REORDER) {
    float rs = 0.0f;
#pragma unroll
    for (int bb = 0; bb < NB; bb++)
#pragma unroll
      for (int r = 0; r < 16; r++) rs = rs + s[bb][r];
    tp.rsp = rs + other_half(rs);
  }
  m = m_new;
}

// O <- alpha O, skipped when the max did not move for any column.
template <int D>
__device__ __forceinline__ void rescale_o(v16f (&accO)[D / 32], float alpha) {
  if (!__all(alpha == 1.0f)) {
#pragma unroll
    for (int ct = 0; ct < D / 32; ct++)
#pragma unroll
      for (int r = 0; r < 16; r++) accO[ct][r] = accO[ct][r] * alpha;
  }
}

// The PV half of a tile (O already rescaled by the tile's alpha): the
// normalizer l = fp16(fp32(alpha l) + rowsum) and O^T += V_hat^T P_hat^T.
template <int D, int KT, bool REORDER, class VOps>
__device__ __forceinline__ void pv_accumulate(const TileP<KT>& tp, const VOps& vops,
                                              v16f (&accO)[D / 32], float& l) {
  constexpr int CT = D / 32, NU = KT / 64;
  const uint4* ph = tp.ph;
  const int* psc = tp.psc;
  const float alpha = tp.alpha;
  // normalizer: l = fp16(fp32(alpha l) + rowsum)
  float rs;
  if constexpr (REORDER) {
    // P-Reordering: the row sum of P_hat comes out of the matrix core, from
    // P_hat against an operand of E2M1 ones (scale 2^0), on the 16x16x128 MFMA
    // (half the matrix work of a 32x32x64 one).  P_hat's registers, laid out as
    // the B operand of the 32x32x64 PV product, read as that MFMA's B operand
    // (lane l: column l % 16, K-slice l / 16) put query c in slices 0 and 2 of
    // column c and query c + 16 in slices 1 and 3.  Row group g of A (rows
    // 4g..4g+3, whose results land in lanes 16g..16g+15) holds ones in slices
    // {0, 2} for even g and {1, 3} for odd g, so lane l receives the row sum of
    // its own query l % 32.
    const int ln = threadIdx.x & 63;
    const uint32_t w = (((ln >> 2) ^ (ln >> 4)) & 1) ? 0u : 0x22222222u;
    const uint4 ones = {w, w, w, w};
    v4f sl = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < NU; u++) sl = mfma16_fp4_unit_a(ones, ph[u], psc[u], sl);
    rs = sl[0];
  } else {
    rs = tp.rsp;
  }
  const float al = alpha * l;
  l = round_f16(al + rs);

  // O^T += V_hat^T P_hat^T
#pragma unroll
  for (int ct = 0; ct < CT; ct++) {
    const int vsc = (int)vops.sc(ct);
#pragma unroll
    for (int u = 0; u < NU; u++) accO[ct] = pv_mfma(u, vops.a(u, ct), vsc, ph[u], psc[u], accO[ct]);
  }
}

// A whole tile: softmax, rescale, normalizer and PV, in that order.
template <int D, int KT, bool REORDER, bool DUMP, class VOps, bool EXPFREE = false>
__device__ __forceinline__ void softmax_pv(v16f (&s)[KT / 32], int kb0, bool need_mask, int lim,
                                           float c, int noclip, const VOps& vops, v16f (&accO)[D / 32],
                                           float& m, float& l, uint8_t* phat_codes_row,
                                           uint8_t* phat_scales_row) {
  TileP<KT> tp;
  softmax_quant<D, KT, REORDER, DUMP, EXPFREE>(s, kb0, need_mask, lim, c, noclip, m, tp, phat_codes_row,
                                      phat_scales_row);
  rescale_o<D>(accO, tp.alpha);
  pv_accumulate<D, KT, REORDER>(tp, vops, accO, l);
}

// o / l from the hardware reciprocal and one residual correction (Markstein):
// q = o r, q' = q + (o - q l) r.  With r within 1 ulp of 1/l this is the
// correctly rounded quotient except in rare boundary cases (then 1 ulp off),
// far below the binary16 rounding that follows.
__device__ __forceinline__ float div_by(float o, float l, float r) {
  const float q = o * r;
  return __builtin_fmaf(__builtin_fmaf(-q, l, o), r, q);
}

// Epilogue: out = fp16(O / l) for the lane's query row (channels 32ct + 8(r/4) + 4hf + r%4).
template <int D>
__device__ __forceinline__ void store_out(uint16_t* orow, const v16f (&accO)[D / 32], float l) {
  const int hf = (threadIdx.x >> 5) & 1;
  const float r = __builtin_amdgcn_rcpf(l);
#pragma unroll
  for (int ct = 0; ct < D / 32; ct++)
#pragma unroll
    for (int r4 = 0; r4 < 4; r4++) {
      uint32_t lo = (uint32_t)float_to_half_bits(div_by(accO[ct][4 * r4 + 0], l, r)) |
                    ((uint32_t)float_to_half_bits(div_by(accO[ct][4 * r4 + 1], l, r)) << 16);
      uint32_t hi = (uint32_t)float_to_half_bits(div_by(accO[ct][4 * r4 + 2], l, r)) |
                    ((uint32_t)float_to_half_bits(div_by(accO[ct][4 * r4 + 3], l, r)) << 16);
      *reinterpret_cast<uint2*>(orow + 32 * ct + 8 * r4 + 4 * hf) = make_uint2(lo, hi);
    }
}

// Smooth-QK multiply and MX quantization of one query row inside the kernel,
// exactly as the quantize pass does it (x = fp32(q * s[j]), one block per 32
// channels): the lane of half hf builds the B operand of k-step s from
// channels 64 s + 32 hf .. + 32, one whole block, so no lane exchange is
// needed.  Every load (the row's binary16 values and its Smooth-QK scales for
// all k-steps) is issued before any is used: one wait on memory instead of two
// per k-step.  qx = NULL gives a zero row (padding columns).
template <int D>
__device__ __forceinline__ void quantize_query_lane(const uint16_t* qx, const float* srow, int noclip,
                                                    uint4 (&qb)[D / 64], uint32_t (&qsc)[(D / 64 + 1) / 2]) {
  constexpr int KS = D / 64, SW = (D / 64 + 1) / 2;
  const int hf = (threadIdx.x >> 5) & 1;
  uint4 raw[KS][4];
  float4 sv[KS][8];
  if (qx) {
#pragma unroll
    for (int s = 0; s < KS; s++)
#pragma unroll
      for (int u = 0; u < 4; u++) raw[s][u] = *reinterpret_cast<const uint4*>(qx + (2 * s + hf) * 32 + 8 * u);
  } else {
#pragma unroll
    for (int s = 0; s < KS; s++)
#pragma unroll
      for (int u = 0; u < 4; u++) raw[s][u] = make_uint4(0, 0, 0, 0);
  }
  if (srow) {
#pragma unroll
    for (int s = 0; s < KS; s++)
#pragma unroll
      for (int u = 0; u < 8; u++) sv[s][u] = *reinterpret_cast<const float4*>(srow + (2 * s + hf) * 32 + 4 * u);
  }
#pragma unroll
  for (int w = 0; w < SW; w++) qsc[w] = 0u;
#pragma unroll
  for (int s = 0; s < KS; s++) {
    float v[32];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const uint32_t w[4] = {raw[s][u].x, raw[s][u].y, raw[s][u].z, raw[s][u].w};
#pragma unroll
      for (int z = 0; z < 4; z++) {
        v[8 * u + 2 * z] = half_to_float((uint16_t)(w[z] & 0xFFFFu));
        v[8 * u + 2 * z + 1] = half_to_float((uint16_t)(w[z] >> 16));
      }
    }
    if (srow) {
#pragma unroll
      for (int u = 0; u < 8; u++) {
        v[4 * u] = v[4 * u] * sv[s][u].x;
        v[4 * u + 1] = v[4 * u + 1] * sv[s][u].y;
        v[4 * u + 2] = v[4 * u + 2] * sv[s][u].z;
        v[4 * u + 3] = v[4 * u + 3] * sv[s][u].w;
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int z = 0; z < 32; z++) amax = fmaxf(amax, fabsf(v[z]));
    const int e = mx_exponent(amax, noclip);
    const float sc = pow2f(e);
    qb[s].x = pack8_fp4(&v[0], sc);
    qb[s].y = pack8_fp4(&v[8], sc);
    qb[s].z = pack8_fp4(&v[16], sc);
    qb[s].w = pack8_fp4(&v[24], sc);
    qsc[s / 2] |= (uint32_t)(qx ? e + 127 : 0) << (16 * (s % 2));
  }
}

struct KParams {
  const uint8_t* q_codes;
  const uint8_t* q_scales;
  const uint16_t* q_f16;
  const float* s;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  uint16_t* out;
  uint8_t* phat_codes;
  uint8_t* phat_scales;
  float* ws_o;
  float* ws_ml;
  int64_t B, Hq, Hkv, N_q, N_kv, Npad_q, Npad_kv;
  int G, num_splits, n_tiles, tiles_per_split;
  int heads_per_wg;  // query heads per prefill workgroup (the rest of its 4 waves are row blocks)
  int slot_rows;     // prefill: row groups per residency slot of a one-round grid (0: longest first)
  int noclip;        // block-exponent rule of P_hat and of an in-kernel quantized Q
  float c;
};

// ---------------------------------------------------------------------------
// Prefill.  Workgroup = 4 wavefronts on KV head (b, g): nh query heads of the
// group x (4 / nh) row blocks of 32 rows.  Grid (B * Hkv * G/nh, row groups);
// row groups run last-first so the longest causal work starts earliest and
// the dispatcher's in-order refill balances the rest.  When the whole grid is
// resident at once there is no refill: the dispatcher hands each CU one
// workgroup of every consecutive slot of (CU count) workgroups, so the row
// groups are laid out in a snake over the slots (longest first in even slots,
// shortest first in odd ones) and the workgroups that share a CU carry
// complementary row ranges.
//
// LDS stage of one tile (KT keys), all in MFMA operand order:
//   [K_hat codes: KT/32 blocks x D/64 k-steps x 64 lanes x 16 B]
//   [V_hat codes: KT/64 units x D/32 channel tiles x 64 lanes x 16 B]
//   [K_hat scales: KT keys x D/32 B][V_hat scales: KT/64 tiles x D x 2 B]
// ---------------------------------------------------------------------------
template <int D, int KT>
struct Stage {
  static constexpr int KS = D / 64, CT = D / 32, NB = KT / 32, NU = KT / 64;
  static constexpr int KC_OFF = 0;
  static constexpr int VC_OFF = KT * D / 2;
  static constexpr int KSC_OFF = KT * D;
  static constexpr int KSC_BYTES = KT * D / 32;
  static constexpr int VSC_OFF = KSC_OFF + KSC_BYTES;
  static constexpr int VSC_BYTES = KT * D / 32;
  static constexpr int BYTES = VSC_OFF + VSC_BYTES;
  static constexpr int N_KC = NB * KS;   // 1 KB pieces of K_hat codes
  static constexpr int N_VC = NU * CT;   // 1 KB pieces of V_hat codes
  // 16-byte units of scale bytes (K_hat then V_hat, one contiguous LDS range)
  static constexpr int SCU = (KSC_BYTES + VSC_BYTES) / 16;
  // per wave: CPW code pieces and SCU/4 units of scale bytes
  static constexpr int CPW = (N_KC + N_VC) / 4;
  static_assert((N_KC + N_VC) % 4 == 0 && SCU % 4 == 0 && SCU / 4 <= 64, "even split over 4 waves");
};

// Tile copies are direct buffer -> LDS transfers (buffer_load_dwordx4 ... lds):
// one instruction moves 16 bytes per lane into LDS lane after lane, so 64
// lanes fill one 1 KB MFMA operand piece of the stage.  Each of the 4
// wavefronts copies CPW code pieces and a quarter of the scale bytes (its
// first SCU/4 lanes).  A piece is a buffer resource on its source tensor (the
// KV head's codes or scales, wave-uniform, in scalar registers) plus a per-lane
// byte offset for the tile at key 0; the tile at kb0 adds kb0 * D/2 bytes (code
// pieces: K_hat rows and 64-token V_hat tiles alike) or kb0 * D/32 (scale
// pieces) through the instruction's scalar offset, so a copy takes no vector
// instruction for its address.
template <int D, int KT>
struct DmaPlan {
  const uint8_t* kc;  // K_hat codes of the KV head
  const uint8_t* vc;  // V_hat codes
  const uint8_t* sc;  // this wave's scale tensor (K_hat's or V_hat's)
  uint32_t code_bytes, scale_bytes;
  int nk;  // pieces j < nk are K_hat codes, the rest V_hat (wave-uniform)
  uint32_t off[Stage<D, KT>::CPW + 1];
  int dst[Stage<D, KT>::CPW + 1];  // LDS offset in the stage (wave-uniform)
};

struct KvBases {
  const uint8_t* kc;  // K_hat codes of (b, g): [Npad][D/2]
  const uint8_t* ks;  // K_hat scales: [Npad][D/32]
  const uint8_t* vc;  // V_hat codes: [Npad/64][D][32]
  const uint8_t* vs;  // V_hat scales: [Npad/64][D][2]
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// A raw buffer resource on a wave-uniform pointer (its two halves read from the
// first lane, so the resource lives in scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const uint8_t* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* q = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, (int)bytes, 0x00020000);
}

// One 16-byte-per-lane copy from base + voff + soff into LDS at `lds` (lane after lane).
__device__ __forceinline__ void copy16_to_lds(const uint8_t* base, uint32_t bytes, uint8_t* lds, uint32_t voff,
                                              int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(uniform_rsrc(base, bytes), (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}

template <int D, int KT>
__device__ __forceinline__ void make_dma_plan(const KvBases& kv, uint32_t code_bytes, uint32_t scale_bytes,
                                              DmaPlan<D, KT>& pl) {
  using S = Stage<D, KT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  pl.kc = kv.kc;
  pl.vc = kv.vc;
  pl.code_bytes = code_bytes;
  pl.scale_bytes = scale_bytes;
  pl.nk = (S::N_KC - wave + 3) / 4;  // pieces i = wave + 4 j below N_KC
#pragma unroll
  for (int j = 0; j < S::CPW; j++) {
    const int i = wave + 4 * j;
    if (i < S::N_KC) {
      const int b = i / S::KS, sk = i % S::KS;
      pl.off[j] = (uint32_t)(32 * b * (D / 2) + 2 * sk * 16 + l32 * (D / 2) + hf * 16);
      pl.dst[j] = S::KC_OFF + i * 1024;
    } else {
      const int jj = i - S::N_KC, u = jj / S::CT, ct = jj % S::CT;
      pl.off[j] = (uint32_t)((u * D + 32 * ct) * 32 + l32 * 32 + 16 * hf);
      pl.dst[j] = S::VC_OFF + jj * 1024;
    }
  }
  // scale units: waves 0-1 copy K_hat's, waves 2-3 V_hat's (KSC_BYTES = VSC_BYTES)
  constexpr int KU = S::KSC_BYTES / 16, PU = S::SCU / 4;
  static_assert(KU == 2 * PU, "each wave's scale units come from one tensor");
  pl.sc = wave < 2 ? kv.ks : kv.vs;
  pl.off[S::CPW] = (uint32_t)((wave < 2 ? wave : wave - 2) * PU * 16 + lane * 16);
  pl.dst[S::CPW] = S::KSC_OFF + wave * PU * 16;
}

// Issue this wave's copies of the tile at kb0 into `stage`.  Completion is
// awaited by the workgroup barrier that ends the iteration (its memory fence
// waits for outstanding vector memory operations).
template <int D, int KT>
__device__ __forceinline__ void dma_tile(const DmaPlan<D, KT>& pl, int kb0, uint8_t* stage) {
  using S = Stage<D, KT>;
#pragma unroll
  for (int j = 0; j < S::CPW; j++)
    copy16_to_lds(j < pl.nk ? pl.kc : pl.vc, pl.code_bytes, stage + pl.dst[j], pl.off[j], kb0 * (D / 2));
  if ((threadIdx.x & 63) < S::SCU / 4)
    copy16_to_lds(pl.sc, pl.scale_bytes, stage + pl.dst[S::CPW], pl.off[S::CPW], kb0 * (D / 32));
}

// V_hat operands read from an LDS stage.
template <int D, int KT>
struct LdsV {
  const uint8_t* st;
  __device__ __forceinline__ uint4 a(int u, int ct) const {
    const int lane = threadIdx.x & 63;
    return *reinterpret_cast<const uint4*>(st + Stage<D, KT>::VC_OFF + (u * (D / 32) + ct) * 1024 + lane * 16);
  }
  __device__ __forceinline__ uint32_t sc(int ct) const {
    const int lane = threadIdx.x & 63, hf = lane >> 5, ch = 32 * ct + (lane & 31);
    const uint8_t* p = st + Stage<D, KT>::VSC_OFF + ch * 2;
    const uint32_t x0 = *reinterpret_cast<const uint16_t*>(p);
    if constexpr (KT == 64) {
      return x0 >> (8 * hf);
    } else {
      // byte 0 <- byte hf of unit 0's pair, byte 1 <- byte hf of unit 1's pair
      const uint32_t x1 = *reinterpret_cast<const uint16_t*>(p + D * 2);
      return __builtin_amdgcn_perm(x1, x0, 0x0C0C0400u + 0x0101u * (uint32_t)hf);
    }
  }
};

// The same operands read into registers up front (the reads overlap the softmax).
template <int D, int KT>
struct LdsVRegs {
  uint4 va[KT / 64][D / 32];
  uint32_t vs[D / 32];
  __device__ __forceinline__ explicit LdsVRegs(const uint8_t* st) {
    const LdsV<D, KT> l{st};
#pragma unroll
    for (int ct = 0; ct < D / 32; ct++) {
#pragma unroll
      for (int u = 0; u < KT / 64; u++) va[u][ct] = l.a(u, ct);
      vs[ct] = l.sc(ct);
    }
  }
  __device__ __forceinline__ uint4 a(int u, int ct) const { return va[u][ct]; }
  __device__ __forceinline__ uint32_t sc(int ct) const { return vs[ct]; }
};

template <int D, int KT, bool CAUSAL, bool REORDER, bool DUMP, bool EXPFREE>
__global__ __launch_bounds__(256, 2) void attn_prefill_kernel(KParams p) {
  using S = Stage<D, KT>;
  constexpr int KS = D / 64, CT = D / 32, SW = (D / 64 + 1) / 2, NB = KT / 32;
  // two stages as separate arrays, so that reads of one are not ordered
  // behind the copies in flight into the other
  __shared__ __attribute__((aligned(16))) uint8_t st0[S::BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t st1[S::BYTES];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hf = lane >> 5, l32 = lane & 31;
  const int nh = p.heads_per_wg, nr = 4 / nh;
  const int64_t chunks = p.G / nh;  // head chunks per KV head
  const int64_t bgc = blockIdx.x;
  const int64_t hc = bgc / (p.B * p.Hkv), bg = bgc % (p.B * p.Hkv);
  const int64_t b = bg / p.Hkv, g = bg % p.Hkv;
  const int64_t h = g * p.G + hc * nh + (wave % nh);
  const int64_t Y = gridDim.y, y = blockIdx.y;
  int64_t rank = y;  // 0 = the longest row group
  if (p.slot_rows > 0) {
    const int64_t sl = y / p.slot_rows, j = y - sl * p.slot_rows;
    if (sl & 1) rank = sl * p.slot_rows + min64(p.slot_rows, Y - sl * p.slot_rows) - 1 - j;
  }
  const int64_t rgrp = Y - 1 - rank;
  const int64_t wg_row0 = rgrp * 32 * nr;
  const int64_t row0 = wg_row0 + 32 * (wave / nh);
  const int64_t bh = b * p.Hq + h;
  (void)chunks;

  KvBases kv;
  kv.kc = p.k_codes + bg * p.Npad_kv * (D / 2);
  kv.ks = p.k_scales + bg * p.Npad_kv * (D / 32);
  kv.vc = p.v_codes + bg * p.Npad_kv * (D / 2);
  kv.vs = p.v_scales + bg * p.Npad_kv * (D / 32);

  const int64_t shift = p.N_kv - p.N_q;  // causal diagonal offset (bottom-right aligned)
  const int64_t wg_last_row = min64(wg_row0 + 32 * nr - 1, p.N_q - 1);
  const int64_t wg_last_key = CAUSAL ? min64(wg_last_row + shift, p.N_kv - 1) : p.N_kv - 1;
  const int tiles = (int)(wg_last_key / KT) + 1;
  const bool wave_active = row0 < p.N_q;
  const int64_t last_row = min64(row0 + 31, p.N_q - 1);
  const int wave_last_key = (int)(CAUSAL ? min64(last_row + shift, p.N_kv - 1) : p.N_kv - 1);
  const int wave_lim = CAUSAL ? (int)min64(row0 + shift, p.N_kv - 1) : (int)(p.N_kv - 1);
  const int64_t qrow = row0 + l32;
  const int lim = CAUSAL ? (int)min64(qrow + shift, p.N_kv - 1) : (int)(p.N_kv - 1);

  // Copy pipeline: tile t+1 is copied into the free stage right after the
  // barrier that ended tile t-1 (the last reads of that stage), so the copy
  // runs under tile t's compute; the barrier that ends tile t waits for it.
  // The first tile's copy is issued before the query work so that it overlaps.
  DmaPlan<D, KT> plan;
  make_dma_plan<D, KT>(kv, (uint32_t)(p.Npad_kv * (D / 2)), (uint32_t)(p.Npad_kv * (D / 32)), plan);
  dma_tile<D, KT>(plan, 0, st0);

  // Q_hat rows of this wave: B operand of S^T, resident for the whole loop.
  uint4 qb[KS];
  uint32_t qsc[SW];
  if (wave_active && p.q_f16) {
    // raw binary16 query: Smooth-QK and quantization here (rows past N_q are zero)
    quantize_query_lane<D>(qrow < p.N_q ? p.q_f16 + (bh * p.N_q + qrow) * D : nullptr,
                           p.s ? p.s + g * D : nullptr, p.noclip, qb, qsc);
  } else if (wave_active) {
    const uint8_t* qr = p.q_codes + (bh * p.Npad_q + qrow) * (D / 2);
#pragma unroll
    for (int s = 0; s < KS; s++) qb[s] = *reinterpret_cast<const uint4*>(qr + (2 * s + hf) * 16);
    row_scales<D>(p.q_scales + (bh * p.Npad_q + qrow) * (D / 32), hf, qsc);
  } else {
#pragma unroll
    for (int s = 0; s < KS; s++) qb[s] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int w = 0; w < SW; w++) qsc[w] = 0;
  }

  uint8_t* phc = nullptr;
  uint8_t* phs = nullptr;
  if constexpr (DUMP) {
    if (wave_active && qrow < p.N_q) {
      phc = p.phat_codes + (bh * p.N_q + qrow) * (p.Npad_kv / 2);
      phs = p.phat_scales + (bh * p.N_q + qrow) * (p.Npad_kv / 32);
    }
  }

  __syncthreads();

  v16f accO[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ct++) accO[ct] = zero16();
  float m = kNegInf, l = 0.0f;
  auto step = [&](int t, const uint8_t* st, uint8_t* nxt) {
    const int kb0 = t * KT;
    if (t + 1 < tiles) dma_tile<D, KT>(plan, kb0 + KT, nxt);
    if (wave_active && kb0 <= wave_last_key) {
      v16f sacc[NB];
      const bool need_mask = (kb0 + KT - 1) > wave_lim;
      if constexpr (D * KT <= 128 * 128) {
        // all K_hat operands read before the S MFMAs, all V_hat operands before the softmax
        uint4 ka[NB][KS];
        uint32_t ksw[NB][SW];
#pragma unroll
        for (int bb = 0; bb < NB; bb++) {
#pragma unroll
          for (int s = 0; s < KS; s++)
            ka[bb][s] = *reinterpret_cast<const uint4*>(st + S::KC_OFF + (bb * KS + s) * 1024 + lane * 16);
          row_scales<D>(st + S::KSC_OFF + (32 * bb + l32) * (D / 32), hf, ksw[bb]);
        }
#pragma unroll
        for (int bb = 0; bb < NB; bb++) sacc[bb] = score_block<D>(ka[bb], ksw[bb], qb, qsc);
        LdsVRegs<D, KT> vops(st);
        softmax_pv<D, KT, REORDER, DUMP, LdsVRegs<D, KT>, EXPFREE>(sacc, kb0, need_mask, lim, p.c, p.noclip, vops,
                                                                  accO, m, l, phc, phs);
      } else {
        // d = 256 with 128-key tiles: the operands would not fit in registers
        // next to O (128) and S^T (64), so they are read block by block
#pragma unroll
        for (int bb = 0; bb < NB; bb++) {
          uint4 ka[KS];
          uint32_t ksw[SW];
#pragma unroll
          for (int s = 0; s < KS; s++)
            ka[s] = *reinterpret_cast<const uint4*>(st + S::KC_OFF + (bb * KS + s) * 1024 + lane * 16);
          row_scales<D>(st + S::KSC_OFF + (32 * bb + l32) * (D / 32), hf, ksw);
          sacc[bb] = score_block<D>(ka, ksw, qb, qsc);
        }
        const LdsV<D, KT> vops{st};
        softmax_pv<D, KT, REORDER, DUMP, LdsV<D, KT>, EXPFREE>(sacc, kb0, need_mask, lim, p.c, p.noclip, vops, accO,
                                                              m, l, phc, phs);
      }
    }
    __syncthreads();
  };
  for (int t = 0; t < tiles; t += 2) {
    step(t, st0, st1);
    if (t + 1 < tiles) step(t + 1, st1, st0);
  }

  if (wave_active && qrow < p.N_q) store_out<D>(p.out + (bh * p.N_q + qrow) * D, accO, l);
}

// ---------------------------------------------------------------------------
// Split-KV: one wavefront per (b, g, chunk), each in a workgroup of its own
// (the wavefronts share nothing).  Its 32 query columns are the
// G * N_q (head-in-group, row) pairs of KV head g (G * N_q <= 32; the rest are
// zero padding).  Q is smoothed and quantized in-kernel from binary16 (or
// read pre-quantized).  Each chunk writes its (m, l, O) partial state.
// ---------------------------------------------------------------------------

// The fused decode kernel reads K_hat / V_hat through buffer resources bounded
// to its KV head's tiles: its register ring requests tiles ahead of the one it
// computes, and a request past the bound returns zeros without touching memory
// (clamping it to the last tile instead read that tile again: 7 % more HBM
// bytes, and 5 % more time on the B=64, 8192-token decode).  Codes are loaded
// with the nontemporal hint: each KV cache byte is read once per step, so its
// stream should not displace cached lines (measured: 5% faster on that decode).
struct KvRsrc {
  __amdgpu_buffer_rsrc_t kc, ks, vc, vs;  // K_hat codes / scales, V_hat codes / scales
};

// Resources for tiles [tb, te) of one (b, g); offsets are then relative to tile tb.
template <int D, int KT>
__device__ __forceinline__ KvRsrc make_kv_rsrc(const KvBases& kv, int tb, int te) {
  constexpr int kWord3 = 0x00020000;  // raw (untyped) buffer
  const int n = te - tb;
  KvRsrc r;
  r.kc = __builtin_amdgcn_make_buffer_rsrc((void*)(kv.kc + (int64_t)tb * KT * (D / 2)), (short)0, n * KT * (D / 2), kWord3);
  r.ks = __builtin_amdgcn_make_buffer_rsrc((void*)(kv.ks + (int64_t)tb * KT * (D / 32)), (short)0, n * KT * (D / 32), kWord3);
  r.vc = __builtin_amdgcn_make_buffer_rsrc((void*)(kv.vc + (int64_t)tb * KT * (D / 2)), (short)0, n * KT * (D / 2), kWord3);
  r.vs = __builtin_amdgcn_make_buffer_rsrc((void*)(kv.vs + (int64_t)tb * KT * (D / 32)), (short)0, n * KT * (D / 32), kWord3);
  return r;
}

__device__ __forceinline__ uint4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);  // aux 2: nontemporal
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// K_hat / V_hat operands of one tile held in registers (split-KV path).
template <int D, int KT>
struct RegOps {
  static constexpr int KS = D / 64, CT = D / 32, NB = KT / 32, NU = KT / 64, SW = (KS + 1) / 2;
  uint4 ka[NB][KS];
  uint32_t ksw[NB][SW];
  uint4 va[NU][CT];
  uint32_t vsw[CT];
  __device__ __forceinline__ uint4 a(int u, int ct) const { return va[u][ct]; }
  __device__ __forceinline__ uint32_t sc(int ct) const { return vsw[ct]; }
};

// Tile t (relative to the resources' first tile) into op: the same operands as
// the prefill kernel's LDS stage, read straight from the cache.
template <int D, int KT>
__device__ __forceinline__ void reg_load_kv(const KvRsrc& r, int t, RegOps<D, KT>& op) {
  const int lane = threadIdx.x & 63, hf = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int bb = 0; bb < KT / 32; bb++) {
    const int key = t * KT + 32 * bb + l32;
#pragma unroll
    for (int s = 0; s < D / 64; s++) op.ka[bb][s] = buf_load16_nt(r.kc, key * (D / 2) + (2 * s + hf) * 16);
    // this key's scale bytes, shifted so that byte 2 * (s % 2) of word s / 2 is block 2 s + hf
    if constexpr (D == 64) {
      op.ksw[bb][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r.ks, key * 2, 0, 0) >> (8 * hf);
    } else if constexpr (D == 128) {
      op.ksw[bb][0] = __builtin_amdgcn_raw_buffer_load_b32(r.ks, key * 4, 0, 0) >> (8 * hf);
    } else {
      const auto x = __builtin_amdgcn_raw_buffer_load_b64(r.ks, key * 8, 0, 0);
      op.ksw[bb][0] = x[0] >> (8 * hf);
      op.ksw[bb][1] = x[1] >> (8 * hf);
    }
  }
#pragma unroll
  for (int ct = 0; ct < D / 32; ct++) {
    const int ch = 32 * ct + l32;
    uint32_t w = 0;
#pragma unroll
    for (int u = 0; u < KT / 64; u++) {
      const int tile = t * (KT / 64) + u;
      op.va[u][ct] = buf_load16_nt(r.vc, (tile * D + ch) * 32 + 16 * hf);
      const uint32_t sb = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r.vs, (tile * D + ch) * 2, 0, 0) >> (8 * hf);
      w |= (sb & 0xFFu) << (8 * u);
    }
    op.vsw[ct] = w;
  }
}

// The split kernel reads the same operands through plain global loads with the
// nontemporal hint (bounded resources measured slower there: 23.2 against
// 20.9 us for one 32768-token sequence at 64 chunks).
__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int D, int KT>
__device__ __forceinline__ void reg_load_k(const KvBases& kv, int kb0, RegOps<D, KT>& op) {
  const int lane = threadIdx.x & 63, hf = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int bb = 0; bb < KT / 32; bb++) {
    const int64_t key = kb0 + 32 * bb + l32;
    const uint8_t* kr = kv.kc + key * (D / 2);
#pragma unroll
    for (int s = 0; s < D / 64; s++) op.ka[bb][s] = load_stream16(kr + (2 * s + hf) * 16);
    row_scales<D>(kv.ks + key * (D / 32), hf, op.ksw[bb]);
  }
}

template <int D, int KT>
__device__ __forceinline__ void reg_load_v(const KvBases& kv, int kb0, RegOps<D, KT>& op) {
  const int lane = threadIdx.x & 63, hf = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int ct = 0; ct < D / 32; ct++) {
    const int64_t ch = 32 * ct + l32;
    uint32_t w = 0;
#pragma unroll
    for (int u = 0; u < KT / 64; u++) {
      const int64_t tile = kb0 / 64 + u;
      op.va[u][ct] = load_stream16(kv.vc + (tile * D + ch) * 32 + 16 * hf);
      const uint32_t sb = (uint32_t)(*reinterpret_cast<const uint16_t*>(kv.vs + (tile * D + ch) * 2)) >> (8 * hf);
      w |= (sb & 0xFFu) << (8 * u);
    }
    op.vsw[ct] = w;
  }
}

// The query operand of a split / decode wavefront: its 32 MFMA columns are the
// G * N_q (head-in-group j, row i) pairs of KV head (b, g), column q = j * N_q + i
// (columns >= G * N_q are zero).  With QRAW the binary16 query is smoothed and
// quantized here exactly as the quantization kernel does it.
struct SplitCols {
  bool real;
  int64_t row;  // flat query row (b*Hq + h)*N_q + i of this lane's column
  int64_t i;    // query index within the sequence
};

__device__ __forceinline__ SplitCols split_cols(const KParams& p, int64_t b, int64_t g) {
  const int l32 = threadIdx.x & 31;
  const int cols = p.G * (int)p.N_q;
  SplitCols c;
  c.real = l32 < cols;
  const int j = c.real ? l32 / (int)p.N_q : 0;  // head within the group
  c.i = c.real ? l32 % p.N_q : p.N_q - 1;
  const int64_t h = g * p.G + j;
  c.row = (b * p.Hq + h) * p.N_q + c.i;
  return c;
}

template <int D, bool QRAW>
__device__ __forceinline__ void split_query(const KParams& p, int64_t b, int64_t g, const SplitCols& cs,
                                            uint4 (&qb)[D / 64], uint32_t (&qsc)[(D / 64 + 1) / 2]) {
  constexpr int KS = D / 64, SW = (D / 64 + 1) / 2;
  const int hf = (threadIdx.x >> 5) & 1;
  const bool real = cs.real;
  const int64_t row = cs.row, i = cs.i;
  const int64_t h = (row / p.N_q) % p.Hq;  // row = (b*Hq + h)*N_q + i
#pragma unroll
  for (int w = 0; w < SW; w++) qsc[w] = 0u;
  if constexpr (QRAW) {
    quantize_query_lane<D>(real ? p.q_f16 + row * D : nullptr, p.s ? p.s + g * D : nullptr, p.noclip, qb,
                           qsc);
  } else {
    const int64_t qr_idx = (b * p.Hq + h) * p.Npad_q + i;
    const uint8_t* qr = p.q_codes + qr_idx * (D / 2);
#pragma unroll
    for (int s = 0; s < KS; s++)
      qb[s] = real ? *reinterpret_cast<const uint4*>(qr + (2 * s + hf) * 16) : make_uint4(0, 0, 0, 0);
    if (real) row_scales<D>(p.q_scales + qr_idx * (D / 32), hf, qsc);
  }
}

template <int D, int KT, bool CAUSAL, bool REORDER, bool DUMP, bool QRAW>
__global__ __launch_bounds__(256) void attn_split_kernel(KParams p) {
  constexpr int KS = D / 64, CT = D / 32, SW = (D / 64 + 1) / 2, NB = KT / 32;
  const int lane = threadIdx.x & 63, hf = lane >> 5, l32 = lane & 31;
  const int64_t wid = (int64_t)blockIdx.x;  // one wavefront per workgroup
  const int64_t total = p.B * p.Hkv * p.num_splits;
  if (wid >= total) return;
  const int chunk = (int)(wid % p.num_splits);
  const int64_t bg = wid / p.num_splits;
  const int64_t b = bg / p.Hkv, g = bg % p.Hkv;

  const int cols = p.G * (int)p.N_q;
  const bool real = l32 < cols;
  const int j = real ? l32 / (int)p.N_q : 0;  // head within the group
  const int64_t i = real ? l32 % p.N_q : p.N_q - 1;
  const int64_t h = g * p.G + j;
  const int64_t row = (b * p.Hq + h) * p.N_q + i;  // flat query row

  uint4 qb[KS];
  uint32_t qsc[SW];
  split_query<D, QRAW>(p, b, g, SplitCols{real, row, i}, qb, qsc);

  KvBases kv;
  kv.kc = p.k_codes + bg * p.Npad_kv * (D / 2);
  kv.ks = p.k_scales + bg * p.Npad_kv * (D / 32);
  kv.vc = p.v_codes + bg * p.Npad_kv * (D / 2);
  kv.vs = p.v_scales + bg * p.Npad_kv * (D / 32);

  const int64_t shift = p.N_kv - p.N_q;
  const int lim = CAUSAL ? (int)min64(i + shift, p.N_kv - 1) : (int)(p.N_kv - 1);
  const int wave_lim = CAUSAL ? (int)min64(shift, p.N_kv - 1) : (int)(p.N_kv - 1);

  uint8_t* phc = nullptr;
  uint8_t* phs = nullptr;
  if constexpr (DUMP) {
    if (real) {
      phc = p.phat_codes + row * (p.Npad_kv / 2);
      phs = p.phat_scales + row * (p.Npad_kv / 32);
    }
  }

  v16f accO[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ct++) accO[ct] = zero16();
  float m = kNegInf, l = 0.0f;
  const int t0 = chunk * p.tiles_per_split;
  const int t1 = p.n_tiles < t0 + p.tiles_per_split ? p.n_tiles : t0 + p.tiles_per_split;
  if (t0 < t1) {
    // Streaming from HBM: three operand sets in a ring keep two tiles in flight
    // while one is computed.  Loads past the chunk re-read its last tile (in
    // bounds, never used); the scheduling barriers keep each load where it is
    // issued instead of letting it sink to its use.
    RegOps<D, KT> o0, o1, o2;
    auto kbc = [&](int t) { return (t < t1 ? t : t1 - 1) * KT; };
    auto load = [&](RegOps<D, KT>& op, int t) {
      reg_load_k<D, KT>(kv, kbc(t), op);
      reg_load_v<D, KT>(kv, kbc(t), op);
      __builtin_amdgcn_sched_barrier(0);
    };
    auto tile = [&](RegOps<D, KT>& op, int t) {
      if (t < t1) {
        const int kb0 = t * KT;
        v16f sacc[NB];
#pragma unroll
        for (int bb = 0; bb < NB; bb++) sacc[bb] = score_block<D>(op.ka[bb], op.ksw[bb], qb, qsc);
        const bool need_mask = (kb0 + KT - 1) > wave_lim;
        softmax_pv<D, KT, REORDER, DUMP>(sacc, kb0, need_mask, lim, p.c, p.noclip, op, accO, m, l, phc, phs);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    load(o0, t0);
    load(o1, t0 + 1);
    for (int t = t0; t < t1; t += 3) {
      load(o2, t + 2);
      tile(o0, t);
      load(o0, t + 3);
      tile(o1, t + 1);
      load(o1, t + 4);
      tile(o2, t + 2);
    }
  }

  if (real && p.num_splits == 1) {
    store_out<D>(p.out + row * D, accO, l);  // a single chunk is the whole pass
  } else if (real) {
    float* wo = p.ws_o + (row * p.num_splits + chunk) * D;
#pragma unroll
    for (int ct = 0; ct < CT; ct++)
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) {
        const float4 o4 = make_float4(accO[ct][4 * r4], accO[ct][4 * r4 + 1], accO[ct][4 * r4 + 2],
                                      accO[ct][4 * r4 + 3]);
        *reinterpret_cast<float4*>(wo + 32 * ct + 8 * r4 + 4 * hf) = o4;
      }
    if (hf == 0) {
      float* ml = p.ws_ml + (row * p.num_splits + chunk) * 2;
      ml[0] = m;
      ml[1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// Split-KV with the merge fused in (decode).  One workgroup per KV head (b, g):
// wave w runs chunks w, w+4, w+8, ... one after another (each from
// (-inf, 0, 0), streaming its tiles through the same register ring as the
// split kernel), and leaves each chunk's (m, l, O) of its real columns in
// LDS.  After a barrier the workgroup merges the C partials in chunk order --
// the same arithmetic as attn_merge_kernel -- and writes the output.  No
// partial state leaves the chip.  LDS: C * cols * (D + 2) floats.
// ---------------------------------------------------------------------------
template <int D, int KT, bool CAUSAL, bool REORDER, bool DUMP, bool QRAW>
__global__ __launch_bounds__(256, (D * KT <= 128 * 64) ? 2 : 1) void attn_decode_kernel(KParams p) {
  constexpr int KS = D / 64, CT = D / 32, SW = (D / 64 + 1) / 2, NB = KT / 32;
  extern __shared__ __attribute__((aligned(16))) float part[];
  const int lane = threadIdx.x & 63, hf = lane >> 5, l32 = lane & 31;
  const int wave = threadIdx.x >> 6;
  const int64_t bg = blockIdx.x;
  const int64_t b = bg / p.Hkv, g = bg % p.Hkv;
  const int C = p.num_splits, tpc = p.tiles_per_split, T = p.n_tiles;
  const int cols = p.G * (int)p.N_q;
  float* part_o = part;                       // [C][cols][D]
  float* part_ml = part + (int64_t)C * cols * D;  // [C][cols][2]

  const SplitCols cs = split_cols(p, b, g);
  uint4 qb[KS];
  uint32_t qsc[SW];
  split_query<D, QRAW>(p, b, g, cs, qb, qsc);

  KvBases kv;
  kv.kc = p.k_codes + bg * p.Npad_kv * (D / 2);
  kv.ks = p.k_scales + bg * p.Npad_kv * (D / 32);
  kv.vc = p.v_codes + bg * p.Npad_kv * (D / 2);
  kv.vs = p.v_scales + bg * p.Npad_kv * (D / 32);

  const int64_t shift = p.N_kv - p.N_q;
  const int lim = CAUSAL ? (int)min64(cs.i + shift, p.N_kv - 1) : (int)(p.N_kv - 1);
  const int wave_lim = CAUSAL ? (int)min64(shift, p.N_kv - 1) : (int)(p.N_kv - 1);

  uint8_t* phc = nullptr;
  uint8_t* phs = nullptr;
  if constexpr (DUMP) {
    if (cs.real) {
      phc = p.phat_codes + cs.row * (p.Npad_kv / 2);
      phs = p.phat_scales + cs.row * (p.Npad_kv / 32);
    }
  }

  v16f accO[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ct++) accO[ct] = zero16();
  float m = kNegInf, l = 0.0f;
  // this wave's positions: chunk k = wave + 4 * (pos / tpc), tile k * tpc + pos % tpc
  const int nck = wave < C ? (C - wave + 3) / 4 : 0;
  const int npos = nck * tpc;
  auto tile_of = [&](int pos) { return (wave + 4 * (pos / tpc)) * tpc + pos % tpc; };
  if (npos > 0) {
    // the split kernel's ring over this wave's positions, with resources that
    // end at the KV head's last tile: a position past the wave's last chunk
    // maps past it and loads nothing
    RegOps<D, KT> o0, o1, o2;
    const KvRsrc rs = make_kv_rsrc<D, KT>(kv, 0, T);
    auto load = [&](RegOps<D, KT>& op, int pos) {
      reg_load_kv<D, KT>(rs, tile_of(pos), op);
      __builtin_amdgcn_sched_barrier(0);
    };
    auto step = [&](RegOps<D, KT>& op, int pos) {
      if (pos < npos) {
        const int t = tile_of(pos);
        if (t < T) {
          const int kb0 = t * KT;
          v16f sacc[NB];
#pragma unroll
          for (int bb = 0; bb < NB; bb++) sacc[bb] = score_block<D>(op.ka[bb], op.ksw[bb], qb, qsc);
          const bool need_mask = (kb0 + KT - 1) > wave_lim;
          softmax_pv<D, KT, REORDER, DUMP>(sacc, kb0, need_mask, lim, p.c, p.noclip, op, accO, m, l, phc, phs);
        }
        if (pos % tpc == tpc - 1) {  // chunk done: its state to LDS, then start the next one
          const int k = wave + 4 * (pos / tpc);
          if (cs.real) {
            float* wo = part_o + ((int64_t)k * cols + l32) * D;
#pragma unroll
            for (int ct = 0; ct < CT; ct++)
#pragma unroll
              for (int r4 = 0; r4 < 4; r4++)
                *reinterpret_cast<float4*>(wo + 32 * ct + 8 * r4 + 4 * hf) =
                    make_float4(accO[ct][4 * r4], accO[ct][4 * r4 + 1], accO[ct][4 * r4 + 2],
                                accO[ct][4 * r4 + 3]);
            if (hf == 0) {
              part_ml[((int64_t)k * cols + l32) * 2] = m;
              part_ml[((int64_t)k * cols + l32) * 2 + 1] = l;
            }
          }
#pragma unroll
          for (int ct = 0; ct < CT; ct++) accO[ct] = zero16();
          m = kNegInf;
          l = 0.0f;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    load(o0, 0);
    load(o1, 1);
    for (int pos = 0; pos < npos; pos += 3) {
      load(o2, pos + 2);
      step(o0, pos);
      load(o0, pos + 3);
      step(o1, pos + 1);
      load(o1, pos + 4);
      step(o2, pos + 2);
    }
  }
  __syncthreads();

  // merge in chunk order: M = max m_k, w_k = 2^(m_k - M), L = sum w_k l_k,
  // A = sum w_k O_k (fp32, sequential), out = fp16(A / fp16(L))
  for (int idx = threadIdx.x; idx < cols * (D / 4); idx += 256) {
    const int q = idx / (D / 4), c4 = idx % (D / 4);
    float M = kNegInf;
    for (int k = 0; k < C; k++) M = fmaxf(M, part_ml[((int64_t)k * cols + q) * 2]);
    float L = 0.0f;
    float A[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < C; k++) {
      const float mk = part_ml[((int64_t)k * cols + q) * 2];
      const float w = (mk == kNegInf) ? 0.0f : exp2_hw(mk - M);
      const float wl = w * part_ml[((int64_t)k * cols + q) * 2 + 1];
      L = L + wl;
      const float4 o = *reinterpret_cast<const float4*>(part_o + ((int64_t)k * cols + q) * D + 4 * c4);
      const float wo[4] = {w * o.x, w * o.y, w * o.z, w * o.w};
#pragma unroll
      for (int z = 0; z < 4; z++) A[z] = A[z] + wo[z];
    }
    const float lf = round_f16(L);
    const int j = q / (int)p.N_q;
    const int64_t row = (b * p.Hq + g * p.G + j) * p.N_q + q % (int)p.N_q;
    const uint32_t lo = (uint32_t)float_to_half_bits(A[0] / lf) | ((uint32_t)float_to_half_bits(A[1] / lf) << 16);
    const uint32_t hi = (uint32_t)float_to_half_bits(A[2] / lf) | ((uint32_t)float_to_half_bits(A[3] / lf) << 16);
    *reinterpret_cast<uint2*>(p.out + row * D + 4 * c4) = make_uint2(lo, hi);
  }
}

// ---------------------------------------------------------------------------
// Merge of split partials, in chunk order: M = max m_k, w_k = 2^(m_k - M),
// L = sum w_k l_k, A = sum w_k O_k (fp32, sequential), out = fp16(A / fp16(L)).
// Workgroup = (query row, slice of 64 channels), four wavefronts.  The partials of
// up to kMergeBatch chunks are loaded by all four wavefronts at once, together
// with the (m, l) pairs, so a merge of that many chunks waits on memory once
// (the loads do not depend on M); they are staged in LDS with the weights w_k
// and w_k l_k, computed one chunk per thread.  Wavefront 0, lane c owning
// channel c, then runs both sums sequentially over the chunks out of LDS.
// Longer chunk lists run in batches of kMergeBatch after M has been reduced.
// ---------------------------------------------------------------------------
constexpr int kMergeBatch = 128;

__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ ws_o,
                                                         const float* __restrict__ ws_ml, int C, int d,
                                                         uint16_t* __restrict__ out) {
  constexpr int PER = kMergeBatch / 4;  // chunks each thread stages per batch
  __shared__ float s_o[kMergeBatch][64];
  __shared__ float s_w[kMergeBatch], s_wl[kMergeBatch];
  __shared__ float s_red[4];
  const int64_t row = blockIdx.x;
  const int t = (int)threadIdx.x, lane = t & 63, wv = t >> 6;
  const int ch = (int)blockIdx.y * 64 + lane;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml + row * C * 2);
  const float* o = ws_o + row * (int64_t)C * d + ch;

  // Every load of the first batch is issued before any is waited on: chunk
  // indices past the end are clamped to the last chunk (in bounds, never used),
  // so no load sits behind a branch.
  const int nb0 = C < kMergeBatch ? C : kMergeBatch;
  float ov[PER];
#pragma unroll
  for (int i = 0; i < PER; i++) ov[i] = o[(int64_t)min(wv + 4 * i, nb0 - 1) * d];
  const float2 st0 = ml[t < C ? t : C - 1];  // chunk t's (m, l), used again for its weight
  float M = t < C ? st0.x : kNegInf;
  for (int k = t + 256; k < C; k += 256) M = fmaxf(M, ml[k].x);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) s_red[wv] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));

  float A = 0.0f, L = 0.0f;
  for (int kb = 0; kb < C; kb += kMergeBatch) {
    const int nb = C - kb < kMergeBatch ? C - kb : kMergeBatch;
    float2 st = st0;
    if (kb > 0) {
      __syncthreads();  // wavefront 0 is done with the previous batch
#pragma unroll
      for (int i = 0; i < PER; i++) ov[i] = o[(int64_t)(kb + min(wv + 4 * i, nb - 1)) * d];
      st = ml[kb + (t < nb ? t : nb - 1)];
    }
#pragma unroll
    for (int i = 0; i < PER; i++)
      if (wv + 4 * i < nb) s_o[wv + 4 * i][lane] = ov[i];
    if (t < nb) {
      const float w = (st.x == kNegInf) ? 0.0f : exp2_hw(st.x - M);
      s_w[t] = w;
      s_wl[t] = w * st.y;
    }
    __syncthreads();
    if (wv == 0) {
#pragma unroll 8
      for (int j = 0; j < nb; j++) {
        L = L + s_wl[j];
        const float wo = s_w[j] * s_o[j][lane];
        A = A + wo;
      }
    }
  }
  if (wv == 0) {
    const float lf = round_f16(L);
    out[row * d + ch] = float_to_half_bits(A / lf);
  }
}

// Compute units of the current device, queried once per device (0 if unknown).
int device_cu_count() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int cus = cache[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

// Workgroups of 256 threads of `kernel` resident at once on one CU of the
// current device (registers and LDS), queried once per device (0 if unknown).
constexpr int kMaxDevices = 64;
int resident_per_cu(const void* kernel, std::atomic<int>* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, 256, 0) != hipSuccess || n <= 0) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int D, int KT, bool CAUSAL, bool REORDER, bool DUMP, bool EXPFREE>
std::atomic<int>* resident_cache() {
  static std::atomic<int> cache[kMaxDevices];
  return cache;
}

template <int D, int KT, bool CAUSAL, bool REORDER, bool DUMP, bool EXPFREE = false>
hipError_t launch_prefill_t(const KParams& kp, hipStream_t stream) {
  const int nh = kp.heads_per_wg, nr = 4 / nh;
  // x = (head chunk, b, g) with the KV head fastest: consecutive workgroups
  // land on consecutive XCDs, so each XCD's L2 serves a fixed set of KV heads
  dim3 grid((unsigned)(kp.B * kp.Hkv * (kp.G / nh)), (unsigned)((kp.N_q + 32 * nr - 1) / (32 * nr)));
  const auto kernel = attn_prefill_kernel<D, KT, CAUSAL, REORDER, DUMP, EXPFREE>;
  const int cus = device_cu_count();
  const int per_cu = resident_per_cu(reinterpret_cast<const void*>(kernel), resident_cache<D, KT, CAUSAL, REORDER, DUMP, EXPFREE>());
  KParams k2 = kp;
  k2.slot_rows = 0;
  const int64_t wgs = (int64_t)grid.x * grid.y;
  if (cus > 0 && per_cu > 0 && wgs <= (int64_t)per_cu * cus) {
    const int64_t slots = (wgs + cus - 1) / cus;  // workgroups each CU receives
    k2.slot_rows = (int)((grid.y + slots - 1) / slots);
  }
  kernel<<<grid, dim3(256), 0, stream>>>(k2);
  return hipGetLastError();
}

// LDS bytes of the fused decode kernel's partial states (0: too large, use the
// split kernel and the merge kernel).
inline size_t decode_lds_bytes(const KParams& kp, int d) {
  const size_t bytes = (size_t)kp.num_splits * kp.G * kp.N_q * (d + 2) * sizeof(float);
  return bytes <= 64 * 1024 ? bytes : 0;
}

template <int D, int KT, bool CAUSAL, bool REORDER, bool DUMP, bool QRAW>
hipError_t launch_split_t(const KParams& kp, hipStream_t stream) {
  // the fused kernel runs one workgroup per (b, g): it needs enough of them to
  // fill the chip; fewer take one wavefront per chunk and a separate merge
  if (kp.num_splits > 1 && kp.B * kp.Hkv >= 128) {
    if (const size_t lds = decode_lds_bytes(kp, D)) {
      attn_decode_kernel<D, KT, CAUSAL, REORDER, DUMP, QRAW>
          <<<dim3((unsigned)(kp.B * kp.Hkv)), dim3(256), lds, stream>>>(kp);
      return hipGetLastError();
    }
  }
  // one wavefront per workgroup: the wavefronts share nothing, and a short grid
  // spreads over twice as many compute units as in workgroups of four (one
  // 32768-token sequence at 64 chunks: 17.9 against 21.2 us)
  const int64_t waves = kp.B * kp.Hkv * kp.num_splits;
  attn_split_kernel<D, KT, CAUSAL, REORDER, DUMP, QRAW><<<dim3((unsigned)waves), dim3(64), 0, stream>>>(kp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || kp.num_splits == 1) return e;
  const int64_t rows = kp.B * kp.Hq * kp.N_q;
  attn_merge_kernel<<<dim3((unsigned)rows, D / 64), dim3(256), 0, stream>>>(kp.ws_o, kp.ws_ml, kp.num_splits, D,
                                                                            kp.out);
  return hipGetLastError();
}

KParams make_params(const AttnLaunch& a) {
  KParams kp;
  kp.q_codes = a.q_codes;
  kp.q_scales = a.q_scales;
  kp.q_f16 = a.q_f16;
  kp.s = a.smooth ? a.s : nullptr;
  kp.k_codes = a.k_codes;
  kp.k_scales = a.k_scales;
  kp.v_codes = a.v_codes;
  kp.v_scales = a.v_scales;
  kp.out = a.out;
  kp.phat_codes = a.phat_codes;
  kp.phat_scales = a.phat_scales;
  kp.ws_o = a.ws_o;
  kp.ws_ml = a.ws_ml;
  kp.B = a.B;
  kp.Hq = a.Hq;
  kp.Hkv = a.Hkv;
  kp.N_q = a.N_q;
  kp.N_kv = a.N_kv;
  kp.Npad_q = a.Npad_q;
  kp.Npad_kv = a.Npad_kv;
  kp.G = (int)(a.Hq / a.Hkv);
  kp.num_splits = a.num_splits;
  kp.n_tiles = (int)((a.N_kv + a.kv_tile - 1) / a.kv_tile);
  kp.tiles_per_split = (kp.n_tiles + a.num_splits - 1) / a.num_splits;
  kp.heads_per_wg = (kp.G % 4 == 0) ? 4 : (kp.G % 2 == 0) ? 2 : 1;
  kp.slot_rows = 0;
  kp.noclip = a.noclip;
  kp.c = (float)(1.4426950408889634073599246810019 / __builtin_sqrt((double)a.d));
  return kp;
}

template <int D, int KT>
hipError_t dispatch_prefill(const AttnLaunch& a, const KParams& kp, hipStream_t st) {
  const bool dump = a.phat_codes != nullptr;
  if (a.phat_mode == 1) {  // exp-free P_hat (reorder = 1, checked by the caller)
    const int k2 = (a.causal ? 2 : 0) | (dump ? 1 : 0);
    switch (k2) {
      case 0: return launch_prefill_t<D, KT, false, true, false, true>(kp, st);
      case 1: return launch_prefill_t<D, KT, false, true, true, true>(kp, st);
      case 2: return launch_prefill_t<D, KT, true, true, false, true>(kp, st);
      default: return launch_prefill_t<D, KT, true, true, true, true>(kp, st);
    }
  }
  const int key = (a.causal ? 4 : 0) | (a.reorder ? 2 : 0) | (dump ? 1 : 0);
  switch (key) {
    case 0: return launch_prefill_t<D, KT, false, false, false>(kp, st);
    case 1: return launch_prefill_t<D, KT, false, false, true>(kp, st);
    case 2: return launch_prefill_t<D, KT, false, true, false>(kp, st);
    case 3: return launch_prefill_t<D, KT, false, true, true>(kp, st);
    case 4: return launch_prefill_t<D, KT, true, false, false>(kp, st);
    case 5: return launch_prefill_t<D, KT, true, false, true>(kp, st);
    case 6: return launch_prefill_t<D, KT, true, true, false>(kp, st);
    default: return launch_prefill_t<D, KT, true, true, true>(kp, st);
  }
}

template <int D, int KT, bool QRAW>
hipError_t dispatch_split_q(const AttnLaunch& a, const KParams& kp, hipStream_t st) {
  const bool dump = a.phat_codes != nullptr;
  const int key = (a.causal ? 4 : 0) | (a.reorder ? 2 : 0) | (dump ? 1 : 0);
  switch (key) {
    case 0: return launch_split_t<D, KT, false, false, false, QRAW>(kp, st);
    case 1: return launch_split_t<D, KT, false, false, true, QRAW>(kp, st);
    case 2: return launch_split_t<D, KT, false, true, false, QRAW>(kp, st);
    case 3: return launch_split_t<D, KT, false, true, true, QRAW>(kp, st);
    case 4: return launch_split_t<D, KT, true, false, false, QRAW>(kp, st);
    case 5: return launch_split_t<D, KT, true, false, true, QRAW>(kp, st);
    case 6: return launch_split_t<D, KT, true, true, false, QRAW>(kp, st);
    default: return launch_split_t<D, KT, true, true, true, QRAW>(kp, st);
  }
}

template <int D, int KT>
hipError_t dispatch_split(const AttnLaunch& a, const KParams& kp, hipStream_t st) {
  return a.q_f16 ? dispatch_split_q<D, KT, true>(a, kp, st) : dispatch_split_q<D, KT, false>(a, kp, st);
}

template <int D>
hipError_t dispatch_prefill_kt(const AttnLaunch& a, const KParams& kp, hipStream_t st) {
  if (a.kv_tile == 128) return dispatch_prefill<D, 128>(a, kp, st);
  return dispatch_prefill<D, 64>(a, kp, st);
}

template <int D>
hipError_t dispatch_split_kt(const AttnLaunch& a, const KParams& kp, hipStream_t st) {
  if constexpr (D <= 128) {
    if (a.kv_tile == 128) return dispatch_split<D, 128>(a, kp, st);
  }
  return dispatch_split<D, 64>(a, kp, st);
}

}  // namespace

hipError_t launch_attn_prefill(const AttnLaunch& a, hipStream_t stream) {
  const KParams kp = make_params(a);
  switch (a.d) {
    case 64: return dispatch_prefill_kt<64>(a, kp, stream);
    case 128: return dispatch_prefill_kt<128>(a, kp, stream);
    default: return dispatch_prefill_kt<256>(a, kp, stream);
  }
}

hipError_t launch_attn_split(const AttnLaunch& a, hipStream_t stream) {
  const KParams kp = make_params(a);
  switch (a.d) {
    case 64: return dispatch_split_kt<64>(a, kp, stream);
    case 128: return dispatch_split_kt<128>(a, kp, stream);
    default: return dispatch_split_kt<256>(a, kp, stream);
  }
}

}  // namespace hifa4

// 4-bit FlashAttention forward for gfx950: prefill, split-KV (decode) and merge.
//
// HiFA4 (arXiv 2607.04302), Abstract: QK^T and PV are both 4-bit
// block-scaled GEMMs, the online-softmax state (m, l) is FP16, and with
// P-Reordering the normalizer is summed from the same quantized P_hat that
// feeds the PV GEMM -- which lets it be produced by that GEMM.
//
// Design on CDNA4 (one wavefront = 32 query rows, tiles of 64 keys):
//  * Scores are computed transposed, S^T = K_hat Q_hat^T, with the scaled
//    FP4 MFMA 32x32x64: A = 32 keys (16-byte rows of K_hat straight from
//    memory), B = the wave's 32 query rows (loop-invariant registers).  The
//    accumulator gives each lane one query column and 16 keys.
//  * One v_permlane32_swap per register pair turns the two 32-key S^T blocks
//    into "lane = (query, 32-key block)": every lane then holds exactly the
//    32 keys that share one P_hat scale.  Block max, exp, block exponent and
//    the E2M1 conversion run in-lane; the row max needs one more swap.
//  * P_hat is then already the B operand of O^T = V_hat^T P_hat^T
//    (A = 32 channels x 64 keys of the token-blocked V_hat, again one
//    16-byte load per lane), so the output accumulator is also "lane =
//    query", and alpha / l never leave their lane.
//  * P-Reordering: one more MFMA with A = all-ones E2M1 codes adds
//    rowsum(P_hat) to the running l -- the normalizer is a row of the same
//    PV product ([V_hat | 1]) instead of a VALU reduction.
#include "hifa4_device.hpp"
#include "hifa4_internal.hpp"

namespace hifa4 {

namespace {

constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

struct KvPtrs {
  const uint8_t* kc;  // K_hat codes of this (b, g), row layout
  const uint8_t* ks;  // K_hat scales
  const uint8_t* vc;  // V_hat codes, token layout
  const uint8_t* vs;  // V_hat scales
  int64_t npad;       // padded KV length
};

// Scale word for the S^T MFMA's k-step s: byte 2*(s%2) of word s/2 holds the
// scale of the 32-channel block (2*s + lane/32).  Built from a row's scale
// bytes by shifting out the other half's byte.
template <int D>
__device__ __forceinline__ void load_row_scales(const uint8_t* row, int hf, uint32_t (&w)[(D / 64 + 1) / 2]) {
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

// One 64-key tile of the online-softmax recurrence for the wave's 32 query
// columns.  lim: last valid key of this lane's query column.
template <int D, bool REORDER, bool DUMP>
__device__ __forceinline__ void attn_tile(const KvPtrs& kv, int kb0, bool need_mask, int lim,
                                          float c, const uint4 (&qb)[D / 64],
                                          const uint32_t (&qsc)[(D / 64 + 1) / 2],
                                          v16f (&accO)[D / 32], v16f& accL, float& m, float& l,
                                          uint8_t* phat_codes_row, uint8_t* phat_scales_row) {
  constexpr int KS = D / 64, CT = D / 32, SW = (D / 64 + 1) / 2;
  const int lane = threadIdx.x & 63, hf = lane >> 5, l32 = lane & 31;

  // ---- operand loads: K_hat rows (A of S^T) and V_hat channel rows (A of O^T)
  uint4 ka[2][KS];
  uint32_t ksw[2][SW];
#pragma unroll
  for (int mi = 0; mi < 2; mi++) {
    const int64_t key = kb0 + 32 * mi + l32;
    const uint8_t* kr = kv.kc + key * (D / 2);
#pragma unroll
    for (int s = 0; s < KS; s++) ka[mi][s] = *reinterpret_cast<const uint4*>(kr + (2 * s + hf) * 16);
    load_row_scales<D>(kv.ks + key * (D / 32), hf, ksw[mi]);
  }
  uint4 va[CT];
  uint32_t vsw[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ct++) {
    const int64_t ch = 32 * ct + l32;
    va[ct] = *reinterpret_cast<const uint4*>(kv.vc + ch * (kv.npad / 2) + kb0 / 2 + 16 * hf);
    vsw[ct] = kv.vs[ch * (kv.npad / 32) + kb0 / 32 + hf];
  }

  // ---- S^T for keys [kb0, kb0+32) and [kb0+32, kb0+64)
  v16f s0 = zero16(), s1 = zero16();
#pragma unroll
  for (int s = 0; s < KS; s++) {
    if (s % 2 == 0) {
      s0 = mfma_fp4<0, 0>(ka[0][s], (int)ksw[0][s / 2], qb[s], (int)qsc[s / 2], s0);
      s1 = mfma_fp4<0, 0>(ka[1][s], (int)ksw[1][s / 2], qb[s], (int)qsc[s / 2], s1);
    } else {
      s0 = mfma_fp4<2, 2>(ka[0][s], (int)ksw[0][s / 2], qb[s], (int)qsc[s / 2], s0);
      s1 = mfma_fp4<2, 2>(ka[1][s], (int)ksw[1][s / 2], qb[s], (int)qsc[s / 2], s1);
    }
  }

  // ---- lane = (query l32, 32-key block hf): X[r] is key 8(r/4) + r%4 of the
  // block, Y[r] the key 4 further.
  float X[16], Y[16];
#pragma unroll
  for (int r = 0; r < 16; r++) {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(s0[r]), __float_as_uint(s1[r]),
                                               false, false);
    X[r] = __uint_as_float(sw[0]);
    Y[r] = __uint_as_float(sw[1]);
  }
  if (need_mask) {
    const int base = kb0 + 32 * hf;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int kx = base + 8 * (r / 4) + (r % 4);
      if (kx > lim) X[r] = kNegInf;
      if (kx + 4 > lim) Y[r] = kNegInf;
    }
  }

  // ---- running max (log2 domain, FP16 state)
  float bm = kNegInf;
#pragma unroll
  for (int r = 0; r < 16; r++) bm = fmaxf(bm, fmaxf(X[r], Y[r]));
  const float smax = fmaxf(bm, other_half(bm));
  const float mt = c * smax;
  const float m_new = round_f16(fmaxf(m, mt));
  const float m_use = (m_new == kNegInf) ? 0.0f : m_new;  // column with no valid key yet
  const float alpha = exp2_hw(m - m_use);

  // ---- P = 2^(S c - m); P_hat block exponent from the block's largest t
#pragma unroll
  for (int r = 0; r < 16; r++) {
    X[r] = exp2_hw(__builtin_fmaf(X[r], c, -m_use));
    Y[r] = exp2_hw(__builtin_fmaf(Y[r], c, -m_use));
  }
  const float tmax = __builtin_fmaf(bm, c, -m_use);
  const float ef = fminf(fmaxf(floorf(tmax) - 2.0f, -127.0f), 127.0f);
  const int e = (int)ef;
  const float psc_f = pow2f(e);
  uint32_t pw[4];
#pragma unroll
  for (int w = 0; w < 4; w++) {
    uint32_t x = cvt_fp4x2<0>(0u, X[4 * w], X[4 * w + 1], psc_f);
    x = cvt_fp4x2<1>(x, X[4 * w + 2], X[4 * w + 3], psc_f);
    x = cvt_fp4x2<2>(x, Y[4 * w], Y[4 * w + 1], psc_f);
    pw[w] = cvt_fp4x2<3>(x, Y[4 * w + 2], Y[4 * w + 3], psc_f);
  }
  const uint4 ph = {pw[0], pw[1], pw[2], pw[3]};
  const int psc = e + 127;
  if constexpr (DUMP) {
    if (phat_codes_row) {
      *reinterpret_cast<uint4*>(phat_codes_row + kb0 / 2 + 16 * hf) = ph;
      phat_scales_row[kb0 / 32 + hf] = (uint8_t)psc;
    }
  }

  // ---- O <- alpha O (skipped when the max did not move for any column)
  if (!__all(alpha == 1.0f)) {
#pragma unroll
    for (int ct = 0; ct < CT; ct++)
#pragma unroll
      for (int r = 0; r < 16; r++) accO[ct][r] = accO[ct][r] * alpha;
  }

  // ---- normalizer
  if constexpr (REORDER) {
    const float al = alpha * l;
#pragma unroll
    for (int r = 0; r < 16; r++) accL[r] = al;
    const uint4 ones = {0x22222222u, 0x22222222u, 0x22222222u, 0x22222222u};  // E2M1 1.0
    accL = mfma_fp4<0, 0>(ones, 127, ph, psc, accL);
    l = round_f16(accL[0]);
  } else {
    float rs = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      rs = rs + X[r];
      rs = rs + Y[r];
    }
    rs = rs + other_half(rs);
    const float al = alpha * l;
    l = round_f16(al + rs);
  }

  // ---- O^T += V_hat^T P_hat^T
#pragma unroll
  for (int ct = 0; ct < CT; ct++) accO[ct] = mfma_fp4<0, 0>(va[ct], (int)vsw[ct], ph, psc, accO[ct]);
  m = m_new;
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
  float c;
};

// ---------------------------------------------------------------------------
// Prefill: block = 4 wavefronts = 128 consecutive query rows of one (b, h).
// Grid (B * Hq, ceil(N_q / 128)); the row blocks run last-first so that the
// longest causal blocks start earliest.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool REORDER, bool DUMP>
__global__ __launch_bounds__(256) void attn_prefill_kernel(KParams p) {
  constexpr int KS = D / 64, CT = D / 32, SW = (D / 64 + 1) / 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, hf = lane >> 5, l32 = lane & 31;
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / p.Hq, h = bh % p.Hq, g = h / p.G;
  const int64_t qblk = (int64_t)gridDim.y - 1 - blockIdx.y;
  const int64_t row0 = qblk * 128 + 32 * wave;
  if (row0 >= p.N_q) return;

  // Q_hat rows of this wave: B operand of S^T, resident for the whole loop.
  const int64_t qrow = row0 + l32;
  const uint8_t* qr = p.q_codes + (bh * p.Npad_q + qrow) * (D / 2);
  uint4 qb[KS];
#pragma unroll
  for (int s = 0; s < KS; s++) qb[s] = *reinterpret_cast<const uint4*>(qr + (2 * s + hf) * 16);
  uint32_t qsc[SW];
  load_row_scales<D>(p.q_scales + (bh * p.Npad_q + qrow) * (D / 32), hf, qsc);

  KvPtrs kv;
  const int64_t bg = b * p.Hkv + g;
  kv.kc = p.k_codes + bg * p.Npad_kv * (D / 2);
  kv.ks = p.k_scales + bg * p.Npad_kv * (D / 32);
  kv.vc = p.v_codes + bg * D * (p.Npad_kv / 2);
  kv.vs = p.v_scales + bg * D * (p.Npad_kv / 32);
  kv.npad = p.Npad_kv;

  const int64_t shift = p.N_kv - p.N_q;  // causal diagonal offset (bottom-right aligned)
  int lim = (int)(p.N_kv - 1);
  if (CAUSAL) lim = (int)min64(qrow + shift, p.N_kv - 1);
  // smallest limit in the wave (its first row) decides when masking is needed
  const int wave_lim = CAUSAL ? (int)min64(row0 + shift, p.N_kv - 1) : (int)(p.N_kv - 1);
  const int64_t last_row = min64(row0 + 31, p.N_q - 1);
  const int64_t last_key = CAUSAL ? min64(last_row + shift, p.N_kv - 1) : p.N_kv - 1;
  const int tiles = (int)(last_key / kKvTile) + 1;

  uint8_t* phc = nullptr;
  uint8_t* phs = nullptr;
  if constexpr (DUMP) {
    if (qrow < p.N_q) {
      phc = p.phat_codes + (bh * p.N_q + qrow) * (p.Npad_kv / 2);
      phs = p.phat_scales + (bh * p.N_q + qrow) * (p.Npad_kv / 32);
    }
  }

  v16f accO[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ct++) accO[ct] = zero16();
  v16f accL = zero16();
  float m = kNegInf, l = 0.0f;
  for (int t = 0; t < tiles; t++) {
    const int kb0 = t * kKvTile;
    const bool need_mask = (kb0 + kKvTile - 1) > wave_lim;
    attn_tile<D, REORDER, DUMP>(kv, kb0, need_mask, lim, p.c, qb, qsc, accO, accL, m, l, phc, phs);
  }

  // ---- out = fp16(O / l): lane holds channels 32ct + 8(r/4) + 4hf + r%4
  if (qrow < p.N_q) {
    uint16_t* orow = p.out + (bh * p.N_q + qrow) * D;
#pragma unroll
    for (int ct = 0; ct < CT; ct++) {
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) {
        uint32_t lo = (uint32_t)float_to_half_bits(accO[ct][4 * r4 + 0] / l) |
                      ((uint32_t)float_to_half_bits(accO[ct][4 * r4 + 1] / l) << 16);
        uint32_t hi = (uint32_t)float_to_half_bits(accO[ct][4 * r4 + 2] / l) |
                      ((uint32_t)float_to_half_bits(accO[ct][4 * r4 + 3] / l) << 16);
        *reinterpret_cast<uint2*>(orow + 32 * ct + 8 * r4 + 4 * hf) = make_uint2(lo, hi);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split-KV: one wavefront per (b, g, chunk).  Its 32 query columns are the
// G * N_q (head-in-group, row) pairs of KV head g (G * N_q <= 32; the rest are
// zero padding).  Q is smoothed and quantized in-kernel from binary16 (or
// read pre-quantized).  Each chunk writes its (m, l, O) partial state.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool REORDER, bool DUMP, bool QRAW>
__global__ __launch_bounds__(256) void attn_split_kernel(KParams p) {
  constexpr int KS = D / 64, CT = D / 32, SW = (D / 64 + 1) / 2;
  const int lane = threadIdx.x & 63, hf = lane >> 5, l32 = lane & 31;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
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
#pragma unroll
  for (int w = 0; w < SW; w++) qsc[w] = 0u;
  if constexpr (QRAW) {
    // Smooth-QK multiply and MX quantization of 32 channels per k-step, in-lane.
    const uint16_t* qx = p.q_f16 + row * D;
#pragma unroll
    for (int s = 0; s < KS; s++) {
      const int cb = 2 * s + hf;
      float v[32];
      if (real) {
#pragma unroll
        for (int u = 0; u < 4; u++) {
          const uint4 raw = *reinterpret_cast<const uint4*>(qx + cb * 32 + 8 * u);
          const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int z = 0; z < 4; z++) {
            v[8 * u + 2 * z] = half_to_float((uint16_t)(w[z] & 0xFFFFu));
            v[8 * u + 2 * z + 1] = half_to_float((uint16_t)(w[z] >> 16));
          }
        }
        if (p.s) {
          const float* sp = p.s + g * D + cb * 32;
#pragma unroll
          for (int z = 0; z < 32; z++) v[z] = v[z] * sp[z];
        }
      } else {
#pragma unroll
        for (int z = 0; z < 32; z++) v[z] = 0.0f;
      }
      float amax = 0.0f;
#pragma unroll
      for (int z = 0; z < 32; z++) amax = fmaxf(amax, fabsf(v[z]));
      const int e = mx_exponent(amax);
      const float sc = pow2f(e);
      qb[s].x = pack8_fp4(&v[0], sc);
      qb[s].y = pack8_fp4(&v[8], sc);
      qb[s].z = pack8_fp4(&v[16], sc);
      qb[s].w = pack8_fp4(&v[24], sc);
      qsc[s / 2] |= (uint32_t)(real ? e + 127 : 0) << (16 * (s % 2));
    }
  } else {
    const int64_t qr_idx = (b * p.Hq + h) * p.Npad_q + i;
    const uint8_t* qr = p.q_codes + qr_idx * (D / 2);
#pragma unroll
    for (int s = 0; s < KS; s++) {
      qb[s] = real ? *reinterpret_cast<const uint4*>(qr + (2 * s + hf) * 16) : make_uint4(0, 0, 0, 0);
    }
    if (real) load_row_scales<D>(p.q_scales + qr_idx * (D / 32), hf, qsc);
  }

  KvPtrs kv;
  kv.kc = p.k_codes + bg * p.Npad_kv * (D / 2);
  kv.ks = p.k_scales + bg * p.Npad_kv * (D / 32);
  kv.vc = p.v_codes + bg * D * (p.Npad_kv / 2);
  kv.vs = p.v_scales + bg * D * (p.Npad_kv / 32);
  kv.npad = p.Npad_kv;

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
  v16f accL = zero16();
  float m = kNegInf, l = 0.0f;
  const int t0 = chunk * p.tiles_per_split;
  const int t1 = p.n_tiles < t0 + p.tiles_per_split ? p.n_tiles : t0 + p.tiles_per_split;
  for (int t = t0; t < t1; t++) {
    const int kb0 = t * kKvTile;
    const bool need_mask = (kb0 + kKvTile - 1) > wave_lim;
    attn_tile<D, REORDER, DUMP>(kv, kb0, need_mask, lim, p.c, qb, qsc, accO, accL, m, l, phc, phs);
  }

  if (real && p.num_splits == 1) {
    // a single chunk is the whole pass: out = fp16(O / l) directly
    uint16_t* orow = p.out + row * D;
#pragma unroll
    for (int ct = 0; ct < CT; ct++)
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) {
        uint32_t lo = (uint32_t)float_to_half_bits(accO[ct][4 * r4 + 0] / l) |
                      ((uint32_t)float_to_half_bits(accO[ct][4 * r4 + 1] / l) << 16);
        uint32_t hi = (uint32_t)float_to_half_bits(accO[ct][4 * r4 + 2] / l) |
                      ((uint32_t)float_to_half_bits(accO[ct][4 * r4 + 3] / l) << 16);
        *reinterpret_cast<uint2*>(orow + 32 * ct + 8 * r4 + 4 * hf) = make_uint2(lo, hi);
      }
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
// Merge of split partials, in chunk order: M = max m_k, w_k = 2^(m_k - M),
// L = sum w_k l_k, A = sum w_k O_k (fp32, sequential), out = fp16(A / fp16(L)).
// One thread per (row, channel).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ ws_o,
                                                         const float* __restrict__ ws_ml,
                                                         int64_t rows, int d, int C,
                                                         uint16_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * d) return;
  const int64_t row = t / d;
  const int ch = (int)(t % d);
  const float* ml = ws_ml + row * C * 2;
  float M = kNegInf;
  for (int k = 0; k < C; k++) M = fmaxf(M, ml[2 * k]);
  float L = 0.0f, A = 0.0f;
  for (int k = 0; k < C; k++) {
    const float mk = ml[2 * k];
    const float w = (mk == kNegInf) ? 0.0f : exp2_hw(mk - M);
    const float wl = w * ml[2 * k + 1];
    L = L + wl;
    const float wo = w * ws_o[(row * C + k) * d + ch];
    A = A + wo;
  }
  const float lf = round_f16(L);
  out[t] = float_to_half_bits(A / lf);
}

template <int D, bool CAUSAL, bool REORDER, bool DUMP>
hipError_t launch_prefill_t(const KParams& kp, hipStream_t stream) {
  dim3 grid((unsigned)(kp.B * kp.Hq), (unsigned)((kp.N_q + 127) / 128));
  attn_prefill_kernel<D, CAUSAL, REORDER, DUMP><<<grid, dim3(256), 0, stream>>>(kp);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool REORDER, bool DUMP, bool QRAW>
hipError_t launch_split_t(const KParams& kp, hipStream_t stream) {
  const int64_t waves = kp.B * kp.Hkv * kp.num_splits;
  dim3 grid((unsigned)((waves + 3) / 4));
  attn_split_kernel<D, CAUSAL, REORDER, DUMP, QRAW><<<grid, dim3(256), 0, stream>>>(kp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || kp.num_splits == 1) return e;
  const int64_t rows = kp.B * kp.Hq * kp.N_q;
  const int64_t n = rows * D;
  attn_merge_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(
      kp.ws_o, kp.ws_ml, rows, D, kp.num_splits, kp.out);
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
  kp.n_tiles = (int)((a.N_kv + kKvTile - 1) / kKvTile);
  kp.tiles_per_split = (kp.n_tiles + a.num_splits - 1) / a.num_splits;
  kp.c = (float)(1.4426950408889634073599246810019 / __builtin_sqrt((double)a.d));
  return kp;
}

template <int D>
hipError_t dispatch_prefill(const AttnLaunch& a, const KParams& kp, hipStream_t st) {
  const bool dump = a.phat_codes != nullptr;
  const int key = (a.causal ? 4 : 0) | (a.reorder ? 2 : 0) | (dump ? 1 : 0);
  switch (key) {
    case 0: return launch_prefill_t<D, false, false, false>(kp, st);
    case 1: return launch_prefill_t<D, false, false, true>(kp, st);
    case 2: return launch_prefill_t<D, false, true, false>(kp, st);
    case 3: return launch_prefill_t<D, false, true, true>(kp, st);
    case 4: return launch_prefill_t<D, true, false, false>(kp, st);
    case 5: return launch_prefill_t<D, true, false, true>(kp, st);
    case 6: return launch_prefill_t<D, true, true, false>(kp, st);
    default: return launch_prefill_t<D, true, true, true>(kp, st);
  }
}

template <int D, bool QRAW>
hipError_t dispatch_split_q(const AttnLaunch& a, const KParams& kp, hipStream_t st) {
  const bool dump = a.phat_codes != nullptr;
  const int key = (a.causal ? 4 : 0) | (a.reorder ? 2 : 0) | (dump ? 1 : 0);
  switch (key) {
    case 0: return launch_split_t<D, false, false, false, QRAW>(kp, st);
    case 1: return launch_split_t<D, false, false, true, QRAW>(kp, st);
    case 2: return launch_split_t<D, false, true, false, QRAW>(kp, st);
    case 3: return launch_split_t<D, false, true, true, QRAW>(kp, st);
    case 4: return launch_split_t<D, true, false, false, QRAW>(kp, st);
    case 5: return launch_split_t<D, true, false, true, QRAW>(kp, st);
    case 6: return launch_split_t<D, true, true, false, QRAW>(kp, st);
    default: return launch_split_t<D, true, true, true, QRAW>(kp, st);
  }
}

template <int D>
hipError_t dispatch_split(const AttnLaunch& a, const KParams& kp, hipStream_t st) {
  return a.q_f16 ? dispatch_split_q<D, true>(a, kp, st) : dispatch_split_q<D, false>(a, kp, st);
}

}  // namespace

hipError_t launch_attn_prefill(const AttnLaunch& a, hipStream_t stream) {
  const KParams kp = make_params(a);
  switch (a.d) {
    case 64: return dispatch_prefill<64>(a, kp, stream);
    case 128: return dispatch_prefill<128>(a, kp, stream);
    default: return dispatch_prefill<256>(a, kp, stream);
  }
}

hipError_t launch_attn_split(const AttnLaunch& a, hipStream_t stream) {
  const KParams kp = make_params(a);
  switch (a.d) {
    case 64: return dispatch_split<64>(a, kp, stream);
    case 128: return dispatch_split<128>(a, kp, stream);
    default: return dispatch_split<256>(a, kp, stream);
  }
}

}  // namespace hifa4

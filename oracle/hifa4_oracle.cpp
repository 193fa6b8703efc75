// CPU oracle for HiFA4's 4-bit FlashAttention forward -- TEST INFRASTRUCTURE.
//
// Plain, slow, single-purpose code that defines the numbers the GPU path must
// reproduce.  Only tests, the smoke check and the benchmark's CPU baseline may
// load it.  It shares no code with the GPU library.
//
// Method source: HiFA4 (arXiv 2607.04302), Abstract -- 4-bit QK^T and PV
// GEMMs, FP16 online-softmax state (m, l), Smooth-QK (static per-channel
// Q*s, K/s after RoPE), P-Reordering (normalizer summed from the same
// quantized P_hat that feeds PV).  The abstract leaves the 4-bit format, the
// calibration formula, the tile shape and every rounding point open; the
// readings taken here are listed next to each function.
//
// Build: g++ -O2 -ffp-contract=off (no -ffast-math): every multiply and add
// below is one IEEE operation in the type written, and fused multiply-adds
// appear only where std::fma is spelled out.
#include "hifa4_oracle.h"

#include <algorithm>
#include <atomic>
#include <cfloat>
#include <cmath>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

std::atomic<int64_t> g_inexact{0};

uint32_t f32_bits(float x) { uint32_t u; std::memcpy(&u, &x, 4); return u; }
float f32_from_bits(uint32_t u) { float x; std::memcpy(&x, &u, 4); return x; }

// binary32 -> binary16, round to nearest, ties to even.
uint16_t f16_rne(float x) {
  const uint32_t u = f32_bits(x);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  const int exp8 = (int)((u >> 23) & 0xFFu);
  const uint32_t mant = u & 0x7FFFFFu;
  if (exp8 == 0xFF) return sign | 0x7C00u | (mant ? 0x200u : 0u);  // inf / nan
  if (exp8 == 0) return sign;  // fp32 subnormals are far below half the fp16 minimum
  int e = exp8 - 127;          // x = 1.mant * 2^e
  const uint32_t full = 0x800000u | mant;  // 24-bit significand
  if (e >= -14) {
    uint32_t m = full >> 13;               // 11 bits incl. the hidden one
    const uint32_t rem = full & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (m & 1u))) m++;
    if (m == 0x800u) { m = 0x400u; e++; }
    if (e > 15) return sign | 0x7C00u;
    return sign | (uint16_t)(((uint32_t)(e + 15) << 10) | (m & 0x3FFu));
  }
  // fp16 subnormal: value = q * 2^-24, q = full * 2^(e + 1 - 0) / 2^0 ... = full >> shift
  const int shift = -(e + 1);  // >= 14
  if (shift > 24) return sign;  // below 2^-25: rounds to zero
  uint32_t q = full >> shift;
  const uint32_t rem = full & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) q++;
  return sign | (uint16_t)q;  // q == 0x400 is the smallest normal, encoded the same way
}

float f16_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
  if (e == 0x1F) return f32_from_bits(sign | 0x7F800000u | (m << 13));
  if (e == 0) {
    float v = (float)m * 5.9604644775390625e-08f;  // m * 2^-24, exact
    return sign ? -v : v;
  }
  return f32_from_bits(sign | ((e - 15 + 127) << 23) | (m << 13));
}

// state rounding: binary16 when the state is FP16, identity otherwise
float round_state(float x, int state_fp16) { return state_fp16 ? f16_to_f32(f16_rne(x)) : x; }

// E2M1 magnitudes by code 0..7 (bit 3 of a code is the sign).
const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

// Round-to-nearest onto the E2M1 grid, ties to the even code, saturating at 6.
int e2m1_rne(double x) {
  const int sign = std::signbit(x) ? 8 : 0;
  const double a = std::fabs(x);
  if (std::isnan(x)) return 7;
  if (a >= 6.0) return sign | 7;
  int best = 0;
  double bestd = a;  // distance to code 0
  for (int c = 1; c < 8; c++) {
    const double dist = std::fabs(a - kE2M1[c]);
    if (dist < bestd || (dist == bestd && (c % 2 == 0) && (best % 2 == 1))) {
      best = c;
      bestd = dist;
    }
  }
  return sign | best;
}

double e2m1_value(int code) { return (code & 8) ? -kE2M1[code & 7] : kE2M1[code & 7]; }

// MX block exponent from the block's largest magnitude a, clamped to [-127, 127].
// rule 0 (the OCP MX rule): floor(log2 a) - 2, where 2 is the emax of E2M1 (its
//   largest value 6 = 1.5 * 2^2); a block whose a * 2^-e lands in [6, 8) saturates.
// rule 1 (no clipping): the smallest e with a * 2^-e <= 6, so nothing saturates.
int mx_exponent_from_amax(double amax, int rule) {
  if (!(amax > 0.0)) return -127;
  int ex;
  std::frexp(amax, &ex);  // amax = fr * 2^ex, fr in [0.5, 1): floor(log2 amax) = ex - 1
  int e = (ex - 1) - 2;
  if (rule == 1 && std::ldexp(amax, -e) > 6.0) e += 1;  // a * 2^-e in [4, 8): one step up
  return std::min(127, std::max(-127, e));
}

void mx_block(const float* x, int n, uint8_t* codes, uint8_t* scale, int rule) {
  double amax = 0.0;
  for (int i = 0; i < n; i++) amax = std::max(amax, std::fabs((double)x[i]));
  const int e = mx_exponent_from_amax(amax, rule);
  for (int i = 0; i < n; i++) codes[i] = (uint8_t)e2m1_rne(std::ldexp((double)x[i], -e));
  *scale = (uint8_t)(e + 127);
}

// Block exponent of P_hat from the largest t = S c - m of the block's valid keys
// (P = 2^t), in the log domain so that it does not depend on the rounding of 2^t:
// rule 0: floor(t_max) - 2 (the OCP rule applied to 2^t_max);
// rule 1: the smallest e with 2^(t_max - e) <= 6 = 1.5 * 2^2, i.e.
//         e = ceil(t_max - log2(3/2)) - 2, the difference taken as one fp32
//         subtraction with log2(3/2) rounded to fp32.
// Both clamped to [-127, 127].
int phat_exponent(float tmax, int rule) {
  int e;
  if (rule == 1) {
    const float lam = (float)std::log2(1.5);
    const float u = tmax - lam;
    e = (int)std::ceil(std::max(u, -200.0f)) - 2;
  } else {
    e = (int)std::floor(std::max(tmax, -200.0f)) - 2;
  }
  return std::min(127, std::max(-127, e));
}

inline void put_nibble(uint8_t* row, int64_t idx, int code) {
  uint8_t& b = row[idx >> 1];
  if (idx & 1) b = (uint8_t)((b & 0x0F) | (code << 4));
  else b = (uint8_t)((b & 0xF0) | (code & 0x0F));
}
inline int get_nibble(const uint8_t* row, int64_t idx) {
  return (row[idx >> 1] >> ((idx & 1) * 4)) & 0xF;
}

// Dequantized value of element idx of an MX row (codes row, scales row).
inline double mx_value(const uint8_t* codes, const uint8_t* scales, int64_t idx) {
  return std::ldexp(e2m1_value(get_nibble(codes, idx)), (int)scales[idx / 32] - 127);
}

// S = fp32 of the dot product of two dequantized rows, summed in fp64.  Every
// product of two dequantized 4-bit values is exact in fp64, and so is the sum
// while the terms' exponents span at most 37 bits (checked by the caller).
float score_f32(const double* a, const double* b, int64_t d) {
  double sum = 0.0;
  for (int64_t x = 0; x < d; x++) sum += a[x] * b[x];
  return (float)sum;
}

template <class F>
void parallel_for(int64_t n, int threads, F&& fn) {
  if (threads < 1) threads = 1;
  if (threads > n) threads = (int)std::max<int64_t>(1, n);
  std::atomic<int64_t> next{0};
  auto work = [&]() {
    for (;;) {
      const int64_t i = next.fetch_add(1);
      if (i >= n) break;
      fn(i);
    }
  };
  std::vector<std::thread> pool;
  for (int t = 1; t < threads; t++) pool.emplace_back(work);
  work();
  for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

uint16_t orc_f16_from_f32(float x) { return f16_rne(x); }
float orc_f32_from_f16(uint16_t h) { return f16_to_f32(h); }
int orc_e2m1_encode(float x) { return e2m1_rne((double)x); }
float orc_e2m1_decode(int code) { return (float)e2m1_value(code & 15); }

void orc_f16_from_f32_array(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = f16_rne(x[i]);
}
void orc_f32_from_f16_array(const uint16_t* h, int64_t n, float* out) {
  for (int64_t i = 0; i < n; i++) out[i] = f16_to_f32(h[i]);
}

float orc_score(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                const uint8_t* k_scales, int64_t d) {
  std::vector<double> a((size_t)d), b((size_t)d);
  for (int64_t x = 0; x < d; x++) {
    a[x] = mx_value(q_codes, q_scales, x);
    b[x] = mx_value(k_codes, k_scales, x);
  }
  return score_f32(a.data(), b.data(), d);
}

int orc_mx_exponent(const float* x, int n, int rule) {
  double amax = 0.0;
  for (int i = 0; i < n; i++) amax = std::max(amax, std::fabs((double)x[i]));
  return mx_exponent_from_amax(amax, rule);
}

void orc_mx_block(const float* x, int n, uint8_t* codes, uint8_t* scale, int rule) {
  mx_block(x, n, codes, scale, rule);
}

int orc_phat_exponent(float tmax, int rule) { return phat_exponent(tmax, rule); }

// Smooth-QK calibration (HiFA4 Abstract: a calibration-static per-channel
// equivalent rescale of Q and K after RoPE).  The formula is not on the page;
// the reading is SmoothQuant's migration rule with strength alpha:
//   s_j = max|K_j|^alpha / max|Q_j|^(1 - alpha),
// maxima over the calibration tokens (and, for Q, over the query heads that
// share KV head g), computed in double and rounded once to fp32; s_j = 1 when
// either maximum is 0.  inv_s = fp32(1 / s).
void orc_calibrate(const uint16_t* q_cal, const uint16_t* k_cal, int64_t B, int64_t Hq,
                   int64_t Hkv, int64_t N, int64_t d, double alpha, float* s, float* inv_s) {
  const int64_t G = Hq / Hkv;
  for (int64_t g = 0; g < Hkv; g++) {
    for (int64_t j = 0; j < d; j++) {
      double qmax = 0.0, kmax = 0.0;
      for (int64_t b = 0; b < B; b++) {
        for (int64_t hh = g * G; hh < (g + 1) * G; hh++)
          for (int64_t n = 0; n < N; n++)
            qmax = std::max(qmax, std::fabs((double)f16_to_f32(q_cal[((b * Hq + hh) * N + n) * d + j])));
        for (int64_t n = 0; n < N; n++)
          kmax = std::max(kmax, std::fabs((double)f16_to_f32(k_cal[((b * Hkv + g) * N + n) * d + j])));
      }
      float sj = 1.0f;
      if (qmax > 0.0 && kmax > 0.0) sj = (float)(std::pow(kmax, alpha) / std::pow(qmax, 1.0 - alpha));
      s[g * d + j] = sj;
      inv_s[g * d + j] = (float)(1.0 / (double)sj);
    }
  }
}

// Q / K quantization along d after the optional Smooth-QK multiply
// x = fp32(x_f16 * mult_j), one MX block per 32 consecutive channels.
void orc_quantize_rows(const uint16_t* x, int64_t B, int64_t H, int64_t Hkv, int64_t N,
                       int64_t Npad, int64_t d, const float* mult, uint8_t* codes,
                       uint8_t* scales, int rule) {
  const int64_t G = (Hkv > 0 && H >= Hkv) ? H / Hkv : 1;
  std::vector<float> blk(32);
  std::vector<uint8_t> c(32);
  for (int64_t b = 0; b < B; b++)
    for (int64_t h = 0; h < H; h++) {
      const int64_t g = h / G;
      for (int64_t n = 0; n < Npad; n++) {
        uint8_t* crow = codes + ((b * H + h) * Npad + n) * (d / 2);
        uint8_t* srow = scales + ((b * H + h) * Npad + n) * (d / 32);
        if (n >= N) {
          std::memset(crow, 0, (size_t)(d / 2));
          std::memset(srow, 0, (size_t)(d / 32));
          continue;
        }
        const uint16_t* xr = x + ((b * H + h) * N + n) * d;
        for (int64_t blkno = 0; blkno < d / 32; blkno++) {
          for (int i = 0; i < 32; i++) {
            const int64_t j = blkno * 32 + i;
            float v = f16_to_f32(xr[j]);
            if (mult) v = v * mult[g * d + j];
            blk[i] = v;
          }
          mx_block(blk.data(), 32, c.data(), &srow[blkno], rule);
          for (int i = 0; i < 32; i++) put_nibble(crow, blkno * 32 + i, c[i]);
        }
      }
    }
}

// V quantization along tokens: one MX block per 32 consecutive token positions
// [32*beta, 32*beta + 32) of one channel; positions >= N count as 0.
void orc_quantize_v(const uint16_t* v, int64_t B, int64_t H, int64_t N, int64_t Npad, int64_t d,
                    uint8_t* codes, uint8_t* scales, int rule) {
  std::vector<float> blk(32);
  std::vector<uint8_t> c(32);
  for (int64_t b = 0; b < B; b++)
    for (int64_t h = 0; h < H; h++)
      for (int64_t j = 0; j < d; j++) {
        uint8_t* crow = codes + ((b * H + h) * d + j) * (Npad / 2);
        uint8_t* srow = scales + ((b * H + h) * d + j) * (Npad / 32);
        for (int64_t beta = 0; beta < Npad / 32; beta++) {
          for (int i = 0; i < 32; i++) {
            const int64_t n = beta * 32 + i;
            blk[i] = (n < N) ? f16_to_f32(v[((b * H + h) * N + n) * d + j]) : 0.0f;
          }
          mx_block(blk.data(), 32, c.data(), &srow[beta], rule);
          for (int i = 0; i < 32; i++) put_nibble(crow, beta * 32 + i, c[i]);
        }
      }
}

// RoPE of binary16 rows before Smooth-QK (the abstract places Smooth-QK after
// RoPE).  The pages do not define RoPE; the reading is the rotate-half form:
// channel j < d/2 pairs with j + d/2 and the pair turns by the angle whose
// cosine and sine the caller tabulates per absolute position p = pos0 + n:
//   r[j]       = fp32(x[j] * cos) - fp32(x[j + d/2] * sin)
//   r[j + d/2] = fp32(x[j + d/2] * cos) + fp32(x[j] * sin)
// each product and sum one fp32 rounding, and r stored as binary16 (the
// binary16 post-RoPE K that the row quantizer takes).
int orc_rope_f16(const uint16_t* x, int64_t B, int64_t H, int64_t N, int64_t d, int64_t pos0,
                 const float* cos_t, const float* sin_t, int64_t n_rope, uint16_t* out) {
  if (B < 0 || H < 0 || N < 0 || d <= 0 || d % 2 != 0 || pos0 < 0 || pos0 + N > n_rope)
    return -1;
  const int64_t half = d / 2;
  for (int64_t r = 0; r < B * H * N; r++) {
    const int64_t p = pos0 + r % N;
    const uint16_t* xr = x + r * d;
    uint16_t* o = out + r * d;
    for (int64_t j = 0; j < half; j++) {
      const float c = cos_t[p * half + j], s = sin_t[p * half + j];
      const float a = f16_to_f32(xr[j]), b = f16_to_f32(xr[j + half]);
      const float ac = a * c, bs = b * s, bc = b * c, as = a * s;
      o[j] = f16_rne(ac - bs);
      o[j + half] = f16_rne(bc + as);
    }
  }
  return 0;
}

int64_t orc_inexact_count(void) { return g_inexact.load(); }
void orc_reset_inexact(void) { g_inexact.store(0); }

// ---------------------------------------------------------------------------
// The attention forward, one query row at a time.
//
// Per row (b, h, i), KV head g = h / (Hq/Hkv), tiles of Bc = kv_tile keys in
// ascending order, keys valid when j < N_kv and (causal) j <= i + N_kv - N_q:
//   S_j    = fp32 of the exact dot product of the dequantized Q_hat row and K_hat row j
//   mt     = fp32(c * max_valid S_j),  c = fp32(log2(e) / sqrt(d))
//   m_new  = fp16(max(m, mt))                       (running max, log2 domain, FP16 state)
//   alpha  = fp32(2^(m - m_new))                    (0 while m = -inf)
//   t_j    = fma(S_j, c, -m_new);  P_j = fp32(2^t_j), results below 2^-126 taken as 0
//   P_hat  = per aligned 32-key block: e = clamp(floor(max_valid t) - 2, -127, 127),
//            P_hat_j = E2M1_rne(P_j * 2^-e) * 2^e   (no valid key: codes 0, e = -127)
//   rs     = sum P_hat_j (reorder = 1, P-Reordering) or sum P_j (reorder = 0)
//   l      = fp16(fp32(fp32(alpha * l) + rs))
//   O_c    = fp32(fp32(alpha * O_c) + fp32(sum_j P_hat_j * V_hat_jc))
//   out_c  = fp16(O_c / l)
// A tile with no valid key for the row changes nothing and is skipped.
// Split-KV (num_splits = C > 1): tiles are dealt to C chunks of ceil(T/C)
// consecutive tiles, each run from (m, l, O) = (-inf, 0, 0), then merged in
// chunk order: M = max m_k, w_k = fp32(2^(m_k - M)), L = sum fp32(w_k * l_k),
// A_c = sum fp32(w_k * O_kc) (fp32, in order), out = fp16(A_c / fp16(L)).
// ---------------------------------------------------------------------------
namespace {

struct RowCtx {
  const orc_attn_params* p;
  int64_t G, T, Tc;
  float c;  // log2(e) / sqrt(d) in fp32
};

struct UnitScratch {
  int64_t bg = -1;                // cached (b, g)
  std::vector<double> kd, vd;     // [N_kv][d] dequantized K_hat, V_hat
  std::vector<int> kexp;          // [N_kv][d/32] K block exponents (quantized mode)
};

void load_kv(const orc_attn_params* p, int64_t b, int64_t g, UnitScratch& u) {
  const int64_t key = b * p->Hkv + g;
  if (u.bg == key) return;
  const int64_t N = p->N_kv, d = p->d, Np = p->Npad_kv;
  u.kd.assign((size_t)(N * d), 0.0);
  u.vd.assign((size_t)(N * d), 0.0);
  u.kexp.assign((size_t)(N * (d / 32)), 0);
  for (int64_t n = 0; n < N; n++) {
    if (p->quantized) {
      const uint8_t* cr = p->k_codes + ((b * p->Hkv + g) * Np + n) * (d / 2);
      const uint8_t* sr = p->k_scales + ((b * p->Hkv + g) * Np + n) * (d / 32);
      for (int64_t j = 0; j < d; j++) u.kd[n * d + j] = mx_value(cr, sr, j);
      for (int64_t blk = 0; blk < d / 32; blk++) u.kexp[n * (d / 32) + blk] = (int)sr[blk] - 127;
    } else {
      const float* kr = p->k_f32 + ((b * p->Hkv + g) * N + n) * d;
      for (int64_t j = 0; j < d; j++) u.kd[n * d + j] = kr[j];
    }
  }
  for (int64_t j = 0; j < d; j++) {
    if (p->quantized) {
      const uint8_t* cr = p->v_codes + ((b * p->Hkv + g) * d + j) * (Np / 2);
      const uint8_t* sr = p->v_scales + ((b * p->Hkv + g) * d + j) * (Np / 32);
      for (int64_t n = 0; n < N; n++) u.vd[n * d + j] = mx_value(cr, sr, n);
    } else {
      for (int64_t n = 0; n < N; n++) u.vd[n * d + j] = p->v_f32[((b * p->Hkv + g) * N + n) * d + j];
    }
  }
  u.bg = key;
}

void run_row(const RowCtx& ctx, int64_t row, int64_t oi, UnitScratch& u) {
  // row: flat id (b*Hq + h)*N_q + i; oi: index of this row in the caller's output arrays
  const orc_attn_params* p = ctx.p;
  const int64_t d = p->d, Nq = p->N_q, Nkv = p->N_kv, Bc = p->kv_tile;
  const int64_t i = row % Nq, bh = row / Nq, h = bh % p->Hq, b = bh / p->Hq;
  const int64_t g = h / ctx.G;
  load_kv(p, b, g, u);
  const int sf16 = p->state_fp16;
  const float c = ctx.c;
  const float NEG_INF = -std::numeric_limits<float>::infinity();

  // dequantized query row
  std::vector<double> qd((size_t)d);
  std::vector<int> qexp((size_t)(d / 32), 0);
  if (p->quantized) {
    const uint8_t* cr = p->q_codes + ((b * p->Hq + h) * p->Npad_q + i) * (d / 2);
    const uint8_t* sr = p->q_scales + ((b * p->Hq + h) * p->Npad_q + i) * (d / 32);
    for (int64_t j = 0; j < d; j++) qd[j] = mx_value(cr, sr, j);
    for (int64_t blk = 0; blk < d / 32; blk++) qexp[blk] = (int)sr[blk] - 127;
  } else {
    const float* qr = p->q_f32 + ((b * p->Hq + h) * Nq + i) * d;
    for (int64_t j = 0; j < d; j++) qd[j] = qr[j];
  }
  const int64_t last = p->causal ? i + Nkv - Nq : Nkv - 1;  // last valid key

  const int64_t C = p->num_splits;
  std::vector<float> mk((size_t)C), lk((size_t)C), Ok((size_t)(C * d));
  std::vector<float> S((size_t)Bc), t((size_t)Bc), P((size_t)Bc), Ph((size_t)Bc);
  std::vector<double> acc((size_t)d);
  const int64_t nt_row = ctx.T;

  for (int64_t k = 0; k < C; k++) {
    float m = NEG_INF, l = 0.0f;
    float* O = &Ok[(size_t)(k * d)];
    for (int64_t j = 0; j < d; j++) O[j] = 0.0f;
    const int64_t t_end = std::min(ctx.T, (k + 1) * ctx.Tc);
    for (int64_t tile = k * ctx.Tc; tile < t_end; tile++) {
      const int64_t tB = tile * Bc, tE = std::min(tB + Bc, Nkv);
      const int64_t vE = std::min(tE, last + 1);  // valid keys: [tB, vE)
      if (vE <= tB) continue;                       // no valid key: exact no-op
      // S for valid keys
      float smax = NEG_INF;
      for (int64_t j = tB; j < vE; j++) {
        const float sj = score_f32(qd.data(), &u.kd[(size_t)(j * d)], d);
        if (p->quantized) {
          int lo = 1 << 30, hi = -(1 << 30);
          for (int64_t blk = 0; blk < d / 32; blk++) {
            const int e = qexp[blk] + u.kexp[j * (d / 32) + blk];
            lo = std::min(lo, e);
            hi = std::max(hi, e);
          }
          if (hi - lo > 37) g_inexact.fetch_add(1);
        }
        S[j - tB] = sj;
        smax = std::max(smax, S[j - tB]);
      }
      const float mt = c * smax;
      const float m_new = round_state(std::max(m, mt), sf16);
      const float alpha = (m == NEG_INF) ? 0.0f : (float)std::exp2((double)m - (double)m_new);
      for (int64_t j = tB; j < tE; j++) {
        const int64_t jj = j - tB;
        if (j < vE) {
          t[jj] = std::fma(S[jj], c, -m_new);
          float pv = (float)std::exp2((double)t[jj]);
          if (pv < FLT_MIN) pv = 0.0f;  // the FP32 exponential has no subnormal results
          P[jj] = pv;
        } else {
          t[jj] = NEG_INF;
          P[jj] = 0.0f;
        }
      }
      // P_hat per aligned 32-key block (tB is a multiple of 32)
      for (int64_t blk0 = tB; blk0 < tE; blk0 += 32) {
        const int64_t blk1 = std::min(blk0 + 32, tE);
        const int64_t v1 = std::min(blk1, vE);
        int e = -127;
        if (v1 > blk0) {
          float tmax = NEG_INF;
          for (int64_t j = blk0; j < v1; j++) tmax = std::max(tmax, t[j - tB]);
          e = phat_exponent(tmax, p->scale_rule);
        }
        for (int64_t j = blk0; j < blk1; j++) {
          const int64_t jj = j - tB;
          int code = 0;
          if (p->quantized) {
            code = (j < v1) ? e2m1_rne(std::ldexp((double)P[jj], -e)) : 0;
            Ph[jj] = (float)std::ldexp(e2m1_value(code), e);
          } else {
            Ph[jj] = P[jj];
          }
          if (p->phat_codes) put_nibble(p->phat_codes + oi * (p->Npad_kv / 2), j, code);
        }
        if (p->phat_scales) p->phat_scales[oi * (p->Npad_kv / 32) + blk0 / 32] = (uint8_t)(e + 127);
      }
      double sp = 0.0, sph = 0.0;
      for (int64_t j = tB; j < tE; j++) { sp += P[j - tB]; sph += Ph[j - tB]; }
      if (p->sum_p) p->sum_p[oi * nt_row + tile] = sp;
      if (p->sum_phat) p->sum_phat[oi * nt_row + tile] = sph;
      const float rs = p->reorder ? (float)sph : (float)sp;
      const float al = alpha * l;
      l = round_state(al + rs, sf16);
      for (int64_t x = 0; x < d; x++) acc[x] = 0.0;
      for (int64_t j = tB; j < vE; j++) {
        const double w = Ph[j - tB];
        const double* vr = &u.vd[(size_t)(j * d)];
        for (int64_t x = 0; x < d; x++) acc[x] += w * vr[x];
      }
      for (int64_t x = 0; x < d; x++) {
        const float ao = alpha * O[x];
        O[x] = ao + (float)acc[x];
      }
      m = m_new;
    }
    mk[k] = m;
    lk[k] = l;
  }

  float* outf = p->out_f32 ? p->out_f32 + oi * d : nullptr;
  uint16_t* outh = p->out_f16 ? p->out_f16 + oi * d : nullptr;
  float m_fin, l_fin;
  if (C == 1) {
    m_fin = mk[0];
    l_fin = lk[0];
    for (int64_t x = 0; x < d; x++) {
      const float o = Ok[x] / l_fin;
      if (outf) outf[x] = o;
      if (outh) outh[x] = f16_rne(o);
    }
  } else {
    float M = NEG_INF;
    for (int64_t k = 0; k < C; k++) M = std::max(M, mk[k]);
    std::vector<float> w((size_t)C);
    for (int64_t k = 0; k < C; k++)
      w[k] = (mk[k] == NEG_INF) ? 0.0f : (float)std::exp2((double)mk[k] - (double)M);
    float L = 0.0f;
    for (int64_t k = 0; k < C; k++) { const float wl = w[k] * lk[k]; L = L + wl; }
    const float lf = round_state(L, sf16);
    for (int64_t x = 0; x < d; x++) {
      float A = 0.0f;
      for (int64_t k = 0; k < C; k++) { const float wo = w[k] * Ok[(size_t)(k * d + x)]; A = A + wo; }
      const float o = A / lf;
      if (outf) outf[x] = o;
      if (outh) outh[x] = f16_rne(o);
    }
    m_fin = M;
    l_fin = lf;
  }
  if (p->m_out) p->m_out[oi] = m_fin;
  if (p->l_out) p->l_out[oi] = l_fin;
}

}  // namespace

int orc_attn(const orc_attn_params* p) {
  if (!p) return -1;
  if (p->B < 0 || p->Hq <= 0 || p->Hkv <= 0 || p->N_q < 0 || p->N_kv <= 0 || p->d <= 0) return -2;
  if (p->Hq % p->Hkv != 0 || p->d % 32 != 0) return -3;
  if (p->kv_tile <= 0 || p->kv_tile % 32 != 0 || p->num_splits < 1) return -4;
  if (p->causal && p->N_q > p->N_kv) return -5;
  if (p->Npad_kv < p->N_kv || p->Npad_kv % 32 != 0 || p->Npad_q < p->N_q) return -6;
  if (p->quantized && (!p->q_codes || !p->q_scales || !p->k_codes || !p->k_scales ||
                       !p->v_codes || !p->v_scales)) return -7;
  if (!p->quantized && (!p->q_f32 || !p->k_f32 || !p->v_f32)) return -7;
  RowCtx ctx;
  ctx.p = p;
  ctx.G = p->Hq / p->Hkv;
  ctx.T = (p->N_kv + p->kv_tile - 1) / p->kv_tile;
  ctx.Tc = (ctx.T + p->num_splits - 1) / p->num_splits;
  ctx.c = (float)(1.4426950408889634073599246810019 / std::sqrt((double)p->d));

  // Rows are visited grouped by (b, g) so that a work unit dequantizes one KV head once.
  const int64_t total = p->B * p->Hq * p->N_q;
  const int64_t n = p->rows ? p->n_rows : total;
  auto row_of = [&](int64_t oi) { return p->rows ? p->rows[oi] : oi; };
  for (int64_t oi = 0; oi < n; oi++)
    if (row_of(oi) < 0 || row_of(oi) >= total) return -8;
  auto group_of = [&](int64_t r) {
    const int64_t bh = r / p->N_q;
    return (bh / p->Hq) * p->Hkv + (bh % p->Hq) / ctx.G;
  };
  std::vector<int64_t> order((size_t)n);
  for (int64_t oi = 0; oi < n; oi++) order[(size_t)oi] = oi;
  std::stable_sort(order.begin(), order.end(),
                   [&](int64_t a, int64_t b2) { return group_of(row_of(a)) < group_of(row_of(b2)); });
  std::vector<std::pair<int64_t, int64_t>> units;  // [begin, end) into order
  for (size_t s0 = 0; s0 < order.size();) {
    size_t e = s0;
    const int64_t gk = group_of(row_of(order[s0]));
    while (e < order.size() && group_of(row_of(order[e])) == gk && e - s0 < 64) e++;
    units.emplace_back((int64_t)s0, (int64_t)e);
    s0 = e;
  }
  int threads = p->threads > 0 ? p->threads : (int)std::max(1u, std::thread::hardware_concurrency());
  threads = (int)std::min<int64_t>(threads, std::max<int64_t>(1, (int64_t)units.size()));
  std::vector<UnitScratch> scratch((size_t)threads);
  std::atomic<int> slot{0};
  std::atomic<int64_t> next{0};
  auto work = [&]() {
    UnitScratch& u = scratch[(size_t)slot.fetch_add(1)];
    for (;;) {
      const int64_t ui = next.fetch_add(1);
      if (ui >= (int64_t)units.size()) break;
      for (int64_t k = units[ui].first; k < units[ui].second; k++) {
        const int64_t oi = order[(size_t)k];
        run_row(ctx, row_of(oi), oi, u);
      }
    }
  };
  std::vector<std::thread> pool;
  for (int t = 1; t < threads; t++) pool.emplace_back(work);
  work();
  for (auto& th : pool) th.join();
  return 0;
}

// fp64 textbook attention on the binary16 inputs (the error reference).
int orc_attn_exact(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B, int64_t Hq,
                   int64_t Hkv, int64_t N_q, int64_t N_kv, int64_t d, int causal,
                   const int64_t* rows, int64_t n_rows, double* out, int threads) {
  if (Hq % Hkv != 0 || (causal && N_q > N_kv) || N_kv <= 0) return -1;
  const int64_t G = Hq / Hkv;
  const int64_t total = B * Hq * N_q;
  const int64_t n = rows ? n_rows : total;
  if (threads <= 0) threads = (int)std::max(1u, std::thread::hardware_concurrency());
  parallel_for(n, threads, [&](int64_t idx) {
    const int64_t row = rows ? rows[idx] : idx;
    const int64_t i = row % N_q, bh = row / N_q, h = bh % Hq, b = bh / Hq, g = h / G;
    const int64_t last = causal ? i + N_kv - N_q : N_kv - 1;
    const uint16_t* qr = q + row * d;
    std::vector<double> s((size_t)(last + 1));
    const double scale = 1.0 / std::sqrt((double)d);
    double mx = -INFINITY;
    for (int64_t j = 0; j <= last; j++) {
      const uint16_t* kr = k + ((b * Hkv + g) * N_kv + j) * d;
      double sum = 0.0;
      for (int64_t x = 0; x < d; x++) sum += (double)f16_to_f32(qr[x]) * (double)f16_to_f32(kr[x]);
      s[j] = sum * scale;
      mx = std::max(mx, s[j]);
    }
    double den = 0.0;
    for (int64_t j = 0; j <= last; j++) { s[j] = std::exp(s[j] - mx); den += s[j]; }
    double* o = out + idx * d;
    for (int64_t x = 0; x < d; x++) o[x] = 0.0;
    for (int64_t j = 0; j <= last; j++) {
      const uint16_t* vr = v + ((b * Hkv + g) * N_kv + j) * d;
      for (int64_t x = 0; x < d; x++) o[x] += s[j] * (double)f16_to_f32(vr[x]);
    }
    for (int64_t x = 0; x < d; x++) o[x] /= den;
  });
  return 0;
}

}  // extern "C"

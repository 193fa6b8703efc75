/*
 * CPU oracle for HiFA4's 4-bit FlashAttention forward: TEST INFRASTRUCTURE ONLY.
 *
 * This library defines, in plain and slow code, the numbers the GPU path must
 * reproduce.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load it; the product library never calls it, and the two share
 * no code, headers, tables or constants.
 *
 * Source: HiFA4 (arXiv 2607.04302), Abstract.  The abstract fixes the pieces:
 * QK^T and PV both run as 4-bit block-scaled GEMMs, the online-softmax state
 * (running max m, normalizer l) is kept in FP16, Smooth-QK is a static
 * per-channel rescale Q*s, K/s applied after RoPE, and P-Reordering sums the
 * normalizer from the same quantized P_hat that feeds the PV GEMM.  The
 * abstract names the HIF4 format without defining it; the 4-bit operands here
 * are MXFP4 (E2M1 elements, one E8M0 scale per 32 along the contraction
 * dimension), see the encoding functions below.
 *
 * Layouts (all row-major, little-endian nibbles: element 2i in the low nibble
 * of byte i):
 *   Q codes  [B][Hq ][Npad_q ][d/2]   scales [B][Hq ][Npad_q ][d/32]
 *   K codes  [B][Hkv][Npad_kv][d/2]   scales [B][Hkv][Npad_kv][d/32]
 *   V codes  [B][Hkv][d][Npad_kv/2]   scales [B][Hkv][d][Npad_kv/32]
 *   out      [B][Hq][N_q][d] binary16 bits
 * Query head h uses KV head h / (Hq/Hkv).
 *
 * Parity pins: every function is checked by tests against closed forms, the
 * format's hand table, fp64 textbook attention and invariants of the method;
 * the only unpinned quantities are those that need the pages' real traces.
 */
#ifndef HIFA4_ORACLE_H
#define HIFA4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* binary16 <-> binary32 (round to nearest even; subnormals kept). */
uint16_t orc_f16_from_f32(float x);
float orc_f32_from_f16(uint16_t h);

void orc_f16_from_f32_array(const float* x, int64_t n, uint16_t* out);
void orc_f32_from_f16_array(const uint16_t* h, int64_t n, float* out);

/* S for one query row and one key row (MX rows of d elements): fp32 of the
 * exact dot product of the dequantized values -- the score used by orc_attn. */
float orc_score(const uint8_t* q_codes, const uint8_t* q_scales, const uint8_t* k_codes,
                const uint8_t* k_scales, int64_t d);

/* E2M1 element: RNE to {0,.5,1,1.5,2,3,4,6}, saturating at 6, sign kept. */
int orc_e2m1_encode(float x);
float orc_e2m1_decode(int code);
/* Block exponent, clamped to [-127, 127], all-zero block -> -127.  rule 0 (OCP MX):
 * floor(log2 max|x|) - 2; rule 1 (no clipping): the smallest e with max|x| * 2^-e <= 6. */
int orc_mx_exponent(const float* x, int n, int rule);
/* Quantize n (<= 32) values into one MX block: codes[i] in 0..15, *scale = e + 127. */
void orc_mx_block(const float* x, int n, uint8_t* codes, uint8_t* scale, int rule);
/* Block exponent of P_hat from the block's largest t (P = 2^t): rule 0: floor(t_max) - 2;
 * rule 1: ceil(fp32(t_max - fp32(log2 1.5))) - 2; clamped to [-127, 127]. */
int orc_phat_exponent(float tmax, int rule);

/* Smooth-QK calibration: s[g][j] = kmax^alpha / qmax^(1-alpha), inv_s = 1/s (fp32). */
void orc_calibrate(const uint16_t* q_cal, const uint16_t* k_cal, int64_t B, int64_t Hq,
                   int64_t Hkv, int64_t N, int64_t d, double alpha, float* s, float* inv_s);

/* Row-wise (along d) quantization of Q or K, optional per-(KV head, channel)
 * multiplier mult[Hkv][d] applied as fp32(x * mult) (Q uses s, K uses inv_s).
 * H is the tensor's own head count; head h reads mult row h / (H / Hkv).
 * Padding rows N..Npad-1 are written as zero codes and scale byte 0.  rule: the
 * block-exponent rule of orc_mx_exponent. */
void orc_quantize_rows(const uint16_t* x, int64_t B, int64_t H, int64_t Hkv, int64_t N,
                       int64_t Npad, int64_t d, const float* mult, uint8_t* codes,
                       uint8_t* scales, int rule);
/* Token-wise (32 tokens per block) quantization of V into [B][H][d][Npad/2]. */
void orc_quantize_v(const uint16_t* v, int64_t B, int64_t H, int64_t N, int64_t Npad, int64_t d,
                    uint8_t* codes, uint8_t* scales, int rule);

/* RoPE (rotate-half: channel j < d/2 pairs with j + d/2) of binary16 rows
 * x [B][H][N][d] at positions pos0 .. pos0+N-1, tables cos/sin [n_rope][d/2]
 * fp32 (row = absolute position):
 *   out[j]       = f16(fp32(x[j] cos) - fp32(x[j+d/2] sin))
 *   out[j + d/2] = f16(fp32(x[j+d/2] cos) + fp32(x[j] sin))
 * Returns 0, or -1 for bad sizes (odd d, pos0 + N > n_rope). */
int orc_rope_f16(const uint16_t* x, int64_t B, int64_t H, int64_t N, int64_t d, int64_t pos0,
                 const float* cos_t, const float* sin_t, int64_t n_rope, uint16_t* out);

typedef struct {
  int64_t B, Hq, Hkv, N_q, N_kv, d;
  int64_t Npad_q, Npad_kv;  /* row counts of the padded Q and K/V layouts */
  int causal, reorder;
  int kv_tile;              /* Bc: keys per tile; the tile partition changes rounding */
  int num_splits;           /* 1 = single pass; C > 1 = split-KV chunks merged in order */
  int quantized;            /* 1: MXFP4 operands; 0: quant-off self-test mode */
  int state_fp16;           /* 1: m, l rounded to binary16; 0: fp32 state self-test mode */
  /* quantized operands (quantized == 1) */
  const uint8_t *q_codes, *q_scales, *k_codes, *k_scales, *v_codes, *v_scales;
  /* real operands (quantized == 0), [B][H][N][d] fp32 */
  const float *q_f32, *k_f32, *v_f32;
  /* outputs */
  uint16_t* out_f16;        /* [B][Hq][N_q][d] (only selected rows written) */
  float* out_f32;           /* optional: O/l before the final binary16 rounding */
  uint8_t *phat_codes, *phat_scales; /* optional P_hat dump [rows][Npad_kv/2], [rows][Npad_kv/32] */
  double *sum_p, *sum_phat; /* optional [rows][n_tiles]: per-tile sums of P and P_hat (NaN: no valid key) */
  float *m_out, *l_out;     /* optional [rows]: final state as floats */
  const int64_t* rows;      /* optional list of flat row ids (b*Hq + h)*N_q + i; NULL = all */
  int64_t n_rows;
  int threads;
  int scale_rule;           /* P_hat block exponent: 0 OCP, 1 no clipping (orc_phat_exponent) */
} orc_attn_params;

/* Returns 0 on success, negative on bad arguments. */
int orc_attn(const orc_attn_params* p);

/* fp64 textbook softmax(Q K^T / sqrt(d)) V on binary16 inputs, causal mask
 * aligned bottom-right.  Q [B][Hq][N_q][d], K/V [B][Hkv][N_kv][d]; out fp64. */
int orc_attn_exact(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B, int64_t Hq,
                   int64_t Hkv, int64_t N_q, int64_t N_kv, int64_t d, int causal,
                   const int64_t* rows, int64_t n_rows, double* out, int threads);

/* Number of S values whose fp64 dot product could have been inexact
 * (exponent spread of the terms above 37 bits) since the last reset. */
int64_t orc_inexact_count(void);
void orc_reset_inexact(void);

#ifdef __cplusplus
}
#endif
#endif

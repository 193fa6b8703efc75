/*
 * hifa4.h -- C ABI of the MI355X (gfx950) 4-bit FlashAttention forward.
 *
 * The operation is the attention operator of HiFA4 (arXiv 2607.04302,
 * "HiFA4: Training-Free 4-bit FlashAttention on Ascend HIF4 NPUs for LLM
 * Inference", Abstract): both QK^T and PV run as 4-bit block-scaled GEMMs, the
 * online-softmax state (running max m and normalizer l) is held in FP16,
 * Smooth-QK rescales Q and K per channel after RoPE with static calibrated
 * scales, and P-Reordering sums the normalizer from the same quantized P_hat
 * that feeds the PV GEMM.  The abstract names the HIF4 4-bit format without
 * defining it; this library uses MXFP4 instead: E2M1 elements (magnitudes 0,
 * 0.5, 1, 1.5, 2, 3, 4, 6, sign in bit 3) with one E8M0 power-of-two scale
 * 2^(k-127) per 32 elements along the contraction dimension.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers named *_f16, codes, scales, s, inv_s, out and workspace are
 *   DEVICE pointers (hipMalloc'd or equivalent) on the current HIP device.
 *   The caller owns every buffer; the library allocates, frees and retains
 *   nothing.  Its only state is the static device scratch of
 *   hifa4_attn_fwd_noalloc (below) and, per host thread, the address ranges of
 *   allocations it has already checked to be device memory (a device pointer
 *   inside one of them is accepted without another runtime query; freeing a
 *   buffer and passing its old address again is the caller's error).
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *   work is enqueued on it; only hifa4_calibrate_smooth synchronizes.
 * - Tensors are row-major.  Raw tensors are binary16, BHSD:
 *   Q [B][Hq][N_q][d], K and V [B][Hkv][N_kv][d].  Query head h reads KV head
 *   h / (Hq / Hkv).
 * - 4-bit layouts (element 2i in the low nibble of byte i; Npad = N rounded
 *   up to a multiple of HIFA4_TOKEN_PAD; padding is written as zero codes
 *   with scale byte 0):
 *     row layout (Q, K):   codes [B][H][Npad][d/2],  scales [B][H][Npad][d/32]
 *                          (blocks of 32 consecutive channels of one token)
 *     tiled token layout (V): codes [B][H][Npad/64][d][32], scales
 *                          [B][H][Npad/64][d][2]: blocks of 32 consecutive
 *                          tokens of one channel; per 64-token tile, each
 *                          channel's two blocks (32 code bytes, 2 scale bytes)
 *                          are contiguous, channel after channel.  Inside a
 *                          block the 32 tokens are stored in the MFMA operand
 *                          order: nibble k (k = k4..k0 in binary) holds token
 *                          (k3 k2 k4 k1 k0) of the block.
 * - Errors: argument checks run first, on the host, and touch no device:
 *   HIFA4_EINVAL (bad sizes, NULL where a buffer is required, misaligned
 *   pointers), HIFA4_EUNSUPPORTED (valid but not built: d not 64/128/256,
 *   kv_tile other than 64 or 128, split-KV with d = 256 and kv_tile 128).
 *   Then HIFA4_ENODEV if no HIP device is visible,
 *   HIFA4_EINVAL for a pointer that is not device memory, HIFA4_ENOSPACE for a
 *   too-small workspace, HIFA4_EHIP if a launch fails.  hifa4_last_error()
 *   returns a thread-local message for the last failing call.  No C++
 *   exception crosses this interface.
 */
#ifndef HIFA4_H
#define HIFA4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HIFA4_TOKEN_PAD 128
#define HIFA4_MAX_NKV 32768 /* l <= 1.5 * N_kv must stay below binary16's 65504 */
/*
 * Block-exponent rules of the 4-bit blocks (scale_rule arguments).  For a block
 * whose largest magnitude is a:
 *   HIFA4_SCALE_OCP    e = floor(log2 a) - 2 (the OCP MX rule; 2 is the exponent
 *                      of E2M1's largest value 6 = 1.5 * 2^2): a block whose
 *                      a * 2^-e lands in [6, 8) saturates its largest elements to 6;
 *   HIFA4_SCALE_NOCLIP the smallest e with a * 2^-e <= 6: nothing saturates.
 * Both clamped to [-127, 127]; an all-zero block gets -127.  For P_hat the rule is
 * applied to P = 2^t through t (t = S c - m, per 32-key block):
 *   OCP: e = floor(t_max) - 2;  NOCLIP: e = ceil(fp32(t_max - fp32(log2 1.5))) - 2.
 * The HiFA4 abstract names its HIF4 format without defining it; the rules are the
 * two readings of an MX-style scale choice, and NOCLIP is the ablation of the default.
 */
#define HIFA4_SCALE_OCP 0
#define HIFA4_SCALE_NOCLIP 1
/*
 * How P_hat's codes are made (phat_mode).  HiFA4's P-Reordering (Abstract) sums the
 * normalizer from P_hat, so with reorder = 1 only P_hat's codes are needed, not P:
 *   HIFA4_PHAT_EXP2     P = 2^t by the hardware exponential, then RNE to E2M1 at the
 *                       block's scale (the reference definition; the default);
 *   HIFA4_PHAT_EXPFREE  the E2M1 code of 2^(t - e) straight from the log-domain value:
 *                       exponent floor(t - e), mantissa from a cubic in the fraction
 *                       that equals 2^f - 1 exactly where 2^(t - e) crosses an E2M1
 *                       rounding boundary.  Same codes as HIFA4_PHAT_EXP2 except within
 *                       a few ulps of a boundary; needs reorder = 1 and the prefill
 *                       kernel (num_splits = 1, not a decode-shaped q_f16 call).
 */
#define HIFA4_PHAT_EXP2 0
#define HIFA4_PHAT_EXPFREE 1

/* Size of the static device scratch of hifa4_attn_fwd_noalloc (16 MiB per device). */
#define HIFA4_NOALLOC_SCRATCH_BYTES (16u << 20)

typedef enum {
  HIFA4_OK = 0,
  HIFA4_EINVAL = 1,
  HIFA4_EUNSUPPORTED = 2,
  HIFA4_ENODEV = 3,
  HIFA4_EHIP = 4,
  HIFA4_ENOSPACE = 5
} hifa4_status;

/* Version of this interface (major * 100 + minor). */
int hifa4_version(void);
const char* hifa4_status_str(hifa4_status s);
/* Message for the last non-OK status returned on this thread ("" if none). */
const char* hifa4_last_error(void);

/*
 * Bytes of one 4-bit tensor in the row layout (v_layout = 0, Q and K) or the
 * tiled token layout (v_layout = 1, V), for B x H x N tokens of d channels.
 * EINVAL for negative sizes or d not a multiple of 32.  Host only.
 */
hifa4_status hifa4_mx4_bytes(int v_layout, int64_t B, int64_t H, int64_t N, int64_t d,
                             size_t* code_bytes, size_t* scale_bytes);

/*
 * Smooth-QK calibration (HiFA4 Abstract: a calibration-static per-channel
 * equivalent rescale of Q and K after RoPE, with no online reduction at
 * inference).  The scale rule is SmoothQuant's migration with strength alpha:
 *   s[g][j]     = max|K_g,j|^alpha / max|Q_j|^(1 - alpha)
 *   inv_s[g][j] = fp32(1 / s[g][j])
 * with the maxima over all B x N_cal calibration tokens (for Q also over the
 * Hq/Hkv query heads that share KV head g) and s = 1 where either maximum is
 * 0.  The maxima are reduced on the device; s is finalized on the host in
 * double and rounded once to fp32, so the call synchronizes `stream`.
 * q_cal_f16 [B][Hq][N_cal][d], k_cal_f16 [B][Hkv][N_cal][d] binary16;
 * s_out, inv_s_out [Hkv][d] fp32 (device).  alpha in [0, 1].
 */
hifa4_status hifa4_calibrate_smooth(const void* q_cal_f16, const void* k_cal_f16, int64_t B,
                                    int64_t Hq, int64_t Hkv, int64_t N_cal, int64_t d,
                                    float alpha, float* s_out, float* inv_s_out, void* stream);

/*
 * Smooth-QK apply + 4-bit quantization (HiFA4 Abstract: Q*s and K/s after
 * RoPE, then 4-bit operands for both GEMMs).
 *   Q: x = fp32(q * s[g][j])      (smooth = 1) or fp32(q) (smooth = 0)
 *   K: x = fp32(k * inv_s[g][j])  (a multiply by the stored reciprocal)
 *   Each block of 32: e from the block's largest |x| by scale_rule
 *   (HIFA4_SCALE_OCP: clamp(floor(log2 max|x|) - 2, -127, 127); all-zero
 *   block: -127), scale byte e + 127, codes RNE_E2M1(x * 2^-e) with ties to
 *   the even code and saturation at +-6.
 *   V: no rescale; blocks of 32 consecutive tokens (token layout).
 * Any of q_f16 / k_f16 / v_f16 may be NULL to skip that tensor (its output
 * pointers are then ignored).  s and inv_s are [Hkv][d] fp32, ignored when
 * smooth = 0.  Codes/scales buffers must hold hifa4_mx4_bytes(...) bytes and
 * be 16-byte aligned.  scale_rule: HIFA4_SCALE_OCP or HIFA4_SCALE_NOCLIP (else
 * EINVAL).  Asynchronous.
 */
hifa4_status hifa4_quantize_qkv(const void* q_f16, const void* k_f16, const void* v_f16,
                                int64_t B, int64_t Hq, int64_t Hkv, int64_t N_q, int64_t N_kv,
                                int64_t d, int smooth, const float* s, const float* inv_s,
                                uint8_t* q_codes, uint8_t* q_scales, uint8_t* k_codes,
                                uint8_t* k_scales, uint8_t* v_codes, uint8_t* v_scales,
                                int scale_rule, void* stream);

/*
 * V_hat layout conversion: a pure re-arrangement of the 4-bit codes and E8M0
 * scale bytes of V_hat (the 4-bit operand of the PV GEMM, HiFA4 Abstract),
 * no value changes, for callers that hold or want V_hat in the canonical
 * token-blocked layout instead of the tiled one the attention kernels read.
 *   canonical: codes [B][H][d][Npad/2], token j of channel c in byte j/2
 *              (even token in the low nibble); scales [B][H][d][Npad/32],
 *              one per 32 consecutive tokens;
 *   tiled:     codes [B][H][Npad/64][d][32], scales [B][H][Npad/64][d][2]
 *              (what hifa4_quantize_qkv writes and hifa4_attn_fwd reads): per
 *              64-token tile and channel its two 32-token blocks, and in each
 *              block's 16 bytes nibble k (k4..k0 in binary) holds the block's
 *              token (k3 k2 k4 k1 k0).
 * Npad = N rounded up to HIFA4_TOKEN_PAD.  to_tiled = 1 converts canonical
 * -> tiled, 0 tiled -> canonical.  Each buffer holds hifa4_mx4_bytes(...)
 * bytes; all four are device pointers, 16-byte aligned, owned by the caller;
 * the outputs must not overlap the inputs.  EINVAL for a NULL or misaligned
 * buffer, negative sizes or d not in {64, 128, 256}; an empty tensor is a
 * no-op.  Asynchronous on `stream`.
 */
hifa4_status hifa4_v_layout(int to_tiled, const uint8_t* codes_in, const uint8_t* scales_in,
                            uint8_t* codes_out, uint8_t* scales_out, int64_t B, int64_t H,
                            int64_t N, int64_t d, void* stream);

/* Buffers of one attention call (all device pointers). */
typedef struct {
  /* Q: either 4-bit (row layout, from hifa4_quantize_qkv) ... */
  const uint8_t* q_codes;
  const uint8_t* q_scales;
  /* ... or raw binary16 [B][Hq][N_q][d], smoothed with `s` (when smooth = 1)
   * and quantized inside the kernel exactly as hifa4_quantize_qkv would
   * (any N_q with num_splits = 1; N_q * Hq/Hkv <= 32 with num_splits > 1). */
  const void* q_f16;
  const float* s;
  /* K row layout, V tiled token layout (from hifa4_quantize_qkv). */
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  /* Output [B][Hq][N_q][d] binary16. */
  void* out_f16;
  /* Scratch for split-KV partial states; hifa4_attn_workspace_bytes(). */
  void* workspace;
  size_t workspace_bytes;
  /* Keys per tile: 64 or 128 (the tile partition fixes the FP16 state's
   * rounding sequence); the split-KV path takes 128 only with d <= 128.
   * 0 selects the default, 64. */
  int kv_tile;
  /* Split-KV: 1 = one pass; C > 1 deals the ceil(N_kv/kv_tile) tiles to C
   * chunks of consecutive tiles, each run from (-inf, 0, 0) and merged in
   * chunk order with FP16 (m, l).  C > 1 requires N_q * Hq/Hkv <= 32.
   * With B * Hkv >= 128 the chunks of a KV head share one workgroup and
   * merge on chip (when their C * Hq/Hkv * N_q * (d + 2) fp32 partial states
   * fit in 64 KB of LDS); otherwise each chunk is a wavefront of its own and
   * the merge runs as a second kernel, so small batches want more chunks (one
   * 32768-token sequence: about 64). */
  int num_splits;
  /* Optional P_hat dump (NULL = off): codes [B][Hq][N_q][Npad_kv/2] and
   * scales [B][Hq][N_q][Npad_kv/32] of every tile a row visits; entries of
   * tiles a row never visits are left as the caller initialized them. */
  uint8_t* phat_codes;
  uint8_t* phat_scales;
  /* Token rows of the K/V layouts (a multiple of HIFA4_TOKEN_PAD, >= N_kv),
   * for a cache allocated larger than N_kv (hifa4_kv_append); 0 means
   * N_kv rounded up to HIFA4_TOKEN_PAD.  The P_hat dump rows use the same
   * count: [..][kv_capacity/2] and [..][kv_capacity/32]. */
  int64_t kv_capacity;
  /* Block-exponent rule of P_hat and of a Q quantized in the kernel (q_f16):
   * HIFA4_SCALE_OCP (0, the default of a zeroed struct) or HIFA4_SCALE_NOCLIP.
   * Pre-quantized Q_hat, K_hat and V_hat carry the rule they were quantized
   * with; a consistent call uses the same rule for all of them. */
  int scale_rule;
  /* HIFA4_PHAT_EXP2 (0, the default of a zeroed struct) or HIFA4_PHAT_EXPFREE. */
  int phat_mode;
} hifa4_attn_args;

/* Workspace bytes hifa4_attn_fwd needs for these sizes (0 when num_splits = 1). */
hifa4_status hifa4_attn_workspace_bytes(int64_t B, int64_t Hq, int64_t N_q, int64_t d,
                                        int num_splits, size_t* bytes);

/*
 * 4-bit FlashAttention forward (HiFA4 Abstract).  Per query row, over tiles
 * of kv_tile keys in ascending order (keys valid when j < N_kv and, if
 * causal, j <= i + N_kv - N_q):
 *   S      = Q_hat K_hat^T                          (4-bit GEMM, fp32 accumulation)
 *   m_new  = fp16(max(m, fp32(c * max S))),  c = fp32(log2(e) / sqrt(d))
 *   alpha  = 2^(m - m_new);   P = 2^(fma(S, c, -m_new))
 *   P_hat  = per 32 keys: e from max t by args->scale_rule (OCP: clamp(floor(max t)
 *            - 2, -127, 127)), E2M1_rne(P / 2^e) * 2^e
 *   reorder = 1 (P-Reordering): [O | l] = alpha * [O | l] + P_hat [V_hat | 1]
 *                                (the normalizer is a column of the PV GEMM)
 *   reorder = 0:                 O = alpha * O + P_hat V_hat,  l = alpha * l + sum P
 *   l      = fp16(l)
 *   out    = fp16(O / l)
 * `smooth` states whether Q_hat/K_hat carry the Smooth-QK scales; with q_f16
 * it makes the kernel multiply Q by s before quantizing.  d in {64, 128,
 * 256}; N_kv in [1, HIFA4_MAX_NKV]; causal requires N_q <= N_kv; N_q = 0 or
 * B = 0 is a successful no-op.  Asynchronous.
 */
hifa4_status hifa4_attn_fwd(int64_t B, int64_t Hq, int64_t Hkv, int64_t N_q, int64_t N_kv,
                            int64_t d, int causal, int smooth, int reorder,
                            const hifa4_attn_args* args, void* stream);

/*
 * The same operation as hifa4_attn_fwd for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, and harnesses that forbid
 * hipMalloc.  Arguments, layouts and results are those of hifa4_attn_fwd, except that
 * args->workspace and args->workspace_bytes are ignored: the split-KV partial states
 * (the only scratch any kernel here uses) go to a static device array of
 * HIFA4_NOALLOC_SCRATCH_BYTES bytes that the library holds on each device it runs on
 * until the process ends.  Calls needing more than that (hifa4_attn_workspace_bytes
 * above the limit) return HIFA4_ENOSPACE on the host, before any device work.  The call
 * allocates and frees nothing.  Every call on one device shares that device's array
 * and each call writes every partial state it later reads, so nothing needs clearing
 * between calls; but calls that overlap in time on one device (different streams, or
 * host threads) race on the array and must be serialized by the caller.
 */
hifa4_status hifa4_attn_fwd_noalloc(int64_t B, int64_t Hq, int64_t Hkv, int64_t N_q,
                                    int64_t N_kv, int64_t d, int causal, int smooth,
                                    int reorder, const hifa4_attn_args* args, void* stream);

/*
 * Decode-time KV-cache append (HiFA4 Abstract: Smooth-QK rescales K after
 * RoPE; both GEMMs take 4-bit operands).  Appends the T new tokens of every
 * (sequence, KV head) at positions pos .. pos+T-1 of a 4-bit cache with
 * kv_capacity token rows (a multiple of HIFA4_TOKEN_PAD, pos + T <=
 * kv_capacity), so that afterwards the cache holds, for positions
 * 0 .. pos+T-1, exactly what hifa4_quantize_qkv writes for the whole
 * post-RoPE sequence (row layout K, tiled token layout V):
 *   K: k_new_f16 [B][Hkv][T][d] binary16 before RoPE.  With tables
 *      (rope_cos, rope_sin [rope_rows][d/2] fp32, row = absolute position,
 *      rope_rows >= pos + T) each row is rotated rotate-half style, channel
 *      j < d/2 paired with j + d/2:
 *        r[j]       = fp32(k[j] cos) - fp32(k[j + d/2] sin)
 *        r[j + d/2] = fp32(k[j + d/2] cos) + fp32(k[j] sin)
 *      and rounded to binary16 (NULL tables: r = k, already rotated).  Then
 *      x = fp32(r * inv_s[g][j]) (smooth = 1) or r, and one MX block per 32
 *      channels into K rows pos .. pos+T-1.
 *   Every block exponent follows scale_rule (HIFA4_SCALE_OCP or HIFA4_SCALE_NOCLIP,
 *   else EINVAL), the same rule the rest of the cache was written with.
 *   V: v_new_f16 [B][Hkv][T][d].  Every 32-position block that the new tokens
 *      touch is quantized again from the binary16 values of all its tokens so
 *      far (positions after pos+T-1 count as 0).  The values of the block
 *      still filling are kept in v_stage_f16 [B][Hkv][32][d] binary16 (slot =
 *      position % 32), which the caller allocates and must not modify
 *      between appends.  Only this call fills it, and its contents matter
 *      for the positions of that block before pos: appends either start at
 *      a multiple of 32 (a fresh cache, pos = 0, needs no initialization)
 *      or continue a cache that earlier appends built.
 * Either k_new_f16 or v_new_f16 may be NULL to skip that tensor (its cache
 * pointers are then ignored).  Cache rows and blocks outside the touched
 * range are left untouched: a cache the decode step reads must hold zero
 * codes and scale bytes there (allocate it zeroed).  d in {64, 128, 256}.
 * Appends on one cache must be issued in position order on one stream.
 * Asynchronous.
 */
hifa4_status hifa4_kv_append(const void* k_new_f16, const void* v_new_f16, int64_t B,
                             int64_t Hkv, int64_t T, int64_t d, int64_t pos,
                             int64_t kv_capacity, const float* rope_cos, const float* rope_sin,
                             int64_t rope_rows, int smooth, const float* inv_s,
                             uint8_t* k_codes, uint8_t* k_scales, uint8_t* v_codes,
                             uint8_t* v_scales, void* v_stage_f16, int scale_rule, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* HIFA4_H */

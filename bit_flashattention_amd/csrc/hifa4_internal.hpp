// Internal declarations shared by the host side of the library (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hifa4 {

constexpr int64_t kTokenPad = 128;  // HIFA4_TOKEN_PAD
constexpr int kKvTile = 64;         // default keys per tile (two 32-key S^T MFMA column blocks)
constexpr int kRowsPerWave = 32;    // query rows (MFMA columns) per wavefront
constexpr int kWavesPerBlock = 4;

inline int64_t pad_tokens(int64_t n) { return (n + kTokenPad - 1) / kTokenPad * kTokenPad; }

hipError_t launch_calib_absmax(const void* q, const void* k, int64_t B, int64_t Hq, int64_t Hkv,
                               int64_t N, int64_t d, float* qmax, float* kmax,
                               hipStream_t stream);
// noclip: block-exponent rule of every 4-bit block written (0: OCP MX, 1: no clipping)
hipError_t launch_quant_rows(const void* x, const float* mult, int64_t B, int64_t H, int64_t Hkv,
                             int64_t N, int64_t d, uint8_t* codes, uint8_t* scales, int noclip,
                             hipStream_t stream);
hipError_t launch_quant_qkv(const void* q, const float* s, const void* k, const float* inv_s,
                            const void* v, int64_t B, int64_t Hq, int64_t Hkv, int64_t N_q,
                            int64_t N_kv, int64_t d, uint8_t* q_codes, uint8_t* q_scales,
                            uint8_t* k_codes, uint8_t* k_scales, uint8_t* v_codes,
                            uint8_t* v_scales, int noclip, hipStream_t stream);

// V_hat canonical <-> tiled layout (to_tiled = 1: canonical -> tiled)
hipError_t launch_v_layout(int to_tiled, const uint8_t* codes_in, const uint8_t* scales_in, uint8_t* codes_out,
                           uint8_t* scales_out, int64_t B, int64_t H, int64_t N, int64_t d, hipStream_t stream);

hipError_t launch_kv_append(const void* k, const void* v, int64_t B, int64_t Hkv, int64_t T,
                            int64_t d, int64_t pos, int64_t cap, const float* cos_t,
                            const float* sin_t, const float* inv_s, uint8_t* k_codes,
                            uint8_t* k_scales, uint8_t* v_codes, uint8_t* v_scales, void* stage,
                            int noclip, hipStream_t stream);

// Everything one attention launch needs (device pointers + sizes).
struct AttnLaunch {
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
  float* ws_o;   // [rows][C][d] fp32 split partial O
  float* ws_ml;  // [rows][C][2] split partial (m, l)
  int64_t B, Hq, Hkv, N_q, N_kv, d;
  int64_t Npad_q, Npad_kv;
  int causal, smooth, reorder, num_splits, kv_tile;
  int noclip;  // block-exponent rule of P_hat and of an in-kernel quantized Q (0: OCP, 1: no clipping)
  int phat_mode;  // P_hat from 2^t by v_exp_f32 (0) or exp-free from t (1; prefill, reorder = 1)
};

hipError_t launch_attn_prefill(const AttnLaunch& a, hipStream_t stream);
hipError_t launch_attn_split(const AttnLaunch& a, hipStream_t stream);

}  // namespace hifa4

// Smooth-QK calibration reduction and the Smooth-QK + 4-bit quantization pass.
//
// HiFA4 (arXiv 2607.04302), Abstract: Smooth-QK is a static per-channel
// rescale Q*s, K/s applied after RoPE; both attention GEMMs take 4-bit
// operands.  The 4-bit format is MXFP4 (E2M1 + one E8M0 scale per 32 along
// the contraction dimension): Q and K are blocked along channels, V along
// tokens.  These kernels are HBM-streaming: each reads binary16 once with
// 16-byte (Q/K) or 8-byte (V) coalesced loads and writes the codes once.
#include "hifa4_device.hpp"
#include "hifa4_internal.hpp"

namespace hifa4 {

// ---------------------------------------------------------------------------
// Calibration maxima: qmax[g][j] = max |Q| over (b, heads of group g, tokens),
// kmax[g][j] = max |K| over (b, tokens).  One thread per (g, j); the inner
// loop walks rows, so a wavefront reads contiguous channels of one row.
// ---------------------------------------------------------------------------
__global__ void calib_absmax_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                    int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                                    float* __restrict__ qmax, float* __restrict__ kmax) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= Hkv * d) return;
  const int64_t g = idx / d, j = idx % d, G = Hq / Hkv;
  float qm = 0.0f, km = 0.0f;
  for (int64_t b = 0; b < B; b++) {
    for (int64_t h = g * G; h < (g + 1) * G; h++) {
      const uint16_t* base = q + ((b * Hq + h) * N) * d + j;
      for (int64_t n = 0; n < N; n++) qm = fmaxf(qm, fabsf(half_to_float(base[n * d])));
    }
    const uint16_t* kb = k + ((b * Hkv + g) * N) * d + j;
    for (int64_t n = 0; n < N; n++) km = fmaxf(km, fabsf(half_to_float(kb[n * d])));
  }
  qmax[idx] = qm;
  kmax[idx] = km;
}

// ---------------------------------------------------------------------------
// Q / K along channels.  One thread per 8 channels of one token row; the four
// threads of an aligned quad form one 32-channel block.  Rows >= N of the
// padded layout are written as zero codes with scale byte 0.
//   x = fp32(x_f16 * mult[g][j])   (mult = s for Q, inv_s for K; NULL: none)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ mult, int64_t H, int64_t G,
    int64_t N, int64_t Npad, int64_t d, int64_t total_threads, uint32_t* __restrict__ codes,
    uint8_t* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total_threads) return;  // total_threads is a multiple of 4: quads stay whole
  const int64_t per_row = d / 8;
  const int64_t row = t / per_row, part = t % per_row;
  const int64_t bh = row / Npad, n = row % Npad;
  float v[8];
  if (n < N) {
    const uint4 raw = *reinterpret_cast<const uint4*>(x + ((bh * N + n) * d + part * 8));
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = half_to_float((uint16_t)(w[i] & 0xFFFFu));
      v[2 * i + 1] = half_to_float((uint16_t)(w[i] >> 16));
    }
    if (mult) {
      const int64_t g = (bh % H) / G;
      const float4* mp = reinterpret_cast<const float4*>(mult + g * d + part * 8);
      const float4 m0 = mp[0], m1 = mp[1];
      v[0] = v[0] * m0.x; v[1] = v[1] * m0.y; v[2] = v[2] * m0.z; v[3] = v[3] * m0.w;
      v[4] = v[4] * m1.x; v[5] = v[5] * m1.y; v[6] = v[6] * m1.z; v[7] = v[7] * m1.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(v[i]));
  amax = quad_max(amax);
  const int e = mx_exponent(amax);
  const uint32_t w = pack8_fp4(v, pow2f(e));
  codes[row * (d / 8) + part] = (n < N) ? w : 0u;
  if ((part & 3) == 0) scales[row * (d / 32) + part / 4] = (n < N) ? (uint8_t)(e + 127) : (uint8_t)0;
}

// ---------------------------------------------------------------------------
// V along tokens, written in the tiled token layout: for each 64-token tile,
// each channel's 32 code bytes (tokens 64t..64t+63, two 32-token blocks) are
// contiguous, channels one after another: codes [B][H][Npad/64][d][32],
// scales [B][H][Npad/64][d][2].  One thread per (4 channels, 32-token block):
// it reads the block's 32 token rows as 8-byte pieces (neighbouring threads
// read neighbouring channels of the same token, so loads coalesce) and writes
// one 16-byte code block + one scale byte per channel.  Tokens >= N count as 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_v_kernel(const uint16_t* __restrict__ v, int64_t N,
                                                      int64_t Npad, int64_t d,
                                                      int64_t total_threads,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total_threads) return;
  const int64_t groups = d / 4, nblk = Npad / 32;
  const int64_t cg = t % groups;
  const int64_t beta = (t / groups) % nblk;
  const int64_t bh = t / (groups * nblk);
  float x[4][32];
#pragma unroll
  for (int i = 0; i < 32; i++) {
    const int64_t n = beta * 32 + i;
    if (n < N) {
      const uint2 raw = *reinterpret_cast<const uint2*>(v + ((bh * N + n) * d + cg * 4));
      x[0][i] = half_to_float((uint16_t)(raw.x & 0xFFFFu));
      x[1][i] = half_to_float((uint16_t)(raw.x >> 16));
      x[2][i] = half_to_float((uint16_t)(raw.y & 0xFFFFu));
      x[3][i] = half_to_float((uint16_t)(raw.y >> 16));
    } else {
      x[0][i] = x[1][i] = x[2][i] = x[3][i] = 0.0f;
    }
  }
  const int64_t tile = bh * (Npad / 64) + beta / 2;
#pragma unroll
  for (int c = 0; c < 4; c++) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(x[c][i]));
    const int e = mx_exponent(amax);
    const float sc = pow2f(e);
    uint4 out;
    out.x = pack8_fp4(&x[c][0], sc);
    out.y = pack8_fp4(&x[c][8], sc);
    out.z = pack8_fp4(&x[c][16], sc);
    out.w = pack8_fp4(&x[c][24], sc);
    const int64_t ch = tile * d + cg * 4 + c;
    *reinterpret_cast<uint4*>(codes + ch * 32 + (beta % 2) * 16) = out;
    scales[ch * 2 + (beta % 2)] = (uint8_t)(e + 127);
  }
}

// ---------------------------------------------------------------------------
// Host launchers (called by the C ABI after validation).
// ---------------------------------------------------------------------------
hipError_t launch_calib_absmax(const void* q, const void* k, int64_t B, int64_t Hq, int64_t Hkv,
                               int64_t N, int64_t d, float* qmax, float* kmax,
                               hipStream_t stream) {
  const int64_t n = Hkv * d;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  calib_absmax_kernel<<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(
      (const uint16_t*)q, (const uint16_t*)k, B, Hq, Hkv, N, d, qmax, kmax);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const void* x, const float* mult, int64_t B, int64_t H, int64_t Hkv,
                             int64_t N, int64_t d, uint8_t* codes, uint8_t* scales,
                             hipStream_t stream) {
  const int64_t Npad = pad_tokens(N);
  const int64_t total = B * H * Npad * (d / 8);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  quant_rows_kernel<<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(
      (const uint16_t*)x, mult, H, H / Hkv, N, Npad, d, total, (uint32_t*)codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_v(const void* v, int64_t B, int64_t H, int64_t N, int64_t d,
                          uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t Npad = pad_tokens(N);
  const int64_t total = B * H * (Npad / 32) * (d / 4);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  quant_v_kernel<<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(
      (const uint16_t*)v, N, Npad, d, total, codes, scales);
  return hipGetLastError();
}

}  // namespace hifa4

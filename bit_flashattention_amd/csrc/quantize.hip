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
// Q / K along channels.  One thread per 32-channel block of one token row
// (64 bytes in, 16 code bytes + 1 scale byte out); consecutive threads cover
// consecutive blocks, so a wavefront reads 4 KB and writes 1 KB contiguously.
// Rows >= N of the padded layout are written as zero codes with scale byte 0.
//   x = fp32(x_f16 * mult[g][j])   (mult = s for Q, inv_s for K; NULL: none)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ mult, int64_t H, int64_t G,
    int64_t N, int64_t Npad, int64_t d, int64_t total_threads, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total_threads) return;
  const int64_t per_row = d / 32;
  const int64_t row = t / per_row, blk = t % per_row;
  const int64_t bh = row / Npad, n = row % Npad;
  u32x4 out = {0u, 0u, 0u, 0u};
  uint8_t sc = 0;
  if (n < N) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + ((bh * N + n) * d + blk * 32));
    float v[32];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const u32x4 raw = src[u];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        v[8 * u + 2 * i] = half_to_float((uint16_t)(raw[i] & 0xFFFFu));
        v[8 * u + 2 * i + 1] = half_to_float((uint16_t)(raw[i] >> 16));
      }
    }
    if (mult) {
      const float4* mp = reinterpret_cast<const float4*>(mult + ((bh % H) / G) * d + blk * 32);
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const float4 mm = mp[u];
        v[4 * u] = v[4 * u] * mm.x;
        v[4 * u + 1] = v[4 * u + 1] * mm.y;
        v[4 * u + 2] = v[4 * u + 2] * mm.z;
        v[4 * u + 3] = v[4 * u + 3] * mm.w;
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(v[i]));
    const int e = mx_exponent(amax);
    const float scale = pow2f(e);
#pragma unroll
    for (int w = 0; w < 4; w++) out[w] = pack8_fp4(&v[8 * w], scale);
    sc = (uint8_t)(e + 127);
  }
  *reinterpret_cast<u32x4*>(codes + row * (d / 2) + blk * 16) = out;
  scales[row * (d / 32) + blk] = sc;
}

// ---------------------------------------------------------------------------
// V along tokens, written in the tiled token layout: for each 64-token tile,
// each channel's 32 code bytes (tokens 64t..64t+63, two 32-token blocks) are
// contiguous, channels one after another: codes [B][H][Npad/64][d][32],
// scales [B][H][Npad/64][d][2].  Inside a 32-token block, nibble k holds
// token operand_key(k) (the PV product's operand order).  One workgroup per 64-token tile: it reads the
// tile's 64 token rows (64 x d binary16, coalesced 16-byte loads) into LDS,
// then each thread quantizes one (channel, 32-token block) from a column of
// the LDS tile and writes its 16 code bytes; the workgroup's writes are one
// contiguous range.  Tokens >= N count as 0.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void quant_v_kernel(const uint16_t* __restrict__ v, int64_t N,
                                                      int64_t Npad, uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  constexpr int ROW = D + 8;  // padded LDS row (binary16 elements): spreads column reads over banks
  __shared__ __attribute__((aligned(16))) uint16_t tile_lds[64 * ROW];
  const int64_t tiles = Npad / 64;
  const int64_t tile = blockIdx.x;  // (b*H + h) * tiles + tile index
  const int64_t bh = tile / tiles, t64 = tile % tiles;
  const int tid = threadIdx.x;
  // load 64 rows x D channels: D/8 16-byte pieces per row
  constexpr int PIECES = 64 * D / 8;
#pragma unroll
  for (int i = tid; i < PIECES; i += 256) {
    const int r = i / (D / 8), c8 = i % (D / 8);
    const int64_t n = t64 * 64 + r;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (n < N) val = *reinterpret_cast<const u32x4*>(v + (bh * N + n) * D + c8 * 8);
    *reinterpret_cast<u32x4*>(&tile_lds[r * ROW + c8 * 8]) = val;
  }
  __syncthreads();
  // (block, channel) pairs: 2 * D of them; a wavefront reads 64 consecutive
  // channels of one LDS row per step (no bank conflicts)
  for (int i = tid; i < 2 * D; i += 256) {
    const int blk = i / D, ch = i % D;
    float x[32];
#pragma unroll
    for (int k = 0; k < 32; k++) x[k] = half_to_float(tile_lds[(blk * 32 + operand_key(k)) * ROW + ch]);
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; k++) amax = fmaxf(amax, fabsf(x[k]));
    const int e = mx_exponent(amax);
    const float sc = pow2f(e);
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; w++) out[w] = pack8_fp4(&x[8 * w], sc);
    *reinterpret_cast<u32x4*>(codes + (tile * D + ch) * 32 + blk * 16) = out;
    scales[(tile * D + ch) * 2 + blk] = (uint8_t)(e + 127);
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
  const int64_t total = B * H * Npad * (d / 32);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  quant_rows_kernel<<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(
      (const uint16_t*)x, mult, H, H / Hkv, N, Npad, d, total, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_v(const void* v, int64_t B, int64_t H, int64_t N, int64_t d,
                          uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t Npad = pad_tokens(N);
  const int64_t tiles = B * H * (Npad / 64);
  if (tiles == 0) return hipSuccess;
  const dim3 grid((unsigned)tiles), block(256);
  const uint16_t* vv = (const uint16_t*)v;
  switch (d) {
    case 64: quant_v_kernel<64><<<grid, block, 0, stream>>>(vv, N, Npad, codes, scales); break;
    case 128: quant_v_kernel<128><<<grid, block, 0, stream>>>(vv, N, Npad, codes, scales); break;
    case 256: quant_v_kernel<256><<<grid, block, 0, stream>>>(vv, N, Npad, codes, scales); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hifa4

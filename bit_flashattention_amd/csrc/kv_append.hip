// Decode-time KV-cache append: RoPE, Smooth-QK and 4-bit quantization of new K
// tokens, and re-quantization of the 32-token V blocks that the new tokens touch.
//
// HiFA4 (arXiv 2607.04302), Abstract: Smooth-QK rescales K per channel after
// RoPE with a static calibrated scale, and both attention GEMMs take 4-bit
// operands.  A cache built by appending tokens therefore holds exactly the
// K_hat / V_hat that quantizing the whole post-RoPE sequence at once gives:
//   K: r = RoPE(k) (rotate-half, channel j < d/2 paired with j + d/2, caller
//      tables), stored as binary16, then x = fp32(r * inv_s[g][j]) and one MX
//      block per 32 channels of the token row;
//   V: one MX block per 32 consecutive positions of a channel.  A block that
//      is still filling is quantized from the binary16 values of its tokens so
//      far (later positions count as 0) and quantized again on every append
//      that adds to it; those values wait in a caller-owned staging buffer
//      [B][Hkv][32][d] until the block is full.
//
// Work split (grid = B*Hkv x chunks, 256 threads): the items are K blocks (one
// token row x 32 channels) and V blocks (one channel x 32 positions).  Only
// chunk 0 of a (b, g) reads the staging buffer (the first touched V block, whose
// older tokens sit there) and only chunk 0 writes it, after a barrier, so no
// other workgroup ever touches it.  HBM-bound; a one-token append is a few
// hundred bytes per (b, g) and is bounded by launch latency.
#include "hifa4_device.hpp"
#include "hifa4_internal.hpp"

namespace hifa4 {

struct AppendArgs {
  const uint16_t* k;      // [B][Hkv][T][d] binary16 before RoPE (NULL: no K)
  const uint16_t* v;      // [B][Hkv][T][d] binary16 (NULL: no V)
  const float* cos_t;     // [rows][d/2], row = absolute position (NULL: no RoPE)
  const float* sin_t;
  const float* inv_s;     // [Hkv][d] (NULL: no Smooth-QK)
  uint8_t* k_codes;       // row layout [B][Hkv][cap][d/2]
  uint8_t* k_scales;      //            [B][Hkv][cap][d/32]
  uint8_t* v_codes;       // tiled token layout [B][Hkv][cap/64][d][32]
  uint8_t* v_scales;      //                    [B][Hkv][cap/64][d][2]
  uint16_t* stage;        // [B][Hkv][32][d] binary16
  int64_t Hkv, T, pos, cap;
  int64_t n_k, n_v;       // K items (T * d/32) and V items after the first block
  int chunks;
};

__device__ __forceinline__ void load32_f16(const uint16_t* p, float (&x)[32]) {
  const u32x4* src = reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int u = 0; u < 4; u++) {
    const u32x4 raw = src[u];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      x[8 * u + 2 * i] = half_to_float((uint16_t)(raw[i] & 0xFFFFu));
      x[8 * u + 2 * i + 1] = half_to_float((uint16_t)(raw[i] >> 16));
    }
  }
}

__device__ __forceinline__ void load32_f32(const float* p, float (&x)[32]) {
  const float4* src = reinterpret_cast<const float4*>(p);
#pragma unroll
  for (int u = 0; u < 8; u++) {
    const float4 f = src[u];
    x[4 * u] = f.x;
    x[4 * u + 1] = f.y;
    x[4 * u + 2] = f.z;
    x[4 * u + 3] = f.w;
  }
}

// One MX block of 32 values: 16 code bytes (value i in nibble i) and the scale byte.
__device__ __forceinline__ void mx32(const float (&x)[32], u32x4& codes, uint8_t& scale) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(x[i]));
  const int e = mx_exponent(amax);
  const float sc = pow2f(e);
#pragma unroll
  for (int w = 0; w < 4; w++) codes[w] = pack8_fp4(&x[8 * w], sc);
  scale = (uint8_t)(e + 127);
}

// K: token t of the call, channels [32 blk, 32 blk + 32).
template <int D>
__device__ void append_k_block(const AppendArgs& a, int64_t bg, int64_t t, int blk) {
  constexpr int HALF = D / 2;
  const int64_t p = a.pos + t;
  const uint16_t* row = a.k + (bg * a.T + t) * D;
  const int j0 = 32 * blk;
  const bool lo = j0 < HALF;
  float x[32];
  load32_f16(row + j0, x);
  if (a.cos_t) {
    // rotate-half: r[j] = x[j] c - x[j + d/2] s (j < d/2), r[j] = x[j] c + x[j - d/2] s
    // (j >= d/2), each product and the sum one fp32 rounding, r kept as binary16
    const int jj = lo ? j0 : j0 - HALF;
    float y[32], c[32], s[32];
    load32_f16(row + (lo ? j0 + HALF : j0 - HALF), y);
    load32_f32(a.cos_t + p * HALF + jj, c);
    load32_f32(a.sin_t + p * HALF + jj, s);
#pragma unroll
    for (int i = 0; i < 32; i++) {
      const float xc = x[i] * c[i], ys = y[i] * s[i];
      x[i] = half_to_float(float_to_half_bits(lo ? xc - ys : xc + ys));
    }
  }
  if (a.inv_s) {
    float m[32];
    load32_f32(a.inv_s + (bg % a.Hkv) * D + j0, m);
#pragma unroll
    for (int i = 0; i < 32; i++) x[i] = x[i] * m[i];
  }
  u32x4 codes;
  uint8_t sc;
  mx32(x, codes, sc);
  *reinterpret_cast<u32x4*>(a.k_codes + (bg * a.cap + p) * (D / 2) + 16 * blk) = codes;
  a.k_scales[(bg * a.cap + p) * (D / 32) + blk] = sc;
}

// V: channel ch of the 32-position block beta, from the staging buffer (positions
// before the call), the new tokens, and zeros after them; written in the tiled
// token layout with nibble k holding position 32 beta + operand_key(k).
template <int D>
__device__ void append_v_block(const AppendArgs& a, int64_t bg, int64_t beta, int ch) {
  const int64_t end = a.pos + a.T;
  float x[32];
#pragma unroll
  for (int k = 0; k < 32; k++) {
    const int64_t n = 32 * beta + operand_key(k);
    uint16_t h = 0;
    if (n < a.pos)
      h = a.stage[(bg * 32 + (n & 31)) * D + ch];
    else if (n < end)
      h = a.v[(bg * a.T + (n - a.pos)) * D + ch];
    x[k] = half_to_float(h);
  }
  u32x4 codes;
  uint8_t sc;
  mx32(x, codes, sc);
  const int64_t tile = bg * (a.cap / 64) + beta / 2;
  *reinterpret_cast<u32x4*>(a.v_codes + (tile * D + ch) * 32 + 16 * (beta & 1)) = codes;
  a.v_scales[(tile * D + ch) * 2 + (beta & 1)] = sc;
}

template <int D>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const int64_t bg = blockIdx.x;
  const int chunk = blockIdx.y, tid = threadIdx.x;
  const int64_t beta0 = a.pos / 32;
  // K blocks and the V blocks after the first one, dealt over all chunks
  const int64_t stride = 256LL * a.chunks;
  for (int64_t i = (int64_t)chunk * 256 + tid; i < a.n_k + a.n_v; i += stride) {
    if (i < a.n_k)
      append_k_block<D>(a, bg, i / (D / 32), (int)(i % (D / 32)));
    else
      append_v_block<D>(a, bg, beta0 + 1 + (i - a.n_k) / D, (int)((i - a.n_k) % D));
  }
  if (chunk != 0 || !a.v) return;
  // the first touched V block (its older positions come from the staging buffer)
  for (int ch = tid; ch < D; ch += 256) append_v_block<D>(a, bg, beta0, ch);
  __syncthreads();  // every read of the staging buffer is done
  // keep the new tokens of the block that is still filling
  const int64_t end = a.pos + a.T;
  if (end % 32 == 0) return;
  const int64_t first = end / 32 * 32 > a.pos ? end / 32 * 32 : a.pos;
  const int64_t cnt = end - first;
  for (int64_t i = tid; i < cnt * D; i += 256) {
    const int64_t n = first + i / D;
    const int ch = (int)(i % D);
    a.stage[(bg * 32 + (n & 31)) * D + ch] = a.v[(bg * a.T + (n - a.pos)) * D + ch];
  }
}

hipError_t launch_kv_append(const void* k, const void* v, int64_t B, int64_t Hkv, int64_t T,
                            int64_t d, int64_t pos, int64_t cap, const float* cos_t,
                            const float* sin_t, const float* inv_s, uint8_t* k_codes,
                            uint8_t* k_scales, uint8_t* v_codes, uint8_t* v_scales, void* stage,
                            hipStream_t stream) {
  if (B == 0 || T == 0 || (!k && !v)) return hipSuccess;
  AppendArgs a;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.cos_t = cos_t;
  a.sin_t = sin_t;
  a.inv_s = inv_s;
  a.k_codes = k_codes;
  a.k_scales = k_scales;
  a.v_codes = v_codes;
  a.v_scales = v_scales;
  a.stage = (uint16_t*)stage;
  a.Hkv = Hkv;
  a.T = T;
  a.pos = pos;
  a.cap = cap;
  a.n_k = k ? T * (d / 32) : 0;
  a.n_v = v ? ((pos + T - 1) / 32 - pos / 32) * d : 0;
  // about four items per thread, at most 128 chunks per (b, g)
  const int64_t per_chunk = 4 * 256;
  int64_t chunks = (a.n_k + a.n_v + per_chunk - 1) / per_chunk;
  chunks = chunks < 1 ? 1 : (chunks > 128 ? 128 : chunks);
  a.chunks = (int)chunks;
  const dim3 grid((unsigned)(B * Hkv), (unsigned)chunks), block(256);
  switch (d) {
    case 64: kv_append_kernel<64><<<grid, block, 0, stream>>>(a); break;
    case 128: kv_append_kernel<128><<<grid, block, 0, stream>>>(a); break;
    default: kv_append_kernel<256><<<grid, block, 0, stream>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace hifa4

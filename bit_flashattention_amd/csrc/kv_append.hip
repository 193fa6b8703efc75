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
// Work split (grid = B*Hkv x (K chunks + V chunks), 256 threads): K octets
// (one token row x 8 channels of the first half and their 8 RoPE partners, one
// lane each, four lanes per MX block pair) are dealt over the K chunks;
// V is handled per 64-position tile, staged through LDS by a whole V-chunk
// workgroup.  Only V chunk 0 of a (b, g) reads the staging buffer (in the first
// touched tile, which holds the positions before the call) and only it writes
// the buffer, after that tile's last barrier, so no other workgroup touches
// it.  HBM-bound in bulk; a one-token append moves about 10 KB per (b, g) and
// is bounded by latency.
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
  int64_t n_k;            // K items: T * d/16 octets of RoPE channel pairs
  int chunks_k, chunks_v; // workgroups per (b, g) for K and for V
  int noclip;             // block-exponent rule (0: OCP, 1: no clipping)
};

// One MX block of 32 values: 16 code bytes (value i in nibble i) and the scale byte.
__device__ __forceinline__ void mx32(const float (&x)[32], u32x4& codes, uint8_t& scale, int noclip) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(x[i]));
  const int e = mx_exponent(amax, noclip);
  const float sc = pow2f(e);
#pragma unroll
  for (int w = 0; w < 4; w++) codes[w] = pack8_fp4(&x[8 * w], sc);
  scale = (uint8_t)(e + 127);
}

// K: token t of the call, lane octet o: channels [8o, 8o + 8) of the first
// half and their RoPE partners [d/2 + 8o, d/2 + 8o + 8).  The four lanes of an
// aligned quad (o = 4b' .. 4b' + 3) hold MX block b' and its partner block
// d/64 + b': each lane loads 16 contiguous bytes of each half (consecutive lanes
// read consecutive bytes), the block maxima are combined over the quad with
// DPP, and each lane writes its 4 code bytes of each block (lane 0 of the quad
// the scale bytes).  Every item of a quad has the same token, so a quad is
// either entirely in range or entirely out.
template <int D>
__device__ __forceinline__ void append_k_oct(const AppendArgs& a, int64_t bg, int64_t g, int64_t t, int o) {
  constexpr int HALF = D / 2;
  const int64_t p = a.pos + t;
  const uint16_t* src = a.k + (bg * a.T + t) * D;
  const int j0 = 8 * o;
  const u32x4 rl = *reinterpret_cast<const u32x4*>(src + j0);
  const u32x4 rh = *reinterpret_cast<const u32x4*>(src + HALF + j0);
  float lo[8], hi[8];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    lo[2 * i] = half_to_float((uint16_t)(rl[i] & 0xFFFFu));
    lo[2 * i + 1] = half_to_float((uint16_t)(rl[i] >> 16));
    hi[2 * i] = half_to_float((uint16_t)(rh[i] & 0xFFFFu));
    hi[2 * i + 1] = half_to_float((uint16_t)(rh[i] >> 16));
  }
  if (a.cos_t) {
    // rotate-half: r[j] = x[j] c - x[j + d/2] s, r[j + d/2] = x[j + d/2] c + x[j] s,
    // each product and each sum one fp32 rounding, r kept as binary16
    const float4* cp = reinterpret_cast<const float4*>(a.cos_t + p * HALF + j0);
    const float4* sp = reinterpret_cast<const float4*>(a.sin_t + p * HALF + j0);
    const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
    const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float ac = lo[i] * c[i], bs = hi[i] * sn[i], bc = hi[i] * c[i], as = lo[i] * sn[i];
      lo[i] = half_to_float(float_to_half_bits(ac - bs));
      hi[i] = half_to_float(float_to_half_bits(bc + as));
    }
  }
  if (a.inv_s) {
    const float4* mp = reinterpret_cast<const float4*>(a.inv_s + g * D + j0);
    const float4* mq = reinterpret_cast<const float4*>(a.inv_s + g * D + HALF + j0);
    const float4 m0 = mp[0], m1 = mp[1], n0 = mq[0], n1 = mq[1];
    const float ml[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    const float mh[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
#pragma unroll
    for (int i = 0; i < 8; i++) {
      lo[i] = lo[i] * ml[i];
      hi[i] = hi[i] * mh[i];
    }
  }
  float al = 0.0f, ah = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    al = fmaxf(al, fabsf(lo[i]));
    ah = fmaxf(ah, fabsf(hi[i]));
  }
  al = quad_max(al);
  ah = quad_max(ah);
  const int el = mx_exponent(al, a.noclip), eh = mx_exponent(ah, a.noclip);
  const int64_t row = bg * a.cap + p;
  const int blk = o / 4, q = o % 4;
  uint8_t* crow = a.k_codes + row * (D / 2);
  *reinterpret_cast<uint32_t*>(crow + 16 * blk + 4 * q) = pack8_fp4(lo, pow2f(el));
  *reinterpret_cast<uint32_t*>(crow + 16 * (blk + HALF / 32) + 4 * q) = pack8_fp4(hi, pow2f(eh));
  if (q == 0) {
    a.k_scales[row * (D / 32) + blk] = (uint8_t)(el + 127);
    a.k_scales[row * (D / 32) + blk + HALF / 32] = (uint8_t)(eh + 127);
  }
}

// V: the touched 32-position blocks of 64-position tile tau.  The workgroup
// stages their binary16 rows in LDS (16-byte loads from the staging buffer for
// positions before the call, from the new tokens, zeros after them), then each
// thread quantizes one (block, channel) column, with nibble k holding position
// 32 beta + operand_key(k), into the tiled token layout.  Ends with a barrier,
// so the LDS tile may be reused and every read of the staging buffer is done.
template <int D>
__device__ void append_v_tile(const AppendArgs& a, int64_t bg, int64_t tau, uint16_t* lds) {
  constexpr int ROW = D + 8;  // padded LDS row (binary16): column reads spread over banks
  const int tid = threadIdx.x;
  const int64_t end = a.pos + a.T;
  const int64_t b_first = a.pos / 32, b_last = (end - 1) / 32;
  const int64_t blo = 2 * tau > b_first ? 2 * tau : b_first;
  const int64_t bhi = 2 * tau + 1 < b_last ? 2 * tau + 1 : b_last;
  const int nblk = (int)(bhi - blo + 1);
  const int r0 = (int)(32 * blo - 64 * tau);
  for (int i = tid; i < 32 * nblk * (D / 8); i += 256) {
    const int r = r0 + i / (D / 8), c8 = i % (D / 8);
    const int64_t n = 64 * tau + r;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (n < a.pos)
      val = *reinterpret_cast<const u32x4*>(a.stage + (bg * 32 + (n & 31)) * D + c8 * 8);
    else if (n < end)
      val = *reinterpret_cast<const u32x4*>(a.v + (bg * a.T + (n - a.pos)) * D + c8 * 8);
    *reinterpret_cast<u32x4*>(&lds[r * ROW + c8 * 8]) = val;
  }
  __syncthreads();
  const int64_t tile = bg * (a.cap / 64) + tau;
  for (int i = tid; i < nblk * D; i += 256) {
    const int64_t beta = blo + i / D;
    const int ch = i % D, rb = (int)(32 * beta - 64 * tau);
    float x[32];
#pragma unroll
    for (int k = 0; k < 32; k++) x[k] = half_to_float(lds[(rb + operand_key(k)) * ROW + ch]);
    u32x4 codes;
    uint8_t sc;
    mx32(x, codes, sc, a.noclip);
    *reinterpret_cast<u32x4*>(a.v_codes + (tile * D + ch) * 32 + 16 * (beta & 1)) = codes;
    a.v_scales[(tile * D + ch) * 2 + (beta & 1)] = sc;
  }
  __syncthreads();
}

template <int D>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[64 * (D + 8)];
  const int64_t bg = blockIdx.x;
  const int tid = threadIdx.x;
  if ((int)blockIdx.y < a.chunks_k) {
    // K blocks, dealt over the K chunks
    const int64_t stride = 256LL * a.chunks_k, g = bg % a.Hkv;
    for (int64_t i = (int64_t)blockIdx.y * 256 + tid; i < a.n_k; i += stride)
      append_k_oct<D>(a, bg, g, i / (D / 16), (int)(i % (D / 16)));
    return;
  }
  // V tiles, dealt over the V chunks
  const int chunk = (int)blockIdx.y - a.chunks_k;
  const int64_t end = a.pos + a.T;
  const int64_t tau0 = a.pos / 64, tau1 = (end - 1) / 64;
  if (chunk == 0) {
    // the first touched tile: its older positions come from the staging buffer
    append_v_tile<D>(a, bg, tau0, lds);
    // every read of the staging buffer is done: keep the new tokens of the
    // block that is still filling.  When that block lies in the tile just
    // quantized, its rows are still in LDS (no second trip to memory).
    if (end % 32 != 0) {
      const int64_t first = end / 32 * 32 > a.pos ? end / 32 * 32 : a.pos;
      const bool in_lds = (end - 1) / 64 == tau0;
      for (int64_t i = tid; i < (end - first) * (D / 8); i += 256) {
        const int64_t n = first + i / (D / 8);
        const int c8 = (int)(i % (D / 8));
        const u32x4 val =
            in_lds ? *reinterpret_cast<const u32x4*>(&lds[(n - 64 * tau0) * (D + 8) + c8 * 8])
                   : *reinterpret_cast<const u32x4*>(a.v + (bg * a.T + (n - a.pos)) * D + c8 * 8);
        *reinterpret_cast<u32x4*>(a.stage + (bg * 32 + (n & 31)) * D + c8 * 8) = val;
      }
    }
  }
  for (int64_t tau = tau0 + 1 + chunk; tau <= tau1; tau += a.chunks_v) append_v_tile<D>(a, bg, tau, lds);
}

hipError_t launch_kv_append(const void* k, const void* v, int64_t B, int64_t Hkv, int64_t T,
                            int64_t d, int64_t pos, int64_t cap, const float* cos_t,
                            const float* sin_t, const float* inv_s, uint8_t* k_codes,
                            uint8_t* k_scales, uint8_t* v_codes, uint8_t* v_scales, void* stage,
                            int noclip, hipStream_t stream) {
  if (B == 0 || T == 0 || (!k && !v)) return hipSuccess;
  AppendArgs a;
  a.noclip = noclip;
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
  a.n_k = k ? T * (d / 16) : 0;
  // separate workgroups for K (one octet of RoPE channel pairs per thread) and
  // V (one 64-position tile each), so a short append's two round trips overlap;
  // at most 128 of each per (b, g)
  const int64_t tiles = v ? (pos + T - 1) / 64 - pos / 64 + 1 : 0;
  const int64_t ck = (a.n_k + 255) / 256;
  a.chunks_k = (int)(ck > 128 ? 128 : ck);
  a.chunks_v = (int)(tiles > 128 ? 128 : tiles);
  const dim3 grid((unsigned)(B * Hkv), (unsigned)(a.chunks_k + a.chunks_v)), block(256);
  switch (d) {
    case 64: kv_append_kernel<64><<<grid, block, 0, stream>>>(a); break;
    case 128: kv_append_kernel<128><<<grid, block, 0, stream>>>(a); break;
    default: kv_append_kernel<256><<<grid, block, 0, stream>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace hifa4

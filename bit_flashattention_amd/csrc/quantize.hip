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
// kmax[g][j] = max |K| over (b, tokens).  Grid (channel groups of 64, g, row
// chunks): lane l of a wavefront owns channel 64 x + l and the four wavefronts
// of a workgroup walk the chunk's rows (the group's Q rows, then its K rows)
// four apart, so every load is 128 contiguous bytes of one row.  The lanes'
// maxima are combined into qmax / kmax (zeroed beforehand) with an integer
// atomic max on the bit patterns: non-negative floats order as their bits, and
// a max is exact in any order.  fmaxf drops NaN inputs, as a sequential scan
// with fmaxf would.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void calib_absmax_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, int64_t B, int64_t Hq,
    int64_t Hkv, int64_t N, int64_t d, int rows_per_wg, float* __restrict__ qmax,
    float* __restrict__ kmax) {
  const int64_t j = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  const int64_t g = blockIdx.y, G = Hq / Hkv;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nq = B * G * N, nrows = nq + B * N;
  const int64_t r0 = (int64_t)blockIdx.z * rows_per_wg;
  if (j >= d) return;
  float qm = 0.0f, km = 0.0f;
#pragma unroll 4
  for (int i = wave; i < rows_per_wg; i += 4) {
    const int64_t r = r0 + i;
    if (r >= nrows) break;
    if (r < nq) {
      const int64_t b = r / (G * N), h = g * G + (r / N) % G, n = r % N;
      qm = fmaxf(qm, fabsf(half_to_float(q[((b * Hq + h) * N + n) * d + j])));
    } else {
      const int64_t rk = r - nq, b = rk / N, n = rk % N;
      km = fmaxf(km, fabsf(half_to_float(k[((b * Hkv + g) * N + n) * d + j])));
    }
  }
  if (qm > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(qmax + g * d + j), __float_as_uint(qm));
  if (km > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(kmax + g * d + j), __float_as_uint(km));
}

// ---------------------------------------------------------------------------
// Q / K along channels.  One thread per 32-channel block of one token row
// (64 bytes in, 16 code bytes + 1 scale byte out); consecutive threads cover
// consecutive blocks, so a wavefront reads 4 KB and writes 1 KB contiguously.
// Rows >= N of the padded layout are written as zero codes with scale byte 0.
//   x = fp32(x_f16 * mult[g][j])   (mult = s for Q, inv_s for K; NULL: none)
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void quant_row_block(const uint16_t* __restrict__ x, const float* __restrict__ mult,
                                                int64_t H, int64_t G, int64_t N, int64_t Npad, int64_t t,
                                                uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                int64_t d_rt, int noclip) {
  const int64_t d = D > 0 ? D : d_rt;
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
    const int e = mx_exponent(amax, noclip);
    const float scale = pow2f(e);
#pragma unroll
    for (int w = 0; w < 4; w++) out[w] = pack8_fp4(&v[8 * w], scale);
    sc = (uint8_t)(e + 127);
  }
  *reinterpret_cast<u32x4*>(codes + row * (d / 2) + blk * 16) = out;
  scales[row * (d / 32) + blk] = sc;
}

// The same quantization with four lanes per 32-channel block (d = 64, 128,
// 256): each lane loads 8 channels (16 bytes, so a wavefront reads 1 KB
// contiguous per instruction), the block max is combined over the lane quad
// with DPP, and each lane writes its 4 code bytes; lane 0 of the quad writes
// the scale byte.  A workgroup covers ROWS consecutive rows of one (b, h)
// (ROWS divides the 128-row padding unit, so no workgroup straddles two heads
// and no per-element division is needed); each thread takes NPT quad slots
// j * 256 + tid and issues all their loads before converting any.
template <int D, int NPT>
struct RowQuads {
  static constexpr int SLOTS_PER_ROW = 4 * (D / 32);
  static constexpr int ROWS = 256 * NPT / SLOTS_PER_ROW;
  static_assert(128 % ROWS == 0, "a workgroup's rows stay inside one head");
};

template <int D, int NPT>
__device__ __forceinline__ void quant_row_quads(const uint16_t* __restrict__ x, const float* __restrict__ mult,
                                                int64_t H, int64_t G, int64_t N, int64_t Npad, int64_t wg,
                                                uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                int noclip) {
  using RQ = RowQuads<D, NPT>;
  const int64_t wgs_per_head = Npad / RQ::ROWS;
  const int64_t bh = wg / wgs_per_head;  // uniform: one division per workgroup
  const int64_t n0 = (wg % wgs_per_head) * RQ::ROWS;
  const float* mrow = mult ? mult + ((bh % H) / G) * D : nullptr;
  const uint16_t* xh = x + bh * N * D;
  uint8_t* ch = codes + (bh * Npad + n0) * (D / 2);
  uint8_t* sh = scales + (bh * Npad + n0) * (D / 32);
  const int tid = threadIdx.x, q = tid & 3;
  u32x4 raw[NPT];
  float4 m0[NPT], m1[NPT];
#pragma unroll
  for (int j = 0; j < NPT; j++) {
    const int s = j * 256 + tid;
    const int r = s / RQ::SLOTS_PER_ROW, blk = (s / 4) % (D / 32);
    raw[j] = u32x4{0u, 0u, 0u, 0u};
    m0[j] = m1[j] = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
    if (n0 + r < N) {
      raw[j] = *reinterpret_cast<const u32x4*>(xh + (n0 + r) * D + blk * 32 + q * 8);
      if (mrow) {
        const float4* mp = reinterpret_cast<const float4*>(mrow + blk * 32 + q * 8);
        m0[j] = mp[0];
        m1[j] = mp[1];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NPT; j++) {
    const int s = j * 256 + tid;
    const int r = s / RQ::SLOTS_PER_ROW, blk = (s / 4) % (D / 32);
    const bool live = n0 + r < N;  // the same for the whole quad
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = half_to_float((uint16_t)(raw[j][i] & 0xFFFFu));
      v[2 * i + 1] = half_to_float((uint16_t)(raw[j][i] >> 16));
    }
    if (mrow) {
      v[0] = v[0] * m0[j].x; v[1] = v[1] * m0[j].y; v[2] = v[2] * m0[j].z; v[3] = v[3] * m0[j].w;
      v[4] = v[4] * m1[j].x; v[5] = v[5] * m1[j].y; v[6] = v[6] * m1[j].z; v[7] = v[7] * m1[j].w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(v[i]));
    amax = quad_max(amax);
    uint32_t out = 0u;
    uint8_t sc = 0;
    if (live) {
      const int e = mx_exponent(amax, noclip);
      out = pack8_fp4(v, pow2f(e));
      sc = (uint8_t)(e + 127);
    }
    *reinterpret_cast<uint32_t*>(ch + r * (D / 2) + blk * 16 + q * 4) = out;
    if (q == 0) sh[r * (D / 32) + blk] = sc;
  }
}

// Any d that is a multiple of 32 (the fused kernel below covers d = 64, 128, 256).
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ mult, int64_t H, int64_t G,
    int64_t N, int64_t Npad, int64_t d, int64_t total_threads, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, int noclip) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total_threads) return;
  quant_row_block<0>(x, mult, H, G, N, Npad, t, codes, scales, d, noclip);
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
__device__ __forceinline__ void quant_v_tile(const uint16_t* __restrict__ v, int64_t N, int64_t Npad,
                                             int64_t tile, uint16_t* tile_lds,
                                             uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                             int noclip) {
  constexpr int ROW = D + 8;  // padded LDS row (binary16 elements): spreads column reads over banks
  const int64_t tiles = Npad / 64;
  const int64_t bh = tile / tiles, t64 = tile % tiles;  // tile = (b*H + h) * tiles + tile index
  const int tid = threadIdx.x;
  // load 64 rows x D channels (D/8 16-byte pieces per row); every load is
  // issued before the first LDS store, so the tile costs one memory round
  // trip per thread, not one per piece
  constexpr int PER_THREAD = 64 * D / 8 / 256;
  u32x4 val[PER_THREAD];
#pragma unroll
  for (int k = 0; k < PER_THREAD; k++) {
    const int i = tid + 256 * k, r = i / (D / 8), c8 = i % (D / 8);
    const int64_t n = t64 * 64 + r;
    val[k] = u32x4{0u, 0u, 0u, 0u};
    if (n < N) val[k] = *reinterpret_cast<const u32x4*>(v + (bh * N + n) * D + c8 * 8);
  }
#pragma unroll
  for (int k = 0; k < PER_THREAD; k++) {
    const int i = tid + 256 * k, r = i / (D / 8), c8 = i % (D / 8);
    *reinterpret_cast<u32x4*>(&tile_lds[r * ROW + c8 * 8]) = val[k];
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
    const int e = mx_exponent(amax, noclip);
    const float sc = pow2f(e);
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; w++) out[w] = pack8_fp4(&x[8 * w], sc);
    *reinterpret_cast<u32x4*>(codes + (tile * D + ch) * 32 + blk * 16) = out;
    scales[(tile * D + ch) * 2 + blk] = (uint8_t)(e + 127);
  }
}

// ---------------------------------------------------------------------------
// Q, K and V of one call in a single launch (d = 64, 128, 256): the first
// blocks quantize one V tile each, the following ones Q rows, then K rows.
// One launch instead of three keeps the HBM stream going across the tensors.
// ---------------------------------------------------------------------------
constexpr int kQuadsPerThread = 4;  // quad slots per thread in the Q / K part

struct QuantArgs {
  const uint16_t* x[2];  // Q, K (NULL: none)
  const float* mult[2];  // s, inv_s (NULL: no Smooth-QK multiply)
  int64_t H[2], G[2], N[2], Npad[2];
  int64_t blocks[2];   // workgroups, each covering RowQuads::ROWS rows of one (b, h)
  uint8_t* codes[2];
  uint8_t* scales[2];
  const uint16_t* v;
  int64_t vN, vNpad, vtiles;
  uint8_t* vcodes;
  uint8_t* vscales;
  int noclip;  // block-exponent rule (0: OCP, 1: no clipping)
};

template <int D>
__global__ __launch_bounds__(256) void quant_qkv_kernel(QuantArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile_lds[64 * (D + 8)];
  int64_t b = blockIdx.x;
  // V tiles first: each is a load -> barrier -> transpose round trip, so they
  // start while the streaming Q / K blocks keep HBM busy
  if (b < a.vtiles) {
    quant_v_tile<D>(a.v, a.vN, a.vNpad, b, tile_lds, a.vcodes, a.vscales, a.noclip);
    return;
  }
  b -= a.vtiles;
#pragma unroll
  for (int i = 0; i < 2; i++) {
    if (b < a.blocks[i]) {
      quant_row_quads<D, kQuadsPerThread>(a.x[i], a.mult[i], a.H[i], a.G[i], a.N[i], a.Npad[i],
                                          b, a.codes[i], a.scales[i], a.noclip);
      return;
    }
    b -= a.blocks[i];
  }
}

// ---------------------------------------------------------------------------
// Host launchers (called by the C ABI after validation).
// ---------------------------------------------------------------------------
hipError_t launch_calib_absmax(const void* q, const void* k, int64_t B, int64_t Hq, int64_t Hkv,
                               int64_t N, int64_t d, float* qmax, float* kmax,
                               hipStream_t stream) {
  const int64_t n = Hkv * d;
  hipError_t e = hipMemsetAsync(qmax, 0, (size_t)n * sizeof(float), stream);
  if (e == hipSuccess) e = hipMemsetAsync(kmax, 0, (size_t)n * sizeof(float), stream);
  if (e != hipSuccess) return e;
  // Q rows then K rows of one group, 64 per workgroup (more when the grid's
  // z dimension would exceed its limit)
  const int64_t rows = B * (Hq / Hkv) * N + B * N;
  int64_t per_wg = 64;
  while ((rows + per_wg - 1) / per_wg > 65535) per_wg *= 2;
  const dim3 grid((unsigned)((d + 63) / 64), (unsigned)Hkv, (unsigned)((rows + per_wg - 1) / per_wg));
  calib_absmax_kernel<<<grid, dim3(256), 0, stream>>>((const uint16_t*)q, (const uint16_t*)k, B, Hq,
                                                      Hkv, N, d, (int)per_wg, qmax, kmax);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const void* x, const float* mult, int64_t B, int64_t H, int64_t Hkv,
                             int64_t N, int64_t d, uint8_t* codes, uint8_t* scales, int noclip,
                             hipStream_t stream) {
  const int64_t Npad = pad_tokens(N);
  const int64_t total = B * H * Npad * (d / 32);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  quant_rows_kernel<<<dim3((unsigned)blocks), dim3(threads), 0, stream>>>(
      (const uint16_t*)x, mult, H, H / Hkv, N, Npad, d, total, codes, scales, noclip);
  return hipGetLastError();
}

hipError_t launch_quant_qkv(const void* q, const float* s, const void* k, const float* inv_s,
                            const void* v, int64_t B, int64_t Hq, int64_t Hkv, int64_t N_q,
                            int64_t N_kv, int64_t d, uint8_t* q_codes, uint8_t* q_scales,
                            uint8_t* k_codes, uint8_t* k_scales, uint8_t* v_codes,
                            uint8_t* v_scales, int noclip, hipStream_t stream) {
  if (d != 64 && d != 128 && d != 256) {  // Q / K only (V needs one of these d)
    hipError_t e = hipSuccess;
    if (q) e = launch_quant_rows(q, s, B, Hq, Hkv, N_q, d, q_codes, q_scales, noclip, stream);
    if (e == hipSuccess && k)
      e = launch_quant_rows(k, inv_s, B, Hkv, Hkv, N_kv, d, k_codes, k_scales, noclip, stream);
    return e;
  }
  QuantArgs a;
  a.noclip = noclip;
  const void* xs[2] = {q, k};
  const float* ms[2] = {s, inv_s};
  const int64_t Hs[2] = {Hq, Hkv}, Ns[2] = {N_q, N_kv};
  uint8_t* cs[2] = {q_codes, k_codes};
  uint8_t* ss[2] = {q_scales, k_scales};
  for (int i = 0; i < 2; i++) {
    a.x[i] = (const uint16_t*)xs[i];
    a.mult[i] = ms[i];
    a.H[i] = Hs[i];
    a.G[i] = Hs[i] / Hkv;
    a.N[i] = Ns[i];
    a.Npad[i] = pad_tokens(Ns[i]);
    // workgroups of RowQuads<d, kQuadsPerThread>::ROWS rows: 256 * kQuadsPerThread
    // quad slots, 4 per 32-channel block
    const int64_t rows_per_wg = 256 * kQuadsPerThread / (4 * (d / 32));
    a.blocks[i] = xs[i] ? B * Hs[i] * (a.Npad[i] / rows_per_wg) : 0;
    a.codes[i] = cs[i];
    a.scales[i] = ss[i];
  }
  a.v = (const uint16_t*)v;
  a.vN = N_kv;
  a.vNpad = pad_tokens(N_kv);
  a.vcodes = v_codes;
  a.vscales = v_scales;
  a.vtiles = v ? B * Hkv * (a.vNpad / 64) : 0;
  const int64_t blocks = a.blocks[0] + a.blocks[1] + a.vtiles;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(256);
  switch (d) {
    case 64: quant_qkv_kernel<64><<<grid, block, 0, stream>>>(a); break;
    case 128: quant_qkv_kernel<128><<<grid, block, 0, stream>>>(a); break;
    default: quant_qkv_kernel<256><<<grid, block, 0, stream>>>(a); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// V_hat layout conversion between the canonical token-blocked layout (codes
// [BH][d][Npad/2], scales [BH][d][Npad/32]) and the tiled layout the kernels
// read (codes [BH][Npad/64][d][32], scales [BH][Npad/64][d][2], each 32-token
// block's nibbles in operand order: nibble k holds token (k3 k2 k4 k1 k0)).
// A pure re-arrangement: 16-bit groups of four nibbles move as a whole, since
// the order keeps bits 1..0 of the token in place.  Operand group G (nibbles
// 4G..4G+3) holds canonical group (G1 G0 G2) of the block.
// ---------------------------------------------------------------------------
namespace {

__device__ __forceinline__ uint4 canonical_to_operand(uint4 c) {
  return make_uint4((c.x & 0xFFFFu) | (c.y << 16), (c.z & 0xFFFFu) | (c.w << 16), (c.x >> 16) | (c.y & 0xFFFF0000u),
                    (c.z >> 16) | (c.w & 0xFFFF0000u));
}

__device__ __forceinline__ uint4 operand_to_canonical(uint4 o) {
  return make_uint4((o.x & 0xFFFFu) | (o.z << 16), (o.x >> 16) | (o.z & 0xFFFF0000u), (o.y & 0xFFFFu) | (o.w << 16),
                    (o.y >> 16) | (o.w & 0xFFFF0000u));
}

// One thread per (head, 64-token tile, channel): its two 32-token blocks (32
// code bytes) and their two scale bytes.  Channel fastest, so the tiled side
// is contiguous across a wavefront.
__global__ __launch_bounds__(256) void v_layout_kernel(int to_tiled, const uint8_t* __restrict__ ci,
                                                      const uint8_t* __restrict__ si, uint8_t* __restrict__ co,
                                                      uint8_t* __restrict__ so, int64_t BH, int64_t ntile, int d) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= BH * ntile * d) return;
  const int c = (int)(idx % d);
  const int64_t r = idx / d, t = r % ntile, bh = r / ntile;
  const int64_t tiled_c = ((bh * ntile + t) * d + c) * 32, tiled_s = ((bh * ntile + t) * d + c) * 2;
  const int64_t canon_c = (bh * d + c) * (ntile * 32) + t * 32, canon_s = (bh * d + c) * (ntile * 2) + t * 2;
  if (to_tiled) {
#pragma unroll
    for (int blk = 0; blk < 2; blk++) {
      const uint4 x = *reinterpret_cast<const uint4*>(ci + canon_c + 16 * blk);
      *reinterpret_cast<uint4*>(co + tiled_c + 16 * blk) = canonical_to_operand(x);
    }
    so[tiled_s] = si[canon_s];
    so[tiled_s + 1] = si[canon_s + 1];
  } else {
#pragma unroll
    for (int blk = 0; blk < 2; blk++) {
      const uint4 x = *reinterpret_cast<const uint4*>(ci + tiled_c + 16 * blk);
      *reinterpret_cast<uint4*>(co + canon_c + 16 * blk) = operand_to_canonical(x);
    }
    so[canon_s] = si[tiled_s];
    so[canon_s + 1] = si[tiled_s + 1];
  }
}

}  // namespace

hipError_t launch_v_layout(int to_tiled, const uint8_t* codes_in, const uint8_t* scales_in, uint8_t* codes_out,
                           uint8_t* scales_out, int64_t B, int64_t H, int64_t N, int64_t d, hipStream_t stream) {
  const int64_t ntile = pad_tokens(N) / 64, total = B * H * ntile * d;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;  // beyond one grid dimension
  v_layout_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      to_tiled, codes_in, scales_in, codes_out, scales_out, B * H, ntile, (int)d);
  return hipGetLastError();
}

}  // namespace hifa4

// Device helpers for the gfx950 4-bit attention kernels.
//
// Register layouts of the scaled FP4 MFMA used throughout
// (v_mfma_scale_f32_32x32x64_f8f6f4 with both formats = E2M1):
//   A (32 x 64):  lane l holds row l % 32, elements k = 32 * (l / 32) + [0, 32)
//                 as 16 bytes, element 2i in the low nibble of byte i; its
//                 E8M0 scale is one byte of a 32-bit register (byte = opsel).
//   B (64 x 32):  lane l holds column l % 32, the same k range and packing.
//   C/D (32 x 32, fp32, 16 registers): lane l, register r holds
//                 column l % 32, row 8 * (r / 4) + 4 * (l / 32) + r % 4.
// So a 4-bit row stored with its 32-element blocks contiguous loads straight
// into an operand: one 16-byte load per lane, one scale byte per lane.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hifa4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 bytes in 4 VGPRs

// Key order inside a 32-key operand block of P_hat (B operand of the PV
// product) and of V_hat (its A operand): nibble k of the block's 16 bytes holds
// key operand_key(k) of the block.  In binary, k = (k4 k3 k2 k1 k0) holds key
// (k3 k2 k4 k1 k0): the S^T accumulator gives lane half hf the keys whose bit 2
// is hf, and packing those first needs no per-element lane exchange.
__host__ __device__ constexpr int operand_key(int k) {
  return (((k >> 3) & 1) << 4) | (((k >> 2) & 1) << 3) | ((k >> 4) << 2) | (k & 3);
}

// One 32x32x64 E2M1 x E2M1 MFMA: acc += (A * 2^(sa-127)) (B * 2^(sb-127)),
// with the scale bytes taken from byte OPA of sa and byte OPB of sb.
template <int OPA, int OPB>
__device__ __forceinline__ v16f mfma_fp4(const uint4& a, int sa, const uint4& b, int sb, v16f acc) {
  v8i A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  v8i B = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc, 4, 4, OPA, sa, OPB, sb);
}

__device__ __forceinline__ v16f mfma_fp4_v(const u32x4& a, int sa, const u32x4& b, int sb, v16f acc) {
  v8i A = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  v8i B = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc, 4, 4, 0, sa, 0, sb);
}

typedef float v4f __attribute__((ext_vector_type(4)));

// One 16x16x128 E2M1 x E2M1 MFMA with A at scale 2^0: acc += A (B * 2^(sb-127)),
// the scale byte taken from byte 0 of sb.
__device__ __forceinline__ v4f mfma16_fp4_unit_a(const uint4& a, const uint4& b, int sb, v4f acc) {
  v8i A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  v8i B = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, acc, 4, 4, 0, 127, 0, sb);
}

__device__ __forceinline__ v16f zero16() {
  v16f z;
#pragma unroll
  for (int i = 0; i < 16; i++) z[i] = 0.0f;
  return z;
}

// Binary16 round-to-nearest-even of an fp32 value, returned as fp32.
__device__ __forceinline__ float round_f16(float x) { return (float)(_Float16)x; }

// v_exp_f32: 2^x, within 1 ulp, results below 2^-126 flushed to 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// MX block exponent from a block's largest magnitude (non-negative, finite),
// clamped to [-127, 127], with 0 and subnormals giving -127:
//   noclip = 0 (the OCP MX rule): floor(log2 a) - 2, read from the exponent
//     field (2 = emax of E2M1); a block whose a * 2^-e lands in [6, 8) saturates;
//   noclip = 1: the smallest e with a * 2^-e <= 6, i.e. one more than the OCP
//     exponent when a's mantissa exceeds 1.5 (6 = 1.5 * 2^2).
__device__ __forceinline__ int mx_exponent(float amax, int noclip) {
  const uint32_t bits = __float_as_uint(amax);
  const int ex = (int)((bits >> 23) & 0xFFu) - 127;
  const int e = ex - 2 + (noclip & (int)((bits & 0x7FFFFFu) > 0x400000u));
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^e as an fp32 value for e in [-127, 127] (2^-127 is subnormal; the
// converter below divides by it exactly).
__device__ __forceinline__ float pow2f(int e) { return __builtin_amdgcn_ldexpf(1.0f, e); }

// Exp-free stand-in for 2^u, for E2M1 rounding only: exponent from floor(u),
// mantissa 1 + r(f) from the fraction f = u - floor(u), where the cubic
// r(f) = f (a + f (b + g f)) equals 2^f - 1 at f = log2 1.25, log2 1.5 and
// log2 1.75 (and at 0).  Those are the fractions at which 2^u crosses an E2M1
// rounding boundary (0.25, 0.75, 1.25, 1.75, 2.5, 3.5 and 5 are 2^k times 1,
// 1.5, 1.25 or 1.75), and r is increasing, so RNE to E2M1 of the result gives
// the code of 2^u itself except within a few ulps of a boundary.  u must be
// finite and at least -126.
__device__ __forceinline__ float expcast_e2m1(float u) {
  constexpr float kA = 0.6950093980189241f, kB = 0.22919986977314274f, kG = 0.07502727831798092f;
  const float f = __builtin_amdgcn_fractf(u);
  const int k = (int)__builtin_floorf(u);
  const float m = __builtin_fmaf(f, __builtin_fmaf(f, __builtin_fmaf(f, kG, kB), kA), 1.0f);
  return __builtin_amdgcn_ldexpf(m, k);
}

// Two E2M1 codes RNE(a / scale), RNE(b / scale) (ties to even, saturating at
// +-6, sign kept) written into byte SEL of `old`: a in the low nibble.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, SEL);
}

// Eight values -> one dword of E2M1 codes (value i in nibble i).
__device__ __forceinline__ uint32_t pack8_fp4(const float* v, float scale) {
  uint32_t w = 0;
  w = cvt_fp4x2<0>(w, v[0], v[1], scale);
  w = cvt_fp4x2<1>(w, v[2], v[3], scale);
  w = cvt_fp4x2<2>(w, v[4], v[5], scale);
  w = cvt_fp4x2<3>(w, v[6], v[7], scale);
  return w;
}

// Lane exchange across the two 32-lane halves: for x, returns x of lane l ^ 32.
__device__ __forceinline__ float other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // r[0] = [x_lo | x_lo], r[1] = [x_hi | x_hi]; lane < 32 wants x_hi, lane >= 32 wants x_lo
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Max over the 4 lanes of an aligned quad (DPP quad permutes).
__device__ __forceinline__ float quad_max(float x) {
  float y = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x = fmaxf(x, y);
  y = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  return fmaxf(x, y);
}

__device__ __forceinline__ float half_to_float(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return (float)v;
}

__device__ __forceinline__ uint16_t float_to_half_bits(float x) {
  _Float16 v = (_Float16)x;
  uint16_t h;
  __builtin_memcpy(&h, &v, 2);
  return h;
}

}  // namespace hifa4

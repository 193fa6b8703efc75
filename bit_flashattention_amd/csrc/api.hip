// C ABI of the library (declared in include/hifa4.h): argument validation,
// kernel selection and launch on the caller's stream.  The operation is the
// HiFA4 attention operator (arXiv 2607.04302, Abstract); this file adds no
// arithmetic of its own except the host-side finalization of the Smooth-QK
// scales from the device-reduced maxima.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/hifa4.h"
#include "hifa4_internal.hpp"

namespace {

thread_local char g_err[512];

hifa4_status fail(hifa4_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

hifa4_status ok() {
  g_err[0] = '\0';
  return HIFA4_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Once a device has been seen the answer cannot change within the process.
std::atomic<bool> g_have_device{false};

hifa4_status check_device() {
  if (g_have_device.load(std::memory_order_relaxed)) return HIFA4_OK;
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess || n <= 0) return fail(HIFA4_ENODEV, "no HIP device visible");
  g_have_device.store(true, std::memory_order_relaxed);
  return HIFA4_OK;
}

// Allocation ranges this thread has already found to be device memory.  A pointer
// inside one of them needs no runtime query: the query takes a lock and a lookup in
// the runtime's allocation map, and an attention call checks up to a dozen buffers,
// most of them inside the same few allocations from one call to the next.  Host and
// unregistered pointers never enter the cache, so they are rejected on every call.
struct DevRange {
  uintptr_t lo, hi;
};
constexpr int kRangeCache = 16;
thread_local DevRange g_ranges[kRangeCache];
thread_local int g_next_range = 0;

bool cached_device(const void* p) {
  const uintptr_t a = (uintptr_t)p;
  for (int i = 0; i < kRangeCache; i++)
    if (a >= g_ranges[i].lo && a < g_ranges[i].hi) return true;
  return false;
}

// Device memory check for a caller buffer (NULL is accepted: callers check
// presence separately).  Host and unregistered pointers are rejected.
hifa4_status check_dev_ptr(const void* p, const char* name) {
  if (!p || cached_device(p)) return HIFA4_OK;
  hipPointerAttribute_t attr;
  memset(&attr, 0, sizeof(attr));
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of an unknown pointer
    return fail(HIFA4_EINVAL, "%s is not a device pointer", name);
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(HIFA4_EINVAL, "%s is not device memory", name);
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p) == hipSuccess && size > 0) {
    g_ranges[g_next_range] = DevRange{(uintptr_t)base, (uintptr_t)base + size};
    g_next_range = (g_next_range + 1) % kRangeCache;
  } else {
    (void)hipGetLastError();
  }
  return HIFA4_OK;
}

hifa4_status hip_fail(hipError_t e, const char* what) {
  return fail(HIFA4_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool supported_d(int64_t d) { return d == 64 || d == 128 || d == 256; }

// Scratch of hifa4_attn_fwd_noalloc: the split-KV partial states (fp32 O, then fp32
// (m, l) pairs) live in this array instead of a caller workspace.  Each device that
// runs the library holds its own copy until the process ends.  Host code never uses
// the array's name as an address: it takes the device address from
// hipGetSymbolAddress once per device and passes that to the kernels.
static __device__ __align__(256) unsigned char scratch[HIFA4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first call on
// that device), or an error status.
hifa4_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HIFA4_EHIP, "attn_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(HIFA4_EUNSUPPORTED, "attn_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(HIFA4_EHIP, "attn_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return HIFA4_OK;
}

}  // namespace

extern "C" {

int hifa4_version(void) { return 105; }

const char* hifa4_status_str(hifa4_status s) {
  switch (s) {
    case HIFA4_OK: return "ok";
    case HIFA4_EINVAL: return "invalid argument";
    case HIFA4_EUNSUPPORTED: return "unsupported configuration";
    case HIFA4_ENODEV: return "no HIP device";
    case HIFA4_EHIP: return "HIP error";
    case HIFA4_ENOSPACE: return "workspace too small";
  }
  return "unknown status";
}

const char* hifa4_last_error(void) { return g_err; }

hifa4_status hifa4_mx4_bytes(int v_layout, int64_t B, int64_t H, int64_t N, int64_t d,
                             size_t* code_bytes, size_t* scale_bytes) {
  if (B < 0 || H < 0 || N < 0 || d <= 0 || d % 32 != 0 || !code_bytes || !scale_bytes)
    return fail(HIFA4_EINVAL, "mx4_bytes: need B, H, N >= 0, d > 0 a multiple of 32, outputs");
  (void)v_layout;  // both layouts hold the same number of codes and scales
  const int64_t np = hifa4::pad_tokens(N);
  *code_bytes = (size_t)(B * H * np * (d / 2));
  *scale_bytes = (size_t)(B * H * np * (d / 32));
  return ok();
}

hifa4_status hifa4_v_layout(int to_tiled, const uint8_t* codes_in, const uint8_t* scales_in,
                            uint8_t* codes_out, uint8_t* scales_out, int64_t B, int64_t H,
                            int64_t N, int64_t d, void* stream) {
  if (!codes_in || !scales_in || !codes_out || !scales_out) return fail(HIFA4_EINVAL, "v_layout: NULL buffer");
  if (B < 0 || H < 0 || N < 0) return fail(HIFA4_EINVAL, "v_layout: negative size");
  if (!supported_d(d)) return fail(HIFA4_EINVAL, "v_layout: d must be 64, 128 or 256");
  if (!aligned(codes_in, 16) || !aligned(scales_in, 16) || !aligned(codes_out, 16) || !aligned(scales_out, 16))
    return fail(HIFA4_EINVAL, "v_layout: buffers must be 16-byte aligned");
  const int64_t np = hifa4::pad_tokens(N);
  const uintptr_t cb = (uintptr_t)(B * H * np * (d / 2)), sb = (uintptr_t)(B * H * np * (d / 32));
  const uintptr_t ci = (uintptr_t)codes_in, co = (uintptr_t)codes_out, si = (uintptr_t)scales_in,
                  so = (uintptr_t)scales_out;
  // [a, a + na) and [b, b + nb) share a byte
  auto overlap = [](uintptr_t a, uintptr_t na, uintptr_t b, uintptr_t nb) { return a < b + nb && b < a + na; };
  if (cb > 0 && (overlap(ci, cb, co, cb) || overlap(ci, cb, so, sb) || overlap(si, sb, co, cb) ||
                 overlap(si, sb, so, sb)))
    return fail(HIFA4_EINVAL, "v_layout: output overlaps input");
  if (B * H * N == 0) return ok();
  hifa4_status st = check_device();
  if (st) return st;
  if ((st = check_dev_ptr(codes_in, "codes_in")) || (st = check_dev_ptr(scales_in, "scales_in")) ||
      (st = check_dev_ptr(codes_out, "codes_out")) || (st = check_dev_ptr(scales_out, "scales_out")))
    return st;
  hipError_t e = hifa4::launch_v_layout(to_tiled ? 1 : 0, codes_in, scales_in, codes_out, scales_out, B, H, N,
                                        d, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "v_layout launch");
  return ok();
}

hifa4_status hifa4_calibrate_smooth(const void* q_cal_f16, const void* k_cal_f16, int64_t B,
                                    int64_t Hq, int64_t Hkv, int64_t N_cal, int64_t d,
                                    float alpha, float* s_out, float* inv_s_out, void* stream) {
  if (!q_cal_f16 || !k_cal_f16 || !s_out || !inv_s_out)
    return fail(HIFA4_EINVAL, "calibrate: NULL buffer");
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N_cal <= 0 || d <= 0 || Hq % Hkv != 0)
    return fail(HIFA4_EINVAL, "calibrate: need positive sizes and Hq %% Hkv == 0");
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return fail(HIFA4_EINVAL, "calibrate: alpha must be in [0, 1]");
  if (!aligned(s_out, 4) || !aligned(inv_s_out, 4)) return fail(HIFA4_EINVAL, "calibrate: misaligned output");
  hifa4_status st = check_device();
  if (st) return st;
  if ((st = check_dev_ptr(q_cal_f16, "q_cal")) || (st = check_dev_ptr(k_cal_f16, "k_cal")) ||
      (st = check_dev_ptr(s_out, "s_out")) || (st = check_dev_ptr(inv_s_out, "inv_s_out")))
    return st;
  hipStream_t hs = (hipStream_t)stream;
  // maxima land in the output buffers, are finalized on the host, then overwritten
  hipError_t e = hifa4::launch_calib_absmax(q_cal_f16, k_cal_f16, B, Hq, Hkv, N_cal, d, s_out,
                                            inv_s_out, hs);
  if (e != hipSuccess) return hip_fail(e, "calibrate launch");
  const size_t n = (size_t)(Hkv * d);
  std::vector<float> qmax(n), kmax(n), s(n), inv(n);
  if ((e = hipMemcpyAsync(qmax.data(), s_out, n * 4, hipMemcpyDeviceToHost, hs)) != hipSuccess ||
      (e = hipMemcpyAsync(kmax.data(), inv_s_out, n * 4, hipMemcpyDeviceToHost, hs)) != hipSuccess ||
      (e = hipStreamSynchronize(hs)) != hipSuccess)
    return hip_fail(e, "calibrate copy-out");
  for (size_t i = 0; i < n; i++) {
    float sj = 1.0f;
    if (qmax[i] > 0.0f && kmax[i] > 0.0f)
      sj = (float)(std::pow((double)kmax[i], (double)alpha) / std::pow((double)qmax[i], 1.0 - (double)alpha));
    s[i] = sj;
    inv[i] = (float)(1.0 / (double)sj);
  }
  if ((e = hipMemcpyAsync(s_out, s.data(), n * 4, hipMemcpyHostToDevice, hs)) != hipSuccess ||
      (e = hipMemcpyAsync(inv_s_out, inv.data(), n * 4, hipMemcpyHostToDevice, hs)) != hipSuccess ||
      (e = hipStreamSynchronize(hs)) != hipSuccess)
    return hip_fail(e, "calibrate copy-in");
  return ok();
}

hifa4_status hifa4_quantize_qkv(const void* q_f16, const void* k_f16, const void* v_f16,
                                int64_t B, int64_t Hq, int64_t Hkv, int64_t N_q, int64_t N_kv,
                                int64_t d, int smooth, const float* s, const float* inv_s,
                                uint8_t* q_codes, uint8_t* q_scales, uint8_t* k_codes,
                                uint8_t* k_scales, uint8_t* v_codes, uint8_t* v_scales,
                                int scale_rule, void* stream) {
  if (scale_rule != HIFA4_SCALE_OCP && scale_rule != HIFA4_SCALE_NOCLIP)
    return fail(HIFA4_EINVAL, "quantize: scale_rule must be HIFA4_SCALE_OCP or HIFA4_SCALE_NOCLIP");
  if (B < 0 || Hq <= 0 || Hkv <= 0 || N_q < 0 || N_kv < 0 || Hq % Hkv != 0)
    return fail(HIFA4_EINVAL, "quantize: need B, N >= 0, Hq, Hkv > 0, Hq %% Hkv == 0");
  if (d <= 0 || d % 32 != 0) return fail(HIFA4_EINVAL, "quantize: d must be a positive multiple of 32");
  if (v_f16 && d != 64 && d != 128 && d != 256)
    return fail(HIFA4_EUNSUPPORTED, "quantize: V needs d in {64, 128, 256}");
  if (smooth && ((q_f16 && !s) || (k_f16 && !inv_s)))
    return fail(HIFA4_EINVAL, "quantize: smooth = 1 needs s (for Q) and inv_s (for K)");
  if ((q_f16 && (!q_codes || !q_scales)) || (k_f16 && (!k_codes || !k_scales)) ||
      (v_f16 && (!v_codes || !v_scales)))
    return fail(HIFA4_EINVAL, "quantize: missing output buffer");
  const void* in[3] = {q_f16, k_f16, v_f16};
  for (int i = 0; i < 3; i++)
    if (in[i] && !aligned(in[i], 16)) return fail(HIFA4_EINVAL, "quantize: input not 16-byte aligned");
  if ((q_f16 && (!aligned(q_codes, 16) || !aligned(q_scales, 16))) ||
      (k_f16 && (!aligned(k_codes, 16) || !aligned(k_scales, 16))) ||
      (v_f16 && (!aligned(v_codes, 16) || !aligned(v_scales, 16))) ||
      (smooth && ((s && !aligned(s, 16)) || (inv_s && !aligned(inv_s, 16)))))
    return fail(HIFA4_EINVAL, "quantize: misaligned buffer");
  hifa4_status st = check_device();
  if (st) return st;
  const void* ptrs[] = {q_f16, k_f16, v_f16, q_codes, q_scales, k_codes, k_scales, v_codes, v_scales,
                        smooth ? s : nullptr, smooth ? inv_s : nullptr};
  const char* names[] = {"q", "k", "v", "q_codes", "q_scales", "k_codes", "k_scales", "v_codes",
                         "v_scales", "s", "inv_s"};
  for (int i = 0; i < 11; i++)
    if ((st = check_dev_ptr(ptrs[i], names[i]))) return st;
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e;
  if ((e = hifa4::launch_quant_qkv(q_f16, smooth ? s : nullptr, k_f16, smooth ? inv_s : nullptr,
                                   v_f16, B, Hq, Hkv, N_q, N_kv, d, q_codes, q_scales, k_codes,
                                   k_scales, v_codes, v_scales, scale_rule, hs)) != hipSuccess)
    return hip_fail(e, "quantize");
  return ok();
}

hifa4_status hifa4_attn_workspace_bytes(int64_t B, int64_t Hq, int64_t N_q, int64_t d,
                                        int num_splits, size_t* bytes) {
  if (!bytes || B < 0 || Hq < 0 || N_q < 0 || d <= 0 || num_splits < 1)
    return fail(HIFA4_EINVAL, "workspace_bytes: bad arguments");
  *bytes = num_splits > 1 ? (size_t)(B * Hq * N_q * num_splits * (d + 2)) * sizeof(float) : 0;
  return ok();
}

}  // extern "C"

// The attention call with its split-KV workspace given explicitly: the caller's
// (hifa4_attn_fwd) or the static scratch (hifa4_attn_fwd_noalloc, scratch = true).
static hifa4_status attn_fwd_impl(int64_t B, int64_t Hq, int64_t Hkv, int64_t N_q, int64_t N_kv,
                                  int64_t d, int causal, int smooth, int reorder,
                                  const hifa4_attn_args* a, bool use_scratch, void* stream) {
  if (!a) return fail(HIFA4_EINVAL, "attn: NULL args");
  if (B < 0 || N_q < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0)
    return fail(HIFA4_EINVAL, "attn: need B, N_q >= 0, Hq, Hkv > 0 and Hq %% Hkv == 0");
  if (N_kv < 1 || N_kv > HIFA4_MAX_NKV)
    return fail(HIFA4_EINVAL, "attn: N_kv must be in [1, %d]", HIFA4_MAX_NKV);
  if (causal && N_q > N_kv) return fail(HIFA4_EINVAL, "attn: causal needs N_q <= N_kv");
  if (d <= 0 || d % 32 != 0) return fail(HIFA4_EINVAL, "attn: d must be a positive multiple of 32");
  if (!supported_d(d)) return fail(HIFA4_EUNSUPPORTED, "attn: d = %lld not built (64, 128, 256)", (long long)d);
  if (B == 0 || N_q == 0) return ok();  // nothing to compute
  if (a->scale_rule != HIFA4_SCALE_OCP && a->scale_rule != HIFA4_SCALE_NOCLIP)
    return fail(HIFA4_EINVAL, "attn: scale_rule must be HIFA4_SCALE_OCP or HIFA4_SCALE_NOCLIP");
  if (a->phat_mode != HIFA4_PHAT_EXP2 && a->phat_mode != HIFA4_PHAT_EXPFREE)
    return fail(HIFA4_EINVAL, "attn: phat_mode must be HIFA4_PHAT_EXP2 or HIFA4_PHAT_EXPFREE");
  if (a->phat_mode == HIFA4_PHAT_EXPFREE && !reorder)
    return fail(HIFA4_EINVAL, "attn: HIFA4_PHAT_EXPFREE needs reorder = 1 (without it the row sum is of P itself)");
  const int kv_tile = a->kv_tile == 0 ? hifa4::kKvTile : a->kv_tile;
  if (kv_tile != 64 && kv_tile != 128) return fail(HIFA4_EUNSUPPORTED, "attn: kv_tile must be 64 or 128");
  if (a->num_splits < 1) return fail(HIFA4_EINVAL, "attn: num_splits must be >= 1");
  const bool q4 = a->q_codes || a->q_scales;
  if (q4 == (a->q_f16 != nullptr)) return fail(HIFA4_EINVAL, "attn: set exactly one of q codes/scales or q_f16");
  if (q4 && (!a->q_codes || !a->q_scales)) return fail(HIFA4_EINVAL, "attn: q codes and scales go together");
  if (a->q_f16 && smooth && !a->s) return fail(HIFA4_EINVAL, "attn: q_f16 with smooth = 1 needs s");
  if (!a->k_codes || !a->k_scales || !a->v_codes || !a->v_scales || !a->out_f16)
    return fail(HIFA4_EINVAL, "attn: missing K/V/out buffer");
  if ((a->phat_codes != nullptr) != (a->phat_scales != nullptr))
    return fail(HIFA4_EINVAL, "attn: phat codes and scales go together");
  const int64_t G = Hq / Hkv;
  if (a->num_splits > 1 && G * N_q > hifa4::kRowsPerWave)
    return fail(HIFA4_EUNSUPPORTED, "attn: split-KV needs N_q * Hq/Hkv <= 32");
  // decode-shaped calls (a few query rows per KV head) take the split-KV kernels,
  // the rest the prefill kernel; both quantize a raw binary16 Q themselves
  const bool split_path = a->num_splits > 1 || (a->q_f16 != nullptr && G * N_q <= hifa4::kRowsPerWave);
  if (split_path && kv_tile == 128 && d > 128)
    return fail(HIFA4_EUNSUPPORTED, "attn: split-KV with d = 256 needs kv_tile 64");
  if (split_path && a->phat_mode == HIFA4_PHAT_EXPFREE)
    return fail(HIFA4_EUNSUPPORTED, "attn: HIFA4_PHAT_EXPFREE is built for the prefill kernel only");
  if (!aligned(a->k_codes, 16) || !aligned(a->v_codes, 16) || !aligned(a->k_scales, 16) ||
      !aligned(a->v_scales, 16) ||
      (a->q_codes && (!aligned(a->q_codes, 16) || !aligned(a->q_scales, 8))) ||
      (a->q_f16 && !aligned(a->q_f16, 16)) || (a->s && !aligned(a->s, 16)) || !aligned(a->out_f16, 8) ||
      (a->phat_codes && !aligned(a->phat_codes, 16)) ||
      (!use_scratch && a->workspace && !aligned(a->workspace, 16)))
    return fail(HIFA4_EINVAL, "attn: misaligned buffer");
  const int64_t cap = a->kv_capacity ? a->kv_capacity : hifa4::pad_tokens(N_kv);
  if (cap < N_kv || cap % hifa4::kTokenPad != 0)
    return fail(HIFA4_EINVAL, "attn: kv_capacity must be a multiple of %d and >= N_kv",
                (int)hifa4::kTokenPad);
  size_t need = 0;
  hifa4_attn_workspace_bytes(B, Hq, N_q, d, a->num_splits, &need);
  if (use_scratch && need > (size_t)HIFA4_NOALLOC_SCRATCH_BYTES)
    return fail(HIFA4_ENOSPACE,
                "attn_noalloc: the split-KV partial states need %zu bytes, more than the %zu-byte "
                "static scratch (use fewer splits, or hifa4_attn_fwd with a workspace)",
                need, (size_t)HIFA4_NOALLOC_SCRATCH_BYTES);
  hifa4_status st = check_device();
  if (st) return st;
  const void* ptrs[] = {a->q_codes, a->q_scales, a->q_f16, a->s, a->k_codes, a->k_scales,
                        a->v_codes, a->v_scales, a->out_f16,
                        use_scratch ? nullptr : a->workspace, a->phat_codes, a->phat_scales};
  const char* names[] = {"q_codes", "q_scales", "q_f16", "s", "k_codes", "k_scales", "v_codes",
                         "v_scales", "out", "workspace", "phat_codes", "phat_scales"};
  for (int i = 0; i < 12; i++)
    if ((st = check_dev_ptr(ptrs[i], names[i]))) return st;
  void* ws = a->workspace;
  if (use_scratch) {
    ws = nullptr;
    if (need > 0 && (st = scratch_address(&ws))) return st;
  } else if (need > 0 && (!a->workspace || a->workspace_bytes < need)) {
    return fail(HIFA4_ENOSPACE, "attn: workspace needs %zu bytes", need);
  }

  hifa4::AttnLaunch L;
  L.q_codes = a->q_codes;
  L.q_scales = a->q_scales;
  L.q_f16 = (const uint16_t*)a->q_f16;
  L.s = a->s;
  L.k_codes = a->k_codes;
  L.k_scales = a->k_scales;
  L.v_codes = a->v_codes;
  L.v_scales = a->v_scales;
  L.out = (uint16_t*)a->out_f16;
  L.phat_codes = a->phat_codes;
  L.phat_scales = a->phat_scales;
  L.ws_o = (float*)ws;
  L.ws_ml = ws ? (float*)ws + B * Hq * N_q * a->num_splits * d : nullptr;
  L.B = B;
  L.Hq = Hq;
  L.Hkv = Hkv;
  L.N_q = N_q;
  L.N_kv = N_kv;
  L.d = d;
  L.Npad_q = hifa4::pad_tokens(N_q);
  L.Npad_kv = cap;
  L.causal = causal ? 1 : 0;
  L.smooth = smooth ? 1 : 0;
  L.reorder = reorder ? 1 : 0;
  L.num_splits = a->num_splits;
  L.kv_tile = kv_tile;
  L.noclip = a->scale_rule == HIFA4_SCALE_NOCLIP ? 1 : 0;
  L.phat_mode = a->phat_mode;
  hipError_t e;
  if (split_path) {
    e = hifa4::launch_attn_split(L, (hipStream_t)stream);
  } else {
    e = hifa4::launch_attn_prefill(L, (hipStream_t)stream);
  }
  if (e != hipSuccess) return hip_fail(e, "attn launch");
  return ok();
}

extern "C" {

hifa4_status hifa4_attn_fwd(int64_t B, int64_t Hq, int64_t Hkv, int64_t N_q, int64_t N_kv,
                            int64_t d, int causal, int smooth, int reorder,
                            const hifa4_attn_args* a, void* stream) {
  return attn_fwd_impl(B, Hq, Hkv, N_q, N_kv, d, causal, smooth, reorder, a, false, stream);
}

hifa4_status hifa4_attn_fwd_noalloc(int64_t B, int64_t Hq, int64_t Hkv, int64_t N_q, int64_t N_kv,
                                    int64_t d, int causal, int smooth, int reorder,
                                    const hifa4_attn_args* a, void* stream) {
  return attn_fwd_impl(B, Hq, Hkv, N_q, N_kv, d, causal, smooth, reorder, a, true, stream);
}

hifa4_status hifa4_kv_append(const void* k_new_f16, const void* v_new_f16, int64_t B,
                             int64_t Hkv, int64_t T, int64_t d, int64_t pos,
                             int64_t kv_capacity, const float* rope_cos, const float* rope_sin,
                             int64_t rope_rows, int smooth, const float* inv_s,
                             uint8_t* k_codes, uint8_t* k_scales, uint8_t* v_codes,
                             uint8_t* v_scales, void* v_stage_f16, int scale_rule, void* stream) {
  if (scale_rule != HIFA4_SCALE_OCP && scale_rule != HIFA4_SCALE_NOCLIP)
    return fail(HIFA4_EINVAL, "kv_append: scale_rule must be HIFA4_SCALE_OCP or HIFA4_SCALE_NOCLIP");
  if (B < 0 || Hkv <= 0 || T < 0 || pos < 0)
    return fail(HIFA4_EINVAL, "kv_append: need B, T, pos >= 0 and Hkv > 0");
  if (d <= 0 || d % 32 != 0) return fail(HIFA4_EINVAL, "kv_append: d must be a positive multiple of 32");
  if (!supported_d(d)) return fail(HIFA4_EUNSUPPORTED, "kv_append: d = %lld not built (64, 128, 256)", (long long)d);
  if (kv_capacity <= 0 || kv_capacity % hifa4::kTokenPad != 0 || pos + T > kv_capacity)
    return fail(HIFA4_EINVAL, "kv_append: kv_capacity must be a positive multiple of %d with pos + T <= kv_capacity",
                (int)hifa4::kTokenPad);
  if ((rope_cos != nullptr) != (rope_sin != nullptr))
    return fail(HIFA4_EINVAL, "kv_append: rope_cos and rope_sin go together");
  if (k_new_f16 && rope_cos && rope_rows < pos + T)
    return fail(HIFA4_EINVAL, "kv_append: the RoPE tables need at least pos + T rows");
  if (k_new_f16 && smooth && !inv_s) return fail(HIFA4_EINVAL, "kv_append: smooth = 1 needs inv_s");
  if ((k_new_f16 && (!k_codes || !k_scales)) || (v_new_f16 && (!v_codes || !v_scales || !v_stage_f16)))
    return fail(HIFA4_EINVAL, "kv_append: missing cache or staging buffer");
  const float* cs = k_new_f16 ? rope_cos : nullptr;
  const float* sn = k_new_f16 ? rope_sin : nullptr;
  const float* is = (k_new_f16 && smooth) ? inv_s : nullptr;
  const void* a16[] = {k_new_f16, v_new_f16, cs, sn, is, k_new_f16 ? k_codes : nullptr,
                       v_new_f16 ? v_codes : nullptr, v_new_f16 ? v_stage_f16 : nullptr};
  for (const void* p : a16)
    if (p && !aligned(p, 16)) return fail(HIFA4_EINVAL, "kv_append: misaligned buffer");
  if (B == 0 || T == 0 || (!k_new_f16 && !v_new_f16)) return ok();
  hifa4_status st = check_device();
  if (st) return st;
  const void* ptrs[] = {k_new_f16, v_new_f16, cs, sn, is,
                        k_new_f16 ? k_codes : nullptr, k_new_f16 ? k_scales : nullptr,
                        v_new_f16 ? v_codes : nullptr, v_new_f16 ? v_scales : nullptr,
                        v_new_f16 ? v_stage_f16 : nullptr};
  const char* names[] = {"k_new", "v_new", "rope_cos", "rope_sin", "inv_s", "k_codes",
                         "k_scales", "v_codes", "v_scales", "v_stage"};
  for (int i = 0; i < 10; i++)
    if ((st = check_dev_ptr(ptrs[i], names[i]))) return st;
  hipError_t e = hifa4::launch_kv_append(k_new_f16, v_new_f16, B, Hkv, T, d, pos, kv_capacity,
                                         cs, sn, is, k_codes, k_scales, v_codes, v_scales,
                                         v_new_f16 ? v_stage_f16 : nullptr,
                                         scale_rule == HIFA4_SCALE_NOCLIP ? 1 : 0, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv_append launch");
  return ok();
}

}  // extern "C"

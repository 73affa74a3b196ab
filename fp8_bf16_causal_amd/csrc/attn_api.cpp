// attn_api.cpp -- the C ABI of libfp8_bf16_causal.so: host-side argument
// checks, device check, parameter folding and kernel dispatch. The contract
// (layout, ownership, error codes) is documented in include/fp8_bf16_causal.h.
#include "fp8_bf16_causal.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "attn_params.h"
#include "attn_launch.h"

namespace {

constexpr double kLog2e = 1.4426950408889634;
constexpr int kMaxDevices = 64;
// 0 = not yet checked, 1 = gfx950, 2 = another architecture
std::atomic<int> g_arch_state[kMaxDevices];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  int st = g_arch_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_LAUNCH;
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? ATTN_OK : ATTN_ERR_UNSUPPORTED;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool finite_positive(float x) { return std::isfinite(x) && x > 0.0f; }

}  // namespace

// Sq query rows (the last Sq positions) over Sk >= Sq key rows.
static int attn_fwd_impl(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
                         int Hkv, int Sq, int Sk, int Dqk, int Dv, int causal, float scale, int dtype,
                         const float* descale_qkv, void* stream, unsigned flags) {
  const int S = Sq;
  // ---- ATTN_ERR_INVALID: malformed arguments
  if (!q || !k || !v || !out) return ATTN_ERR_INVALID;
  if (lse && ((uintptr_t)lse & 3u)) return ATTN_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_ERR_INVALID;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || S <= 0 || Sk < S || Dqk <= 0 || Dv <= 0) return ATTN_ERR_INVALID;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID;
  if (!std::isfinite(scale) || scale < 0.0f) return ATTN_ERR_INVALID;
  const unsigned known = ATTN_FLAG_EXACT_P | ATTN_FLAG_NO_BLOCKSCALE | ATTN_FLAG_DESCALE_DEVICE;
  if ((flags & ~known) != 0u) return ATTN_ERR_INVALID;
  // device-resident factors are read by the kernels; host ones here
  const bool dev_descale = (flags & ATTN_FLAG_DESCALE_DEVICE) != 0u;
  float dq = 1.0f, dk = 1.0f, dv = 1.0f;
  if (dev_descale) {
    if (!descale_qkv || ((uintptr_t)descale_qkv & 3u)) return ATTN_ERR_INVALID;
  } else if (descale_qkv) {
    dq = descale_qkv[0];
    dk = descale_qkv[1];
    dv = descale_qkv[2];
    if (!finite_positive(dq) || !finite_positive(dk) || !finite_positive(dv)) return ATTN_ERR_INVALID;
  }
  // the base-2 score scale the kernels use, scale dq dk log2(e), must be a
  // finite float (for device factors only the host part can be checked)
  const double cd = (double)scale * dq * dk * kLog2e;
  if (!(cd <= 3.4e38)) return ATTN_ERR_INVALID;
  // element counts of the largest tensor, whole and per batch entry, checked
  // step by step so that no product itself overflows; the kernels address one
  // batch entry with 32-bit byte offsets (2 bytes per element at most)
  const int64_t dmax = Dqk > Dv ? Dqk : Dv;
  int64_t per_batch = 0, whole = 0;
  if (__builtin_mul_overflow((int64_t)Sk, (int64_t)(Hq > Hkv ? Hq : Hkv), &per_batch) ||
      __builtin_mul_overflow(per_batch, dmax * 2, &per_batch) || __builtin_mul_overflow(per_batch, (int64_t)B, &whole))
    return ATTN_ERR_INVALID;
  if (per_batch >= (INT64_C(1) << 32)) return ATTN_ERR_INVALID;
  const int64_t nqb = ((int64_t)S + fbc::kBQ - 1) / fbc::kBQ;
  const int64_t grid = (int64_t)B * Hq * nqb;
  if (grid > 0x7fffffff) return ATTN_ERR_INVALID;

  // ---- ATTN_ERR_UNSUPPORTED: outside what the library implements
  if (causal != 1) return ATTN_ERR_UNSUPPORTED;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
  if (!((Dqk == 128 && Dv == 128) || (Dqk == 192 && Dv == 128))) return ATTN_ERR_UNSUPPORTED;
  if (dtype == ATTN_BF16 && flags != 0u) return ATTN_ERR_UNSUPPORTED;
  const int dev_rc = check_device();
  if (dev_rc != ATTN_OK) return dev_rc;

  fbc::AttnParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.S = S;
  p.Sk = Sk;
  p.G = Hq / Hkv;
  p.nqb = (int)nqb;
  p.xcd_group = ((int64_t)B * Hkv) % fbc::kXcds == 0 ? 1 : 0;
  // softmax in base 2: p = 2^((s - m) c). A zero scale (all scores equal) is
  // kept positive so that masked scores (-inf) still map to zero weight.
  p.c = (float)(cd > 1e-30 ? cd : 1e-30);
  p.dv = dv;
  p.scale = scale;
  p.dscale = dev_descale ? descale_qkv : nullptr;
  p.lse = lse;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // clear a stale error so the launch check below is ours
  const int mode = (int)(flags & (ATTN_FLAG_EXACT_P | ATTN_FLAG_NO_BLOCKSCALE));
  const hipError_t e = dtype == ATTN_FP8_E4M3 ? fbc::launch_attn_fwd_fp8(p, Dqk, mode, (int)grid, st)
                                              : fbc::launch_attn_fwd_bf16(p, Dqk, (int)grid, st);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

extern "C" int attn_fwd_ex(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int S,
                           int Dqk, int Dv, int causal, float scale, int dtype, const float* descale_qkv,
                           void* stream, unsigned flags) {
  return attn_fwd_impl(q, k, v, out, nullptr, B, Hq, Hkv, S, S, Dqk, Dv, causal, scale, dtype, descale_qkv, stream,
                       flags);
}

extern "C" int attn_fwd_lse(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
                            int Hkv, int S, int Dqk, int Dv, int causal, float scale, int dtype,
                            const float* descale_qkv, void* stream, unsigned flags) {
  if (!lse) return ATTN_ERR_INVALID;
  return attn_fwd_impl(q, k, v, out, lse, B, Hq, Hkv, S, S, Dqk, Dv, causal, scale, dtype, descale_qkv, stream,
                       flags);
}

extern "C" int attn_fwd_prefix(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
                               int Hkv, int Sq, int Sk, int Dqk, int Dv, int causal, float scale, int dtype,
                               const float* descale_qkv, void* stream, unsigned flags) {
  return attn_fwd_impl(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, Dqk, Dv, causal, scale, dtype, descale_qkv, stream,
                       flags);
}

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int S,
                        int Dqk, int Dv, int causal, float scale, int dtype) {
  return attn_fwd_ex(q, k, v, out, B, Hq, Hkv, S, Dqk, Dv, causal, scale, dtype, nullptr, nullptr, 0u);
}

extern "C" int attn_quantize_e4m3(const void* x, void* y, float* scale, long long rows, int dim, int hadamard, void* stream) {
  if (!x || !y || !scale) return ATTN_ERR_INVALID;
  if (!aligned16(x) || !aligned16(y) || ((uintptr_t)scale & 3u)) return ATTN_ERR_INVALID;
  if (rows <= 0 || (hadamard != 0 && hadamard != 1)) return ATTN_ERR_INVALID;
  if (dim != 64 && dim != 128 && dim != 192 && dim != 256) return ATTN_ERR_UNSUPPORTED;
  if (rows > (long long)(INT64_MAX / 256)) return ATTN_ERR_INVALID;
  const int dc = check_device();
  if (dc != ATTN_OK) return dc;
  (void)hipGetLastError();
  const hipError_t e = fbc::launch_quantize_e4m3(x, y, scale, (int64_t)rows, dim, hadamard, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK:
      return "success";
    case ATTN_ERR_INVALID:
      return "invalid argument (null or misaligned pointer, bad size, Hq % Hkv != 0, bad scale/descale, unknown flags)";
    case ATTN_ERR_UNSUPPORTED:
      return "unsupported (non-causal, unknown dtype, head dims other than 128/128 or 192/128, flags with BF16, or not gfx950)";
    case ATTN_ERR_LAUNCH:
      return "HIP runtime error while querying the device or launching the kernel";
    default:
      return "unknown error code";
  }
}

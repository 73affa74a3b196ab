// abi_host_check.cpp -- drives the C ABI's host-side paths (attn_api.cpp)
// against stubbed HIP calls (hip_stub.cpp): every rejection, the device check
// on a gfx950 and on another architecture, and the parameters handed to the
// launchers. Built with AddressSanitizer and UBSan by tests/test_host_sanitized.py.
// Prints one line per failed check and exits non-zero if any failed.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>

#include "attn_params.h"
#include "fp8_bf16_causal.h"

extern "C" {
void stub_set_device(int d);
int stub_launches(void);
const fbc::AttnParams* stub_last_params(void);
int stub_last_kind(void);
int stub_last_grid(void);
int stub_last_mode(void);
int stub_last_dqk(void);
}

static int g_fail = 0;
#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      std::printf("FAILED line %d: %s\n", __LINE__, #cond);             \
      ++g_fail;                                                         \
    }                                                                   \
  } while (0)

// fake device addresses: 16-byte aligned, never dereferenced by the host code
static void* const P = (void*)(uintptr_t)(1u << 20);
static void* addr_at(uintptr_t off) { return (void*)((uintptr_t)P + off); }

static int call(int B, int Hq, int Hkv, int S, int Dqk, int Dv, float scale, int dtype, const float* ds = nullptr,
                unsigned flags = 0, void* q = P, void* out = P) {
  return attn_fwd_ex(q, P, P, out, B, Hq, Hkv, S, Dqk, Dv, 1, scale, dtype, ds, nullptr, flags);
}

int main(int argc, char** argv) {
  const bool other_arch = argc > 1 && std::strcmp(argv[1], "other-arch") == 0;
  const float nan = std::nanf(""), inf = INFINITY;
  const int launches0 = stub_launches();

  // ---- rejected before the device is queried (same on every architecture)
  CHECK(attn_fwd(nullptr, P, P, P, 1, 4, 2, 128, 128, 128, 1, 0.1f, ATTN_BF16) == ATTN_ERR_INVALID);
  CHECK(call(1, 4, 2, 128, 128, 128, 0.1f, ATTN_BF16, nullptr, 0, addr_at(8)) == ATTN_ERR_INVALID);
  CHECK(call(0, 4, 2, 128, 128, 128, 0.1f, ATTN_BF16) == ATTN_ERR_INVALID);
  CHECK(call(1, 6, 4, 128, 128, 128, 0.1f, ATTN_BF16) == ATTN_ERR_INVALID);
  CHECK(call(1, 4, 2, -5, 128, 128, 0.1f, ATTN_BF16) == ATTN_ERR_INVALID);
  CHECK(call(1, 4, 2, 128, 128, 128, nan, ATTN_BF16) == ATTN_ERR_INVALID);
  CHECK(call(1, 4, 2, 128, 128, 128, inf, ATTN_BF16) == ATTN_ERR_INVALID);
  CHECK(call(1, 4, 2, 128, 128, 128, -0.5f, ATTN_BF16) == ATTN_ERR_INVALID);
  const float bad_ds[][3] = {{nan, 1, 1}, {1, 0, 1}, {1, 1, -2}, {1, inf, 1}};
  for (const auto& d : bad_ds) CHECK(call(1, 4, 2, 128, 128, 128, 0.1f, ATTN_FP8_E4M3, d) == ATTN_ERR_INVALID);
  CHECK(call(1, 4, 2, 128, 128, 128, 0.1f, ATTN_FP8_E4M3, nullptr, 8u) == ATTN_ERR_INVALID);
  CHECK(call(1 << 20, 1 << 10, 1 << 10, 1 << 30, 128, 128, 0.1f, ATTN_BF16) == ATTN_ERR_INVALID);
  CHECK(call(1, 1 << 12, 1 << 12, 1 << 22, 128, 128, 0.1f, ATTN_BF16) == ATTN_ERR_INVALID);
  CHECK(attn_fwd_lse(P, P, P, P, nullptr, 1, 4, 2, 128, 128, 128, 1, 0.1f, ATTN_BF16, nullptr, nullptr, 0) ==
        ATTN_ERR_INVALID);
  CHECK(attn_fwd_prefix(P, P, P, P, nullptr, 1, 4, 2, 300, 200, 128, 128, 1, 0.1f, ATTN_BF16, nullptr, nullptr, 0) ==
        ATTN_ERR_INVALID);
  CHECK(attn_quantize_e4m3(P, P, (float*)addr_at(2), 10, 128, 0, nullptr) == ATTN_ERR_INVALID);
  CHECK(attn_quantize_e4m3(P, P, (float*)P, 10, 128, 2, nullptr) == ATTN_ERR_INVALID);
  // unsupported on every device
  CHECK(attn_fwd(P, P, P, P, 1, 4, 2, 128, 128, 128, 0, 0.1f, ATTN_BF16) == ATTN_ERR_UNSUPPORTED);
  CHECK(call(1, 4, 2, 128, 64, 64, 0.1f, ATTN_BF16) == ATTN_ERR_UNSUPPORTED);
  CHECK(call(1, 4, 2, 128, 128, 128, 0.1f, 7) == ATTN_ERR_UNSUPPORTED);
  CHECK(call(1, 4, 2, 128, 128, 128, 0.1f, ATTN_BF16, nullptr, ATTN_FLAG_EXACT_P) == ATTN_ERR_UNSUPPORTED);
  CHECK(attn_quantize_e4m3(P, P, (float*)P, 10, 96, 0, nullptr) == ATTN_ERR_UNSUPPORTED);
  CHECK(stub_launches() == launches0);
  // a device index past the library's table
  stub_set_device(1000);
  CHECK(call(1, 4, 2, 128, 128, 128, 0.1f, ATTN_BF16) == ATTN_ERR_UNSUPPORTED);
  stub_set_device(0);
  CHECK(stub_launches() == launches0);

  if (other_arch) {
    // ---- a device that is not gfx950: valid calls are refused, nothing launches
    CHECK(attn_fwd(P, P, P, P, 1, 4, 2, 128, 128, 128, 1, 0.1f, ATTN_BF16) == ATTN_ERR_UNSUPPORTED);
    CHECK(call(2, 8, 2, 1000, 192, 128, 0.07f, ATTN_FP8_E4M3) == ATTN_ERR_UNSUPPORTED);
    CHECK(attn_quantize_e4m3(P, P, (float*)P, 10, 128, 1, nullptr) == ATTN_ERR_UNSUPPORTED);
    CHECK(stub_launches() == launches0);
  } else {
    // ---- gfx950: launches with the folded parameters
    CHECK(attn_fwd(P, addr_at(16), addr_at(32), addr_at(48), 2, 8, 2, 1000, 128, 128, 1, 0.125f, ATTN_BF16) == ATTN_OK);
    CHECK(stub_launches() == launches0 + 1 && stub_last_kind() == 0 && stub_last_dqk() == 128);
    const fbc::AttnParams* p = stub_last_params();
    CHECK(p->q == P && p->k == addr_at(16) && p->v == addr_at(32) && p->out == addr_at(48));
    CHECK(p->B == 2 && p->Hq == 8 && p->Hkv == 2 && p->S == 1000 && p->Sk == 1000 && p->G == 4);
    CHECK(p->nqb == 4 && stub_last_grid() == 2 * 8 * 4);
    CHECK(p->xcd_group == 0 && p->lse == nullptr && p->dv == 1.0f);
    CHECK(std::fabs(p->c - 0.125f * 1.4426950408889634f) <= 1e-7f);
    const float ds[3] = {0.5f, 0.25f, 3.0f};
    CHECK(call(1, 32, 8, 16384, 192, 128, 0.07f, ATTN_FP8_E4M3, ds, ATTN_FLAG_NO_BLOCKSCALE) == ATTN_OK);
    p = stub_last_params();
    CHECK(stub_last_kind() == 1 && stub_last_dqk() == 192 && stub_last_mode() == 2);
    CHECK(p->xcd_group == 1 && p->nqb == 64 && stub_last_grid() == 32 * 64 && p->dv == 3.0f);
    CHECK(std::fabs(p->c - 0.07f * 0.125f * 1.4426950408889634f) <= 1e-7f);
    // scale 0 keeps the folded base-2 scale positive
    CHECK(call(1, 2, 2, 5, 128, 128, 0.0f, ATTN_BF16) == ATTN_OK && stub_last_params()->c == 1e-30f);
    // queries after a key prefix
    float* lse = (float*)addr_at(64);
    CHECK(attn_fwd_prefix(P, P, P, P, lse, 1, 4, 4, 300, 1000, 128, 128, 1, 0.1f, ATTN_BF16, nullptr, nullptr, 0) ==
          ATTN_OK);
    p = stub_last_params();
    CHECK(p->S == 300 && p->Sk == 1000 && p->lse == lse && p->nqb == 2);
    CHECK(attn_quantize_e4m3(P, P, (float*)P, 10, 128, 1, nullptr) == ATTN_OK && stub_last_kind() == 2);
  }
  for (int c : {(int)ATTN_OK, (int)ATTN_ERR_INVALID, (int)ATTN_ERR_UNSUPPORTED, (int)ATTN_ERR_LAUNCH, 99})
    CHECK(attn_strerror(c) != nullptr && std::strlen(attn_strerror(c)) > 0);
  std::printf("%s: %d failed\n", other_arch ? "other-arch" : "gfx950", g_fail);
  return g_fail ? 1 : 0;
}

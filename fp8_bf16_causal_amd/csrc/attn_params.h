// attn_params.h -- the launch parameter block of the attention kernels and the
// work-decomposition constants, shared by the host-side dispatch
// (attn_api.cpp, plain C++) and the kernels (attn_common.h).
#pragma once

namespace fbc {

// Work decomposition: 8 waves per workgroup (two per SIMD), 32 query rows
// per wave, 256 query rows per workgroup.
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kQW = 32;
constexpr int kBQ = kWaves * kQW;
constexpr int kXcds = 8;      // MI355X: 8 accelerator complex dies, each with its own L2
constexpr int kOStride = 272; // epilogue staging: bytes per 128-wide BF16 output row in LDS

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int B, Hq, Hkv, S;  // S: query rows
  int Sk;             // key rows (>= S); query i sits at position i + Sk - S
  int G;          // Hq / Hkv
  int nqb;        // query blocks per head, ceil(S / kBQ)
  int xcd_group;  // 1: every KV head's workgroups run on one XCD
  float c;        // softmax scale * dq * dk * log2(e) (> 0), folded on the host
  float dv;       // output dequantisation factor
  float scale;    // softmax scale (for factors read on the device)
  const float* dscale;  // NULL, or device {dq, amax_q, dk, amax_k, dv, amax_v}: the
                        // kernel folds dq, dk and reads dv itself, as the host does
  float* lse;     // NULL, or [B][Hq][S]: each row's log-sum-exp of its logits
};

}  // namespace fbc

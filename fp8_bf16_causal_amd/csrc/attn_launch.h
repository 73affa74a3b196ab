// attn_launch.h -- internal launchers of the attention kernels (not part of
// the public ABI; see include/fp8_bf16_causal.h for that).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fbc {

struct AttnParams;

// One workgroup of 512 threads per (batch, query head, 256-row query block);
// grid = B * Hq * ceil(S / 256). dqk is 128 or 192 (Dv is 128).
// mode: ATTN_FLAG_* bits (0 = the method as the pages give it)
hipError_t launch_attn_fwd_fp8(const AttnParams& p, int dqk, int mode, int grid, hipStream_t stream);
hipError_t launch_attn_fwd_bf16(const AttnParams& p, int dqk, int grid, hipStream_t stream);

// FP8 quantize prologue: clear, amax, convert (three kernels on `stream`).
// dim is 64, 128, 192 or 256; scale points to 2 device floats.
hipError_t launch_quantize_e4m3(const void* x, void* y, float* scale, int64_t rows, int dim, int hadamard,
                                hipStream_t stream);

}  // namespace fbc

// attn_quant.hip -- the FP8 quantize prologue for gfx950: per-tensor e4m3fn
// quantisation of a BF16 tensor viewed as rows of `dim` elements, with an
// optional Hadamard rotation of every row (for Q and K).
//
// [spbcomputers.ru ZYFA article, section "Точность: ошибка FP8 ниже, чем у
// AITER" and the FAQ entry on the Hadamard rotation; captivela.com "Zyphra
// Luncurkan ZYFA", section "Akurasi Jauh Lebih Baik, Bukan Cuma Cepat":
// quantising Q, K and V dominates the FP8 error of a full model; a Hadamard
// rotation of Q and K roughly halves it. One orthogonal H on both leaves
// Q K^T unchanged.]
//
// Readings: the rotation is the normalised Walsh-Hadamard transform of each
// row in blocks of 128 elements (rows whose length is a multiple of 128) or
// 64; s = amax / 448 (1 if amax = 0); code = e4m3fn(y / s), nearest even.
// Every code is decided in IEEE fp32: the butterflies run over index bits
// 0, 1, ... in that order, (a, b) -> (a + b, a - b), followed by one multiply
// by the fp32 constant 1/sqrt(n); y / s and amax / 448 are correctly rounded
// divisions.
//
// Layout: one wave per row, lane l holding elements 64 j + l (j < dim / 64),
// so index bits 0-5 are lane bits (butterflies across lanes) and bit 6 is j
// (in-lane). Three kernels on one stream: clear the amax word, reduce amax
// (the rotated values' when rotating) with a vector atomic max on the float
// bits, then rotate again, scale and convert. HBM-bound: 2 reads of the
// input, 1 write of the codes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace fbc {

constexpr int kQuantThreads = 256;  // 4 waves per workgroup, one row per wave at a time

template <int J>
struct RowVals {
  float v[J];
};

// Load row r (lane l: elements 64 j + l), rotated if HAD (block n = 128 or 64).
template <int J, bool HAD, int N>
__device__ inline RowVals<J> load_row(const uint16_t* x, int64_t r, int lane) {
  RowVals<J> a;
  const uint16_t* row = x + r * (64 * J);
#pragma unroll
  for (int j = 0; j < J; ++j) a.v[j] = __builtin_bit_cast(float, (uint32_t)row[64 * j + lane] << 16);
  if constexpr (HAD) {
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {  // index bits 0..5: across lanes
      const bool upper = (lane & h) != 0;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const float partner = __shfl_xor(a.v[j], h, 64);
        a.v[j] = upper ? partner - a.v[j] : a.v[j] + partner;
      }
    }
    if constexpr (N == 128) {  // index bit 6: in-lane, j even / odd
#pragma unroll
      for (int j = 0; j + 1 < J; j += 2) {
        const float p = a.v[j], q = a.v[j + 1];
        a.v[j] = p + q;
        a.v[j + 1] = p - q;
      }
    }
    const float norm = N == 128 ? 0.08838834764831845f : 0.125f;  // fp32(1/sqrt(N))
#pragma unroll
    for (int j = 0; j < J; ++j) a.v[j] *= norm;
  }
  return a;
}

__global__ void quant_clear_kernel(float* scale) {
  if (threadIdx.x == 0) scale[1] = 0.0f;
}

template <int J, bool HAD, int N>
__global__ __launch_bounds__(kQuantThreads) void quant_amax_kernel(const uint16_t* x, float* scale, int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kQuantThreads / 64);
  float m = 0.0f;
  for (int64_t r = wave; r < rows; r += nwaves) {
    const RowVals<J> a = load_row<J, HAD, N>(x, r, lane);
#pragma unroll
    for (int j = 0; j < J; ++j) m = fmaxf(m, fabsf(a.v[j]));
  }
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) m = fmaxf(m, __shfl_xor(m, h, 64));
  // workgroup maximum through LDS, then one vector atomic per workgroup (all
  // atomics of the grid meet at one address): non-negative floats order like
  // their bit patterns
  __shared__ float wmax[kQuantThreads / 64];
  if (lane == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = wmax[0];
#pragma unroll
    for (int w = 1; w < kQuantThreads / 64; ++w) b = fmaxf(b, wmax[w]);
    if (b > 0.0f) atomicMax((unsigned int*)(scale + 1), __builtin_bit_cast(unsigned int, b));
  }
}

template <int J, bool HAD, int N>
__global__ __launch_bounds__(kQuantThreads) void quant_convert_kernel(const uint16_t* x, uint8_t* y, float* scale,
                                                                      int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kQuantThreads / 64);
  const float amax = scale[1];
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) scale[0] = s;
  for (int64_t r = wave; r < rows; r += nwaves) {
    const RowVals<J> a = load_row<J, HAD, N>(x, r, lane);
    uint8_t* row = y + r * (64 * J);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float q = a.v[j] / s;
      row[64 * j + lane] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(q, 0.0f, 0, false) & 0xFF);
    }
  }
}

template <int J, bool HAD, int N>
static hipError_t launch_quant_t(const void* x, void* y, float* scale, int64_t rows, hipStream_t stream) {
  const int64_t waves_needed = rows;
  int64_t blocks = (waves_needed + kQuantThreads / 64 - 1) / (kQuantThreads / 64);
  if (blocks > 16384) blocks = 16384;
  // the reduction grid is smaller: its atomics serialise at one address
  const int64_t rblocks = blocks < 1024 ? blocks : 1024;
  hipLaunchKernelGGL(quant_clear_kernel, dim3(1), dim3(64), 0, stream, scale);
  hipLaunchKernelGGL((quant_amax_kernel<J, HAD, N>), dim3((unsigned)rblocks), dim3(kQuantThreads), 0, stream,
                     (const uint16_t*)x, scale, rows);
  hipLaunchKernelGGL((quant_convert_kernel<J, HAD, N>), dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream,
                     (const uint16_t*)x, (uint8_t*)y, scale, rows);
  return hipGetLastError();
}

hipError_t launch_quantize_e4m3(const void* x, void* y, float* scale, int64_t rows, int dim, int hadamard,
                                hipStream_t stream) {
  switch (dim) {
    case 64:
      return hadamard ? launch_quant_t<1, true, 64>(x, y, scale, rows, stream)
                      : launch_quant_t<1, false, 64>(x, y, scale, rows, stream);
    case 128:
      return hadamard ? launch_quant_t<2, true, 128>(x, y, scale, rows, stream)
                      : launch_quant_t<2, false, 128>(x, y, scale, rows, stream);
    case 192:
      return hadamard ? launch_quant_t<3, true, 64>(x, y, scale, rows, stream)
                      : launch_quant_t<3, false, 64>(x, y, scale, rows, stream);
    default:
      return hadamard ? launch_quant_t<4, true, 128>(x, y, scale, rows, stream)
                      : launch_quant_t<4, false, 128>(x, y, scale, rows, stream);
  }
}

}  // namespace fbc

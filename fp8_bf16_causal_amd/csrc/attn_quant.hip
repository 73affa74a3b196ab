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
// Layout: the tensor is a flat array of n-element blocks (n = 128 or 64, the
// rotation's block; whole rows hold whole blocks). Without the rotation a
// wave takes 512 consecutive elements per step, each lane 8 (one 16-byte
// load). With it a wave takes 2048 per step, each lane 32 consecutive ones
// (four 16-byte loads): index bits 0-4 of an element are in-lane, so five
// butterfly stages run in registers, and the last one or two are lane bits
// (DPP moves within quads). Three kernels on one stream: clear the amax word,
// reduce amax (of the rotated values when rotating) with one vector atomic
// max per workgroup on the float bits, then (rotate again,) scale and
// convert. HBM-bound without the rotation, vector-ALU-bound with it (the
// convert pass spends about 14.5 instructions per element): 2 reads of the
// input, 1 write of the codes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace fbc {

constexpr int kQuantThreads = 256;  // 4 waves per workgroup
constexpr int kWaveElems = 512;     // elements per wave per step, 8 per lane

typedef int qv4i __attribute__((ext_vector_type(4)));
typedef int qv2i __attribute__((ext_vector_type(2)));

// x from lane (lane ^ HL) of the same quad (HL = 1, 2), by a DPP quad
// permutation.
template <int HL>
__device__ inline float lane_xor(float x) {
  static_assert(HL == 1 || HL == 2, "lane distances within a quad");
  const int v = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), HL == 1 ? 0xB1 : 0x4E, 0xF, 0xF, true);
  return __builtin_bit_cast(float, v);  // quad_perm [1, 0, 3, 2] or [2, 3, 0, 1]
}

// The 8 elements e0 .. e0+7 of lane `lane` (e0 = 8 * lane within the wave's 512).
__device__ inline void load8(const uint16_t* x, int64_t e0, bool valid, float v[8]) {
  qv4i w = {0, 0, 0, 0};
  if (valid) w = *(const qv4i*)(x + e0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __builtin_bit_cast(float, (uint32_t)w[i] << 16);
    v[2 * i + 1] = __builtin_bit_cast(float, (uint32_t)w[i] & 0xFFFF0000u);
  }
}

__global__ void quant_clear_kernel(float* scale) {
  if (threadIdx.x == 0) scale[1] = 0.0f;
}

__global__ __launch_bounds__(kQuantThreads) void quant_amax_kernel(const uint16_t* x, float* scale, int64_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kQuantThreads / 64);
  // eight 512-element chunks per wave and step: eight independent 16-byte
  // loads in flight per lane (this pass runs on a small grid; four measured
  // 2.7% slower)
  float m = 0.0f;
  for (int64_t base = wave * 8 * kWaveElems; base < n; base += nwaves * 8 * kWaveElems) {
    float v[8][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t e0 = base + j * kWaveElems + 8 * lane;
      load8(x, e0, e0 < n, v[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[j][i]));
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

__global__ __launch_bounds__(kQuantThreads) void quant_convert_kernel(const uint16_t* x, uint8_t* y, float* scale,
                                                                      int64_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kQuantThreads / 64);
  const float amax = scale[1];
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) scale[0] = s;
  // y / s correctly rounded, from the correctly rounded reciprocal r = 1/s:
  // q0 = y r is within one ulp of y / s, the remainder y - s q0 is exact
  // (one fma), and q0 + r (y - s q0) rounds to the correctly rounded quotient
  // (Markstein's theorem) as long as nothing underflows, which holds for
  // s >= 2^-69. Smaller scales take the plain division. The remainder is
  // formed as s q0 - y and subtracted: the same value, but for y = -0 the
  // last step adds -0 to -0 and keeps the quotient's sign (y - s q0 would
  // turn it into +0).
  const float r = 1.0f / s;
  const bool fast = s >= 0x1p-69f;
  for (int64_t base = wave * kWaveElems; base < n; base += nwaves * kWaveElems) {
    const int64_t e0 = base + 8 * lane;
    const bool valid = e0 < n;
    float v[8];
    load8(x, e0, valid, v);
    float q[8];
    if (fast) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q0 = v[i] * r;
        q[i] = fmaf(-fmaf(q0, s, -v[i]), r, q0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = v[i] / s;
    }
    qv2i out;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * i], q[4 * i + 1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * i + 2], q[4 * i + 3], w, true);
      out[i] = w;
    }
    if (valid) *(qv2i*)(y + e0) = out;
  }
}

// ---- rotation: 32 consecutive elements per lane
// With the rotation each lane holds 32 consecutive elements (index bits 0-4
// of a block) from four 16-byte loads, so five butterfly stages run in
// registers, one add or subtract per element and stage; the remaining index
// bits (5 and 6 of a 128-element block, 5 of a 64-element one) are lane bits
// 0 and 1: quad-permutation DPP moves and one multiply-add with +-1 per
// element and stage (a + b on the lane holding a, a - b on the lane holding
// b, each rounded once as the plain sum). A wave takes 2048 consecutive
// elements per step. Every code is decided in the precision and order stated
// above.
constexpr int kHadLaneElems = 32;
constexpr int kHadWaveElems = 64 * kHadLaneElems;

// The 32 elements of lane `lane` from element e0, as BF16 pairs. FULL: the
// wave's whole step lies below n; else elements at or past n read as zeros
// (whole lanes, as n is a multiple of the 64-element block).
template <bool FULL>
__device__ inline void load32(const uint16_t* x, int64_t e0, int64_t n, qv4i w[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (FULL) {
      w[j] = *(const qv4i*)(x + e0 + 8 * j);
    } else {
      w[j] = (qv4i){0, 0, 0, 0};
      if (e0 < n) w[j] = *(const qv4i*)(x + e0 + 8 * j);
    }
  }
}

// v = the rotated, not yet normalised, 32 elements held in w.
template <int N>
__device__ inline void rotate32(const qv4i w[4], int lane, float v[32]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * j + 2 * i] = __builtin_bit_cast(float, (uint32_t)w[j][i] << 16);
      v[8 * j + 2 * i + 1] = __builtin_bit_cast(float, (uint32_t)w[j][i] & 0xFFFF0000u);
    }
  // index bits 0..4: in-lane, (a, b) -> (a + b, a - b)
#pragma unroll
  for (int h = 1; h < 32; h <<= 1)
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if ((i & h) == 0) {
        const float p = v[i], q = v[i + h];
        v[i] = p + q;
        v[i + h] = p - q;
      }
  // index bit 5 (and 6 at n = 128): lane bit 0 (and 1)
  {
    const float sgn = (lane & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = fmaf(v[i], sgn, lane_xor<1>(v[i]));
  }
  if constexpr (N == 128) {
    const float sgn = (lane & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = fmaf(v[i], sgn, lane_xor<2>(v[i]));
  }
}

template <int N>
__global__ __launch_bounds__(kQuantThreads) void quant_amax_had_kernel(const uint16_t* x, float* scale, int64_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kQuantThreads / 64);
  // max |z| over the unnormalised rotated values: rounding the product with
  // the positive constant 1/sqrt(n) is monotone, so the maximum of the
  // normalised values is the normalised maximum
  // two wave steps per iteration: eight 16-byte loads in flight per lane
  float m = 0.0f;
  for (int64_t wbase = wave * 2 * kHadWaveElems; wbase < n; wbase += nwaves * 2 * kHadWaveElems) {
    qv4i w[2][4];
    if (wbase + 2 * kHadWaveElems <= n) {  // wave-uniform: only the last steps are partial
#pragma unroll
      for (int u = 0; u < 2; ++u) load32<true>(x, wbase + u * kHadWaveElems + kHadLaneElems * lane, n, w[u]);
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u) load32<false>(x, wbase + u * kHadWaveElems + kHadLaneElems * lane, n, w[u]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float v[32];
      rotate32<N>(w[u], lane, v);
#pragma unroll
      for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
    }
  }
  m *= N == 128 ? 0.08838834764831845f : 0.125f;  // fp32(1/sqrt(N))
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) m = fmaxf(m, __shfl_xor(m, h, 64));
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

// One wave step of the convert pass: rotate, normalise, divide by s, convert,
// store 32 codes per lane. FAST: y / s from the reciprocal (as in
// quant_convert_kernel), else the plain division. FULL: the whole step lies
// below n.
template <int N, bool FAST, bool FULL>
__device__ inline void convert_had_step(const uint16_t* x, uint8_t* y, int64_t e0, int64_t n, int lane, float s,
                                        float r) {
  const float norm = N == 128 ? 0.08838834764831845f : 0.125f;
  qv4i w[4];
  load32<FULL>(x, e0, n, w);
  float v[32];
  rotate32<N>(w, lane, v);
#pragma unroll
  for (int k = 0; k < 2; ++k) {  // 16 codes per 16-byte store
    float q[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float yv = v[16 * k + i] * norm;
      if constexpr (FAST) {
        const float q0 = yv * r;
        q[i] = fmaf(-fmaf(q0, s, -yv), r, q0);
      } else {
        q[i] = yv / s;
      }
    }
    qv4i out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // the first convert fills the low half of a register whose high half
      // the second one writes: its old contents do not matter (an empty asm
      // definition, no instruction)
      int w;
      asm volatile("" : "=v"(w));
      w = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * i], q[4 * i + 1], w, false);
      out[i] = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * i + 2], q[4 * i + 3], w, true);
    }
    if (FULL || e0 < n) *(qv4i*)(y + e0 + 16 * k) = out;
  }
}

template <int N>
__global__ __launch_bounds__(kQuantThreads) void quant_convert_had_kernel(const uint16_t* x, uint8_t* y, float* scale,
                                                                          int64_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kQuantThreads / 64);
  const float amax = scale[1];
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) scale[0] = s;
  const float r = 1.0f / s;
  // (wbase + step <= n is wave-uniform: only the last steps are partial)
  if (s >= 0x1p-69f) {
    for (int64_t wbase = wave * kHadWaveElems; wbase < n; wbase += nwaves * kHadWaveElems) {
      if (wbase + kHadWaveElems <= n)
        convert_had_step<N, true, true>(x, y, wbase + kHadLaneElems * lane, n, lane, s, r);
      else
        convert_had_step<N, true, false>(x, y, wbase + kHadLaneElems * lane, n, lane, s, r);
    }
  } else {
    for (int64_t wbase = wave * kHadWaveElems; wbase < n; wbase += nwaves * kHadWaveElems)
      convert_had_step<N, false, false>(x, y, wbase + kHadLaneElems * lane, n, lane, s, r);
  }
}

template <int N>
static hipError_t launch_quant_had(const void* x, void* y, float* scale, int64_t n, hipStream_t stream) {
  int64_t blocks = (n + kHadWaveElems * (kQuantThreads / 64) - 1) / (kHadWaveElems * (kQuantThreads / 64));
  if (blocks > 16384) blocks = 16384;
  const int64_t rblocks = blocks < 1024 ? blocks : 1024;
  hipLaunchKernelGGL(quant_clear_kernel, dim3(1), dim3(64), 0, stream, scale);
  hipLaunchKernelGGL((quant_amax_had_kernel<N>), dim3((unsigned)rblocks), dim3(kQuantThreads), 0, stream,
                     (const uint16_t*)x, scale, n);
  hipLaunchKernelGGL((quant_convert_had_kernel<N>), dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream,
                     (const uint16_t*)x, (uint8_t*)y, scale, n);
  return hipGetLastError();
}

static hipError_t launch_quant_plain(const void* x, void* y, float* scale, int64_t n, hipStream_t stream) {
  int64_t blocks = (n + kWaveElems * (kQuantThreads / 64) - 1) / (kWaveElems * (kQuantThreads / 64));
  if (blocks > 16384) blocks = 16384;
  // the reduction grid is smaller: its atomics serialise at one address
  const int64_t rblocks = blocks < 1024 ? blocks : 1024;
  hipLaunchKernelGGL(quant_clear_kernel, dim3(1), dim3(64), 0, stream, scale);
  hipLaunchKernelGGL(quant_amax_kernel, dim3((unsigned)rblocks), dim3(kQuantThreads), 0, stream, (const uint16_t*)x,
                     scale, n);
  hipLaunchKernelGGL(quant_convert_kernel, dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream, (const uint16_t*)x,
                     (uint8_t*)y, scale, n);
  return hipGetLastError();
}

hipError_t launch_quantize_e4m3(const void* x, void* y, float* scale, int64_t rows, int dim, int hadamard,
                                hipStream_t stream) {
  const int64_t n = rows * dim;  // a multiple of 64: blocks of 64 (and of 128 when dim is) never straddle rows
  if (!hadamard) return launch_quant_plain(x, y, scale, n, stream);
  return dim % 128 == 0 ? launch_quant_had<128>(x, y, scale, n, stream) : launch_quant_had<64>(x, y, scale, n, stream);
}

}  // namespace fbc

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
// rotation's block; whole rows hold whole blocks). A wave takes 512
// consecutive elements per step, each lane 8 (one 16-byte load): index bits
// 0-2 of an element are in-lane, bits 3.. are lane bits, so the butterflies
// for bits 0-2 run in registers and the rest across 8 or 16 lanes (DPP
// moves within 16-lane rows). Three
// kernels on one stream: clear the amax word, reduce amax (of the rotated
// values when rotating) with one vector atomic max per workgroup on the float
// bits, then rotate again, scale and convert (8-byte stores). HBM-bound:
// 2 reads of the input, 1 write of the codes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.h"

namespace fbc {

constexpr int kQuantThreads = 256;  // 4 waves per workgroup
constexpr int kWaveElems = 512;     // elements per wave per step, 8 per lane

typedef int qv4i __attribute__((ext_vector_type(4)));
typedef int qv2i __attribute__((ext_vector_type(2)));

// x from lane (lane ^ HL) of the same 16-lane row (HL = 1, 2, 4, 8), by DPP
// moves: quad permutations for 1 and 2, half-row mirror then quad reversal
// for 4 ((i ^ 7) ^ 3 = i ^ 4), rotation by 8 for 8.
template <int HL>
__device__ inline float lane_xor(float x) {
  int v = __builtin_bit_cast(int, x);
  if constexpr (HL == 1) {
    v = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);  // quad_perm [1, 0, 3, 2]
  } else if constexpr (HL == 2) {
    v = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);  // quad_perm [2, 3, 0, 1]
  } else if constexpr (HL == 4) {
    v = __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true);  // row_half_mirror
    v = __builtin_amdgcn_mov_dpp(v, 0x1B, 0xF, 0xF, true);   // quad_perm [3, 2, 1, 0]
  } else {
    static_assert(HL == 8, "lane distances within a 16-lane row");
    v = __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, true);  // row_ror:8
  }
  return __builtin_bit_cast(float, v);
}

// One butterfly stage across lanes at distance HL: the lane whose index bit
// is clear holds a and gets a + b, its partner holds b and gets a - b; both
// as one fused multiply-add with +-1, rounded once like the plain sum.
template <int HL>
__device__ inline void cross_lane_stage(float v[8], int lane) {
  const float sgn = (lane & HL) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = fmaf(v[i], sgn, lane_xor<HL>(v[i]));
}

// The 8 elements e0 .. e0+7 of lane `lane` (e0 = 8 * lane within the wave's
// 512), rotated by the normalised Walsh-Hadamard transform of block N if HAD.
template <bool HAD, int N>
__device__ inline void load8(const uint16_t* x, int64_t e0, bool valid, int lane, float v[8]) {
  qv4i w = {0, 0, 0, 0};
  if (valid) w = *(const qv4i*)(x + e0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __builtin_bit_cast(float, (uint32_t)w[i] << 16);
    v[2 * i + 1] = __builtin_bit_cast(float, (uint32_t)w[i] & 0xFFFF0000u);
  }
  if constexpr (HAD) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)  // index bits 0..2: in-lane
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if ((i & h) == 0) {
          const float p = v[i], q = v[i + h];
          v[i] = p + q;
          v[i + h] = p - q;
        }
    // index bits 3..: across lanes (bit 3 + j of the block index is lane bit j)
    cross_lane_stage<1>(v, lane);
    cross_lane_stage<2>(v, lane);
    cross_lane_stage<4>(v, lane);
    if constexpr (N == 128) cross_lane_stage<8>(v, lane);
    const float norm = N == 128 ? 0.08838834764831845f : 0.125f;  // fp32(1/sqrt(N))
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= norm;
  }
}

__global__ void quant_clear_kernel(float* scale) {
  if (threadIdx.x == 0) scale[1] = 0.0f;
}

template <bool HAD, int N>
__global__ __launch_bounds__(kQuantThreads) void quant_amax_kernel(const uint16_t* x, float* scale, int64_t n) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kQuantThreads / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (kQuantThreads / 64);
  // four 512-element chunks per wave and step: four independent 16-byte
  // loads in flight per lane (this pass runs on a small grid)
  float m = 0.0f;
  for (int64_t base = wave * 4 * kWaveElems; base < n; base += nwaves * 4 * kWaveElems) {
    float v[4][8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t e0 = base + j * kWaveElems + 8 * lane;
      load8<HAD, N>(x, e0, e0 < n, lane, v[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
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

template <bool HAD, int N>
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
  // s >= 2^-69. Smaller scales take the plain division.
  const float r = 1.0f / s;
  const bool fast = s >= 0x1p-69f;
  for (int64_t base = wave * kWaveElems; base < n; base += nwaves * kWaveElems) {
    const int64_t e0 = base + 8 * lane;
    const bool valid = e0 < n;
    float v[8];
    load8<HAD, N>(x, e0, valid, lane, v);
    float q[8];
    if (fast) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q0 = v[i] * r;
        // (copysign keeps -0: the correction would turn it into +0)
        q[i] = copysignf(fmaf(fmaf(-q0, s, v[i]), r, q0), v[i]);
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

template <bool HAD, int N>
static hipError_t launch_quant_t(const void* x, void* y, float* scale, int64_t n, hipStream_t stream) {
  int64_t blocks = (n + kWaveElems * (kQuantThreads / 64) - 1) / (kWaveElems * (kQuantThreads / 64));
  if (blocks > 16384) blocks = 16384;
  // the reduction grid is smaller: its atomics serialise at one address
  const int64_t rblocks = blocks < 1024 ? blocks : 1024;
  hipLaunchKernelGGL(quant_clear_kernel, dim3(1), dim3(64), 0, stream, scale);
  hipLaunchKernelGGL((quant_amax_kernel<HAD, N>), dim3((unsigned)rblocks), dim3(kQuantThreads), 0, stream,
                     (const uint16_t*)x, scale, n);
  hipLaunchKernelGGL((quant_convert_kernel<HAD, N>), dim3((unsigned)blocks), dim3(kQuantThreads), 0, stream,
                     (const uint16_t*)x, (uint8_t*)y, scale, n);
  return hipGetLastError();
}

hipError_t launch_quantize_e4m3(const void* x, void* y, float* scale, int64_t rows, int dim, int hadamard,
                                hipStream_t stream) {
  const int64_t n = rows * dim;  // a multiple of 64: blocks of 64 (and of 128 when dim is) never straddle rows
  if (dim % 128 == 0)
    return hadamard ? launch_quant_t<true, 128>(x, y, scale, n, stream) : launch_quant_t<false, 128>(x, y, scale, n, stream);
  return hadamard ? launch_quant_t<true, 64>(x, y, scale, n, stream) : launch_quant_t<false, 64>(x, y, scale, n, stream);
}

}  // namespace fbc

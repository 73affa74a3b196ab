// attn_fwd_bf16.hip -- causal prefill attention forward, BF16 inputs and
// output, for gfx950 (MI355X).
//
// The operation [ZYFA abstract, "ZYFA: Speed and Accuracy of FP8
// FlashAttention on AMD CDNA4" (airebao.com); spbcomputers.ru ZYFA article,
// opening paragraphs: BF16 kernels alongside the FP8 ones, causal forward]:
// FlashAttention forward with an exact online softmax,
//   S = Q K^T, m = running row max, P = 2^((S - m) c) rounded to BF16,
//   O = sum P V / sum P, rescaled by 2^((m_old - m_new) c) when m rises.
// Readings: the row sum accumulates the fp32 probabilities (before their BF16
// rounding); the running max is updated once per key tile.
//
// Tiling (gfx950-specific): 8 waves x 32 query rows per workgroup; K/V tiles
// of BK keys staged through LDS, double-buffered. S^T = K Q^T and
// O^T = V^T P^T both run on v_mfma_f32_32x32x16_bf16, so each lane holds one
// query (l%32): row maxima and sums are in-lane plus one permlane32 swap, and
// the probabilities feed the P V instruction straight from registers. V stays
// row-major in LDS; the V^T operand is read with ds_read_b64_tr_b16.
#include "attn_common.h"
#include "attn_launch.h"

namespace fbc {

template <int DQK, int BK>
struct Bf16Layout {
  static constexpr int kBK = BK;
  static constexpr int kDv = 128;
  static constexpr int kNsb = BK / 32;                 // 32-key blocks per tile
  static constexpr int kKStride = DQK * 2 + 16;        // padded K row (bytes)
  static constexpr int kVStride = kDv * 2 + 32;        // padded V row (bytes)
  static constexpr int kKTile = BK * kKStride;
  static constexpr int kVTile = BK * kVStride;
  static constexpr int kStage = kKTile + kVTile;
  static constexpr int kLoop = 2 * kStage;
  static constexpr int kEpi = kWaves * kQW * kOStride;
  static constexpr int kLds = kLoop > kEpi ? kLoop : kEpi;
  static constexpr int kKChunksPerRow = DQK * 2 / 16;
  static constexpr int kKPerThread = BK * kKChunksPerRow / kThreads;
  static constexpr int kVPerThread = BK * (kDv * 2 / 16) / kThreads;
};

template <int DQK, int BK>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_bf16_kernel(AttnParams p) {
  using L = Bf16Layout<DQK, BK>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[L::kLds];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  int b, h, qb;
  map_block(p, blockIdx.x, b, h, qb);
  const int S = p.S;
  const int kvh = h / p.G;
  const int q0 = qb * kBQ, qw0 = q0 + wave * kQW;
  const int n_tiles = (min(q0 + kBQ, S) + BK - 1) / BK;
  const int wave_tiles = qw0 < S ? (min(qw0 + kQW, S) - 1) / BK + 1 : 0;

  const size_t q_rs = (size_t)p.Hq * DQK * 2, k_rs = (size_t)p.Hkv * DQK * 2, v_rs = (size_t)p.Hkv * L::kDv * 2;
  const uint8_t* Qg = (const uint8_t*)p.q + (size_t)b * S * q_rs + (size_t)h * DQK * 2;
  const uint8_t* Kg = (const uint8_t*)p.k + (size_t)b * S * k_rs + (size_t)kvh * DQK * 2;
  const uint8_t* Vg = (const uint8_t*)p.v + (size_t)b * S * v_rs + (size_t)kvh * L::kDv * 2;

  // Q^T operand: lane (query l32, half g) holds Q[q][16t + 8g .. +7] per step t.
  v8bf qf[DQK / 16];
  {
    const int qrow = qw0 + l32;
#pragma unroll
    for (int t = 0; t < DQK / 16; ++t) {
      v4i x = {0, 0, 0, 0};
      if (qrow < S) x = ld_global16(Qg + (size_t)qrow * q_rs + (16 * t + 8 * g) * 2);
      qf[t] = __builtin_bit_cast(v8bf, x);
    }
  }

  v4i kst[L::kKPerThread], vst[L::kVPerThread];
  auto stage_load = [&](int t) {
    const int k0 = t * BK;
#pragma unroll
    for (int u = 0; u < L::kKPerThread; ++u) {
      const int x = tid + kThreads * u, row = x / L::kKChunksPerRow, c = x % L::kKChunksPerRow;
      const int j = k0 + row;
      kst[u] = j < S ? ld_global16(Kg + (size_t)j * k_rs + 16 * c) : (v4i){0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < L::kVPerThread; ++u) {
      const int x = tid + kThreads * u, row = x >> 4, c = x & 15;
      const int j = k0 + row;
      vst[u] = j < S ? ld_global16(Vg + (size_t)j * v_rs + 16 * c) : (v4i){0, 0, 0, 0};
    }
  };
  auto stage_store = [&](int buf) {
    uint8_t* Kl = lds + buf * L::kStage;
    uint8_t* Vl = Kl + L::kKTile;
#pragma unroll
    for (int u = 0; u < L::kKPerThread; ++u) {
      const int x = tid + kThreads * u, row = x / L::kKChunksPerRow, c = x % L::kKChunksPerRow;
      st_lds16(Kl + row * L::kKStride + 16 * c, kst[u]);
    }
#pragma unroll
    for (int u = 0; u < L::kVPerThread; ++u) {
      const int x = tid + kThreads * u, row = x >> 4, c = x & 15;
      st_lds16(Vl + row * L::kVStride + 16 * c, vst[u]);
    }
  };

  // V^T operand of v_mfma_f32_32x32x16_bf16, read with ds_read_b64_tr_b16:
  // lane (d = 32 db + l%32, half g) needs the keys whose probabilities sit in
  // the P operand: for block sb and step hh, 8(r/4) + 4g + r%4 + 32 sb + 16 hh
  // for r = 0..7, i.e. 4 consecutive keys at +0 and 4 more at +8.
  int vrd;
  {
    const int G = lane >> 4, pp = lane & 15, br = pp >> 2, w = pp & 3;
    vrd = (4 * (G >> 1) + br) * L::kVStride + (16 * (G & 1) + 4 * w) * 2;
  }

  v16f oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = (v16f){};
  float m = -INFINITY, lsum = 0.0f;
  const float c = p.c;

  stage_load(0);
  stage_store(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) stage_load(t + 1);
    if (t < wave_tiles) {
      const uint8_t* Kl = lds + buf * L::kStage;
      const uint8_t* Vl = Kl + L::kKTile;
      const int k0 = t * BK;

      v16f s[L::kNsb];
#pragma unroll
      for (int sb = 0; sb < L::kNsb; ++sb) s[sb] = (v16f){};
#pragma unroll
      for (int t16 = 0; t16 < DQK / 16; ++t16) {
#pragma unroll
        for (int sb = 0; sb < L::kNsb; ++sb) {
          const v4i kx = ld_lds16(Kl + (sb * 32 + l32) * L::kKStride + (16 * t16 + 8 * g) * 2);
          s[sb] = mfma_32x32x16_bf16(__builtin_bit_cast(v8bf, kx), qf[t16], s[sb]);
        }
      }

      if (k0 + BK - 1 > qw0) {
        const int qi = qw0 + l32;
#pragma unroll
        for (int sb = 0; sb < L::kNsb; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + sb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key > qi) s[sb][r] = -INFINITY;
          }
      }

      float mt = s[0][0];
#pragma unroll
      for (int sb = 0; sb < L::kNsb; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[sb][r]);
      mt = max_xor32(mt);
      const float mn = fmaxf(m, mt);
      const float alpha = (m == mn) ? 1.0f : __builtin_amdgcn_exp2f((m - mn) * c);
      m = mn;
      const float nmc = -mn * c;

      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
        lsum *= alpha;
      }

#pragma unroll
      for (int sb = 0; sb < L::kNsb; ++sb) {
        float pr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          pr[r] = __builtin_amdgcn_exp2f(fmaf(s[sb][r], c, nmc));
          lsum += pr[r];
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const v4i pw = {(int)pack_bf16(pr[8 * hh + 0], pr[8 * hh + 1]), (int)pack_bf16(pr[8 * hh + 2], pr[8 * hh + 3]),
                          (int)pack_bf16(pr[8 * hh + 4], pr[8 * hh + 5]), (int)pack_bf16(pr[8 * hh + 6], pr[8 * hh + 7])};
          const v8bf pf = __builtin_bit_cast(v8bf, pw);
          const uint8_t* vb = Vl + vrd + (sb * 32 + 16 * hh) * L::kVStride;
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const v4s lo = lds_read_tr16(vb + db * 64);
            const v4s hi = lds_read_tr16(vb + db * 64 + 8 * L::kVStride);
            const v4i vv = {__builtin_bit_cast(v2i, lo).x, __builtin_bit_cast(v2i, lo).y,
                            __builtin_bit_cast(v2i, hi).x, __builtin_bit_cast(v2i, hi).y};
            oacc[db] = mfma_32x32x16_bf16(__builtin_bit_cast(v8bf, vv), pf, oacc[db]);
          }
        }
      }
    }
    if (t + 1 < n_tiles) stage_store(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lanes l and l^32 hold partial sums of one query.
  const float l_tot = sum_xor32(lsum);
  uint8_t* Ol = lds + wave * kQW * kOStride;
  if (wave_tiles > 0) {
    const float inv = p.dv / l_tot;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const v2i w = {(int)pack_bf16(oacc[db][4 * rq + 0] * inv, oacc[db][4 * rq + 1] * inv),
                       (int)pack_bf16(oacc[db][4 * rq + 2] * inv, oacc[db][4 * rq + 3] * inv)};
        *(v2i*)(Ol + l32 * kOStride + (32 * db + 8 * rq + 4 * g) * 2) = w;
      }
  }
  __syncthreads();
  if (wave_tiles > 0) {
    uint8_t* Og = (uint8_t*)p.out;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int x = lane + 64 * u, row = x >> 4, cc = x & 15;
      const int qrow = qw0 + row;
      if (qrow < S)
        *(v4i*)(Og + (((size_t)b * S + qrow) * p.Hq + h) * (L::kDv * 2) + 16 * cc) =
            ld_lds16(Ol + row * kOStride + 16 * cc);
    }
  }
}

template <int DQK, int BK>
static hipError_t launch_bf16(const AttnParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<DQK, BK>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_bf16(const AttnParams& p, int dqk, int grid, hipStream_t stream) {
  if (dqk == 128) return launch_bf16<128, 128>(p, grid, stream);
  return launch_bf16<192, 64>(p, grid, stream);
}

}  // namespace fbc

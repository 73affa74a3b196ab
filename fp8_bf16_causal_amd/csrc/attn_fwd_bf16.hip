// attn_fwd_bf16.hip -- causal prefill attention forward, BF16 inputs and
// output, for gfx950 (MI355X).
//
// The operation [ZYFA abstract, "ZYFA: Speed and Accuracy of FP8
// FlashAttention on AMD CDNA4" (airebao.com); spbcomputers.ru ZYFA article,
// opening paragraphs: BF16 kernels alongside the FP8 ones, causal forward]:
// FlashAttention forward with an exact online softmax,
//   S = Q K^T, m = running row max, P = 2^((S - m) c) rounded to BF16,
//   O = sum P V / sum P, rescaled by 2^((m_old - m_new) c) when m rises.
// Readings: the row sum accumulates the BF16-rounded probabilities (the
// weights the P V product actually applies); the reference max is updated per key tile, lazily (only when the
// tile max exceeds it by more than 8 binades), with an exact rescale then.
//
// Tiling (gfx950-specific): 8 waves x 32 query rows per workgroup; K/V tiles
// of BK keys staged in LDS by direct-to-LDS loads, double-buffered, with the
// same two-group ping-pong schedule as the FP8 kernel. S^T = K Q^T and
// O^T = V^T P^T both run on v_mfma_f32_32x32x16_bf16, so each lane holds one
// query (l%32): row maxima are in-lane plus one permlane32 swap, and the
// probabilities feed the P V instruction straight from registers. The row
// sums come from one more (16x16x32) matrix instruction per 16 keys. V stays
// row-major in LDS (rows permuted); the V^T operand is read with
// ds_read_b64_tr_b16.
#include <type_traits>

#include "attn_common.h"
#include "attn_launch.h"

namespace fbc {

template <int DQK, int BK>
struct Bf16Layout {
  static constexpr int kBK = BK;
  static constexpr int kDv = 128;
  static constexpr int kNsb = BK / 32;                // 32-key blocks per tile
  static constexpr bool kHi = DQK == 192;             // K columns 128..191 kept apart
  // one 16-byte padding chunk per LDS row: additive chunk offsets, and
  // consecutive rows start in different bank groups
  static constexpr int kKLoStride = 272;              // K[:, 0:128]  (256 data bytes)
  static constexpr int kKHiStride = 144;              // K[:, 128:192] (128 data bytes)
  static constexpr int kVStride = 272;                // V (256 data bytes)
  static constexpr int kKLoTile = BK * kKLoStride;
  static constexpr int kKHiTile = kHi ? BK * kKHiStride : 0;
  static constexpr int kKTile = kKLoTile + kKHiTile;
  static constexpr int kVTile = BK * kVStride;
  static constexpr int kLoop = 2 * (kKTile + kVTile);
  static constexpr int kEpi = kWaves * kQW * kOStride;
  static constexpr int kLds = kLoop > kEpi ? kLoop : kEpi;
};

// V's LDS row for key k of the tile: inside each group of 16 keys the two
// 2-bit fields of k swap. One ds_read_b64_tr_b16 pass serves two 16-lane
// groups that read the same 4 consecutive keys at 32-byte-apart columns; the
// swap puts those 4 rows 4 bank groups apart under the 272-byte stride.
__device__ inline int vrow_bf16(int k) { return (k & ~15) | ((k & 3) << 2) | ((k >> 2) & 3); }

// Ping-pong schedule, as in the FP8 kernel: group 1 (waves 4-7) one phase
// behind group 0 (waves 0-3), one workgroup barrier per tile, so the two
// waves of a SIMD alternate between
//   X_t: O^T += V^T P_{t-1}^T and its row sums, then S_t^T = K_t Q^T   [matrix cores]
//   Y_t: mask, maxima, rescale, P_t = 2^((S - m) c) -> BF16             [vector ALU]
// Each group copies one operand with direct-to-LDS loads issued at the start
// of its softmax phase: group 1 loads V_t before X_t and waits for it after
// X_t; group 0 loads K_{t+1} after X_t and waits at the end of Y_t; both
// waits precede the barrier after which the tile is first read. Each load
// overwrites a buffer last read before the previous barrier, so double
// buffers suffice; splitting the loads (and their address arithmetic) between
// the groups keeps their softmax phases the same length.
template <int DQK, int BK>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_bf16_kernel(AttnParams p) {
  using L = Bf16Layout<DQK, BK>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[L::kLds];
  uint8_t* const Kbuf = lds;
  uint8_t* const Vbuf = lds + 2 * L::kKTile;

  // the wave index is wave-uniform: keep it (and all phase control) in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int l32 = lane & 31, g = lane >> 5;
  int b, h, qb;
  map_block(p, blockIdx.x, b, h, qb);
  const int S = p.S, Sk = p.Sk, off = Sk - S;  // query i sees keys j <= i + off
  const int kvh = h / p.G;
  const int q0 = qb * kBQ, qw0 = q0 + wave * kQW;
  const int n_tiles = (min(q0 + kBQ, S) + off + BK - 1) / BK;
  const int wave_tiles = qw0 < S ? (min(qw0 + kQW, S) - 1 + off) / BK + 1 : 0;

  const uint32_t q_rs = (uint32_t)p.Hq * DQK * 2, k_rs = (uint32_t)p.Hkv * DQK * 2,
                 v_rs = (uint32_t)p.Hkv * L::kDv * 2;
  const uint8_t* Qg = (const uint8_t*)p.q + (size_t)b * S * q_rs + (size_t)h * DQK * 2;
  const uint8_t* Kg = (const uint8_t*)p.k + (size_t)b * Sk * k_rs + (size_t)kvh * DQK * 2;
  const uint8_t* Vg = (const uint8_t*)p.v + (size_t)b * Sk * v_rs + (size_t)kvh * L::kDv * 2;

  // Q^T operand: lane (query l32, half g) holds Q[q][16t + 8g .. +7] per step t,
  // loaded from global memory once per wave (no other wave uses these rows, so
  // an LDS copy would bring no reuse).
  v8bf qf[DQK / 16];
  {
    const int qrow = qw0 + l32;
#pragma unroll
    for (int t = 0; t < DQK / 16; ++t) {
      v4i x = {0, 0, 0, 0};
      if (qrow < S) x = ld_global16(Qg + ((uint32_t)qrow * q_rs + (16 * t + 8 * g) * 2));
      qf[t] = __builtin_bit_cast(v8bf, x);
    }
  }

  // Loads are issued at the start of a softmax phase, so that no wave starts
  // a matrix phase behind a burst of its own memory instructions.
  constexpr int kLoadWaves = kWaves / 2;
  const int lw = wave & (kLoadWaves - 1);  // index within the wave's group
  auto identity = [](int r) { return r; };
  // per-lane source offsets computed once; each tile goes through a buffer
  // resource from its first key to the end of key Sk - 1 (rows past it: zeros)
  TileLoader<BK, 17, 16, kLoadWaves, 0> kld;
  TileLoader<BK, 9, 8, kLoadWaves, 2> khld;
  TileLoader<BK, 17, 16, kLoadWaves, 0> vld;
  // group 1 copies the first K tile, group 0 all later ones
  kld.init(k_rs, lw, lane, identity);
  if constexpr (L::kHi) khld.init(k_rs, lw, lane, identity);
  if (grp == 1) vld.init(v_rs, lw, lane, vrow_bf16);
  auto issue_k = [&](int t) {
    uint8_t* Kl = Kbuf + (t & 1) * L::kKTile;
    const int k0 = t * BK;
    const uint32_t bytes = (uint32_t)(Sk - k0) * k_rs;
    const uint8_t* src = Kg + (size_t)k0 * k_rs;
    kld.issue(make_rsrc(src, bytes), Kl);
    if constexpr (L::kHi) khld.issue(make_rsrc(src + 256, bytes - 256), Kl + L::kKLoTile);
  };
  auto issue_v = [&](int t) {
    uint8_t* Vl = Vbuf + (t & 1) * L::kVTile;
    const int k0 = t * BK;
    vld.issue(make_rsrc(Vg + (size_t)k0 * v_rs, (uint32_t)(Sk - k0) * v_rs), Vl);
  };

  // V^T operand of v_mfma_f32_32x32x16_bf16 via ds_read_b64_tr_b16: lane
  // (d = 32 db + l%32, half g) needs the keys whose probabilities sit in the P
  // operand: for block sb, step hh and half eh, keys 32 sb + 16 hh + 8 eh +
  // 4 g + 0..3. In 16-lane group G (d0 = 32 db + 16 (G & 1), g = G >> 1),
  // lanes 4 br + w read key ... + br, elements d0 + 4w .. +3; with the row
  // permutation the per-lane part is (4 br + (G >> 1)) rows and the rest is an
  // additive offset of (32 sb + 16 hh + 2 eh) rows + 64 db bytes.
  int vrd;
  {
    const int G = lane >> 4, pp = lane & 15, br = pp >> 2, w = pp & 3;
    vrd = (4 * br + (G >> 1)) * L::kVStride + 32 * (G & 1) + 8 * w;
  }
  // K operand: block sb reads row sb*32 + l32, bytes 32 t16 + 16 g (D columns
  // 16 t16 + 8 g .. +7)
  const int krd = l32 * L::kKLoStride + 16 * g;
  const int khrd = l32 * L::kKHiStride + 16 * g;

  v16f oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) oacc[db] = (v16f){};
  float m = -INFINITY;
  // Row sums of the rounded probabilities on the matrix cores: per 16 keys,
  // one v_mfma_f32_16x16x32_bf16 of a selector against the P operand. Lane l
  // of P holds 8 keys of query l%32; in the 16x16 instruction it supplies
  // column l%16 and the K slots of lane group l/16. The selector (A: row
  // l%16, K slots of group l/16) is 1 where bit 2 of l equals bit 4, so D
  // rows 0-3 and 8-11 add lane groups 0 and 2 (query n) and rows 4-7 and
  // 12-15 groups 1 and 3 (query n + 16); lane l's four D registers (rows
  // 4 (l/16) ..) then all hold the running sum of query l%32. The eight
  // instructions of a tile alternate between two accumulators (rs, rs2), so
  // that issued back to back they do not wait on one another.
  v4f rs = {0.0f, 0.0f, 0.0f, 0.0f}, rs2 = {0.0f, 0.0f, 0.0f, 0.0f};
  v8bf sel;
  {
    const __bf16 e = ((lane >> 2) & 1) == ((lane >> 4) & 1) ? (__bf16)1.0f : (__bf16)0.0f;
    sel = (v8bf){e, e, e, e, e, e, e, e};
  }
  const float c = p.c;

  v16f s[L::kNsb];           // S_t^T, from X_t to Y_t
  v8bf pf[L::kNsb][2];       // P_t as the B operand of the P V instruction, from Y_t to X_{t+1}
#pragma unroll
  for (int sb = 0; sb < L::kNsb; ++sb) pf[sb][0] = pf[sb][1] = (v8bf){};

  // X_t: the matrix phase of tile t (P V of tile t-1, then Q K^T of tile t).
  auto phase_x = [&](int tt) {
    __builtin_amdgcn_s_setprio(1);
    const bool do_pv = tt >= 1 && tt - 1 < wave_tiles;
    const bool do_qk = tt < wave_tiles;
    const uint8_t* Kl = Kbuf + (tt & 1) * L::kKTile;
    const uint8_t* Vl = Vbuf + ((tt - 1) & 1) * L::kVTile;
    // PV step i = (sb * 2 + hh) * 4 + db
    auto read_v = [&](int i) {
      const int db = i & 3, hh = (i >> 2) & 1, sb = i >> 3;
      const uint8_t* vb = Vl + vrd + (32 * sb + 16 * hh) * L::kVStride + 64 * db;
      const v2i lo = __builtin_bit_cast(v2i, lds_read_tr16(vb));
      const v2i hi = __builtin_bit_cast(v2i, lds_read_tr16(vb + 2 * L::kVStride));
      return __builtin_bit_cast(v8bf, (v4i){lo.x, lo.y, hi.x, hi.y});
    };
    // QK step i = t16 * kNsb + sb
    auto read_k = [&](int i) {
      const int sb = i % L::kNsb, t16 = i / L::kNsb;
      const uint8_t* kp = t16 < 8 ? Kl + sb * 32 * L::kKLoStride + krd + 32 * t16
                                  : Kl + L::kKLoTile + sb * 32 * L::kKHiStride + khrd + 32 * (t16 - 8);
      return __builtin_bit_cast(v8bf, ld_lds16(kp));
    };
    constexpr int kPvSteps = L::kNsb * 2 * 4;
    constexpr int kQkSteps = L::kNsb * (DQK / 16);
    // S_{tt-1} was consumed by Y_{tt-1}: end its live range (no instruction)
#pragma unroll
    for (int sb = 0; sb < L::kNsb; ++sb) asm volatile("" : "=v"(s[sb]));
    // Operand fragments are read kDepth MFMA steps ahead of their use (a
    // 32x32x16 BF16 instruction lasts 32 cycles, so two steps would not cover
    // the LDS latency), in one ring that runs from the P V steps into the
    // Q K steps. Ring slots are compile-time constants.
    constexpr int kDepth = 3;
    constexpr int kRing = kDepth + 1;
    v8bf fr[kRing];
    // Q K steps; step i uses ring slot (B + i) % kRing
    auto qk_steps = [&](auto base) {
      constexpr int B = decltype(base)::value;
#pragma unroll
      for (int i = 0; i < kQkSteps; ++i) {
        if (i + kDepth < kQkSteps) fr[(B + i + kDepth) % kRing] = read_k(i + kDepth);
        const int sb = i % L::kNsb;
        s[sb] = mfma_32x32x16_bf16(fr[(B + i) % kRing], qf[i / L::kNsb], i < L::kNsb ? (v16f){} : s[sb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (do_pv) {
#pragma unroll
      for (int j = 0; j < kDepth; ++j) fr[j] = read_v(j);
      __builtin_amdgcn_sched_barrier(0);
      // the row sums first: their operands are in registers, so they run
      // while the first V fragments arrive from LDS
#pragma unroll
      for (int j = 0; j < kPvSteps / 4; ++j) {
        if (j & 1) rs2 = mfma_16x16x32_bf16(sel, pf[j >> 1][j & 1], rs2);
        else rs = mfma_16x16x32_bf16(sel, pf[j >> 1][j & 1], rs);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < kPvSteps; ++i) {
        const int jn = i + kDepth;
        if (jn < kPvSteps)
          fr[jn % kRing] = read_v(jn);
        else if (do_qk)
          fr[jn % kRing] = read_k(jn - kPvSteps);
        oacc[i & 3] = mfma_32x32x16_bf16(fr[i % kRing], pf[i >> 3][(i >> 2) & 1], oacc[i & 3]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if (do_qk) {
#pragma unroll
      for (int j = 0; j < kDepth; ++j) fr[(kPvSteps + j) % kRing] = read_k(j);
    }
    if (do_qk) qk_steps(std::integral_constant<int, kPvSteps>{});
    __builtin_amdgcn_s_setprio(0);
  };

  // Y_t: the softmax phase of tile t.
  auto phase_y = [&](int tt) {
    const int k0 = tt * BK;
    if (k0 + BK - 1 > qw0 + off) {  // the tile crosses this wave's diagonal
      const int d = qw0 + off - k0 + l32 - 4 * g;
#pragma unroll
      for (int sb = 0; sb < L::kNsb; ++sb) mask_block_causal(s[sb], d - 32 * sb);
    }
    float mt = s[0][0];
#pragma unroll
    for (int sb = 0; sb < L::kNsb; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[sb][r]);
    mt = max_xor32(mt);
    // Lazy running max: the reference m moves (and the accumulators are
    // rescaled) only when the tile max exceeds it by more than 8 binades;
    // probabilities up to 2^8 are exact in BF16's range and O / l does not
    // depend on the reference point.
    const float mn = (mt - m) * c > 8.0f ? mt : m;
    const float alpha = (m == mn) ? 1.0f : __builtin_amdgcn_exp2f((m - mn) * c);
    m = mn;
    const float nmc = -mn * c;
    if (__any(alpha != 1.0f)) {
      // keep this a real branch: the multiplies are skipped on most tiles
      asm volatile("" ::: "memory");
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
      rs *= alpha;
      rs2 *= alpha;
    }
    // P = 2^(S c - m c) rounded to BF16 (the next matrix phase adds the row
    // sums of exactly these rounded weights)
#pragma unroll
    for (int sb = 0; sb < L::kNsb; ++sb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t pw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * hh + 2 * e;
          pw[e] = pack_bf16(__builtin_amdgcn_exp2f(fmaf(s[sb][r], c, nmc)),
                            __builtin_amdgcn_exp2f(fmaf(s[sb][r + 1], c, nmc)));
        }
        pf[sb][hh] = __builtin_bit_cast(v8bf, (v4i){(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3]});
      }
    }
  };

  if (grp == 1) issue_k(0);
  wait_vmem();
  lds_barrier();

  // One copy of the tile loop per group (simpler live ranges), one barrier
  // B_t per tile. Group 0 stages K tiles, group 1 V tiles; between B_{t-1}
  // and B_t, K_{t+1} and V_t overwrite the buffers of K_{t-1} and V_{t-2},
  // last read by X_{t-1} before B_{t-1}, while X_t reads K_t and V_{t-1}.
  if (grp == 0) {
    for (int t = 0; t <= n_tiles; ++t) {
      phase_x(t);                              // X_t
      if (t < n_tiles) {                       // Y_t, loads K_{t+1}
        if (t + 1 < n_tiles) issue_k(t + 1);
        if (t < wave_tiles) phase_y(t);
        wait_vmem();                           // K_{t+1} is first read in X_{t+1}
      }
      lds_barrier();                           // B_t
    }
  } else {
    for (int t = 0; t <= n_tiles; ++t) {
      if (t < n_tiles) issue_v(t);            // Y_{t-1}, loads V_t
      if (t >= 1 && t - 1 < wave_tiles) phase_y(t - 1);
      phase_x(t);                              // X_t
      if (t < n_tiles) wait_vmem();            // V_t is first read in X_{t+1}
      lds_barrier();                           // B_t
    }
  }

  // ---- epilogue
  const float l_tot = rs[0] + rs2[0];
  uint8_t* Ol = lds + wave * kQW * kOStride;
  if (wave_tiles > 0) {
    const float inv = p.dv / l_tot;
    // log-sum-exp of the row's logits: sum_j 2^(c s_j) = 2^(c m) l
    if (p.lse != nullptr && g == 0 && qw0 + l32 < S)
      p.lse[((size_t)b * p.Hq + h) * S + qw0 + l32] = (m * c + __builtin_amdgcn_logf(l_tot)) * kLn2;
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
    uint8_t* Og = (uint8_t*)p.out + ((size_t)b * S * p.Hq + h) * (L::kDv * 2);
    const uint32_t o_rs = (uint32_t)p.Hq * L::kDv * 2;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int x = lane + 64 * u, row = x >> 4, cc = x & 15;
      const int qrow = qw0 + row;
      if (qrow < S) *(v4i*)(Og + ((uint32_t)qrow * o_rs + 16 * cc)) = ld_lds16(Ol + row * kOStride + 16 * cc);
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

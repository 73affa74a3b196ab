// attn_fwd_fp8.hip -- causal prefill attention forward, FP8 e4m3 inputs, BF16
// output, for gfx950 (MI355X).
//
// The method [ZYFA abstract, "ZYFA: Speed and Accuracy of FP8 FlashAttention
// on AMD CDNA4" (airebao.com), techniques (1)-(3); spbcomputers.ru ZYFA
// article, section "Три приёма, которые дали ускорение"; captivela.com
// "Zyphra Luncurkan ZYFA", section "Tiga Trik ZYFA Biar Cepat dan Akurat"]:
//  * S = Q K^T and O += P V run on the FP8 matrix cores;
//  * "Lean P": a probability's e4m3 code is written straight from its score:
//    read as an integer, the code of 2^x is about 8x + C, so one fused
//    multiply-add and one float->u8 convert replace the exponential;
//  * each 64-key block of a row gets its own power of two 2^k before
//    rounding, so blocks far below the row max keep normal e4m3 codes; the
//    scaled matrix instruction applies 2^-k through its E8M0 operand scale;
//  * the row sum is taken over the rounded probabilities with one extra
//    matrix instruction against an all-ones operand (16 rows), and the output
//    is divided by it;
//  * two waves share each SIMD and ping-pong: one issues matrix instructions
//    while the other computes probabilities, in an order fixed by the
//    instruction stream.
//
// Readings where the pages leave a step open: C = 55.63 (minimax constant,
// the only narrow window meeting the pages' 7.5 percent bound); the block
// exponent k = floor(8 - t_max), t_max the block's largest log2 probability
// relative to the reference max, kept in [0, 127] (E8M0 range); the reference
// max is updated per 128-key tile, lazily: only when the tile max exceeds it
// by more than 8 binades, and the accumulators are rescaled exactly then.
//
// Tiling (gfx950-specific, not from the pages): a workgroup of 8 waves owns
// 256 consecutive query rows of one head; each wave owns 32 rows. K and V
// tiles of 128 keys are staged in LDS, in three buffers each, and shared by
// the 8 waves.
//  * S^T = K Q^T on v_mfma_scale_f32_32x32x64_f8f6f4 (neutral scales): each
//    lane then holds one query (l%32) and 64 of the tile's keys, so row maxima
//    are in-lane plus one permlane32 swap.
//  * The P codes go straight into the B operand of the same 32x32x64
//    instruction computing O^T = V^T P^T: a lane's 16 scores of one 32-key
//    block become 16 code bytes in accumulator order, two blocks (one 64-key
//    scale block) per instruction, so each lane's scale byte is 127 - k of
//    its own query and block. The V^T operand is read from LDS in the
//    matching key order (ds_read_b64_tr_b8).
//  * The same P operand against an all-ones A operand gives the rounded row
//    sum: one more 32x32x64 instruction per 64-key block (a 16x16x128 one
//    would mix the scales of two queries in one K block).
//  * K and V are copied global -> LDS by direct-to-LDS loads (no staging
//    registers) into row-major tiles of 128-byte rows whose 16-byte chunks
//    are XOR-swizzled per row, so that the reads of the Q K and P V steps
//    (including the transposing reads building the V^T operand) are free of
//    bank conflicts without padding (at head dim 192, K's first 128 columns
//    chunk-major, its last 64 in padded rows).
#include <type_traits>

#include "attn_common.h"
#include "attn_launch.h"

namespace fbc {

constexpr float kLeanPC = 55.63f;
// lazy running-max threshold, in binades (log2 units)
constexpr float kLazyLog2 = 8.0f;

// K[:, 0:128] tile without padding (used at head dim 192): 16-row groups of
// 2 KiB, chunk-major inside a group, so the 16-byte chunk c of row r sits at
// slot 128 (r / 16) + 16 c + r % 16. Sixteen rows' copies of one chunk are
// then 256 contiguous bytes (a conflict-free ds_read_b128 for 16 lanes), the
// reads stay additive in (block, chunk), and a tile is 16 direct-to-LDS
// instructions, four per wave of the loading group. (At head dim 192
// this layout measured 6% faster than padded rows; at 128, K uses the
// swizzled row-major tile below.)
struct KLoLoader {
  static constexpr int kRegs = 4;
  uint32_t off[kRegs];
  int wave;
  template <typename KeyOf>
  __device__ void init(uint32_t row_stride, int wave_, int lane, KeyOf) {
    wave = wave_;
#pragma unroll
    for (int u = 0; u < kRegs; ++u) {
      const int n = (wave + 4 * u) * 64 + lane;  // LDS slot written by this lane
      const int r = ((n >> 7) << 4) | (n & 15), c = (n >> 4) & 7;
      off[u] = (uint32_t)r * row_stride + 16u * (uint32_t)c;
    }
  }
  __device__ void issue_spare(rsrc_t r, uint32_t lds_tile, uint32_t, int u) const {
    buf_load_lds16_at(r, off[u], lds_tile + (uint32_t)(wave + 4 * u) * 1024u);
  }
};

// Tiles of 128-byte rows without padding (K at head dim 128, V at both head
// dims): the 16-byte chunk c of row r sits at byte r * 128 + 16 (c ^ swz(r)).
// A 1 KiB direct-to-LDS instruction then fills 8 whole rows, each lane
// fetching one chunk (8 lanes cover a row's 128 contiguous bytes), and a
// tile is exactly 16 instructions, four per wave of the loading group.
// kswz makes the ds_read_b128 of the Q K steps (lanes 0-31 read rows 0-31 at
// one chunk) free of bank conflicts: any 8 consecutive rows, and the 8 even
// or 8 odd rows of any 16, get distinct chunk positions. vswz does the same
// for the ds_read_b64_tr_b8 of the P V steps, where a 16-lane group reads one
// chunk of the 8 rows {0-3, 8-11} (or {4-7, 12-15}) of a 16-key group and
// two groups read neighbouring chunks of the same rows.
__device__ inline int kswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ inline int vswz(int r) { return (r & 3) | ((r >> 1) & 4); }

template <int NW, int (*Swz)(int)>
struct SwizLoader {
  static constexpr int kRegs = 16 / NW;  // 1 KiB instructions per wave
  static_assert(16 % NW == 0, "a tile is 16 instructions");
  uint32_t off[kRegs];
  int wave;
  template <typename KeyOf>
  __device__ void init(uint32_t row_stride, int wave_, int lane, KeyOf) {
    wave = wave_;
#pragma unroll
    for (int u = 0; u < kRegs; ++u) {
      const int r = 8 * (wave + NW * u) + (lane >> 3), c = (lane & 7) ^ Swz(r);
      off[u] = (uint32_t)r * row_stride + 16u * (uint32_t)c;
    }
  }
  __device__ void issue_spare(rsrc_t r, uint32_t lds_tile, uint32_t, int u) const {
    buf_load_lds16_at(r, off[u], lds_tile + (uint32_t)(wave + NW * u) * 1024u);
  }
};

template <int DQK>
struct Fp8Layout {
  static constexpr int kBK = 128;                     // keys per tile
  static constexpr int kDv = 128;
  static constexpr bool kHi = DQK == 192;             // K columns 128..191 kept apart
  // K[:, 128:192] rows carry one 16-byte padding chunk, so that a row's
  // chunks sit at additive offsets and consecutive rows start in different
  // bank groups.
  static constexpr int kKHiStride = 80;
  static constexpr bool kKCm = kHi;                   // K[:, 0:128] chunk-major (KLoLoader), else swizzled
  static constexpr int kKLoTile = kBK * 128;
  static constexpr int kKHiTile = kHi ? kBK * kKHiStride : 0;
  static constexpr int kKTile = kKLoTile + kKHiTile;
  static constexpr int kVTile = kBK * 128;            // swizzled
  static constexpr int kStages = 3;                   // buffers per operand
  static constexpr int kSpare = kStages * (kKTile + kVTile);  // 1 KiB target of idle loads
  static constexpr int kLoop = kSpare + 1024;
  static constexpr int kEpi = kWaves * kQW * kOStride;
  static constexpr int kLds = kLoop > kEpi ? kLoop : kEpi;
};

// Ping-pong schedule. The workgroup's 8 waves form two groups (waves w and
// w + 4 share a SIMD). Group 0 runs X_t then Y_t, group 1 Y_{t-1} then X_t,
// where a wave's phases alternate
//   X_t: O^T += V^T P_{t-1}^T (and the row-sum MFMAs), then S_t^T = K_t Q^T  [matrix cores]
//   Y_t: softmax of S_t: maxima, block exponents, Lean P codes, rescale       [vector ALU]
// so on every SIMD one wave issues matrix instructions while its partner
// computes probabilities, then they swap. One workgroup barrier per tile,
// after group 0's Y_t and group 1's X_t, orders the tile copies (below); the
// swap in the middle of a tile is left to the instruction stream (a wave that
// finishes its phase early starts the next one, and the matrix wave keeps the
// higher issue priority).
// [spbcomputers.ru ZYFA article and captivela.com "Zyphra Luncurkan ZYFA",
// sections on the three techniques: two waves per SIMD, one on the matrix
// cores while the other computes probabilities, order enforced by the
// instruction stream because the hardware does not track MFMA completion.]
//
// Within X_t the operand fragments are read from LDS two MFMA steps ahead (K
// four at head dim 128) in one ring that runs from the P V steps into the
// Q K steps; the phase starts
// by reading the first two V fragments (the softmax phase, the longer of the
// two, then carries no LDS reads of the next tile). Each tile's row sums come
// from matrix instructions against a ones operand into S's last block, which
// is free until the fourth Q K step; they are issued first, while the V
// fragments arrive (their operands are in registers), and one register of the
// result joins the running sum l. This keeps the registers within budget without spills: a
// spilled register is reloaded through the vector-memory counter, and that
// wait would also cover the tile copies still in flight.
//
// K/V staging (three buffers per operand): each group copies one operand with
// direct-to-LDS instructions issued together at the start of its softmax
// phase (issued later, spread through the phase or in the matrix phase, they
// measured no faster). Between the barriers B_{t-1} and B_t (the one after
// tile t), group 1 loads V_{t+1} during Y_{t-1} and group 0 loads K_{t+2}
// during Y_t, while both groups' X_t read K_t and V_{t-1}: every load
// overwrites a buffer whose last reads (X_{t-1}) ended before B_{t-1}. A wave
// waits for a tile at the end of the softmax phase before the barrier that
// precedes the tile's first read, with the tile it has just issued still in
// flight (vmcnt = one tile's loads). Every softmax phase issues the same
// loads, also for tiles past the workgroup's last (empty range: zeros into a
// free buffer), so that no branch surrounds them.
// MODE: 0 for the method; bit 0 = exact e4m3 rounding of 2^x instead of the
// Lean P code, bit 1 = no per-block exponent (ablations).
template <int DQK, int MODE>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_fp8_kernel(AttnParams p) {
  using L = Fp8Layout<DQK>;
  constexpr bool kExactP = (MODE & 1) != 0;
  constexpr bool kBlockScale = (MODE & 2) == 0;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[L::kLds];
  uint8_t* const Kbuf = lds;                            // kStages x kKTile
  uint8_t* const Vbuf = lds + L::kStages * L::kKTile;   // kStages x kVTile

  // the wave index is wave-uniform: keep it (and all phase control) in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int l32 = lane & 31, g = lane >> 5;
  int b, h, qb;
  map_block(p, blockIdx.x, b, h, qb);
  const int S = p.S, Sk = p.Sk, off = Sk - S;  // query i sees keys j <= i + off
  const int kvh = h / p.G;
  const int q0 = qb * kBQ, qw0 = q0 + wave * kQW;
  const int n_tiles = (min(q0 + kBQ, S) + off + L::kBK - 1) / L::kBK;
  const int wave_tiles = qw0 < S ? (min(qw0 + kQW, S) - 1 + off) / L::kBK + 1 : 0;

  const uint32_t q_rs = (uint32_t)p.Hq * DQK, k_rs = (uint32_t)p.Hkv * DQK, v_rs = (uint32_t)p.Hkv * L::kDv;
  const uint8_t* Qg = (const uint8_t*)p.q + (size_t)b * S * q_rs + (size_t)h * DQK;
  const uint8_t* Kg = (const uint8_t*)p.k + (size_t)b * Sk * k_rs + (size_t)kvh * DQK;
  const uint8_t* Vg = (const uint8_t*)p.v + (size_t)b * Sk * v_rs + (size_t)kvh * L::kDv;

  // Q^T operand of S^T = K Q^T: lane (query l32, half g) holds, per 64-wide
  // step t, Q[q][64t + 16g .. +15] and Q[q][64t + 32 + 16g .. +15]. Q goes
  // straight from global memory into these registers, once per wave: each
  // element is used by one wave only, so staging it in LDS would add a write,
  // a read and a barrier for no reuse, and the 16-byte loads already read
  // each 64-byte step of a row whole (2 lanes x 2 loads per row and step).
  v8i qf[DQK / 64];
  {
    const int qrow = qw0 + l32;
#pragma unroll
    for (int t = 0; t < DQK / 64; ++t) {
      v4i lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
      if (qrow < S) {
        const uint8_t* src = Qg + ((uint32_t)qrow * q_rs + 64 * t + 16 * g);
        lo = ld_global16(src);
        hi = ld_global16(src + 32);
      }
      qf[t] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
  }

  // Each tile goes through a buffer resource that starts at its first key and
  // ends with key Sk - 1: rows past the sequence arrive as zeros (finite
  // values whose keys every stored query masks). Group 0 (waves 0-3) copies K
  // tiles, group 1 (waves 4-7) V tiles.
  constexpr int kGroupWaves = kWaves / 2;
  const int gw = wave & (kGroupWaves - 1);
  std::conditional_t<L::kKCm, KLoLoader, SwizLoader<kGroupWaves, kswz>> kld;
  TileLoader<L::kBK, 5, 4, kGroupWaves, 2> khld;
  SwizLoader<kGroupWaves, vswz> vld;
  constexpr int kKLoads = decltype(kld)::kRegs + (L::kHi ? decltype(khld)::kRegs : 0);
  constexpr int kVLoads = decltype(vld)::kRegs;
  // load u of this wave's share of K tile t (u = 0 .. kKLoads-1)
  // Tiles t >= n_tiles (past the workgroup's last tile) are loaded too, with
  // an empty range: zeros into a buffer the schedule has already freed, so
  // the loads need no branch.
  // The buffer's LDS offset and the descriptors are computed once per tile;
  // the returned issuer takes u = 0 .. kKLoads-1 (K) or kVLoads-1 (V).
  const uint32_t spare = lds_offset(lds) + L::kSpare;
  const uint32_t kbase = lds_offset(Kbuf), vbase = lds_offset(Vbuf);
  auto k_tile = [&](int t) {
    const uint32_t Kl = kbase + ring_offset<L::kStages>(t, L::kKTile);
    const int k0 = t * L::kBK;
    const uint8_t* src = Kg + (size_t)k0 * k_rs;
    const bool live = t < n_tiles;
    const uint32_t bytes = live ? (uint32_t)(Sk - k0) * k_rs : 0u;  // through the end of key row Sk - 1's slot
    const rsrc_t r = make_rsrc(src, bytes);
    const rsrc_t rh = make_rsrc(src + 128, live ? bytes - 128 : 0u);
    return [&, Kl, r, rh](int u) {
      if (u < decltype(kld)::kRegs)
        kld.issue_spare(r, Kl, spare, u);
      else if constexpr (L::kHi)
        khld.issue_spare(rh, Kl + L::kKLoTile, spare, u - decltype(kld)::kRegs);
    };
  };
  auto v_tile = [&](int t) {
    const uint32_t Vl = vbase + ring_offset<L::kStages>(t, L::kVTile);
    const int k0 = t * L::kBK;
    const uint32_t bytes = t < n_tiles ? (uint32_t)(Sk - k0) * v_rs : 0u;
    const rsrc_t r = make_rsrc(Vg + (size_t)k0 * v_rs, bytes);
    return [&, Vl, r](int u) { vld.issue_spare(r, Vl, spare, u); };
  };

  // V^T operand of O^T = V^T P^T (32x32x64): A lane (dv row i, half g) byte
  // 16 h + 4 e + x pairs with the P code of key 32 (2 ks + h) + 8 e + 4 g + x
  // (the key the S^T accumulator of lane (., g) holds in register 4 e + x).
  // Read j (bytes 8j .. 8j+7) covers keys 16 j + 64 ks + {8 e' + 4 g + x}: in
  // each 16-lane group, lanes 2k and 2k+1 address the two 8-byte halves of
  // the 16 dv columns of the k-th of those keys. d-block dvb reads dv columns
  // 32 dvb + 16 (G & 1) .. +15, logical chunk 2 dvb + (G & 1) of the key's row;
  // vrd[dvb] is that chunk's swizzled offset in the lane's row (the swizzle
  // depends on key bits 0, 1 and 3 only, the same for every j and ks).
  int vrd[4];
  {
    const int G = lane >> 4, cc = lane & 15, k = cc >> 1;
    const int key = 8 * (k >> 2) + 4 * (G >> 1) + (k & 3);
    const int h = (G & 1) ^ vswz(key);
#pragma unroll
    for (int dvb = 0; dvb < 4; ++dvb) vrd[dvb] = key * 128 + 16 * ((2 * dvb) ^ h) + 8 * (cc & 1);
  }
  // K operand: block sb reads row sb*32 + l32, logical chunks 4 t6 + g and
  // 4 t6 + 2 + g; krd[q] is the swizzled offset of chunk g + 2q in the lane's
  // row (head dim 128). At head dim 192 the chunk-major part is additive.
  int krd[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    krd[q] = L::kKCm ? (l32 >> 4) * 2048 + g * 256 + (l32 & 15) * 16 + 512 * q : l32 * 128 + 16 * ((g + 2 * q) ^ kswz(l32));
  const int khrd = l32 * L::kKHiStride + 16 * g;

  // PV step i = 4 ks + dvb
  auto read_v = [&](const uint8_t* Vl, int i) {
    const uint8_t* vp = Vl + vrd[i & 3] + 64 * 128 * (i >> 2);
    const v2i r0 = lds_read_tr8(vp);
    const v2i r1 = lds_read_tr8(vp + 16 * 128);
    const v2i r2 = lds_read_tr8(vp + 32 * 128);
    const v2i r3 = lds_read_tr8(vp + 48 * 128);
    return (v8i){r0.x, r0.y, r1.x, r1.y, r2.x, r2.y, r3.x, r3.y};
  };
  // QK step i = t6 * 4 + sb: K rows sb*32 + l32, bytes 64 t6 + 16 g and +32
  auto read_k = [&](const uint8_t* Kl, int i) {
    const int sb = i & 3, t6 = i >> 2;
    if (t6 >= 2) {
      const uint8_t* kp = Kl + L::kKLoTile + sb * 32 * L::kKHiStride + khrd;
      const v4i lo = ld_lds16(kp), hi = ld_lds16(kp + 32);
      return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
    const uint8_t* kp = Kl + sb * 4096;
    const v4i lo = ld_lds16(kp + krd[2 * t6]), hi = ld_lds16(kp + krd[2 * t6 + 1]);
    return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  };

  // O^T in four 32x32 blocks (lane (query l32, g), register r: dv row
  // 32 dvb + 8 (r/4) + 4 g + r%4). l: the query's running sum of the rounded
  // probabilities (each tile's sum comes from a matrix instruction against a
  // ones operand, every register of whose result holds it; only register 0 is
  // kept).
  v16f oacc[4];
  float l = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) oacc[d] = (v16f){};
  float m = -INFINITY;  // running max of the raw scores of query qw0 + l32
  // the base-2 score scale lives in a vector register: as a scalar it would be
  // spilled and reloaded every tile under this kernel's scalar-register pressure
  float c = p.c;
  float dv = p.dv;
  if (p.dscale != nullptr) {
    // dequantisation factors left on the device by the quantize prologue:
    // folded in the same precision and order as the host folds its own
    const double cd = (double)p.scale * p.dscale[0] * p.dscale[2] * 1.4426950408889634;
    c = (float)(cd > 1e-30 ? cd : 1e-30);
    dv = p.dscale[4];
  }
  asm volatile("" : "+v"(c));
  const float c8 = 8.0f * c;

  v16f s[4];     // S_t^T, from X_t to Y_t
  v8i P[2];      // P_t codes (64-key block ks in P[ks]), from Y_t to X_{t+1}
  int sc[2] = {127, 127};  // E8M0 scale bytes of P[0], P[1]: 127 - k
#pragma unroll
  for (int q = 0; q < 2; ++q) P[q] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};

  // X_t: the matrix phase of tile t (P V of tile t-1, then Q K^T of tile t).
  auto phase_x = [&](int tt) {
    // ================= X_tt: matrix phase
    // One operand ring (V two MFMA steps deep, K kKA) runs through the P V
    // steps into the Q K steps; scheduling barriers keep the compiler from hoisting
    // every LDS read of the phase to its top.
    __builtin_amdgcn_s_setprio(1);
    const bool do_pv = tt >= 1 && tt - 1 < wave_tiles;
    const bool do_qk = tt < wave_tiles;
    const uint8_t* Kl = Kbuf + ring_offset<L::kStages>(tt, L::kKTile);
    const uint8_t* Vl = Vbuf + ring_offset<L::kStages>(tt + L::kStages - 1, L::kVTile);
    constexpr int kQkSteps = 4 * (DQK / 64);
    // S_{tt-1} was consumed by Y_{tt-1}: end its live range here (an empty
    // asm definition, no instruction) so it does not occupy registers
    // through the P V half of this phase.
    asm volatile("" : "=v"(s[0]), "=v"(s[1]), "=v"(s[2]), "=v"(s[3]));
    // Q K fragments are read kKA steps ahead (four at head dim 128, where the
    // K reads meet the other waves' operand reads and the tile copies in the
    // LDS and need the longer lead; two at 192, where the registers for a
    // third are not free)
    constexpr int kKA = DQK == 128 ? 4 : 2;
    constexpr int kKR = kKA + 1;
    v8i kf[kKR];
    v8i q0;  // Q fragment 0 for the Q K steps
    // this tile's row sums go through S's block 3, free until Q K step 3
    if (do_pv) {
      const v8i ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                        0x38383838, 0x38383838, 0x38383838, 0x38383838};  // e4m3 1.0
      v8i vf[3];
      vf[0] = read_v(Vl, 0);
      vf[1] = read_v(Vl, 1);
      __builtin_amdgcn_sched_barrier(0);
      // the row sums first: their operands are in registers, so they run
      // while the first V fragments arrive from LDS
      s[3] = mfma_32x32x64_fp8(ones, P[0], (v16f){}, 127, sc[0]);
      __builtin_amdgcn_sched_barrier(0);
      s[3] = mfma_32x32x64_fp8(ones, P[1], s[3], 127, sc[1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ks = i >> 2, dvb = i & 3;
        if (i + 2 < 8) vf[(i + 2) % 3] = read_v(Vl, i + 2);
        if (i >= 8 - kKA) kf[i - (8 - kKA)] = read_k(Kl, i - (8 - kKA));  // the first Q K steps
        if (i == 7) q0 = qf[0];
        oacc[dvb] = mfma_32x32x64_fp8(vf[i % 3], P[ks], oacc[dvb], 127, sc[ks]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kKA; ++j) kf[j] = read_k(Kl, j);
      q0 = qf[0];
      s[3] = (v16f){};
    }
    if (do_qk) {
#pragma unroll
      for (int i = 0; i < kQkSteps; ++i) {
        if (i + kKA < kQkSteps) kf[(i + kKA) % kKR] = read_k(Kl, i + kKA);
        if (i == 3) l += s[3][0];  // three steps after the row-sum instruction
        s[i & 3] = mfma_32x32x64_fp8(kf[i % kKR], i < 4 ? q0 : qf[i >> 2], i < 4 ? (v16f){} : s[i & 3], 127, 127);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      l += s[3][0];
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // Y_t: the softmax phase of tile t. ld(u), u = 0..7, issues this wave's
  // u-th tile load of the phase (or nothing).
  auto phase_y = [&](int tt, auto&& ld) {
    // ================= Y_tt: softmax phase
    const int k0 = tt * L::kBK;
#pragma unroll
    for (int u = 0; u < 8; ++u) ld(u);  // this phase's tile loads, first
    __builtin_amdgcn_sched_barrier(0);
    if (k0 + L::kBK - 1 > qw0 + off) {  // the tile crosses this wave's diagonal (or lies past it)
      const int d = qw0 + off - k0 + l32 - 4 * g;
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) mask_block_causal(s[sb], d - 32 * sb);
    }
    // per-(row, 64-key block) maxima and the running max
    // (four independent chains, one per 32x32 block)
    float ma0 = s[0][0], ma1 = s[1][0], mb0 = s[2][0], mb1 = s[3][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      ma0 = fmaxf(ma0, s[0][r]);
      ma1 = fmaxf(ma1, s[1][r]);
      mb0 = fmaxf(mb0, s[2][r]);
      mb1 = fmaxf(mb1, s[3][r]);
    }
    float ma = fmaxf(ma0, ma1), mb = fmaxf(mb0, mb1);
    max_xor32_pair(ma, mb);
    // Lazy running max: the reference m moves (and the accumulators are
    // rescaled) only when the tile max exceeds it by more than kLazyLog2
    // binades; otherwise probabilities up to 2^kLazyLog2 are encoded relative
    // to the old m, which the per-block exponent absorbs (k >= 0 keeps every
    // code <= 120). O / l does not depend on the reference point.
    // (Without block exponents the reference max moves on every rise, so the
    // encoded probabilities stay in [0, 1]: the plain FP8 softmax.)
    constexpr float kLazy = kBlockScale ? kLazyLog2 : 0.0f;
    const float mt = fmaxf(ma, mb);
    const bool rises = (mt - m) * c > kLazy;
    // move the reference and rescale the accumulators when it rises (rare:
    // the factor and its exponential are computed only then)
    if (__any(rises)) {
      // keep this a real branch: the multiplies are skipped on most tiles
      asm volatile("" ::: "memory");
      const float mn = rises ? mt : m;
      const float alpha = rises ? __builtin_amdgcn_exp2f((m - mn) * c) : 1.0f;
      m = mn;
#pragma unroll
      for (int d = 0; d < 4; ++d) oacc[d] *= alpha;
      l *= alpha;
    }
    const float mn = m;
    // block exponents: the block max lands in (2^7, 2^8]
    const float ka = kBlockScale ? fminf(fmaxf(floorf(8.0f - (ma - mn) * c), 0.0f), 127.0f) : 0.0f;
    const float kb = kBlockScale ? fminf(fmaxf(floorf(8.0f - (mb - mn) * c), 0.0f), 127.0f) : 0.0f;
    // Lean P: code = u8(8 c s + C + 8k - 8 c m); exact (ablation): the e4m3
    // rounding of 2^(c s + k - c m). Four codes per dword, in accumulator
    // order: P[ks] dword d holds registers 4(d%4) .. +3 of s[2 ks + d/4].
    const float bias_a = kExactP ? fmaf(-c, mn, ka) : fmaf(-c8, mn, kLeanPC + 8.0f * ka);
    const float bias_b = kExactP ? fmaf(-c, mn, kb) : fmaf(-c8, mn, kLeanPC + 8.0f * kb);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const float bias = ks == 0 ? bias_a : bias_b;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {  // block s[2 ks + hb] -> dwords 4 hb .. 4 hb + 3 of P[ks]
        const v16f& sv = s[2 * ks + hb];
        if constexpr (kExactP) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x0 = __builtin_amdgcn_exp2f(fmaf(sv[4 * j + 0], c, bias));
            const float x1 = __builtin_amdgcn_exp2f(fmaf(sv[4 * j + 1], c, bias));
            const float x2 = __builtin_amdgcn_exp2f(fmaf(sv[4 * j + 2], c, bias));
            const float x3 = __builtin_amdgcn_exp2f(fmaf(sv[4 * j + 3], c, bias));
            uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
            w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, (int)w, true);
            P[ks][4 * hb + j] = (int)w;
          }
        } else {
          // the four dwords are built side by side (multiply-adds for byte x,
          // then the four converts inserting it), so that no instruction
          // waits on the one just before it
          uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            float f[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) f[j] = fmaf(sv[4 * j + x], c8, bias);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = __builtin_amdgcn_cvt_pk_u8_f32(f[j], x, w[j]);
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) P[ks][4 * hb + j] = (int)w[j];
        }
      }
    }
    sc[0] = 127 - (int)ka;
    sc[1] = 127 - (int)kb;
  };

  if (grp == 0) {
    auto identity = [](int r) { return r; };
    kld.init(k_rs, gw, lane, identity);
    if constexpr (L::kHi) khld.init(k_rs, gw, lane, identity);
#pragma unroll
    for (int u = 0; u < kKLoads; ++u) {
      k_tile(0)(u);
      k_tile(1)(u);
    }
  } else {
    vld.init(v_rs, gw, lane, 0);
#pragma unroll
    for (int u = 0; u < kVLoads; ++u) {
      v_tile(0)(u);
      v_tile(1)(u);
    }
  }
  wait_vmem();
  lds_barrier();

  // Each group runs its own copy of the tile loop, so that S never has to
  // stay live across the loop's back edge in group 0 and P never in group 1.
  // Both copies execute one barrier per tile. Every wave runs a softmax phase
  // for every tile of the workgroup's range, also past its own diagonal (all
  // keys masked there) or with all of its rows past S (never stored): the
  // phase carries the group's tile loads, and the probabilities it makes are
  // never used.
  if (grp == 0) {
    for (int t = 0; t <= n_tiles; ++t) {
      phase_x(t);                              // X_t
      if (t < n_tiles) {                       // Y_t, loads K_{t+2}
        const auto ldk = k_tile(t + 2);
        phase_y(t, [&](int u) {
          if (u < kKLoads) ldk(u);
        });
        wait_vmem_all_but<kKLoads>();          // K_{t+1} (loaded in Y_{t-1}), first read in X_{t+1}
      }
      lds_barrier();                           // B_t
    }
  } else {
    for (int t = 0; t <= n_tiles; ++t) {
      if (t >= 1) {                            // Y_{t-1}, loads V_{t+1}
        const auto ldv = v_tile(t + 1);
        phase_y(t - 1, [&](int u) {
          if (u < kVLoads) ldv(u);
        });
        wait_vmem_all_but<kVLoads>();          // V_t (loaded in Y_{t-2}), first read in X_{t+1}
      }
      phase_x(t);                              // X_t
      lds_barrier();                           // B_t
    }
  }
  // the last loads (of tiles past the range) write LDS that the epilogue reuses
  wait_vmem();
  lds_barrier();

  // ---- epilogue: O / l * dv -> BF16, staged through LDS for coalesced rows.
  uint8_t* Ol = lds + wave * kQW * kOStride;
  if (wave_tiles > 0) {
    const float inv = dv / l;
    // log-sum-exp of the row's logits: sum_j 2^(c s_j) = 2^(c m) l
    if (p.lse != nullptr && g == 0 && qw0 + l32 < S)
      p.lse[((size_t)b * p.Hq + h) * S + qw0 + l32] = (m * c + __builtin_amdgcn_logf(l)) * kLn2;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int col = 32 * d + 8 * e + 4 * g;
        const v2i w = {(int)pack_bf16(oacc[d][4 * e] * inv, oacc[d][4 * e + 1] * inv),
                       (int)pack_bf16(oacc[d][4 * e + 2] * inv, oacc[d][4 * e + 3] * inv)};
        *(v2i*)(Ol + l32 * kOStride + col * 2) = w;
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

template <int DQK, int MODE>
static hipError_t launch_fp8(const AttnParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<DQK, MODE>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int DQK>
static hipError_t launch_fp8_mode(const AttnParams& p, int mode, int grid, hipStream_t stream) {
  switch (mode) {
    case 0: return launch_fp8<DQK, 0>(p, grid, stream);
    case 1: return launch_fp8<DQK, 1>(p, grid, stream);
    case 2: return launch_fp8<DQK, 2>(p, grid, stream);
    default: return launch_fp8<DQK, 3>(p, grid, stream);
  }
}

hipError_t launch_attn_fwd_fp8(const AttnParams& p, int dqk, int mode, int grid, hipStream_t stream) {
  if (dqk == 128) return launch_fp8_mode<128>(p, mode, grid, stream);
  return launch_fp8_mode<192>(p, mode, grid, stream);
}

}  // namespace fbc

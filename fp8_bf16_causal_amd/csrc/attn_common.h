// attn_common.h -- shared pieces of the gfx950 causal prefill attention kernels:
// vector types, matrix-core and cross-lane wrappers, LDS helpers and the
// workgroup -> (batch, head, query block) mapping (the launch parameter block
// is in attn_params.h).
//
// Register layouts used throughout (gfx950, wave64; measured on the device):
//  * v_mfma_f32_32x32x16_bf16: A lane (i = l%32, g = l/32) holds A[i][8g .. 8g+7],
//    B lane (j, g) holds B[8g .. 8g+7][j]; D lane (j = l%32, g) register r holds
//    D[8(r/4) + 4g + r%4][j].
//  * v_mfma_scale_f32_32x32x64_f8f6f4: a lane's bytes 0-15 are K-half 0 and
//    bytes 16-31 K-half 1 (byte b of A lane (i, g) pairs with byte b of B lane
//    (j, g)); the E8M0 scale of (row or column i, K-half kb) is the byte taken
//    from lane i + 32*kb. D layout as for the 32x32 bf16 instruction.
//  * v_mfma_scale_f32_16x16x128_f8f6f4: lane (i = l%16, g = l/16) bytes 0-15
//    cover K in [0, 64), bytes 16-31 cover K in [64, 128); the scale of
//    (i, 32-wide K block kb) comes from lane i + 16*kb. D lane (j = l%16, g)
//    register r holds D[4g + r][j].
//  * v_mfma_f32_16x16x32_bf16: A lane (i = l%16, g = l/16) holds row i at the
//    K slots of lane group g, B lane (j, g) column j at the same K slots; D
//    lane (j = l%16, g) register r holds D[4g + r][j].
//  * buffer_load_dwordx4 ... lds: lane l's 16 bytes land at M0 + 16 l; lanes
//    whose offset lies past the buffer resource's range write zeros.
//  * ds_read_b64_tr_b8: within each 16-lane group, lanes 2b and 2b+1 supply
//    the addresses of the two 8-byte halves of "row" b (b = 0..7); lane c
//    receives byte c of each of the 8 rows.
//  * ds_read_b64_tr_b16: within each 16-lane group, lanes 4b..4b+3 supply the
//    four 8-byte quarters of row b (b = 0..3); lane c receives element c of
//    each of the 4 rows.
//  * v_permlane32_swap(x, y): x' = [x.lo32, y.lo32], y' = [x.hi32, y.hi32].
//  * v_permlane16_swap(x, y) on 16-lane rows R0..R3:
//    x' = [x.R0, y.R0, x.R2, y.R2], y' = [x.R1, y.R1, x.R3, y.R3].
//  * v_cvt_pk_u8_f32 rounds half to even and saturates to [0, 255]; -inf and
//    NaN give 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_params.h"

namespace fbc {

typedef __attribute__((address_space(3))) uint8_t lds_u8;

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.69314718055994531f;

// Workgroup -> (batch, query head, query block). Heaviest (latest) query blocks
// first, so the causal tail finishes on light work. Workgroups are dispatched
// to XCDs round-robin (bid % 8); when the KV heads split evenly over the XCDs,
// each XCD takes whole KV heads and walks them one at a time, so the
// workgroups resident on an XCD stream the same K/V tiles through its L2.
__device__ inline void map_block(const AttnParams& p, int bid, int& b, int& h, int& qb) {
  const int per_head = p.G * p.nqb;
  int kvh, s;
  if (p.xcd_group) {
    const int x = bid % kXcds, slot = bid / kXcds;
    kvh = x + kXcds * (slot / per_head);
    s = slot % per_head;
    qb = p.nqb - 1 - s / p.G;
  } else {
    const int nkv = p.B * p.Hkv;
    qb = p.nqb - 1 - bid / (nkv * p.G);
    s = bid % (nkv * p.G);
    kvh = s / p.G;
  }
  const int gi = s % p.G;
  b = kvh / p.Hkv;
  h = (kvh % p.Hkv) * p.G + gi;
}

__device__ inline v16f mfma_32x32x64_fp8(v8i a, v8i b, v16f c, int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}
__device__ inline v16f mfma_32x32x16_bf16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline v4f mfma_16x16x32_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ inline float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ inline uint32_t as_u(float f) { return __builtin_bit_cast(uint32_t, f); }

// max over the two 32-lane halves: every lane gets max(x[l], x[l ^ 32])
__device__ inline float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(as_u(x), as_u(x), false, false);
  return fmaxf(as_f(r[0]), as_f(r[1]));
}
// The maxima over lanes l and l ^ 32 of two values at once: two swaps of
// lane halves instead of two per value.
__device__ inline void max_xor32_pair(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(as_u(a), as_u(b), false, false);
  const float t = fmaxf(as_f(r[0]), as_f(r[1]));  // lanes 0-31: max of a, lanes 32-63: max of b
  const auto u = __builtin_amdgcn_permlane32_swap(as_u(t), as_u(t), false, false);
  a = as_f(u[0]);
  b = as_f(u[1]);
}
// Causal mask of one 32x32 block of S^T (32 keys x 32 queries, accumulator
// layout): register r of lane (query l32, half g) holds key 8 (r/4) + 4 g +
// r%4 of the block. With d = (query - first key of the block) - 4 g, that key
// is hidden iff d < 8 (r/4) + r%4, and its score becomes -inf. One element at
// a time through VCC, two wait states between the compare and the select: the
// compiler's own form keeps 16 lane masks in scalar register pairs at once,
// which crowds the scalar register file of these kernels.
__device__ inline void mask_block_causal(v16f& s, int d) {
  const float ninf = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float x = s[r];
    asm volatile("v_cmp_gt_i32 vcc, %2, %1\n\ts_nop 1\n\tv_cndmask_b32 %0, %0, %3, vcc"
                 : "+v"(x)
                 : "v"(d), "i"(8 * (r >> 2) + (r & 3)), "v"(ninf)
                 : "vcc");
    s[r] = x;
  }
}


__device__ inline v2i lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(lds_u8*)p);
}
__device__ inline v4s lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(lds_u8*)p);
}

__device__ inline v4i ld_global16(const uint8_t* p) { return *(const v4i*)p; }

// s_waitcnt vmcnt(0): every vector-memory load of this wave (including
// direct-to-LDS ones) has completed.
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): all but this wave's N most recently issued vector-memory
// loads have completed (they complete in issue order).
template <int N>
__device__ inline void wait_vmem_all_but() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | 0x0F70 | (N & 15));
}
// Workgroup barrier without a memory fence. __syncthreads() also waits for
// every outstanding global load of the wave (vmcnt(0)), which would stall each
// slot on the direct-to-LDS loads still in flight for a later slot. This one
// waits only for the wave's own LDS operations (no LDS read may still be in
// flight when another wave overwrites a buffer after the barrier); callers
// wait_vmem() before the barrier that publishes a direct-to-LDS tile. The
// memory clobber keeps the compiler from moving memory accesses across it.
// The LDS wait is the compiler's own instruction rather than part of the asm,
// so the compiler knows that no LDS read is pending after the barrier and
// inserts no wait of its own before the first LDS reads of the next phase.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
  asm volatile("s_barrier" ::: "memory");
}
// Buffer resource (raw, no stride) over `bytes` bytes from `base`. The
// hardware range-checks every lane of a buffer load against it: lanes at or
// past the end read zero instead of memory. Word 3 is the gfx9 default
// (32-bit data format).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// buffer_load_dwordx4 ... lds: lane l's 16 bytes from voff land at
// lds_base + 16 l (lds_base wave-uniform); out-of-range lanes write zeros.
__device__ inline void buf_load_lds16(rsrc_t r, uint32_t voff, uint8_t* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds_u8*)lds_base, 16,
                                           (int)voff, 0, 0, 0);
}
// The same with the LDS destination as a byte offset into the workgroup's LDS
// (no generic-pointer conversion, so no null check on the way).
__device__ inline uint32_t lds_offset(const uint8_t* p) { return (uint32_t)(uintptr_t)(const lds_u8*)p; }
__device__ inline void buf_load_lds16_at(rsrc_t r, uint32_t voff, uint32_t lds_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(uintptr_t)lds_off, 16,
                                           (int)voff, 0, 0, 0);
}

// Direct-to-LDS copy of a key tile through a buffer resource whose range ends
// at the sequence's last row, so rows past it arrive as zeros. LDS row r has
// CS 16-byte chunks: the first CD hold bytes [0, 16 CD) of key row key_of(r)
// (relative to the resource's first row); the lanes writing the padding
// chunks read from out of range, so they write zeros and fetch nothing. The
// per-lane source offsets are computed once, so issuing a tile costs no
// vector instructions. The kInsts 1 KiB instructions
// are dealt round-robin to the NW waves; the remainder goes to the waves
// whose (wave + ROT) % NW is below it, so that loaders with different ROT
// balance each other.
template <int ROWS, int CS, int CD, int NW, int ROT>
struct TileLoader {
  static constexpr int kInsts = ROWS * CS / 64;
  static constexpr int kFull = kInsts / NW;
  static constexpr int kRem = kInsts % NW;
  static constexpr int kRegs = kFull + (kRem ? 1 : 0);
  static_assert(ROWS * CS % 64 == 0, "tile must be a whole number of 1 KiB loads");
  uint32_t off[kRegs];
  int wave;
  int rem_inst;  // index of this wave's remainder instruction, or -1 (wave-uniform)

  template <typename KeyOf>
  __device__ static uint32_t lane_offset(int i, int lane, uint32_t row_stride, KeyOf key_of) {
    const int n = i * 64 + lane, r = n / CS, pos = n - r * CS;
    return pos < CD ? (uint32_t)key_of(r) * row_stride + 16u * (uint32_t)pos : kOutOfRange;
  }
  template <typename KeyOf>
  __device__ void init(uint32_t row_stride, int wave_, int lane, KeyOf key_of) {
    wave = wave_;
#pragma unroll
    for (int u = 0; u < kFull; ++u) off[u] = lane_offset(wave + NW * u, lane, row_stride, key_of);
    rem_inst = -1;
    if constexpr (kRem != 0) {
      const int rw = (wave + ROT) % NW;
      rem_inst = rw < kRem ? kFull * NW + rw : -1;
      // a wave without a remainder instruction issues one anyway, out of
      // range (its lanes write zeros to a spare LDS area): see issue_spare
      off[kFull] = rem_inst < 0 ? kOutOfRange : lane_offset(rem_inst, lane, row_stride, key_of);
    }
  }
  // a source offset past any buffer resource's range (ranges stay below 2^31)
  static constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;
  // r: resource whose byte 0 is the tile's first key row and whose range ends
  // with the sequence's last row
  __device__ void issue(rsrc_t r, uint8_t* lds_tile) const {
#pragma unroll
    for (int u = 0; u < kRegs; ++u) issue_one(r, lds_tile, u);
  }
  // instruction u (0 .. kRegs-1) of this wave's share; u must be a constant
  __device__ void issue_one(rsrc_t r, uint8_t* lds_tile, int u) const {
    if (u < kFull)
      buf_load_lds16(r, off[u], lds_tile + (wave + NW * u) * 1024);
    else if (rem_inst >= 0)
      buf_load_lds16(r, off[kFull], lds_tile + rem_inst * 1024);
  }
  // The same without a branch: every wave issues kRegs instructions (so a
  // vmcnt wait can count one tile's loads); one without a remainder
  // instruction sends its last to `spare` (1 KiB of LDS nobody reads), from
  // out of range, so it writes zeros there.
  // lds_tile and spare are LDS byte offsets
  __device__ void issue_spare(rsrc_t r, uint32_t lds_tile, uint32_t spare, int u) const {
    if (u < kFull)
      buf_load_lds16_at(r, off[u], lds_tile + (uint32_t)(wave + NW * u) * 1024u);
    else
      buf_load_lds16_at(r, off[kFull], rem_inst >= 0 ? lds_tile + (uint32_t)rem_inst * 1024u : spare);
  }
};

// Byte offset of buffer (t mod N) in a ring of N buffers of `bytes` each.
// The index passes through an empty asm statement so that the compiler treats
// it as an opaque scalar: otherwise it strength-reduces every LDS address
// built from it into a register of its own.
template <int N>
__device__ inline int ring_offset(int t, int bytes) {
  int i = t % N;
  asm volatile("" : "+s"(i));
  return i * bytes;
}

__device__ inline v4i ld_lds16(const uint8_t* p) { return *(const v4i*)p; }

__device__ inline uint32_t pack_bf16(float lo, float hi) {
  v2bf v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace fbc

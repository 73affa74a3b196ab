/*
 * fp8_bf16_causal.h -- C ABI of the MI355X (gfx950) causal prefill attention
 * forward library, libfp8_bf16_causal.so.
 *
 * The operation: causal prefill FlashAttention forward,
 *   out = softmax(Q K^T * scale + causal mask) V,
 * with BF16 or FP8 e4m3 inputs and BF16 output, for one MI355X.
 *   [ZYFA abstract, "ZYFA: Speed and Accuracy of FP8 FlashAttention on AMD
 *    CDNA4" (airebao.com page): prefill kernels for the MI355X, FlashAttention
 *    with the softmax between the two matrix products;
 *    spbcomputers.ru ZYFA article, opening paragraphs and FAQ: causal forward
 *    only, FP8 e4m3 and BF16, an interface compatible with flash_attn_func,
 *    no decode and no paged KV.]
 *
 * Conventions (flash_attn_func's public ones, where the pages give none):
 *   - layout (batch, seq, heads, dim), contiguous:
 *       q   [B][S][Hq][Dqk]
 *       k   [B][S][Hkv][Dqk]
 *       v   [B][S][Hkv][Dv]
 *       out [B][S][Hq][Dv]   always BF16
 *   - grouped-query attention: query head h reads KV head h / (Hq / Hkv);
 *   - queries and keys have the same length S; key j is visible to query i
 *     iff j <= i;
 *   - FP8 inputs are OCP e4m3fn codes (torch.float8_e4m3fn) with one
 *     dequantisation factor per tensor: the score scale is scale*dq*dk and dv
 *     multiplies the output.
 *
 * FP8 softmax: each probability's e4m3 code is written directly from its
 * score with one multiply-add and one integer convert (the code of 2^x is
 * about 8x plus a constant); each 64-key block of a row is scaled by a power
 * of two before rounding and the scaled matrix instruction removes the factor;
 * the output is divided by the sum of the already-rounded probabilities.
 *   [spbcomputers.ru ZYFA article, section "Три приёма, которые дали
 *    ускорение"; captivela.com "Zyphra Luncurkan ZYFA", section "Tiga Trik
 *    ZYFA Biar Cepat dan Akurat"; ZYFA abstract, techniques (1) and (3).]
 *
 * Memory and threading: every pointer is device memory owned by the caller.
 * The library allocates nothing, keeps no pointer after returning and needs
 * no workspace. Calls are asynchronous: they return once the kernel is
 * enqueued on the stream; out is valid after the stream synchronises. Calls
 * on different streams are independent; the library holds no mutable state.
 *
 * Errors: every entry point returns an int; nothing else crosses the ABI.
 * Arguments are checked on the host before anything is enqueued; on an error
 * return nothing was launched and out is untouched.
 */
#ifndef FP8_BF16_CAUSAL_H
#define FP8_BF16_CAUSAL_H

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k and v. out is always BF16. */
enum { ATTN_BF16 = 0, ATTN_FP8_E4M3 = 1 };

/*
 * attn_fwd_ex flags: ablations of the FP8 softmax (dtype ATTN_FP8_E4M3 only).
 * They reproduce the comparisons the pages draw [spbcomputers.ru ZYFA
 * article, sections "Три приёма, которые дали ускорение" and "Точность":
 * exact e4m3 rounding of each probability versus the one-FMA code, 5.9 versus
 * 7.5 percent worst-case error, and matrix-core busy time; captivela.com
 * "Zyphra Luncurkan ZYFA", section "Tiga Trik ZYFA Biar Cepat dan Akurat",
 * third trick: per-block scaling for blocks far below the row maximum].
 *   ATTN_FLAG_EXACT_P        each probability is 2^x evaluated in fp32 and
 *                            rounded to e4m3 (nearest, ties to even) instead
 *                            of the one-FMA code
 *   ATTN_FLAG_NO_BLOCKSCALE  no per-64-key-block power of two: every block
 *                            keeps exponent 0 (plain probabilities in [0, 1])
 * The two may be combined.
 */
enum { ATTN_FLAG_EXACT_P = 1u, ATTN_FLAG_NO_BLOCKSCALE = 2u };

/*
 * ATTN_FLAG_DESCALE_DEVICE (dtype ATTN_FP8_E4M3 only; combines with the
 * ablation flags): descale_qkv is a device pointer (4-byte aligned) to six
 * floats {dq, amax_q, dk, amax_k, dv, amax_v}, the layout three
 * attn_quantize_e4m3 calls produce when their scale buffers lie back to back
 * (scale, scale + 2, scale + 4). The kernels read dq, dk and dv at launch, so
 * a caller can quantise Q, K and V and run the attention on one stream, or in
 * one graph, with no host round trip. The factors are not validated (a
 * quantize call always writes finite positive ones); the score scale is folded
 * exactly as for host factors, so the output is bit-identical to a call with
 * the same values passed from the host. Reading the pages: the factors are the
 * per-tensor scales of the quantisation step [spbcomputers.ru ZYFA article,
 * section "Точность: ошибка FP8 ниже, чем у AITER"].
 */
enum { ATTN_FLAG_DESCALE_DEVICE = 4u };

/* Return codes. */
enum {
  ATTN_OK = 0,
  /* a null or misaligned pointer (q, k, v, out must be 16-byte aligned), a
   * size <= 0, Hq not a multiple of Hkv, scale negative or not finite, a
   * descale factor <= 0 or not finite, a score scale scale*dq*dk*log2(e)
   * beyond the float range, a flags word with unknown bits, a null or
   * misaligned descale_qkv with ATTN_FLAG_DESCALE_DEVICE, or sizes whose
   * products overflow the index types (one batch entry of q, k, v or out must
   * stay below 4 GiB; the workgroup count B*Hq*ceil(S/256) below 2^31) */
  ATTN_ERR_INVALID = -1,
  /* causal == 0 (the method is causal-only), an unknown dtype, a head-dim
   * pair other than (Dqk, Dv) = (128, 128) or (192, 128), flags with dtype
   * ATTN_BF16, or a current device that is not gfx950 */
  ATTN_ERR_UNSUPPORTED = -2,
  /* the HIP runtime reported an error when querying the device or launching */
  ATTN_ERR_LAUNCH = -3
};

/*
 * attn_fwd: causal prefill attention forward on the current device's null
 * stream, with all dequantisation factors equal to 1.
 *
 *   q, k, v  device pointers to the inputs, dtype elements, layout above
 *   out      device pointer to B*S*Hq*Dv BF16 values (written entirely)
 *   B, Hq, Hkv, S, Dqk, Dv   sizes; Hq % Hkv == 0
 *   causal   must be 1
 *   scale    softmax scale (flash_attn_func's default is 1/sqrt(Dqk)), >= 0
 *   dtype    ATTN_BF16 or ATTN_FP8_E4M3
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int S, int Dqk,
             int Dv, int causal, float scale, int dtype);

/*
 * attn_fwd_ex: attn_fwd with per-tensor dequantisation factors and a stream.
 *
 *   descale_qkv  host pointer to {dq, dk, dv}, or NULL for {1, 1, 1}; read
 *                during the call only (with ATTN_FLAG_DESCALE_DEVICE: a device
 *                pointer to six floats, read by the kernels, see above)
 *   stream       a hipStream_t created on the current device (the device the
 *                pointers belong to and whose architecture is checked), or
 *                NULL for that device's null stream
 *   flags        0, or ATTN_FLAG_* bits (FP8 only): ablations of the FP8
 *                softmax, device-resident dequantisation factors
 */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* out, int B, int Hq, int Hkv, int S, int Dqk,
                int Dv, int causal, float scale, int dtype, const float* descale_qkv, void* stream,
                unsigned flags);

/*
 * attn_fwd_lse: attn_fwd_ex that also writes each row's log-sum-exp, the
 * second result a merge of partial attention over key ranges needs (as in a
 * context-parallel split of the keys: O = sum_r exp(lse_r - lse) O_r with
 * lse = ln sum_r exp(lse_r)). The pages do not describe this output; it is
 * read from the online-softmax state every forward kernel keeps (the running
 * max m and the row sum l):
 *   lse[(b*Hq + h)*S + i] = ln sum_{j<=i} exp(scale*dq*dk*<q_i, k_j>)
 *                        ~= ln(2) * (m c + log2 l),  c = scale*dq*dk*log2(e),
 * where l sums the probabilities the P V product applies: BF16-rounded (within
 * ln(1 + 2^-8) ~ 0.0039 of the exact value: BF16 keeps 8 significant bits),
 * or, for FP8, the Lean P codes with their block scales (within about 0.094:
 * a code in e4m3's normal range decodes to 0.927-1.073 times its probability,
 * keys more than about 13 binades below their block's maximum add at most
 * 0.0043 of the sum, and the FP8 matrix instruction that sums the codes
 * truncates each product within its group of 8 to 2^(E - 13), E the group's
 * largest exponent sum, at most 1.4% downwards; the FP8 scores carry the same
 * truncation, which moves the log-sum-exp by at most their error).
 *   lse   device pointer to B*Hq*S floats (4-byte aligned), written entirely;
 *         float32, natural log, layout [B][Hq][S]
 * Other arguments and errors as attn_fwd_ex; a null or misaligned lse is
 * ATTN_ERR_INVALID. The output O is bit-identical to attn_fwd_ex's.
 */
int attn_fwd_lse(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv, int S,
                 int Dqk, int Dv, int causal, float scale, int dtype, const float* descale_qkv, void* stream,
                 unsigned flags);

/*
 * attn_fwd_prefix: Sq queries after a prefix of keys. The queries are the last
 * Sq positions of a sequence of Sk >= Sq keys: query i sits at position
 * i + Sk - Sq and sees keys j <= i + Sk - Sq (flash_attn_func's causal
 * alignment when the key sequence is longer, bottom-right). With Sq = Sk this
 * is attn_fwd_lse (or attn_fwd_ex when lse is NULL). Together with the
 * log-sum-exp it lets a caller split the keys of one query block into ranges
 * and merge the partial results (context parallelism). The pages do not
 * describe this case; it reuses the same kernels with the diagonal moved by
 * Sk - Sq.
 *   q     B*Sq*Hq*Dqk elements, layout [B][Sq][Hq][Dqk]
 *   k, v  [B][Sk][Hkv][Dqk], [B][Sk][Hkv][Dv]
 *   out   [B][Sq][Hq][Dv] BF16, written entirely
 *   lse   NULL, or B*Hq*Sq floats ([B][Hq][Sq], 4-byte aligned)
 * Other arguments and errors as attn_fwd_ex; Sk < Sq is ATTN_ERR_INVALID.
 */
int attn_fwd_prefix(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv,
                    int Sq, int Sk, int Dqk, int Dv, int causal, float scale, int dtype, const float* descale_qkv,
                    void* stream, unsigned flags);

/*
 * attn_quantize_e4m3: the FP8 quantize prologue. Per-tensor e4m3fn
 * quantisation of a BF16 tensor viewed as `rows` rows of `dim` elements,
 * optionally rotating every row by a normalised Hadamard transform first (for
 * Q and K: one orthogonal H on both leaves Q K^T unchanged).
 *   [spbcomputers.ru ZYFA article, section "Точность: ошибка FP8 ниже, чем у
 *    AITER" and the FAQ entry on the Hadamard rotation; captivela.com "Zyphra
 *    Luncurkan ZYFA", section "Akurasi Jauh Lebih Baik, Bukan Cuma Cepat":
 *    quantising Q, K and V dominates a full model's FP8 attention error, and a
 *    Hadamard rotation of Q and K roughly halves it.]
 * Definition (every step in IEEE fp32): y = the row, or its Walsh-Hadamard
 * transform in blocks of n = 128 elements (dim a multiple of 128) or n = 64,
 * butterflies over index bits 0, 1, ... then one multiply by fp32(1/sqrt(n));
 * amax = max |y| over the tensor; s = amax / 448 (1 if amax = 0); code =
 * e4m3fn(y / s), rounded to nearest, ties to even. attn_fwd takes the codes
 * with descale s.
 *
 *   x         device pointer to rows*dim BF16 values (16-byte aligned)
 *   y         device pointer to rows*dim bytes (16-byte aligned), receives the
 *             e4m3fn codes
 *   scale     device pointer to 2 floats (4-byte aligned): scale[0] receives
 *             s, scale[1] amax; overwritten (also used as the reduction word)
 *   rows      >= 1
 *   dim       64, 128, 192 or 256
 *   hadamard  0 or 1
 *   stream    a hipStream_t of the current device, or NULL for its null
 *             stream
 * Errors: ATTN_ERR_INVALID for a null or misaligned pointer, rows <= 0 or a
 * hadamard flag other than 0/1; ATTN_ERR_UNSUPPORTED for another dim or a
 * device that is not gfx950; ATTN_ERR_LAUNCH for a HIP error. Asynchronous
 * like attn_fwd; x must not overlap y or scale.
 */
int attn_quantize_e4m3(const void* x, void* y, float* scale, long long rows, int dim, int hadamard, void* stream);

/* A static, human-readable description of a return code (never NULL). */
const char* attn_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* FP8_BF16_CAUSAL_H */

/*
 * fa.h -- C ABI of the MI355X (gfx950) fused exact attention library
 * (forward in bf16 and FP8, grouped-head and decode-shaped forwards, and
 * the bf16 backward).
 *
 * The library computes O = softmax(scale * Q K^T) V and the row logsumexp,
 * tile by tile with an online softmax, without ever writing the N x N score
 * matrix to memory (wmrh.cn FlashAttention V3 article, sections 一.1 and
 * 二.1; "FlashAttention-3：用异步流水榨出 Hopper 的 Attention 性能",
 * section "Online Softmax 仍是精确合并的核心").  An FP8 E4M3 variant uses
 * per-block scales and a random-sign Hadamard rotation of Q and K (same
 * explainer, sections "Block Quantization 为什么优于 Per-Tensor Scale" and
 * "Incoherent Processing 如何摊平离群值").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller.  The
 *   library allocates no memory (entry points that need scratch memory
 *   take a caller-owned workspace; fa_fwd_bf16_decode_noalloc uses a static
 *   device buffer instead) and keeps no state besides per-device caches of
 *   the architecture check, the compute-unit count and that buffer's
 *   address; it is safe to call from several host threads.
 * - Tensors are dense row-major ("contiguous").  Layout [B, H, N, d] means
 *   element (b, h, n, i) sits at ((b * H + h) * N + n) * d + i.
 * - Every pointer must be 16-byte aligned (FA_ERR_ALIGN otherwise).
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *   the call returns without waiting.  Faults inside a kernel surface at the
 *   caller's next synchronisation.
 * - Return value: FA_OK (0) or a negative FA_ERR_* code.  Arguments are
 *   validated before any device work is issued; on an error nothing is
 *   enqueued and no output is touched.  Nothing is printed and no C++
 *   exception crosses the ABI.
 * - There is no fallback: a case the kernels do not cover is an error,
 *   never a slower path.  The kernels are built for gfx950 only; any other
 *   device gives FA_ERR_DEVICE.
 * - Causal masking: query row i attends to key j iff j <= i when queries
 *   and keys have the same length N; the entry points for Nq queries and
 *   Nk keys align the mask bottom-right, j <= i + Nk - Nq.
 * - logsumexp is the natural log of sum_j exp(scale * q_i . k_j) over the
 *   keys row i attends to, fp32 [B, H, N].
 */
#ifndef EXACT_ATTENTION_FA_H
#define EXACT_ATTENTION_FA_H

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 2

enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL_PTR = -1, /* a required pointer is NULL                              */
  FA_ERR_SHAPE = -2,    /* B, H or N < 1, >= 2^40 elements, or N * d * 2 >= 2^31   */
  FA_ERR_HEADDIM = -3,  /* d not supported by this entry point                     */
  FA_ERR_ARG = -4,      /* causal not 0/1, scale not finite and > 0, bad flags     */
  FA_ERR_ALIGN = -5,    /* a pointer is not 16-byte aligned                        */
  FA_ERR_DEVICE = -6,   /* no device, or the current device is not gfx950          */
  FA_ERR_LAUNCH = -7,   /* the kernel launch itself failed                         */
  FA_ERR_WORKSPACE = -8, /* workspace missing or smaller than the split count needs */
  FA_ERR_SCRATCH = -9    /* the call needs more than the static scratch buffer holds  */
};

/* Flags of fa_fp8_prep. */
#define FA_PREP_TRANSPOSE 1u  /* write x8 transposed, [B, H, d, fa_fp8_vt_ld(N)]       */
#define FA_PREP_PER_TENSOR 2u /* one scale for the whole tensor (the comparison mode) */
#define FA_PREP_POW2_SCALE 4u /* power-of-two scales (a variant for V, the PV operand); no rotation */

/*
 * fa_fwd_bf16 -- exact attention forward, bf16 operands, fp32 accumulation.
 *
 *   q, k, v : bf16 [B, H, N, d]   (read only)
 *   o       : fp32 [B, H, N, d]   (every element written)
 *   lse     : fp32 [B, H, N]      (every element written, natural log)
 *   d       : 64, 128 or 256      (FA_ERR_HEADDIM otherwise)
 *   causal  : 0 or 1
 *   softmax_scale : finite, > 0 (the usual value is 1/sqrt(d)).
 *
 * Any N >= 1 is accepted; tiles past N are masked.
 */
int fa_fwd_bf16(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H, int N, int d,
                int causal, float softmax_scale, void* stream);

/*
 * fa_fwd_bf16_gqa -- the same forward for grouped- and multi-query heads
 * and unequal query / key lengths (the FA3 explainer names grouped and
 * multi-query KV heads and short queries against long keys among the shapes
 * a kernel meets, section "为什么 Causal Shape 可能更难调度", and lists
 * "Q/K 不同长度" among what tests must cover, section "正确性验证要覆盖异步边界").
 *
 *   q    : bf16 [B, Hq, Nq, d]      k, v : bf16 [B, Hkv, Nk, d]   (read only)
 *   o    : fp32 [B, Hq, Nq, d]      lse  : fp32 [B, Hq, Nq]       (every element written)
 *   Hq   : a multiple of Hkv; query head h reads KV head h / (Hq / Hkv)
 *   causal : 1 = bottom-right alignment, query i sees keys j <= i + Nk - Nq
 *            (a single query sees every key; Nq = Nk is fa_fwd_bf16's mask).
 *            A query that sees no key (Nq > Nk) gets o = 0 and lse = -inf.
 *   d, softmax_scale : as fa_fwd_bf16.
 *
 * FA_ERR_SHAPE also when Hkv < 1, Nk < 1 or Hq % Hkv != 0.
 */
int fa_fwd_bf16_gqa(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Hq, int Hkv,
                    int Nq, int Nk, int d, int causal, float softmax_scale, void* stream);

/*
 * fa_fwd_bf16_varlen -- the forward over a batch of sequences of different
 * lengths packed end to end (the FA3 explainer names variable-length
 * batches among the shapes kernels are dispatched on, section "安装了包，
 * 为什么可能没有用上 FA3", and asks tests to cover very short and empty
 * ranges in them, section "正确性验证要覆盖异步边界").
 *
 *   q        : bf16 [total_q, Hq, d]    k, v : bf16 [total_k, Hkv, d]  (token-major)
 *   o        : fp32 [total_q, Hq, d]    lse  : fp32 [Hq, total_q]
 *   cu_seqlens_q, cu_seqlens_k : int32 [B + 1] DEVICE arrays, nondecreasing
 *              from 0 to total_q (total_k): sequence b owns query rows
 *              cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1 and key rows
 *              cu_seqlens_k[b] .. cu_seqlens_k[b+1] - 1.  Values are clamped
 *              into [0, total] on the device, so no access leaves the tensors.
 *   max_seqlen_q : at least the largest query count of any sequence (sizes
 *              the grid).  The device cannot report a longer sequence: its
 *              query rows beyond max_seqlen_q are left unwritten, so the
 *              caller must pass the true maximum.
 *   Hq, Hkv, d, causal, softmax_scale : as fa_fwd_bf16_gqa, applied to each
 *              sequence on its own (causal bottom-right per sequence; a query
 *              that sees no key, e.g. in a sequence with no keys, gets o = 0
 *              and lse = -inf).  Empty sequences are allowed.
 *
 * Rows of o and lse that belong to no sequence are not written.
 * FA_ERR_SHAPE also when total_q * Hq * d * 2 or total_k * Hkv * d * 2 is
 * >= 2^31 (rows are addressed with 32-bit byte offsets) or a size is negative;
 * FA_ERR_ALIGN when a cu_seqlens array is not 4-byte aligned.
 */
int fa_fwd_bf16_varlen(const void* q, const void* k, const void* v, float* o, float* lse, const int* cu_seqlens_q,
                       const int* cu_seqlens_k, int B, int Hq, int Hkv, int total_q, int total_k, int max_seqlen_q,
                       int d, int causal, float softmax_scale, void* stream);

/*
 * Decode-shaped forward: a few queries per head against a long key/value
 * sequence.  The FA3 explainer (sections "GQA/MQA 为何改变 Kernel 任务数量"
 * and "Prefill、Decode 和训练的收益不同") names split-KV and packing the
 * query heads of a KV head as what gives such shapes enough parallel work.
 * The result is that of fa_fwd_bf16_gqa (same arguments, same bottom-right
 * causal reading, O = 0 and lse = -inf for a query that sees no key); only
 * the work split differs:
 *
 *  - The G = Hq / Hkv query heads of a KV head, times Nq queries, are packed
 *    into 32-row blocks, so one read of a K/V tile serves up to 32 rows.
 *  - The keys of each KV head are cut into `splits` chunks of whole 32-key
 *    tiles, one workgroup per (batch, KV head, chunk, row block).  When more
 *    than one chunk is used, each chunk's normalised O_c and lse_c go to the
 *    workspace, and a second kernel on the same stream merges them by
 *    lse = ln sum_c exp(lse_c), O = sum_c exp(lse_c - lse) O_c.
 *
 * fa_fwd_bf16_decode_splits -- the chunk count the forward will use.
 *   num_splits >= 1: that many, reduced to the number of non-empty chunks
 *   (every chunk holds ceil(tiles / num_splits) tiles).  num_splits = 0: a
 *   cost model's choice for a device with num_cus compute units (HBM time
 *   of the K/V stream in rounds of resident workgroups, plus the partial
 *   results' traffic and one more launch when there is more than one chunk).
 *   Host only, no device needed.  Returns >= 1, or FA_ERR_SHAPE /
 *   FA_ERR_HEADDIM as fa_fwd_bf16_decode would, or FA_ERR_ARG for a
 *   negative count or num_splits = 0 without num_cus.
 *
 * fa_fwd_bf16_decode_workspace -- bytes of workspace for `splits` chunks:
 *   0 when splits = 1, else splits * B * Hq * Nq * (d + 1) * 4.
 *   FA_ERR_ARG for sizes < 1 or an unsupported d.
 *
 * fa_fwd_bf16_decode -- the forward.
 *   q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, softmax_scale: as
 *   fa_fwd_bf16_gqa (also FA_ERR_SHAPE when (Nk + 32) * d * 2 >= 2^31).
 *   num_splits : >= 1, reduced as fa_fwd_bf16_decode_splits does
 *                (FA_ERR_ARG for < 1).
 *   workspace  : device memory, 16-byte aligned, owned by the caller, at
 *                least fa_fwd_bf16_decode_workspace(effective splits) bytes
 *                (FA_ERR_WORKSPACE otherwise); unused, and may be NULL,
 *                when the effective count is 1.  Its contents on entry do
 *                not matter, and on return they are scratch.  Calls that
 *                share a workspace must not overlap in time.
 */
int fa_fwd_bf16_decode_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d, int num_splits, int num_cus);
long long fa_fwd_bf16_decode_workspace(int B, int Hq, int Nq, int d, int splits);
int fa_fwd_bf16_decode(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Hq, int Hkv,
                       int Nq, int Nk, int d, int causal, float softmax_scale, int num_splits, void* workspace,
                       long long workspace_bytes, void* stream);

/*
 * fa_fwd_bf16_decode_noalloc -- fa_fwd_bf16_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It allocates nothing; the chunk partials
 * go to a static device buffer of FA_DECODE_SCRATCH_BYTES (16 MiB) that the
 * library holds on every device it runs on until the process ends.
 *
 *   q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, causal, softmax_scale: as
 *   fa_fwd_bf16_decode.
 *   num_splits : >= 1 as fa_fwd_bf16_decode (FA_ERR_SCRATCH when that
 *                count's partials, fa_fwd_bf16_decode_workspace bytes, exceed
 *                the buffer), or 0 for the cost model's count on the current
 *                device, lowered until the partials fit.
 *
 * The first call on a device looks the buffer up (hipGetSymbolAddress); make
 * it outside graph capture.  Every call on a device shares that device's
 * buffer and leaves its partials there: calls that overlap in time on one
 * device (several streams or host threads) race and must be ordered by the
 * caller.  The buffer needs no clearing: each chunk writes all of its
 * partial rows before the merge reads them.  Results are bit-identical to
 * fa_fwd_bf16_decode with the same effective split count.
 */
#define FA_DECODE_SCRATCH_BYTES (16ll << 20)
int fa_fwd_bf16_decode_noalloc(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Hq,
                               int Hkv, int Nq, int Nk, int d, int causal, float softmax_scale, int num_splits,
                               void* stream);

/*
 * fa_bwd_bf16 -- exact attention backward: dQ, dK, dV of the forward above
 * for an upstream gradient dO, recomputing P from the saved logsumexp
 * (the derivative of the forward's definition, wmrh.cn FlashAttention V3
 * article, section 一.1; the FA3 explainer lists dQ, dK, dV among what a
 * correctness suite must cover, section "正确性验证要覆盖异步边界"):
 *   D = rowsum(dO * O), dV = P^T dO, dS = P * (dO V^T - D),
 *   dQ = scale dS K, dK = scale dS^T Q.
 *
 *   q, k, v, dout : bf16 [B, H, N, d]   (read only; the forward's inputs)
 *   o             : fp32 [B, H, N, d]   (read only; the forward's output)
 *   lse           : fp32 [B, H, N]      (read only; the forward's logsumexp)
 *   dq, dk, dv    : fp32 [B, H, N, d]   (every element written)
 *   delta_ws      : fp32 [B, H, N]      caller-owned workspace, overwritten
 *                                       with D (the library allocates nothing)
 *   d             : 64, 128 or 256      (FA_ERR_HEADDIM otherwise)
 *   causal, softmax_scale : as for the forward, and equal to its values.
 *
 * Also FA_ERR_SHAPE when N * d * 4 >= 2^31.  The kernels run in order on
 * `stream`: D, then dK/dV (one launch, or a dV launch and a dK launch: always
 * at d = 256, at d = 128 when the grid fills the device), then dQ; no
 * atomics, so results are deterministic.
 */
int fa_bwd_bf16(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dout,
                float* dq, float* dk, float* dv, float* delta_ws, int B, int H, int N, int d, int causal,
                float softmax_scale, void* stream);

/*
 * fa_bwd_bf16_gqa -- the same backward for grouped- and multi-query heads
 * (queries and keys of equal length N): the backward of fa_fwd_bf16_gqa
 * with Nq = Nk = N.  Query head h reads KV head h / (Hq / Hkv), so a KV
 * head's dK, dV are the sums of the gradients of the Hq / Hkv query heads
 * that read it (the chain rule through the shared head).
 *
 *   q, dout       : bf16 [B, Hq, N, d]    k, v   : bf16 [B, Hkv, N, d]
 *   o             : fp32 [B, Hq, N, d]    lse    : fp32 [B, Hq, N]
 *   dq            : fp32 [B, Hq, N, d]    dk, dv : fp32 [B, Hkv, N, d]
 *   delta_ws      : fp32 [B, Hq, N]       caller-owned workspace
 *   Hq            : a multiple of Hkv (FA_ERR_SHAPE otherwise, or for Hkv < 1)
 *   everything else as fa_bwd_bf16 (which is this call with Hkv = Hq).
 */
int fa_bwd_bf16_gqa(const void* q, const void* k, const void* v, const float* o, const float* lse, const void* dout,
                    float* dq, float* dk, float* dv, float* delta_ws, int B, int Hq, int Hkv, int N, int d,
                    int causal, float softmax_scale, void* stream);

/*
 * fa_fp8_prep -- one pass over one tensor that produces the FP8 operands of
 * fa_fwd_fp8 ("Incoherent Processing" and "Block Quantization" sections of
 * the FA3 explainer cited above; E4M3 largest value 448 from the wmrh.cn
 * article, section 三.3).
 *
 *   x       : bf16 [B, H, N, d]  (read only)
 *   signs   : int8 [H, d] of +1/-1, or NULL.  When given, each row is
 *             rotated, y = x diag(signs[h]) H_d / sqrt(d) with H_d the
 *             Sylvester Hadamard matrix (apply the same signs to Q and K;
 *             never to V).  NULL: y = x.  Device memory, 16-byte aligned
 *             like every pointer here (FA_ERR_ALIGN otherwise).
 *   x8      : uint8 E4M3 (OCP e4m3fn) codes of y / s:
 *             [B, H, N, d] by default, or with FA_PREP_TRANSPOSE the
 *             transposed [B, H, d, ld] with ld = fa_fp8_vt_ld(N); columns
 *             N..ld-1 are written as zero codes.  In the transposed layout
 *             the keys of each row are stored in groups of four (one 32-bit
 *             word each) and, within every aligned run of 64 keys, word w
 *             holds key group 2 (w % 8) + w / 8: the even groups first, then
 *             the odd ones, which is the key order of fa_fwd_fp8's PV
 *             operand.
 *   x_scale : fp32 [B, H, ceil(N / 128)]: s = amax(|y|) / 448 over each block
 *             of 128 rows (all of d); s = 1 for an all-zero block.  With
 *             FA_PREP_POW2_SCALE, s = 2^ceil(log2(amax / 448)) instead (the
 *             smallest power of two with amax / s <= 448): a variant for V,
 *             whose scale the PV product then takes as an exact block
 *             exponent, at the cost of up to one bit of V's range.  With
 *             FA_PREP_PER_TENSOR, amax runs over the whole tensor and every
 *             entry holds the same s.
 *   d       : 128.
 *   flags   : OR of FA_PREP_TRANSPOSE, FA_PREP_PER_TENSOR and
 *             FA_PREP_POW2_SCALE (FA_ERR_ARG for any other bit, or for
 *             FA_PREP_POW2_SCALE together with signs).
 *
 * Codes are round-to-nearest-even of clamp(y * 448 / amax, -448, 448), the
 * product formed in fp32 (one code step from the exact quotient's rounding
 * where that quotient lies within fp32 rounding of a tie); with
 * FA_PREP_POW2_SCALE of y / s (exact).
 * Per-tensor mode issues three kernels on `stream` (block amaxes into
 * x_scale, quantise with the tensor amax reduced from them, then the
 * scales); block mode issues one.  Calls that share an x_scale buffer
 * must be ordered on one stream.
 */
int fa_fp8_prep(const void* x, void* x8, float* x_scale, const signed char* signs, int B, int H, int N, int d,
                unsigned flags, void* stream);

/* Row stride (in elements) of the transposed V produced by fa_fp8_prep:
 * N rounded up to a multiple of 128.  Returns 0 for N < 1. */
int fa_fp8_vt_ld(int N);

/*
 * fa_fwd_fp8 -- exact-attention forward on FP8 E4M3 operands made by
 * fa_fp8_prep (Q and K rotated with the same signs, V transposed).  Both
 * products run on FP8 matrix instructions with fp32 accumulation; the
 * softmax state is fp32 ("FP8 Attention 仍然不等于 FP8 全链路" section of the
 * FA3 explainer).  Scores are descaled by s_Q,i * s_K,j per block pair; the
 * V block scale is applied in the PV product.  Probabilities P in (0, 1]
 * enter the PV product as E4M3(P * 2^7 * mu_j), mu_j the mantissa in
 * [1, 2) of the key block's V scale, whose exponent goes to the matrix
 * instruction's power-of-two block scale; l sums the unrounded P.
 *
 *   q8, k8  : uint8 [B, H, N, d]
 *   v8t     : uint8 [B, H, d, fa_fp8_vt_ld(N)] (padding columns must be 0)
 *   q_scale, k_scale, v_scale : fp32 [B, H, ceil(N / 128)], positive
 *             normal floats (as fa_fp8_prep writes them: amax / 448, or
 *             powers of two with FA_PREP_POW2_SCALE, where mu_j = 1)
 *   o, lse  : as in fa_fwd_bf16
 *   d       : 128.
 *
 * The exponent reference of P (the running row max rounded up to a whole
 * power of two) moves once per block of fa_fp8_ref_block(N, causal) keys:
 * the kernel's key tile, which P of that block is quantised against
 * ("Online Softmax 仍是精确合并的核心": each block rescales the running
 * state; the block length is the kernel's choice).
 */
int fa_fwd_fp8(const void* q8, const void* k8, const void* v8t, const float* q_scale, const float* k_scale,
               const float* v_scale, float* o, float* lse, int B, int H, int N, int d, int causal,
               float softmax_scale, void* stream);

/* Keys per exponent-reference step of fa_fwd_fp8 for N keys (the key tile
 * of the kernel it runs): 128 for non-causal N >= 1024 and causal
 * N >= 4096, 64 otherwise; it divides the 128-row scale block.  Only the
 * rounding of P depends on it.  FA_ERR_SHAPE for N < 1, FA_ERR_ARG for
 * causal not 0/1.  Host only: no device work. */
int fa_fp8_ref_block(int N, int causal);

/* Static description of a status code (never NULL). */
const char* fa_status_string(int status);

/* FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_FA_H */

/*
 * attn.h - C ABI of the gfx950 (MI355X) exact-attention library (libattn.so).
 *
 * Three operations:
 *
 *   attn_fwd           O = softmax(scale * Q K^T) V, computed tile by tile with
 *                      an online softmax so the score matrix never reaches HBM;
 *                      also returns LSE, the natural-log softmax denominator.
 *   attn_decode_paged  the same definition for one query row per sequence
 *                      against a paged KV cache, split over the keys, with the
 *                      partial results merged by their log-sum-exps.
 *   attn_bwd           dQ, dK, dV of the forward for an upstream dO, with the
 *                      probabilities recomputed from the forward's LSE.
 * attn_fwd_varlen and attn_bwd_varlen are attn_fwd and attn_bwd over packed
 * sequences of different lengths; attn_fwd_alibi and attn_bwd_alibi add an
 * ALiBi bias; attn_fwd_fp8 takes FP8 (E4M3) inputs with per-tensor descales.
 *
 * Definitions followed (page titles and sections):
 *  - attention as the fused softmax(QK^T/sqrt(d))V, bf16, head dim 128, BSHD
 *    or BHSD without transposes, arbitrary lengths including cross-attention:
 *    "MoonMath AI open-sources a HIP attention kernel for AMD MI300X that beats
 *    AITER v3", definition and scope paragraphs;
 *  - tiling with a running row max m and denominator l, merged per block as
 *    m' = max(m, m_new), l' = l*exp(m - m') + l_new: "IO-aware tiling strategy
 *    in FlashAttention-4", body;
 *  - shared K/V heads for several query heads (MQA/GQA), paged KV cache with
 *    16-token pages and an int32 block table: "Engineering the FlashAttention-4
 *    kernel port to ROCm: HIP migration and multi-query inference
 *    optimisation", multi-query section;
 *  - causal (upper-triangular) masking: "Reverse engineering Flash Attention
 *    4's proprietary fused attention kernel", point 1;
 *  - the key split with a merge of partials for the tail: MoonMath page,
 *    third-Q-tile paragraph;
 *  - launching on the caller's stream so the call overlaps a larger
 *    pipeline: MoonMath page, use-case paragraph;
 *  - updating the shared KV cache inside the attention call (the current
 *    token's K/V appended, then attended): "Reverse engineering Flash
 *    Attention 4's proprietary fused attention kernel", first point;
 *  - three rounding rules for the bf16 output (to nearest with ties to even,
 *    to nearest with ties away from zero, toward zero): MoonMath page,
 *    numerics and benchmark paragraphs.
 *
 * Conventions common to every entry point
 *  - bf16 tensors are passed as raw device pointers to IEEE bfloat16 data;
 *    d (head dim) is innermost and contiguous.  Every entry point takes
 *    d = 128; attn_fwd and attn_fwd_rounded also take d = 64 and d = 256, and
 *    attn_bwd also takes d = 64.  Any other d returns ATTN_ERR_UNSUPPORTED.
 *  - Pointers are device pointers, 16-byte aligned.  The caller allocates and
 *    owns every buffer (inputs, outputs, tables, workspace); the library never
 *    allocates, frees or synchronises.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued on it and the call returns; buffers must stay alive until
 *    the stream has passed the launch.  Results are bitwise deterministic for
 *    identical inputs and shapes (no atomics in the arithmetic, fixed order).
 *  - Outputs must not alias inputs.
 *  - Every argument check runs before any HIP call; a failed check returns its
 *    status and enqueues nothing.  A launch the runtime rejects returns
 *    ATTN_ERR_LAUNCH.  Faults inside kernels surface at the caller's next
 *    synchronisation, as HIP defines.
 *  - Reading taken for GQA: query head h uses K/V head h / (Hq / Hkv).
 *  - Reading taken for causal with Sq != Sk: bottom-right alignment, key j is
 *    visible from query i iff j <= i + (Sk - Sq).  A query row that sees no key
 *    gets O = 0 and LSE = -inf.
 *  - The scale is applied in fp32 to fp32 scores (never folded into bf16 Q).
 *  - O is rounded to bf16 with round-to-nearest-even by attn_fwd and
 *    attn_decode_paged; their *_rounded variants take the rule as an argument.
 *    The rule applies to the final fp32 -> bf16 conversion of O only; the
 *    probabilities inside the kernels are rounded to nearest even as always,
 *    and LSE does not depend on it.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_VERSION 13

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,        /* a required pointer is NULL                    */
  ATTN_ERR_SHAPE = -2,       /* a size is < 1, Hq % Hkv != 0, size overflow    */
  ATTN_ERR_UNSUPPORTED = -3, /* head dim not taken by the entry point, page_size
                                != 16, bad layout/rounding, scale not finite > 0 */
  ATTN_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned               */
  ATTN_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required     */
  ATTN_ERR_LAUNCH = -6,      /* the HIP runtime rejected a launch              */
  ATTN_ERR_DEVICE = -7       /* no usable gfx950 device / device query failed  */
} attn_status;

enum { ATTN_BSHD = 0, ATTN_BHSD = 1 };

/*
 * Rounding rule of the final fp32 -> bf16 conversion of O:
 *   ATTN_ROUND_RTNE  to nearest, ties to the value with an even last bit
 *   ATTN_ROUND_RTNA  to nearest, ties away from zero; from half a spacing past
 *                    the largest finite bf16 the result is +-inf
 *   ATTN_ROUND_RTZ   toward zero (truncation); finite values never become inf
 * In every rule NaN stays NaN and +-0, +-inf keep their sign.
 */
enum { ATTN_ROUND_RTNE = 0, ATTN_ROUND_RTNA = 1, ATTN_ROUND_RTZ = 2 };

/*
 * attn_fwd - fused exact attention forward (prefill, self- or cross-attention).
 *
 *   q    bf16, layout `layout`: BSHD [B, Sq, Hq, d] or BHSD [B, Hq, Sq, d]
 *   k, v bf16, same layout:     BSHD [B, Sk, Hkv, d] or BHSD [B, Hkv, Sk, d]
 *   o    bf16 output, same layout and shape as q
 *   lse  fp32 output [B, Hq, Sq] (contiguous, for both layouts); natural log of
 *        sum_j exp(scale * q_i . k_j) over the visible keys j
 *   B, Hq, Hkv, Sq, Sk >= 1, Hq % Hkv == 0, d in {64, 128, 256}
 *   scale  finite float32 (1/sqrt(d) is the usual value)
 *   causal 0 or 1
 *
 * Size limits (ATTN_ERR_SHAPE): the K/V rows of one (batch, kv head) are
 * addressed with 32-bit byte offsets, so (Sk - 1) * row stride * 2 + 2 * d
 * must stay below 2^31 (row stride = Hkv * d elements in BSHD, d in BHSD), and
 * the workgroup count (B * Hq * ceil(Sq / rows per workgroup)) must stay below
 * 2^31.
 *
 * Returns ATTN_OK or an attn_status error.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
             int layout, void* stream);

/*
 * attn_fwd_rounded - attn_fwd with the rounding rule of O as an argument
 * ("MoonMath AI open-sources a HIP attention kernel for AMD MI300X that beats
 * AITER v3", benchmark paragraph: every shape is measured under RTNE, RTNA and
 * RTZ).  `rounding` is one of ATTN_ROUND_*; any other value returns
 * ATTN_ERR_UNSUPPORTED.  Every other argument, limit and status is as for
 * attn_fwd, which is attn_fwd_rounded with ATTN_ROUND_RTNE.  O under the three
 * rules comes from the same fp32 values, so the results differ by at most one
 * bf16 spacing per element; LSE is identical.
 */
int attn_fwd_rounded(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                     int layout, int rounding, void* stream);

/*
 * attn_prep_v_bytes / attn_prep_v / attn_fwd_prepped - attn_fwd_rounded in
 * two steps, with V prepared once as the P.V product reads it.  Where each
 * operand lives is what sets the speed of the kernels in "MoonMath AI
 * open-sources a HIP attention kernel for AMD MI300X that beats AITER v3"
 * (data-placement paragraph); here the fp16 V^T tiles the matrix cores read
 * are written once per K/V head, instead of being converted and transposed
 * in LDS by every query-tile workgroup.  The result is bit-identical to
 * attn_fwd_rounded on the same inputs.
 *
 * attn_prep_v_bytes(B, Hq, Hkv, Sk, d): bytes of the prepared tiles, or 0
 *   for an unsupported head dim and for invalid sizes.  d = 128:
 *   B * Hkv * ceil(Sk / 64) * 16384, or B * Hkv * ceil(Sk / 32) * 8192 when
 *   Hq / Hkv is a multiple of 4 (the kernel for those groups works on 32-key
 *   tiles); d = 256: B * Hkv * ceil(Sk / 32) * 16384; d = 64:
 *   B * Hkv * ceil(Sk / 64) * 8192 (fp16 V rows; that kernel reads V^T by
 *   transposing LDS reads).
 * attn_prep_v(v, B, Hq, Hkv, Sk, d, layout, vt, vt_bytes, stream): writes
 *   the tiles of v (bf16, attn_fwd's k/v layout) into vt (device memory,
 *   16-byte aligned, at least attn_prep_v_bytes; owned by the caller).  Each
 *   value is rounded to fp16 (nearest even); |v| >= 65520 becomes +-inf,
 *   which attn_fwd_prepped detects and answers with the bf16 path, as
 *   attn_fwd does.  Returns ATTN_OK without work where the size is 0;
 *   ATTN_ERR_WORKSPACE if vt is NULL or smaller, ATTN_ERR_ALIGN,
 *   ATTN_ERR_SHAPE (one head's tiles, about Sk * 2 * d bytes, must stay
 *   below 2^32 bytes),
 *   ATTN_ERR_UNSUPPORTED for another layout.
 * attn_fwd_prepped(q, k, v, vt, vt_bytes, o, lse, ...): attn_fwd_rounded,
 *   reading V^T from vt, which must hold attn_prep_v's output for this v
 *   with the same B, Hkv, Sk, layout (not checked; v itself is still read
 *   by the bf16 path).  vt is not written; the call may be repeated with
 *   other q on the same prepared tiles.  Where attn_prep_v_bytes is 0, vt
 *   is ignored.  Otherwise vt NULL returns ATTN_ERR_NULL, too small
 *   ATTN_ERR_WORKSPACE, misaligned ATTN_ERR_ALIGN.  Other arguments,
 *   limits and statuses as for attn_fwd_rounded.
 */
size_t attn_prep_v_bytes(int B, int Hq, int Hkv, int Sk, int d);
int attn_prep_v(const void* v, int B, int Hq, int Hkv, int Sk, int d, int layout, void* vt,
                size_t vt_bytes, void* stream);
int attn_fwd_prepped(const void* q, const void* k, const void* v, const void* vt,
                     size_t vt_bytes, void* o, float* lse, int B, int Hq, int Hkv, int Sq, int Sk,
                     int d, float scale, int causal, int layout, int rounding, void* stream);

/*
 * attn_fwd_alibi - attn_fwd_rounded with an ALiBi linear position bias: for
 * query head h, -alibi_slopes[h] * |i + Sk - Sq - j| is added to the scaled
 * score of query row i and key j before the softmax (query positions aligned
 * to the end of the keys, as the causal mask is), and LSE is that of the
 * biased scores.  ALiBi support is what "IO-aware tiling strategy in
 * FlashAttention-4" (integration paragraph) asks a drop-in kernel to check;
 * the bias form is the ALiBi method's own (per-head slopes, linear in the
 * distance).
 *
 *   alibi_slopes  device fp32 [Hq], 4-byte aligned, finite values (device
 *                 data: not checked); NULL returns ATTN_ERR_NULL
 * Everything else is as for attn_fwd_rounded.
 */
int attn_fwd_alibi(const void* q, const void* k, const void* v, void* o, float* lse,
                   const float* alibi_slopes, int B, int Hq, int Hkv, int Sq, int Sk, int d,
                   float scale, int causal, int layout, int rounding, void* stream);

/*
 * attn_fwd_fp8 - attn_fwd on FP8 inputs.  Q, K and V are bytes in the OCP
 * 8-bit E4M3 format ("FN": sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, subnormals, no infinity, largest finite 448), each tensor with one
 * fp32 descale factor: the attention of attn_fwd is computed on the real
 * values descale_q*q, descale_k*k, descale_v*v.  The pages name FP8 inputs
 * as a variant and say that FP8 handling falls back to FP16 on ROCm
 * ("Engineering the FlashAttention-4 kernel port to ROCm", HIP migration
 * section; "IO-aware tiling strategy in FlashAttention-4", monitoring
 * paragraph): Q.K^T runs on the FP8 matrix core (exact products, fp32
 * accumulation: the scores of the exactly widened values), V is widened
 * exactly to fp16 inside the kernel and P.V runs on fp16 MFMA with fp32
 * accumulation.
 *
 *   q, k, v      device E4M3 bytes in `layout` (BSHD [B,S,H,128] or BHSD
 *                [B,H,S,128]), 16-byte aligned, finite values (the E4M3 NaN
 *                encoding s.1111.111 propagates to the rows it touches)
 *   descale_*    positive finite fp32; scale*descale_q*descale_k*log2(e) and
 *                descale_v must be normal fp32 values, otherwise
 *                ATTN_ERR_UNSUPPORTED
 *   o, lse       as for attn_fwd (O bf16 rounded to nearest even in q's
 *                layout, LSE fp32 [B,Hq,Sq] of the descaled scores)
 * d must be 128.  Everything else (shapes, GQA, causal alignment, empty rows,
 * errors, stream) is as for attn_fwd.
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, float descale_q, float descale_k,
                 float descale_v, void* o, float* lse, int B, int Hq, int Hkv, int Sq, int Sk,
                 int d, float scale, int causal, int layout, void* stream);

/*
 * attn_fwd_varlen - attn_fwd over a batch of packed sequences of different
 * lengths (variable-length batching, which the MoonMath page lists among what
 * its kernel lacks: "MoonMath AI open-sources a HIP attention kernel for AMD
 * MI300X that beats AITER v3", limitations paragraph).  Sequence b is query
 * rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] ..
 * cu_seqlens_k[b+1]-1; each sequence is one attn_fwd problem of its own
 * lengths (causal alignment, empty-row rule and GQA mapping as for attn_fwd).
 *
 *   q     bf16 [total_q, Hq, d] (packed rows, d innermost)
 *   k, v  bf16 [total_k, Hkv, d]
 *   o     bf16 output [total_q, Hq, d]
 *   lse   fp32 output [Hq, total_q]
 *   cu_seqlens_q, cu_seqlens_k  device int32 [B + 1], 4-byte aligned:
 *         0 = cu[0] <= cu[1] <= ... <= cu[B] = total; a sequence may be
 *         empty; one with keys but no query rows writes nothing, one with
 *         query rows but no keys gets O = 0 and LSE = -inf
 *   max_seqlen_q  >= every query length (it sizes the launch; rows of a
 *         longer sequence past it are not written)
 *   B, Hq, Hkv, total_q, total_k, max_seqlen_q >= 1, Hq % Hkv == 0, d == 128
 *   rounding  one of ATTN_ROUND_* for O
 *
 * Each sequence's O and LSE equal, bit for bit, those of attn_fwd_rounded on
 * that sequence alone (the same kernel runs both: groups of 4k query heads
 * the GQA kernel, other groups the 256-row kernel).
 *
 * The offsets live on the device and are not read by the host; out-of-order
 * or out-of-range values are clamped to [0, total] (memory-safe, results for
 * such sequences unspecified).  Size limits (ATTN_ERR_SHAPE):
 * (total_k - 1) * Hkv * 256 + 256 < 2^31 and B * Hq * ceil(max_seqlen_q / R)
 * < 2^31, R = 64 when Hq / Hkv is a multiple of 4, else 256.  Other statuses
 * as for attn_fwd_rounded.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int Hq,
                    int Hkv, int total_q, int total_k, int max_seqlen_q, int d, float scale,
                    int causal, int rounding, void* stream);

/*
 * attn_decode_workspace_bytes - device workspace that attn_decode_paged needs
 * for its split partials (fp32 partial outputs and their LSEs), for a batch of
 * B sequences, Hq query heads and block tables of max_blocks_per_seq entries:
 * B * Hq * (S * 129 + 1) * 4 bytes with S = ceil(max_blocks_per_seq / 4) + 1
 * partial results per (sequence, head).  Returns 0 for invalid sizes.
 */
size_t attn_decode_workspace_bytes(int B, int Hq, int max_blocks_per_seq);

/*
 * attn_decode_paged - one decode step: attention of one query row per
 * (sequence, query head) against every cached token, over a paged KV cache.
 *
 *   q            bf16 [B, Hq, d]
 *   k_cache,     bf16 [num_pages, page_size, Hkv, d]: token t of sequence b
 *   v_cache      is slot t % 16 of page block_table[b, t / 16]
 *   block_table  int32 [B, max_blocks_per_seq]; entries p < ceil(seq_lens[b]/16)
 *                must lie in [0, num_pages); entries beyond are never read
 *   seq_lens     int32 [B], 1 <= seq_lens[b] <= max_blocks_per_seq * 16,
 *                counting every cached token (the current one included);
 *                B <= 65535 and max_blocks_per_seq <= 262140
 *   o            bf16 output [B, Hq, d]
 *   lse          fp32 output [B, Hq]
 *   page_size == 16, d == 128, Hq % Hkv == 0
 *   workspace    device memory of at least
 *                attn_decode_workspace_bytes(B, Hq, max_blocks_per_seq) bytes;
 *                its contents on entry do not matter
 *
 * The table and seq_lens live on the device and are not read by the host, so
 * their preconditions are documented, not checked; out-of-contract values stay
 * memory-safe: a length is clamped to [0, 16 * max_blocks_per_seq], a table
 * entry outside [0, num_pages) is not dereferenced and its 16 tokens are left
 * out, and a sequence left with no tokens gets O = 0 and LSE = -inf.  Cache
 * slots past a sequence's end may hold any bits (NaN included): they are
 * never used.
 */
int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* seq_lens, void* o,
                      float* lse, int B, int Hq, int Hkv, int d, int page_size,
                      int max_blocks_per_seq, int num_pages, float scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged_rounded - attn_decode_paged with the rounding rule of O
 * (one of ATTN_ROUND_*, else ATTN_ERR_UNSUPPORTED) as an argument; the same
 * rules as attn_fwd_rounded, applied when the merged fp32 output is written.
 * Everything else is as for attn_decode_paged, which is this call with
 * ATTN_ROUND_RTNE.
 */
int attn_decode_paged_rounded(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, void* o,
                              float* lse, int B, int Hq, int Hkv, int d, int page_size,
                              int max_blocks_per_seq, int num_pages, float scale, int rounding,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged_append - one decode step that first appends the current
 * token to the paged KV cache: token seq_lens[b] - 1 of sequence b (the
 * lengths count it) gets K row k_new[b] and V row v_new[b], written into slot
 * (seq_lens[b] - 1) % 16 of page block_table[b, (seq_lens[b] - 1) / 16] of
 * k_cache / v_cache, and the attention runs over all seq_lens[b] tokens with
 * those rows ("Reverse engineering Flash Attention 4's proprietary fused
 * attention kernel", first point: the KV-cache update fused with the
 * attention; paged format as for attn_decode_paged).
 *
 *   k_new, v_new  bf16 [B, Hkv, d], 16-byte aligned, not aliasing the caches
 *   k_cache,      as for attn_decode_paged, but written: after the call the
 *   v_cache       current tokens' slots hold the new rows; no other byte of
 *                 the caches changes.  The previous contents of those slots
 *                 are never read (they may hold any bits).
 *   rounding      one of ATTN_ROUND_* for O
 * Everything else (shapes, workspace, limits, statuses) is as for
 * attn_decode_paged; a NULL k_new or v_new returns ATTN_ERR_NULL.  The result
 * equals writing the rows into the caches and then calling
 * attn_decode_paged_rounded, bit for bit, in one launch sequence.  If the
 * table entry of the current token's page is outside [0, num_pages) nothing
 * is written and that page's tokens are left out, as in attn_decode_paged.
 */
int attn_decode_paged_append(const void* q, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, const int32_t* block_table,
                             const int32_t* seq_lens, void* o, float* lse, int B, int Hq,
                             int Hkv, int d, int page_size, int max_blocks_per_seq,
                             int num_pages, float scale, int rounding, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged_noalloc - attn_decode_paged (RTNE) without a workspace
 * argument and without any allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The split partials go to a device array the library
 * owns (64 MiB = 67108864 bytes per GPU, held until the process ends, its
 * address looked up once per device); the library calls no allocating
 * routine.
 *
 *   arguments: as for attn_decode_paged, less workspace and workspace_bytes
 *
 * Limit: attn_decode_workspace_bytes(B, Hq, max_blocks_per_seq) must be at
 * most 67108864, else ATTN_ERR_WORKSPACE (checked before any HIP call).  A
 * failed lookup of the array's device address returns ATTN_ERR_DEVICE.
 * Every call on a GPU uses that GPU's one array, and nothing in it needs to
 * start cleared (every partial is written before it is read), so the contents
 * an earlier call left do no harm; calls that overlap on one GPU (different
 * streams, or threads) race on the array and must not be issued.
 */
int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, void* o,
                              float* lse, int B, int Hq, int Hkv, int d, int page_size,
                              int max_blocks_per_seq, int num_pages, float scale, void* stream);

/*
 * attn_bwd_workspace_bytes - device workspace that attn_bwd needs: two fp32
 * values per query row (the row term D_i = dO_i . O_i and the LSE in log2
 * units), 8 * B * Hq * Sq bytes.  Returns 0 for invalid sizes.
 */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Sq);

/*
 * attn_bwd - gradients dQ, dK, dV of attn_fwd's O for an upstream gradient
 * dO, recomputing the probabilities from the forward's LSE instead of storing
 * them ("IO-aware tiling strategy in FlashAttention-4", backward-pass
 * paragraph: only the row statistics are kept and S/P are recomputed;
 * "Reverse engineering Flash Attention 4's proprietary fused attention
 * kernel", point 2).  What is returned is the gradient of sum(dO * O) with
 * respect to Q, K and V of the forward's definition (same GQA mapping, causal
 * alignment and scale); a K/V head's dK and dV are summed over the query
 * heads that share it.
 *
 *   q, k, v      the forward's inputs, as for attn_fwd
 *   o, lse       the forward's outputs for these inputs (attn_fwd with the
 *                same arguments; O under any rounding rule)
 *   dout         bf16, same layout and shape as q
 *   dq           bf16 output, same layout and shape as q
 *   dk, dv       bf16 outputs, same layout and shape as k
 *   workspace    device memory of at least attn_bwd_workspace_bytes(B, Hq, Sq)
 *                bytes; its contents on entry do not matter
 *   B, Hq, Hkv, Sq, Sk, scale, causal, layout: as for attn_fwd
 *   d            128 or 64 (64 not with attn_bwd_alibi)
 *
 * Rows that see no key (causal with Sq > Sk) get dQ = 0 and add nothing to dK
 * and dV.  Products run in bf16 with fp32 accumulation (P and dS rounded to
 * bf16 to nearest even); the outputs are rounded to bf16 to nearest even.
 * Size limits (ATTN_ERR_SHAPE): (Sq + 64) * q row stride * 2 and
 * (Sk + 64) * k row stride * 2 must stay below 2^31 (row stride = heads * d
 * elements in BSHD, d in BHSD), B and Hq at most 65535.
 * Returns ATTN_OK or an attn_status error; every check runs before any HIP
 * call.  Deterministic: no atomics, fixed summation order.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
             int Sk, int d, float scale, int causal, int layout, void* workspace,
             size_t workspace_bytes, void* stream);

/*
 * attn_bwd_alibi - attn_bwd for attn_fwd_alibi: the gradients of the forward
 * with the ALiBi bias (the bias does not depend on Q, K or V, so it enters
 * only the recomputed probabilities).  alibi_slopes as for attn_fwd_alibi
 * (the same values the forward used); o and lse from attn_fwd_alibi.
 * Everything else is as for attn_bwd.
 */
int attn_bwd_alibi(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, const float* alibi_slopes,
                   int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                   int layout, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd_varlen - attn_bwd for packed sequences (the backward of
 * attn_fwd_varlen): each sequence's gradients are those of its own problem.
 *
 *   q, k, v, o, dout, dq, dk, dv  packed as for attn_fwd_varlen
 *                 (q, o, dout, dq [total_q, Hq, d]; k, v, dk, dv
 *                 [total_k, Hkv, d])
 *   lse           fp32 [Hq, total_q], as attn_fwd_varlen writes it
 *   cu_seqlens_q, cu_seqlens_k  device int32 [B + 1], as for attn_fwd_varlen
 *   max_seqlen_q, max_seqlen_k  >= every query / key length (they size the
 *                 launches; rows or keys of a longer sequence past them are
 *                 not written)
 *   workspace     at least attn_bwd_workspace_bytes(1, Hq, total_q) bytes
 * Key rows of a sequence with no query rows get dK = dV = 0.  Size limits
 * (ATTN_ERR_SHAPE): (total + 64) * heads * 256 < 2^31 for q and k, Hq <=
 * 65535.  Other arguments, checks and statuses as for attn_bwd.
 */
int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q,
                    const int32_t* cu_seqlens_k, int B, int Hq, int Hkv, int total_q,
                    int total_k, int max_seqlen_q, int max_seqlen_k, int d, float scale,
                    int causal, void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* attn_status_string(int status);

/* ATTN_VERSION of the built library. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */

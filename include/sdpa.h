/*
 * libsdpa — exact scaled dot-product attention forward on MI355X (gfx950).
 *
 * Computes O = softmax(Q K^T * scale + mask) V over the last (key) axis, with
 * the score matrix never written to memory.  The operation is the one built
 * from reshape, two batched products, a scale, an additive 0/-inf causal mask
 * and a last-axis softmax in the tensai autograd guide (section
 * "Attention の組み立て"), the exact dense kernel of the HOF Flash Attention
 * essay (distillative.ai, section 4 "カーネル"), and the dense / paged
 * attention entry points of the ruDNN user guide (sections 2 and 9).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Layout: q is [B, Hq, Sq, D], k and v are [B, Hkv, Sk, D], out is
 *    [B, Hq, Sq, D]; all contiguous, row-major, innermost dimension D
 *    (the (batch, head, seq, headDim) layout of the tensai guide).
 *  - Grouped K/V: Hq must be a multiple of Hkv; query head h reads K/V head
 *    h / (Hq / Hkv) (contiguous groups; ruDNN guide section 9 requires only
 *    divisibility).
 *  - dtype: q, k, v and out share one element type, SDPA_BF16, SDPA_F16 or
 *    SDPA_F32 (the ruDNN guide's F32/F16/BF16 inputs, sections 9 and 10).
 *    Products accumulate in fp32; softmax statistics (running max, sum,
 *    log-sum-exp) are fp32; the output is rounded to the input type (round to
 *    nearest even), as the ruDNN guide's normalisation ops do (section 7).
 *    On the 16-bit paths the softmax weights are rounded to the input type
 *    before the product with V, and the running denominator is the fp32 sum
 *    of those same rounded weights; scores, the running max and Q are never
 *    rounded.
 *  - Pointers: every tensor pointer (q, k, v, out, key_lens, workspace) is a
 *    DEVICE pointer on the current HIP device, owned by the caller.  The
 *    library allocates nothing and keeps no per-call state, except the one
 *    static device scratch array of sdpa_decode_noalloc (below).
 *  - stream: a hipStream_t passed as void* (NULL = the null stream).  Work is
 *    enqueued and the call returns; out is valid once the stream has reached
 *    that point.  The library never synchronises.
 *  - Errors: arguments are validated on the host before any HIP call; on
 *    error nothing is launched and out is left untouched.  A launch failure
 *    returns SDPA_ERR_HIP.  There is no fallback kernel: a valid call that no
 *    kernel covers returns SDPA_ERR_UNSUPPORTED (the ruDNN guide's rule that
 *    an automatic choice falls back only for unsupported configurations and
 *    never hides an execution failure, section 10).
 *  - Not checked (device data): finiteness of q, k, v, and key_lens values.
 *    Contract: 1 <= key_lens[b] <= Sk.  A value above Sk acts as Sk; a value
 *    <= 0 leaves every key of that batch hidden and its output rows NaN
 *    (0/0, the literal result of normalising an empty softmax).
 *  - Aliasing: out must not overlap q, k, v, key_lens or the workspace
 *    (ruDNN guide section 11: outputs may not overlap inputs).
 *  - Concurrency: calls are reentrant; calls on different streams do not
 *    interact.  Calls that share a decode workspace must be ordered on one
 *    stream (ruDNN guide section 9: a split workspace is reused only with the
 *    same shapes and one ordered queue).
 */
#ifndef LIBSDPA_SDPA_H
#define LIBSDPA_SDPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SDPA_OK = 0,
    SDPA_ERR_INVALID_ARGUMENT = 1, /* bad pointer, size, flag or aliasing       */
    SDPA_ERR_UNSUPPORTED = 2,      /* valid, but no kernel covers it (e.g. D)    */
    SDPA_ERR_WORKSPACE = 3,        /* decode workspace missing or too small      */
    SDPA_ERR_HIP = 4               /* a HIP runtime call or launch failed        */
} sdpa_status_t;

typedef enum { SDPA_F32 = 0, SDPA_BF16 = 1, SDPA_F16 = 2 } sdpa_dtype_t;

/* Mask flags, combinable with |. */
enum {
    SDPA_MASK_NONE = 0,
    SDPA_MASK_CAUSAL = 1,      /* key j visible to query i iff j <= i (needs Sq == Sk);
                                  tensai guide: 0 on and below the diagonal, -inf above */
    SDPA_MASK_KEY_PADDING = 2  /* key j of batch b visible iff j < key_lens[b]          */
};

/* Largest split count of the decode path (ruDNN guide section 9: 2..=32 splits,
 * plus the unsplit case 1). */
#define SDPA_MAX_SPLITS 32

/*
 * Prefill / full forward.
 *   q        device [B, Hq, Sq, D], dtype
 *   k, v     device [B, Hkv, Sk, D], dtype
 *   B, Hq, Hkv, Sq, Sk, D   sizes, all >= 1, Hq % Hkv == 0
 *   scale    finite, > 0; multiplies the scores before the mask is added
 *   mask_kind  SDPA_MASK_* flags; SDPA_MASK_CAUSAL requires Sq == Sk
 *   key_lens device int32 [B] when mask_kind has SDPA_MASK_KEY_PADDING, else NULL
 *   out      device [B, Hq, Sq, D], dtype; written completely
 *   dtype    SDPA_BF16, SDPA_F16 or SDPA_F32
 *   stream   hipStream_t as void*
 * Supported head dims: SDPA_BF16 / SDPA_F16 any multiple of 8 from 8 to 1024
 * (ruDNN user guide section 9 allows up to 1024): up to 128 on the 64- and
 * 128-wide kernels, with the dims past D read as zeros on chip; from 136 to
 * 256 on paired waves that split the head dim in two and add each other's
 * partial scores in LDS (with a bias: two workgroups per query block each
 * produce 128 output dims and both compute the scores); above 256 on a
 * kernel that splits the head dim over 4, 6 or 8 waves of 128 dims per
 * 32-row query block (partial scores summed in LDS).  Any other D from 1 to
 * 1023 on the same kernels with Q, K and V read element by element (rows of
 * such a width are not 16-byte aligned); not with a bias.  SDPA_F32 any
 * multiple of 4 from 4 to 128 (the 64- and 128-wide fp32 kernels, likewise;
 * when the grid of 32-row query blocks fits the CUs, each block's keys are
 * split over its workgroup's waves and their softmax states merged).  One
 * head (Sq*D or Sk*D elements) must be under 2 GiB (SDPA_ERR_UNSUPPORTED
 * otherwise).
 */
sdpa_status_t sdpa_forward(const void *q, const void *k, const void *v,
                           int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D,
                           float scale, int mask_kind, const int32_t *key_lens,
                           void *out, int dtype, void *stream);

/*
 * sdpa_forward that also writes each row's log-sum-exp, the statistic the
 * backward recomputes the probabilities from (ruDNN guide section 11: the
 * backward keeps no score matrix).
 *   lse      device float [B, Hq, Sq]: lse_i = ln(sum_j exp(scale * s_ij))
 *            over the visible keys j of row i (natural log, scaled-score
 *            units), -inf for a row with no visible key
 * Every other argument as sdpa_forward; lse must not overlap any tensor.
 * Supported: the dtypes and head dims of sdpa_forward.
 */
sdpa_status_t sdpa_forward_lse(const void *q, const void *k, const void *v,
                               int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk,
                               int64_t D, float scale, int mask_kind, const int32_t *key_lens,
                               void *out, float *lse, int dtype, void *stream);

/*
 * Forward with a general additive mask: O = softmax(Q K^T * scale + bias +
 * mask) V, the tensai guide's Add(mask) with an arbitrary mask tensor
 * ("Attention の組み立て"), combinable with the causal / key-padding flags.
 *   bias       device [B or 1, Hq or 1, Sq, Sk], dtype; element (b, h, i, j)
 *              at bias[b * bias_stride_b + h * bias_stride_h + i * Sk + j]
 *              (a stride of 0 broadcasts over that axis).  Finite values or
 *              -inf (hides the key); a row left with no visible key is NaN
 *              (lse -inf).
 *   lse        NULL, or device float [B, Hq, Sq] as in sdpa_forward_lse
 * Every other argument as sdpa_forward.  The bias is read once per 128-row
 * query block (and output slice, 128 < D <= 256; by every wave above 256).
 * Supported: dtype SDPA_BF16 or SDPA_F16, D a multiple of 8 up to 1024, bias
 * rows 16-byte aligned (Sk, bias_stride_b and bias_stride_h multiples of 8,
 * pointer 16-byte aligned), one head's bias (Sq * Sk elements) under 2 GiB
 * (SDPA_ERR_UNSUPPORTED otherwise).  out and lse must not overlap the bias.
 */
sdpa_status_t sdpa_forward_bias(const void *q, const void *k, const void *v,
                                int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk,
                                int64_t D, float scale, int mask_kind, const int32_t *key_lens,
                                const void *bias, int64_t bias_stride_b, int64_t bias_stride_h,
                                void *out, float *lse, int dtype, void *stream);

/*
 * Bytes of device workspace sdpa_backward needs (0 if the sizes are invalid):
 * 8 bytes per query row, rows of a head padded to an even count.
 */
size_t sdpa_backward_workspace_size(int64_t B, int64_t Hq, int64_t Sq);

/*
 * Attention backward (ruDNN guide section 11; the derivative of the tensai
 * guide's attention block): the gradients of a loss L through
 * O = softmax(Q K^T * scale + mask) V, given dout = dL/dO,
 *   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - rowsum(dO o O)),
 *   dQ = scale dS K,  dK = scale dS^T Q,
 * with P recomputed as exp(scale * s_ij - lse_i) (hidden keys 0).  A K/V head's
 * dK and dV sum over its Hq / Hkv query heads; rows with no visible key
 * contribute nothing and get dQ = 0; keys at or past key_lens[b] get dK = dV = 0.
 *   q, out, dout   device [B, Hq, Sq, D], dtype (out: the forward's output)
 *   k, v           device [B, Hkv, Sk, D], dtype
 *   lse            device float [B, Hq, Sq] from sdpa_forward_lse
 *   scale, mask_kind, key_lens   as in the forward call
 *   dq             device [B, Hq, Sq, D], dtype; written completely
 *   dk, dv         device [B, Hkv, Sk, D], dtype; written completely
 *   workspace      device buffer of at least sdpa_backward_workspace_size bytes
 * Up to D = 128 two kernels are enqueued on stream: a query-parallel pass
 * (dQ, and each row's rowsum(dO o O) into the workspace) then a key-parallel
 * pass (dK, dV); above 128 three (a row-statistics pass first, then the two
 * passes with the head dim split over 2 or 4 waves of 128 dims).
 * Every sum runs in a fixed order: the result is bitwise reproducible (the
 * guide's ordered, atomic-free reduction).  Accumulation is fp32; P and dS are
 * rounded to dtype before their products, and the gradients to dtype at the end.
 * Outputs and workspace must not overlap each other or any input.
 * Supported: dtype SDPA_BF16 or SDPA_F16, D any width up to 512 (ruDNN user
 * guide section 9; SDPA_ERR_UNSUPPORTED above); a width that is not a
 * multiple of 8 is read and written element by element.  SDPA_F32 (section
 * 9: F32 inputs), D a multiple of 4 up to 128: three kernels (the row
 * statistics, then the dQ and the dK/dV passes on fp32 MFMA), P and dS kept
 * in fp32.
 */
sdpa_status_t sdpa_backward(const void *q, const void *k, const void *v, const void *out,
                            const void *dout, const float *lse,
                            int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk, int64_t D,
                            float scale, int mask_kind, const int32_t *key_lens,
                            void *dq, void *dk, void *dv,
                            void *workspace, size_t workspace_bytes, int dtype, void *stream);

/*
 * The backward of sdpa_forward_bias (tensai guide, "Attention の組み立て":
 * the additive mask enters after Scale, before Softmax): dq, dk, dv as
 * sdpa_backward with P recomputed from the biased scores, and optionally the
 * bias gradient, which is dS = P o (dP - rowsum(dO o O)) itself.
 *   lse        device float [B, Hq, Sq] from sdpa_forward_bias with this bias
 *   bias, bias_stride_b, bias_stride_h   as in sdpa_forward_bias
 *   dbias      NULL, or device [B, Hq, Sq, Sk], dtype, 16-byte aligned:
 *              written completely (0 at hidden keys); for a bias broadcast
 *              over batch or heads the caller sums it over those axes
 * Every other argument as sdpa_backward (same workspace size).  The bias is
 * read by both passes; dbias is written by the query-parallel one.  Outputs
 * and workspace must not overlap each other or any input.
 * Supported: dtype SDPA_BF16 or SDPA_F16, D a multiple of 8 up to 128, bias
 * rows 16-byte aligned (Sk and the strides multiples of 8), one head's bias
 * (Sq * Sk elements) under 2 GiB (SDPA_ERR_UNSUPPORTED otherwise).
 */
sdpa_status_t sdpa_backward_bias(const void *q, const void *k, const void *v, const void *out,
                                 const void *dout, const float *lse,
                                 int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk,
                                 int64_t D, float scale, int mask_kind, const int32_t *key_lens,
                                 const void *bias, int64_t bias_stride_b, int64_t bias_stride_h,
                                 void *dq, void *dk, void *dv, void *dbias,
                                 void *workspace, size_t workspace_bytes, int dtype, void *stream);

/*
 * Bytes of device workspace sdpa_backward_atomic needs (0 if the sizes are
 * invalid): the row statistics of sdpa_backward_workspace_size, then an fp32
 * dQ accumulator [B, Hq, Sq, D], each section 256-byte aligned.
 */
size_t sdpa_backward_atomic_workspace_size(int64_t B, int64_t Hq, int64_t Sq, int64_t D);

/*
 * The attention backward with an atomic dQ reduction (ruDNN guide section 11:
 * the history gradients by fp32 atomic addition, next to the ordered
 * reduction of sdpa_backward).  Same arguments, results and contract as
 * sdpa_backward except the workspace (sdpa_backward_atomic_workspace_size)
 * and the order of dQ's sums: three kernels are enqueued — row statistics
 * and a zeroed accumulator; one key-parallel pass that forms dK, dV and adds
 * every key block's share of dQ into the accumulator with fp32 atomics; and
 * the conversion dQ = scale * accumulator rounded to dtype.  dK and dV are
 * bitwise reproducible; dQ's summation order varies from call to call, so
 * dQ is not.  One head's accumulator (Sq * D floats) must be under 2 GiB.
 */
sdpa_status_t sdpa_backward_atomic(const void *q, const void *k, const void *v, const void *out,
                                   const void *dout, const float *lse,
                                   int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t Sk,
                                   int64_t D, float scale, int mask_kind, const int32_t *key_lens,
                                   void *dq, void *dk, void *dv,
                                   void *workspace, size_t workspace_bytes, int dtype, void *stream);

/*
 * Bytes of device workspace sdpa_block_forward needs (0 if the sizes are
 * invalid): q, k, v and the attention output, each [B, heads, S, model/heads]
 * in the input dtype, 256-byte aligned.
 */
size_t sdpa_block_workspace_size(int64_t B, int64_t S, int64_t model);

/*
 * The multi-head attention block of the tensai guide ("Attention の組み立て"):
 *   q, k, v = heads(x . wq), heads(x . wk), heads(x . wv)
 *   y       = heads^-1(softmax(q k^T * scale + mask) v) . wo
 * where heads reshapes (batch, seq, model) to (batch, seq, head, headDim)
 * and swaps seq and head, and heads^-1 undoes it.
 *   x              device [B, S, model], dtype
 *   wq, wk, wv, wo device [model, model], dtype (x is multiplied on the left)
 *   heads          model % heads == 0; headDim = model / heads
 *   scale, mask_kind, key_lens   as in sdpa_forward (with Sq = Sk = S)
 *   y              device [B, S, model], dtype; written completely
 *   workspace      device buffer of at least sdpa_block_workspace_size bytes
 * Three kernels are enqueued: the q, k, v projections in one launch (written
 * straight into head layout), the attention, and the output projection
 * (reading the attention output from head layout).  Products accumulate in
 * fp32; q, k, v, the attention output and y are rounded to dtype.
 * Supported: dtype SDPA_BF16 or SDPA_F16, headDim a multiple of 8 up to 1024,
 * x and each weight under 2 GiB.  y and the workspace must not overlap each
 * other or any input.
 */
sdpa_status_t sdpa_block_forward(const void *x, const void *wq, const void *wk, const void *wv,
                                 const void *wo, int64_t B, int64_t S, int64_t model,
                                 int64_t heads, float scale, int mask_kind,
                                 const int32_t *key_lens, void *y, void *workspace,
                                 size_t workspace_bytes, int dtype, void *stream);

/*
 * Bytes of device workspace sdpa_decode needs for these sizes (0 if the sizes
 * are invalid).  Layout, fp32, 256-byte aligned sections:
 *   o_part [B, Hq, num_splits, Dp] normalised partial outputs, Dp = D
 *                                  rounded up to a multiple of 4 (the
 *                                  padding floats are unspecified)
 *   lse    [B, Hq, num_splits]     natural-log log-sum-exp of each partial
 * Split s covers keys [s*C, min((s+1)*C, len_b)) with C = ceil(Sk / num_splits)
 * and len_b = key_lens[b] (or Sk); an empty split holds o_part = 0, lse = -inf.
 * (ruDNN guide section 9: split partial statistics and the merge are FP32.)
 */
size_t sdpa_decode_workspace_size(int64_t B, int64_t Hq, int64_t D, int num_splits);

/*
 * Single-query decode with split-KV and a log-sum-exp merge (ruDNN guide
 * section 9, split history).  Equivalent to sdpa_forward with Sq = 1 and no
 * causal mask: every cached key below key_lens[b] (or Sk) is visible.
 *   q          device [B, Hq, 1, D]
 *   k, v       device [B, Hkv, Sk, D]
 *   key_lens   device int32 [B] or NULL (all Sk keys valid)
 *   num_splits 1..SDPA_MAX_SPLITS
 *   workspace  device buffer of at least sdpa_decode_workspace_size() bytes
 *   out        device [B, Hq, 1, D]
 * Two kernels are enqueued on stream: the split pass, then the merge.
 * Supported: dtype SDPA_BF16 or SDPA_F16, D any width up to 1024 (a width
 * that is not a multiple of 8 is read element by element; above 128 each
 * wave's LDS ring holds two 16-key steps instead of four;
 * above 256 the split pass runs on the head-dim-split kernel of
 * sdpa_forward, with up to 32 query heads of a K/V group as its rows, and
 * writes the same partials).
 */
sdpa_status_t sdpa_decode(const void *q, const void *k, const void *v,
                          int64_t B, int64_t Hq, int64_t Hkv, int64_t Sk, int64_t D,
                          float scale, const int32_t *key_lens, int num_splits,
                          void *workspace, size_t workspace_bytes,
                          void *out, int dtype, void *stream);

/* Bytes of the static device scratch array behind sdpa_decode_noalloc: room
 * for the decode partials of B=64, Hq=32, D=128 at 32 splits (33.8 MB) with
 * headroom.  Every GPU the library runs on holds one copy from module load
 * until the process ends. */
#define SDPA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * sdpa_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  Arguments, results, kernels and errors are
 * those of sdpa_decode; the split partials go to a file-scope device array of
 * SDPA_NOALLOC_SCRATCH_BYTES (one per GPU, its address looked up once per
 * device on the first call there).  The call itself allocates nothing: no
 * hipMalloc, hipFree or allocating library routine.
 *   Returns SDPA_ERR_WORKSPACE, launching nothing, when
 *   sdpa_decode_workspace_size(B, Hq, D, num_splits) exceeds
 *   SDPA_NOALLOC_SCRATCH_BYTES.
 *   Concurrency: every call on one GPU shares that GPU's scratch, so calls
 *   that overlap in time on one GPU (different streams, or host threads
 *   without ordering) race and may return wrong results; order them on one
 *   stream.  The scratch keeps the last call's partials; nothing in it needs
 *   clearing between calls.
 */
sdpa_status_t sdpa_decode_noalloc(const void *q, const void *k, const void *v,
                                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Sk, int64_t D,
                                  float scale, const int32_t *key_lens, int num_splits,
                                  void *out, int dtype, void *stream);

/*
 * Paged attention over a shared K/V page cache (ruDNN guide section 9): packed
 * queries of several sequences, prefill chunks and decode alike, each query
 * attending to the cached keys of its own sequence through that sequence's
 * page table.  Split-KV with the same log-sum-exp merge as sdpa_decode.
 *   q            device [queries, Hq, D]
 *   k_cache      device [pages, page_size, Hkv, D]
 *   v_cache      device [pages, page_size, Hkv, Dv]: the value head dim Dv
 *                may differ from D (the guide's K [.., Hkv, D], V [.., Hkv,
 *                Dv], output [.., Hq, Dv])
 *   block_tables device int32 [num_seqs, max_pages_per_seq]: logical key j of
 *                sequence s is slot j % page_size of physical page
 *                block_tables[s][j / page_size]
 *   seq_lens     device int32 [num_seqs]: cached keys of each sequence
 *   query_seq    device int32 [queries]: the sequence of each query
 *   query_pos    device int32 [queries]: zero-based absolute position of each
 *                query within its sequence (used by the causal flag)
 *   max_seq_len  host: bound on seq_lens; splits cover [0, max_seq_len) in
 *                chunks of ceil(max_seq_len / num_splits) keys rounded up to a
 *                multiple of 16.  Must be <= max_pages_per_seq * page_size.
 *   causal       0: query t sees keys j < seq_lens[s]; 1: additionally only
 *                j <= query_pos[t] (absolute positions: a chunk of new queries
 *                at the end of a sequence is aligned bottom-right)
 *   num_splits   1..SDPA_MAX_SPLITS
 *   workspace    device buffer of at least
 *                sdpa_decode_workspace_size(queries, Hq, Dv, num_splits) bytes
 *                (same layout as sdpa_decode's with B = queries, D = Dv)
 *   out          device [queries, Hq, Dv]
 * Two kernels are enqueued on stream: the split pass, then the merge.
 * Supported: dtype SDPA_BF16 or SDPA_F16, D and Dv any width up to 1024
 * (when either is above 256 the split pass runs on the head-dim-split
 * kernel, as in sdpa_decode, its waves covering the larger of the two;
 * widths that are not multiples of 8 read element by element);
 * page_size a multiple of 16 (SDPA_ERR_UNSUPPORTED otherwise).
 * Not checked (device data), with the kernels' behaviour outside the
 * contract: seq_lens above max_seq_len act as max_seq_len; a query_seq outside
 * [0, num_seqs), a negative query_pos under the causal flag, or a sequence
 * with no cached key leave the query with no visible key (NaN output row); a
 * block_tables entry outside [0, pages) is never read: its keys are hidden.
 */
sdpa_status_t sdpa_paged_attention(const void *q, const void *k_cache, const void *v_cache,
                                   int64_t queries, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv,
                                   int64_t pages, int64_t page_size, const int32_t *block_tables,
                                   int64_t num_seqs, int64_t max_pages_per_seq,
                                   const int32_t *seq_lens, const int32_t *query_seq,
                                   const int32_t *query_pos, int64_t max_seq_len, float scale,
                                   int causal, int num_splits, void *workspace,
                                   size_t workspace_bytes, void *out, int dtype, void *stream);

/*
 * Packed prefill chunks over the same page cache (ruDNN guide section 9:
 * packed variable-length prefill): query-tiled, each K/V page of a sequence
 * read once per 128 query rows of its chunk.  The queries of sequence s are
 * the packed rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 of q and are the
 * last n_s = cu_seqlens_q[s+1] - cu_seqlens_q[s] tokens of the sequence (they
 * are already in the cache): row i of the chunk sits at absolute position
 * seq_lens[s] - n_s + i.  Equivalent to sdpa_paged_attention with those
 * query_seq / query_pos.
 *   q             device [total_q, Hq, D]
 *   k_cache       device [pages, page_size, Hkv, D]
 *   v_cache       device [pages, page_size, Hkv, Dv] (Dv may differ from D)
 *   block_tables  device int32 [num_seqs, max_pages_per_seq] (as above)
 *   seq_lens      device int32 [num_seqs]: cached keys, the chunk included
 *   cu_seqlens_q  device int32 [num_seqs + 1]: 0 = cu[0] <= cu[1] <= ... <=
 *                 cu[num_seqs] = total_q
 *   max_q         host: bound on the chunk lengths (sizes the grid)
 *   max_seq_len   host: bound on seq_lens, <= max_pages_per_seq * page_size
 *   causal        0: every cached key of the sequence is visible; 1: only
 *                 keys j <= the row's absolute position
 *   out           device [total_q, Hq, Dv]
 *   lse           device fp32 [total_q, Hq] or NULL: natural-log log-sum-exp
 *                 of each row's scaled scores (-inf for a row with no visible
 *                 key), the input sdpa_paged_backward needs
 * One kernel is enqueued; no workspace.  Supported: dtype SDPA_BF16 or
 * SDPA_F16, D and Dv any width up to 1024 (when either is above 256 on the
 * head-dim-split kernel; otherwise a value head dim above 128 in two 128-dim
 * output slices; widths that are not multiples of 8 read element by
 * element); page_size a multiple of
 * 16 (SDPA_ERR_UNSUPPORTED otherwise).
 * Not checked (device data), with the kernel's behaviour outside the
 * contract: cu_seqlens_q entries are clamped into [0, total_q] (no row outside
 * out is ever written); a chunk longer than max_q is only computed for its
 * first ceil(max_q / 128) * 128 rows (the rest are not written);
 * seq_lens above max_seq_len act as max_seq_len; rows left with no visible
 * key are NaN; a block_tables entry outside [0, pages) is never read and its
 * keys are hidden.
 */
sdpa_status_t sdpa_paged_prefill(const void *q, const void *k_cache, const void *v_cache,
                                 int64_t total_q, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv,
                                 int64_t pages,
                                 int64_t page_size, const int32_t *block_tables, int64_t num_seqs,
                                 int64_t max_pages_per_seq, const int32_t *seq_lens,
                                 const int32_t *cu_seqlens_q, int64_t max_q, int64_t max_seq_len,
                                 float scale, int causal, void *out, float *lse, int dtype,
                                 void *stream);

/*
 * Bytes of device workspace sdpa_paged_backward needs (0 if the sizes or the
 * dtype are invalid): Q, dO, O and dQ of every sequence at its absolute
 * positions [num_seqs, Hq, max_seq_len, W] (in dtype), K, V, dK and dV of its
 * reachable keys [num_seqs, Hkv, max_seq_len, W], their fp32 log-sum-exp and
 * the dense backward's statistics; W = max(D, Dv) rounded up to a multiple
 * of 8 (16-bit) or W = D (SDPA_F32).
 */
size_t sdpa_paged_backward_workspace_size(int64_t num_seqs, int64_t Hq, int64_t Hkv,
                                          int64_t max_seq_len, int64_t D, int64_t Dv, int dtype);

/*
 * Backward of sdpa_paged_prefill (ruDNN guide section 11: the paged plan's
 * attention backward returns dq and the history gradients dk, dv and
 * recomputes the probabilities from the forward's log-sum-exp).  For a loss
 * L with dL/dout = dout:
 *   dq        device [total_q, Hq, D]: dL/dq
 *   dk_cache  device [pages, page_size, Hkv, D]: dL/dk_cache
 *   dv_cache  device [pages, page_size, Hkv, Dv]: dL/dv_cache; in both,
 *             every slot a sequence's keys j < seq_lens[s] sit in gets that
 *             key's gradient, every other slot 0 (written in full)
 * Inputs as sdpa_paged_prefill (V of its own width Dv), plus its out and lse
 * (fp32 [total_q, Hq]) and dout [total_q, Hq, Dv].  Each sequence's chunk
 * rows are placed at their absolute positions in dense per-sequence tensors
 * in the workspace (with the zero rows of absent positions adding nothing),
 * zero-padded to the common width W (zero dims change no score, row term or
 * gradient of the true dims); the dense ordered backward runs on them
 * (causal flag and key limit seq_lens), and the gradients' true dims are
 * scattered back: deterministic, no atomics.  Several kernels are enqueued
 * on stream.  Supported: SDPA_BF16 or SDPA_F16 with D and Dv any width up to
 * 512, or SDPA_F32 with Dv = D a multiple of 4 up to 128 (the fp32 dense
 * backward, all in fp32); page_size a multiple of 16 (SDPA_ERR_UNSUPPORTED
 * otherwise).
 * Outputs and the workspace must overlap no input and each other.
 * Not checked (device data): as sdpa_paged_prefill; in addition every table
 * entry a sequence's keys j < seq_lens[s] use must lie in [0, pages) (an
 * entry outside reads as zero keys and values) and no physical page may be
 * reached by two sequences (such a page gets one sequence's gradient).  The
 * work scales with num_seqs * max_seq_len rows, not with the chunk lengths.
 */
sdpa_status_t sdpa_paged_backward(const void *q, const void *k_cache, const void *v_cache,
                                  const void *out, const void *dout, const float *lse,
                                  int64_t total_q, int64_t Hq, int64_t Hkv, int64_t D, int64_t Dv,
                                  int64_t pages, int64_t page_size, const int32_t *block_tables,
                                  int64_t num_seqs, int64_t max_pages_per_seq,
                                  const int32_t *seq_lens, const int32_t *cu_seqlens_q,
                                  int64_t max_seq_len, float scale, int causal, void *dq,
                                  void *dk_cache, void *dv_cache, void *workspace,
                                  size_t workspace_bytes, int dtype, void *stream);

/* Static English name of a status code; never NULL. */
const char *sdpa_status_string(int status);

/* Detail of the last failed call on this host thread ("" if none); valid
 * until the next call on the same thread. */
const char *sdpa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBSDPA_SDPA_H */

/*
 * cpattn.h - C ABI of libcpattn.so: load-balanced context-parallel causal attention and
 * grouped-query decode attention for AMD Instinct MI355X (gfx950).
 *
 * Conventions for every call below
 *  - Pointers named for tensors are DEVICE pointers (hipMalloc'd or torch CUDA storage) unless
 *    the comment says host. The caller owns every buffer; the library allocates nothing per call
 *    and keeps no pointer after it returns.
 *  - Tensors are dense, row-major, innermost dimension last, with the shapes given.
 *  - Calls that take `stream` enqueue work on that hipStream_t (NULL = the null stream) and
 *    return without synchronising. Results are ready when the stream reaches that point.
 *  - Every shape, dtype, alignment and pointer check runs on the host before any HIP call.
 *    A failed check returns CPA_EINVAL (bad argument) or CPA_ENOTSUP (valid but unsupported
 *    combination, or a device that is not gfx950) and enqueues nothing. A HIP launch or runtime
 *    failure returns CPA_EHIP. cpattn_last_error() then gives a message for the calling thread.
 *  - Preconditions that live in device memory (position and length values) cannot be checked
 *    without a synchronisation. Kernels clamp them so that no access leaves the buffers, but
 *    the numbers produced for out-of-range values are unspecified.
 *  - Batch 0, zero rows or zero sequences are valid and enqueue nothing.
 *
 * Load-balanced order ("Add context parallelism", MaxText PR 1445, Description): the sequence
 * of length S is cut into 2*cp chunks of c = S/(2*cp) tokens; rank r keeps chunk r followed by
 * chunk 2*cp-1-r, so every rank sees about the same number of causal (query, key) pairs. For
 * cp = 2 and S = 8 this gives 0,1,6,7 | 2,3,4,5. The "permuted" sequence is the concatenation of
 * the ranks' shards in rank order, which is what an all-gather of the shards returns. Permuted
 * slot j holds original position src(j) = r*c + w if w < c, else (2*cp-1-r)*c + (w-c), where
 * r = j / (2c), w = j % (2c).
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CPA_OK = 0,
  CPA_EINVAL = -22,   /* an argument is invalid (shape, divisibility, null or misaligned pointer) */
  CPA_ENOTSUP = -95,  /* valid but unsupported here (head dim, dtype, device other than gfx950)  */
  CPA_EHIP = -1000    /* a HIP runtime call or kernel launch failed                              */
} cpa_status;

typedef enum {
  CPA_F32 = 0,   /* IEEE float32 storage, float32 arithmetic                                 */
  CPA_BF16 = 1   /* bfloat16 storage, float32 accumulation                                   */
} cpa_dtype;

/* Message for the last non-OK status returned on the calling thread (never NULL). */
const char* cpattn_last_error(void);

/* ---------------------------------------------------------------------------------------------
 * Index helpers (host only, no HIP call).
 * ------------------------------------------------------------------------------------------- */

/* Original token position held by permuted slot j, i.e. src(j) above.
 * Returns -1 if seq < 1, cp < 1, seq % (2*cp) != 0 or j is outside [0, seq). */
int64_t cp_load_balance_source_index(int64_t seq, int32_t cp, int64_t j);

/* Writes src(row_begin + i) for i in [0, row_count) to out_host (HOST int32 array of row_count
 * entries). Rank r's query positions are row_begin = r*2c, row_count = 2c.
 * CPA_EINVAL for the same conditions as above, for a window outside [0, seq), or seq >= 2^31. */
int cp_load_balance_positions(int64_t seq, int32_t cp, int64_t row_begin, int64_t row_count,
                              int32_t* out_host);

/* ---------------------------------------------------------------------------------------------
 * Load-balance permutation: the token reorder that "Add context parallelism" (PR 1445,
 * Description) performs with a gather along the sequence axis. Both calls are bit copies: rows
 * are moved as raw bytes, so any dtype works and the round trip is exact.
 *
 * A tensor is viewed as [outer, seq, row_bytes]: every dimension before the sequence axis folds
 * into `outer`, every dimension after it into `row_bytes` (e.g. Q [B,S,H,D] bf16 has outer = B,
 * row_bytes = H*D*2; an LSE [B,H,S] fp32 permuted along S has outer = B*H, row_bytes = 4).
 * The window [row_begin, row_begin + row_count) selects slots of the PERMUTED order; the full
 * permutation is row_begin = 0, row_count = seq. A rank's own share is row_begin = r*2c,
 * row_count = 2c.
 * ------------------------------------------------------------------------------------------- */

/* Gather. src: [outer, seq, row_bytes] in original token order.
 * dst: [outer, row_count, row_bytes]; dst[o, i] = src[o, src(row_begin + i)].
 * src and dst must not overlap. CPA_EINVAL if seq % (2*cp) != 0, cp < 1, the window leaves
 * [0, seq), row_bytes < 1, or a pointer is NULL while the copy is non-empty. */
int cp_load_balance_permute(const void* src, void* dst, int64_t outer, int64_t seq,
                            int64_t row_bytes, int32_t cp, int64_t row_begin, int64_t row_count,
                            void* stream);

/* Scatter, the exact inverse. src: [outer, row_count, row_bytes] holding permuted slots
 * [row_begin, row_begin + row_count). dst: [outer, seq, row_bytes] in original order;
 * dst[o, src(row_begin + i)] = src[o, i]. Rows of dst outside the window's images are left
 * untouched, so calling it once per rank (or once with the full window) rebuilds the whole
 * tensor. Same errors as cp_load_balance_permute. */
int cp_load_balance_unpermute(const void* src, void* dst, int64_t outer, int64_t seq,
                              int64_t row_bytes, int32_t cp, int64_t row_begin, int64_t row_count,
                              void* stream);

/* ---------------------------------------------------------------------------------------------
 * Causal grouped-query attention forward for one context-parallel rank ("Add context
 * parallelism", PR 1445, Description: keys and values all-gathered, queries sharded on the
 * sequence, tokens and mask reordered for balance; unit test of "Add support for EP to context
 * parallelism in self-attention", PR 2023: the sharded result equals un-sharded dot-product
 * attention).
 *
 *   q_shard     [B, sq, Hq, Dqk]  the rank's query rows (in its shard order)
 *   k           [B, seq, Hkv, Dqk] all keys in PERMUTED (all-gathered) order
 *   v           [B, seq, Hkv, Dv]  all values in permuted order
 *   q_positions [sq] int32, original position of each query row; NULL means the rank's own
 *               shard, src(rank*2c + i), in which case sq must equal 2c = seq/cp
 *   o           [B, sq, Hq, Dv] same dtype as q (output)
 *   lse         [B, Hq, sq] float32 (output, may be NULL): natural-log log-sum-exp of the scaled
 *               logits of each row
 *
 * For row i and query head h (kv head g = h / (Hq/Hkv)), key j is visible iff
 * src(j) <= q_positions[i] (a token sees itself):
 *   O[b,i,h,:] = sum_j softmax_j(scale * q.k_j) * v_j,  LSE[b,h,i] = ln sum_j exp(scale*q.k_j).
 * Precision: float32 accumulation; for bf16 the probabilities are rounded to bf16 before the PV
 * product and the row sum uses the same rounded values.
 * Supported (dtype, Dqk, Dv): bf16 with (64,64), (128,128), (192,128); f32 with (64,64),
 * (128,128). Others return CPA_ENOTSUP.
 * CPA_EINVAL if seq % (2*cp) != 0, rank outside [0, cp), hq % hkv != 0, a needed pointer is NULL
 * or not 16-byte aligned, scale is not finite and positive, or q_positions == NULL with
 * sq != seq/cp. Device precondition: 0 <= q_positions[i] < seq. */
int cp_attention_fwd(const void* q_shard, const void* k, const void* v,
                     const int32_t* q_positions, void* o, float* lse,
                     int32_t batch, int32_t seq, int32_t sq, int32_t hq, int32_t hkv,
                     int32_t d_qk, int32_t d_v, int32_t dtype, float softmax_scale,
                     int32_t cp, int32_t rank, void* stream);

/* cp_attention_fwd_ws: cp_attention_fwd with an optional caller workspace, which lets the bf16
 * forward balance small grids in time as well as in work. "Add context parallelism" (PR 1445,
 * Description) balances the ranks so that they take a similar amount of work and hence time;
 * inside one rank, a grid with fewer than two 256-row work items per compute unit (the 8192-token
 * shape at cp = 4) is otherwise timed by its heaviest row block. With the workspace, the visible
 * key tiles of heavy row blocks are cut into pieces computed by separate workgroups, each writing
 * an unnormalised output with its running maximum and row sum, and a second kernel merges them
 * (O = sum_i w_i o_i / sum_i w_i l_i, w_i = exp(m_i - max m)). Same arguments, results and
 * errors as cp_attention_fwd, plus:
 *   workspace, workspace_bytes: device scratch of at least cp_attention_fwd_workspace_bytes(...)
 *            bytes, owned by the caller, 16-byte aligned; contents on entry do not matter; calls
 *            sharing one workspace must not overlap. NULL, a smaller workspace, explicit
 *            q_positions or float32 inputs run exactly as cp_attention_fwd (no split).
 * cp_attention_fwd_workspace_bytes: the bytes the split needs for the rank's own shard of this
 * shape (q_positions == NULL, sq = seq / cp); 0 when this shape is not split (grids with enough
 * work items, float32) or the arguments are invalid. */
size_t cp_attention_fwd_workspace_bytes(int32_t batch, int32_t seq, int32_t hq, int32_t hkv,
                                        int32_t d_qk, int32_t d_v, int32_t dtype, int32_t cp,
                                        int32_t rank);

int cp_attention_fwd_ws(const void* q_shard, const void* k, const void* v,
                        const int32_t* q_positions, void* o, float* lse,
                        int32_t batch, int32_t seq, int32_t sq, int32_t hq, int32_t hkv,
                        int32_t d_qk, int32_t d_v, int32_t dtype, float softmax_scale,
                        int32_t cp, int32_t rank, void* workspace, size_t workspace_bytes,
                        void* stream);

/* ---------------------------------------------------------------------------------------------
 * Backward pass of cp_attention_fwd for one rank ("Add context parallelism", PR 1445,
 * Description: context parallelism serves training on long sequences, so each rank also
 * differentiates its shard's attention). From the forward's inputs, its O and LSE, and the
 * upstream gradient dO (the chain rule through the forward's definition):
 *   D_i = dO_i . O_i,  P_ij = exp(scale q_i . k_j - LSE_i) over visible keys,
 *   dS_ij = P_ij (dO_i . v_j - D_i),  dQ_i = scale sum_j dS_ij k_j,
 *   dK_j = scale sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i,
 * with dK and dV of a kv head summed over the query heads of its group. dK and dV cover every
 * key of the gathered K/V but only this rank's query rows: summing them over the ranks (a
 * reduce-scatter on several GPUs) gives the full gradients.
 *
 *   q_shard, k, v, q_positions, batch, seq, sq, hq, hkv, d_qk, d_v, softmax_scale, cp, rank:
 *            exactly as passed to cp_attention_fwd
 *   o        [B, Sq, Hq, Dv] and lse [B, Hq, Sq] float32: that forward call's outputs
 *   d_o      [B, Sq, Hq, Dv], dtype of q
 *   dq       [B, Sq, Hq, Dqk] float32 (output)
 *   dk, dv   [B, seq, Hkv, Dqk | Dv] float32 (output), in the gathered key order
 *   workspace, workspace_bytes: at least cp_attention_bwd_workspace_bytes(batch, sq, hq) bytes of
 *            caller-owned device scratch; contents on entry do not matter; calls sharing one
 *            workspace must not overlap. With at least
 *            cp_attention_bwd_split_workspace_bytes(...) bytes (and q_positions == NULL), a grid
 *            too small to balance itself (the 8192-token shape at cp = 4) also computes dQ of its
 *            heavy 256-row blocks in pieces of their key range, which this workspace holds until a
 *            last kernel adds them in a fixed order; the ranks then take about equal time (the
 *            balance in time that "Add context parallelism" asks of the shards). A smaller
 *            workspace runs unsplit; both give dQ to within float32 rounding of each other.
 * Supported: bf16 with (d_qk, d_v) in {(64, 64), (128, 128), (192, 128)}; CPA_ENOTSUP otherwise. CPA_EINVAL
 * for the forward's argument errors, null pointers (all tensors are required), tensors not
 * 16-byte aligned (lse and q_positions: 4-byte), or a workspace that is too small. */
size_t cp_attention_bwd_workspace_bytes(int32_t batch, int32_t sq, int32_t hq);

/* cp_attention_bwd_split_workspace_bytes: the workspace bytes with which cp_attention_bwd also
 * splits the dQ of heavy row blocks for the rank's own shard of this shape (sq = seq / cp); equal
 * to cp_attention_bwd_workspace_bytes(batch, seq / cp, hq) when the shape is not split (grids
 * with enough work items); 0 when the arguments are invalid or unsupported. */
size_t cp_attention_bwd_split_workspace_bytes(int32_t batch, int32_t seq, int32_t hq, int32_t hkv,
                                              int32_t d_qk, int32_t d_v, int32_t dtype, int32_t cp,
                                              int32_t rank);

int cp_attention_bwd(const void* q_shard, const void* k, const void* v, const void* o, const float* lse,
                     const void* d_o, const int32_t* q_positions, float* dq, float* dk, float* dv,
                     int32_t batch, int32_t seq, int32_t sq, int32_t hq, int32_t hkv, int32_t d_qk,
                     int32_t d_v, int32_t dtype, float softmax_scale, int32_t cp, int32_t rank,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Grouped-query single-token decode attention ("Add Pallas GPU decode attention in Maxtext
 * inference", PR 1066, Description: decode calls a grouped-query attention kernel; Tests: the
 * cache is filled by a prefill and grows to the target length). The newest token attends to
 * cache entries 0 .. lengths[b]-1 of its sequence. Split-K over the cache length: a first kernel
 * writes per-split (max, sum, unnormalised output) partials into `workspace`, a second merges
 * them with log-sum-exp weights.
 *
 *   q        [B, Hq, D]
 *   k_cache  [B, Hkv, max_len, D]   (each (b, kv head) slab contiguous)
 *   v_cache  [B, Hkv, max_len, D]
 *   lengths  [B] int32 (device), valid entries per sequence; device precondition
 *            0 <= lengths[b] <= max_len. Entries at index >= lengths[b] are never read. A
 *            length of 0 (an empty cache slice) gives O = 0 and LSE = -inf.
 *   o        [B, Hq, D] same dtype as q (output)
 *   lse      [B, Hq] float32 (output, may be NULL)
 *   workspace, workspace_bytes: device scratch of at least gqa_decode_workspace_bytes(...)
 *            bytes, owned by the caller, holding the split partials between the two passes.
 *            Its contents on entry do not matter. Calls sharing one workspace must not overlap.
 * Supported: bf16 and f32 with D in {64, 128}. CPA_EINVAL for hq % hkv != 0, null or misaligned
 * pointers, a workspace that is too small, or a non-positive scale. */
/* gqa_decode_workspace_bytes: batch x hq x nsplit x (d + 2) floats of split partials, with
 * nsplit = ceil(max_len / 128) for max_len <= 1024 (short caches take 128-key splits, so that
 * they still fill the part) and ceil(max_len / 256) beyond; 0 for a non-positive argument. */
size_t gqa_decode_workspace_bytes(int32_t batch, int32_t hq, int32_t hkv, int32_t max_len, int32_t d);

int gqa_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* lengths, void* o, float* lse,
                         int32_t batch, int32_t hq, int32_t hkv, int32_t d, int32_t max_len,
                         int32_t dtype, float softmax_scale,
                         void* workspace, size_t workspace_bytes, void* stream);

/* gqa_decode_attention_noalloc: gqa_decode_attention for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, results and errors as gqa_decode_attention, minus the workspace: the split
 * partials go to a static device array of CPATTN_DECODE_NOALLOC_SCRATCH_BYTES bytes inside the
 * library (one per GPU, held until the process ends; its address is looked up once per device on
 * the first call there). The call performs no hipMalloc or hipFree and calls no allocating routine.
 *   Limit: gqa_decode_workspace_bytes(batch, hq, hkv, max_len, d) must not exceed
 *   CPATTN_DECODE_NOALLOC_SCRATCH_BYTES (16 MiB: e.g. batch 24, 48 query heads, max_len 2048,
 *   d 128 needs 4.8 MiB); larger calls return CPA_EINVAL with a message and enqueue nothing.
 *   Every call on one GPU shares that GPU's array and leaves its partials there: calls that
 *   overlap on one GPU (other streams, or other threads) race and give undefined results;
 *   calls ordered on one stream are safe. */
#define CPATTN_DECODE_NOALLOC_SCRATCH_BYTES (16u << 20)

int gqa_decode_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* lengths, void* o, float* lse,
                                 int32_t batch, int32_t hq, int32_t hkv, int32_t d, int32_t max_len,
                                 int32_t dtype, float softmax_scale, void* stream);

/* ---------------------------------------------------------------------------------------------
 * Merge of decode results over a cache split along its length ("rename context to
 * context_autoregressive", PR 1453, Description: a separate context-parallel axis for
 * autoregressive inference, which shards the cache by length). Each of `parts` shards holds a
 * disjoint slice of every sequence's cache entries and runs gqa_decode_attention on it; this call
 * combines their results exactly as one decode over the whole cache would:
 *   M = max_r lse_r,  w_r = exp(lse_r - M),  O = sum_r w_r o_r / sum_r w_r,  LSE = M + ln sum_r w_r.
 *
 *   o_parts   [parts, B, Hq, D] in dtype (device), each part's normalised output
 *   lse_parts [parts, B, Hq] float32 (device), each part's natural-log LSE; -inf marks an empty
 *             slice (weight 0; its o_parts entries are not read into the sum)
 *   o         [B, Hq, D] in dtype (output); lse [B, Hq] float32 (output, may be NULL)
 * A (b, h) with every part empty gets O = 0 and LSE = -inf. o may not overlap o_parts.
 * CPA_EINVAL for parts < 1, negative sizes, d < 1, an unknown dtype, a null pointer or a pointer
 * not aligned to its element size. */
int gqa_decode_merge(const void* o_parts, const float* lse_parts, void* o, float* lse, int32_t parts,
                     int32_t batch, int32_t hq, int32_t d, int32_t dtype, void* stream);

/* ---------------------------------------------------------------------------------------------
 * int8 KV cache ("rename context to context_autoregressive", PR 1453, Description: the decode
 * benchmark runs with the KV cache quantized to int8). The page names the setting, not its
 * arithmetic; the reading implemented is symmetric absmax quantization with one float32 scale per
 * cached row (sequence, kv head, position):
 *   amax = max_d |x_d|,  scale = amax / 127,  code_d = round_half_even(x_d / scale) in [-127, 127],
 * with both divisions correctly rounded in float32; a row of zeros gets scale 0 and codes 0.
 *
 * kv_cache_quantize_int8: quantizes `rows` rows of `d` values.
 *   x       [rows, d] in dtype (CPA_BF16 or CPA_F32, device), finite values
 *   codes   [rows, d] int8 (device, output); scales [rows] float32 (device, output)
 * CPA_EINVAL for negative rows, d < 1, an unknown dtype, a null pointer or x / scales not aligned
 * to their element size. rows == 0 returns CPA_OK without touching the device. */
int kv_cache_quantize_int8(const void* x, int8_t* codes, float* scales, int64_t rows, int32_t d,
                           int32_t dtype, void* stream);

/* gqa_decode_attention_int8kv: gqa_decode_attention over a quantized cache; K and V are read as
 * code * scale, everything else (lengths, GQA grouping, outputs, workspace) is as there.
 *   q        [B, Hq, 128] bf16 (device)
 *   k_codes, v_codes   [B, Hkv, max_len, 128] int8 (device, 16-byte aligned)
 *   k_scales, v_scales [B, Hkv, max_len] float32 (device), the per-row scales
 *   lengths  [B] int32 (device), 0 <= lengths[b] <= max_len; entries at or past a length are not
 *            used (they may hold anything); a length of 0 gives O = 0 and LSE = -inf
 *   o        [B, Hq, 128] bf16 (output); lse [B, Hq] float32 (output, may be NULL)
 *   workspace, workspace_bytes: at least gqa_decode_workspace_bytes(B, Hq, Hkv, max_len, 128)
 *            bytes of caller-owned device scratch; calls sharing one workspace must not overlap.
 * Supported: head dim 128, B <= 65535, Hkv * ceil((Hq / Hkv) / 16) <= 65535. CPA_ENOTSUP for other
 * head dims; CPA_EINVAL for bad sizes, null or misaligned pointers, a small workspace or a
 * non-positive scale. */
int gqa_decode_attention_int8kv(const void* q, const int8_t* k_codes, const int8_t* v_codes,
                                const float* k_scales, const float* v_scales, const int32_t* lengths,
                                void* o, float* lse, int32_t batch, int32_t hq, int32_t hkv, int32_t d,
                                int32_t max_len, float softmax_scale, void* workspace,
                                size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */

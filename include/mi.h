/*
 * mi.h - C ABI of libmi.so: attention-state merging and split-KV paged decode
 * on AMD MI355X (gfx950).
 *
 * An attention state is a pair (v, s) for one query over a subset of keys:
 * v[D] is the softmax-normalised output over that subset and s is the subset's
 * log-sum-exp of scores in base 2 (s = natural LSE * log2(e)). States over
 * disjoint key subsets merge exactly; the merge is commutative and associative
 * ("F2 hints: merge_state, base-2 LSE merge", sections 1 and 2).
 *
 * Conventions shared by every entry point:
 *  - Empty state: s = -inf, v = 0 (same page, section 5). Merging only empty
 *    states yields s = -inf and v = 0, never NaN.
 *  - Every s read by a merge is sanitised first: NaN and +inf count as -inf,
 *    i.e. "no weight" ("FlashAttention's empty-row LSE", section 2.2). A state
 *    with zero weight contributes nothing, even if its v holds NaN.
 *  - s / lse values are always fp32, base 2.
 *  - Arithmetic is fp32 with exp2/log2; v outputs are rounded to nearest even
 *    into the requested dtype.
 *  - Pointers are device pointers unless a name ends in _host. Every pointer is
 *    borrowed: the caller allocates and frees; the library never allocates,
 *    frees or synchronises and keeps no state between calls.
 *  - stream is a hipStream_t passed as void*; NULL is the default stream.
 *    Calls enqueue work and return; device faults surface at the caller's next
 *    synchronisation.
 *  - Arguments are validated on the host before anything is enqueued. A
 *    non-MI_OK status means nothing was enqueued (except MI_ERR_HIP, returned
 *    when a launch itself fails).
 *  - Every output element is written, including those of empty rows and empty
 *    splits.
 *  - Tensors are dense and row-major ("C order") in the shapes given below.
 *    16-bit and fp32 tensors must be 16-byte aligned.
 */
#ifndef MI_H_
#define MI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MI_F16 = 0, MI_BF16 = 1, MI_F32 = 2 } mi_dtype;

typedef enum {
  MI_OK = 0,
  MI_ERR_NULL = 1,        /* a required pointer is NULL */
  MI_ERR_SHAPE = 2,       /* a size is negative/zero where it must be positive, or inconsistent */
  MI_ERR_DTYPE = 3,       /* dtype code out of range or not allowed for this argument */
  MI_ERR_UNSUPPORTED = 4, /* valid but not built: head dim, page size, group size, alignment,
                             or a launch past 2^32 work-items */
  MI_ERR_HIP = 5,         /* a HIP launch failed */
  MI_ERR_ALIAS = 6,       /* outputs overlap inputs other than by exact in-place aliasing */
  MI_ERR_SCRATCH = 7      /* the work needs more than the library's static scratch holds */
} mi_status;

/* Human-readable name of a status code (static storage, never NULL). */
const char* mi_status_string(mi_status status);

/*
 * Merge two states per row ("F2 hints: merge_state, base-2 LSE merge",
 * section 3; empty states, section 5).
 *   v_a, v_b : [S, H, D] of v_dtype        s_a, s_b : [S, H] fp32, base 2
 *   v_out    : [S, H, D] of out_dtype      s_out    : [S, H] fp32 (may be NULL)
 * For each row r = pos*H + h: m = max(s_a, s_b); w = 2^(s - m) (0 for an
 * empty state); v = (w_a v_a + w_b v_b) / (w_a + w_b); s = m + log2(w_a + w_b).
 * In-place use is allowed: v_out may equal v_a or v_b when out_dtype ==
 * v_dtype, and s_out may equal s_a or s_b. Any other overlap is MI_ERR_ALIAS.
 * S == 0 is a no-op. D must be a positive multiple of 8, at most 512.
 */
mi_status mi_merge_state(const void* v_a, const float* s_a, const void* v_b, const float* s_b,
                         void* v_out, float* s_out, int64_t S, int32_t H, int32_t D,
                         mi_dtype v_dtype, mi_dtype out_dtype, void* stream);

/*
 * Merge N states per (pos, h) ("F2 hints: merge_state, base-2 LSE merge",
 * section 4): the N states sit between position and head.
 *   v     : [S, N, H, D] of v_dtype      s     : [S, N, H] fp32, base 2
 *   v_out : [S, H, D] of out_dtype       s_out : [S, H] fp32 (may be NULL)
 * s[pos, n, h] is at flat offset (pos*N + n)*H + h. The result is the merge of
 * the N states; N == 1 sanitises and copies. Used with fp32 v, H = 1 and
 * S = B*Hq it is the combine of split-KV decode ("L3 hints: split-KV decode and
 * LSE merge", section 3). Outputs must not overlap inputs. S == 0 is a no-op.
 * D must be a positive multiple of 8, at most 512.
 */
mi_status mi_merge_states(const void* v, const float* s, void* v_out, float* s_out, int64_t S,
                          int32_t N, int32_t H, int32_t D, mi_dtype v_dtype, mi_dtype out_dtype,
                          void* stream);

/*
 * N-state merge over two levels, for few positions with many states each (the
 * many-index-set case of "F2 hints", section 7): each position's N states are
 * cut into slices merged in parallel into fp32 partial states (level 1), then
 * the partials are merged (level 2, the section-4 merge again). Same inputs,
 * outputs and rules as mi_merge_states; results equal up to rounding order.
 *   workspace : fp32 device buffer of at least the bytes reported by
 *               mi_merge_states_workspace (may be NULL when that is 0, in
 *               which case this is one launch of mi_merge_states); it must not
 *               overlap any other argument. Two launches on `stream`.
 */
mi_status mi_merge_states_two_level(const void* v, const float* s, void* v_out, float* s_out,
                                    int64_t S, int32_t N, int32_t H, int32_t D,
                                    mi_dtype v_dtype, mi_dtype out_dtype, float* workspace,
                                    size_t ws_bytes, void* stream);

/* Workspace bytes mi_merge_states_two_level needs for this shape (0: one level
 * suffices). Host only. */
mi_status mi_merge_states_workspace(int64_t S, int32_t N, int32_t H, int32_t D,
                                    size_t* ws_bytes);

/*
 * Two-state merge in place with an optional per-position mask (the
 * merge_state_in_place variant named in "F2 hints: merge_state, base-2 LSE
 * merge", section 7; section 3 for the merge itself).
 *   v, s       : [S, H, D] of v_dtype and [S, H] fp32 base 2, read and updated
 *   v_other,
 *   s_other    : [S, H, D] of v_dtype and [S, H] fp32, read only
 *   mask       : [S] bytes (device, may be NULL = merge every position);
 *                positions whose byte is 0 are left exactly as they were
 *                (their s is not even sanitised); the others get
 *                merge((v, s), (v_other, s_other)).
 * No overlap between v/s and the other arguments. S == 0 is a no-op. D must be
 * a positive multiple of 8, at most 512.
 */
mi_status mi_merge_state_in_place(void* v, float* s, const void* v_other, const float* s_other,
                                  const uint8_t* mask, int64_t S, int32_t H, int32_t D,
                                  mi_dtype v_dtype, void* stream);

/*
 * Fold an attention sink into each state ("FlashAttention's empty-row LSE",
 * table of section 0 and the FlashMLA branch of section 2.1): the sink acts
 * as one extra key of logit sink[h] whose value is 0, i.e. a merge with the
 * state (v = 0, s = sink[h] * log2 e). v is scaled by 2^s / (2^s + 2^sink2)
 * and s becomes log2(2^s + 2^sink2), sink2 = sink * log2 e.
 *   v, s    : [S, H, D] of v_dtype, [S, H] fp32 base 2
 *   sink    : [H] fp32 (device), natural-log logits, one per head; -inf means
 *             no sink, and NaN / +inf count as -inf like any LSE
 *   v_out   : [S, H, D] of out_dtype; s_out : [S, H] fp32 (may be NULL)
 * An empty state becomes (0, sink2). In-place use is allowed (v_out == v when
 * out_dtype == v_dtype, s_out == s); any other overlap is MI_ERR_ALIAS.
 * S == 0 is a no-op. D must be a positive multiple of 8, at most 512.
 */
mi_status mi_merge_sink(const void* v, const float* s, const float* sink, void* v_out,
                        float* s_out, int64_t S, int32_t H, int32_t D, mi_dtype v_dtype,
                        mi_dtype out_dtype, void* stream);

/*
 * Merge index sets of any size ("F2 hints", section 4's N-state merge over
 * variable-length sets; section 7's many-index-set variant).
 *   v      : [total, H, D] of v_dtype      s : [total, H] fp32 base 2
 *   indptr : [S + 1] int32 (device); set p is the states indptr[p] ..
 *            indptr[p+1] - 1 (entries are clamped to [0, total]; an empty set
 *            gives (0, -inf))
 *   v_out  : [S, H, D] of out_dtype        s_out : [S, H] fp32 (may be NULL)
 * Each (p, h) is served by one or more whole waves, so a set of thousands of
 * states is merged without a second launch. With indptr[p] = p * N it is
 * mi_merge_states on [S, N, H, D]. Used with fp32 v and H = Hq it is the
 * combine of per-sequence split decode. Outputs must not overlap inputs.
 * S == 0 is a no-op. D must be a positive multiple of 8, at most 512.
 */
mi_status mi_merge_states_varlen(const void* v, const float* s, const int32_t* indptr,
                                 int64_t total, void* v_out, float* s_out, int64_t S, int32_t H,
                                 int32_t D, mi_dtype v_dtype, mi_dtype out_dtype, void* stream);

/*
 * Choose the number of KV splits for one decode step ("L3 hints: split-KV
 * decode and LSE merge", section 6: make B*Hkv*splits a few times the compute
 * unit count while each split keeps several pages; do not split when B*Hkv is
 * already large). Host only; ctx_lens_host is a HOST array of B lengths.
 * Rule: the smallest of {1, 4, 16, 64} with B*Hkv*splits >= 2*num_cus (64 if
 * none), then step down through the set while the longest sequence would give
 * a split fewer than 8 pages. Writes the choice to *num_splits_out.
 * num_cus <= 0 asks the current HIP device for its compute unit count.
 */
mi_status mi_plan_splits(int32_t B, int32_t Hkv, const int32_t* ctx_lens_host, int32_t page_size,
                         int32_t num_cus, int32_t* num_splits_out);

/*
 * Page range [*p_start, *p_end) of split `split` for a sequence of ctx tokens
 * ("L3 hints: split-KV decode and LSE merge", section 2):
 *   num_pages = ceil(ctx / page_size); per = ceil(num_pages / num_splits);
 *   p_start = split * per; p_end = min(p_start + per, num_pages).
 * The split is empty when p_end <= p_start. Host only; the decode kernels use
 * the same formula on the device.
 */
mi_status mi_split_range(int32_t ctx, int32_t page_size, int32_t num_splits, int32_t split,
                         int32_t* p_start, int32_t* p_end);

/*
 * Split-KV paged decode, pass 1 only (Flash-Decoding's producer, "L3 hints:
 * split-KV decode and LSE merge", sections 1-5): one workgroup per
 * (split, kv head, sequence) runs an online softmax over its split's pages and
 * writes that split's normalised output and base-2 LSE. An empty split writes
 * o = 0, lse = -inf.
 *   q          : [B, Hq, D] of kv_dtype (one new token per sequence)
 *   k_cache,
 *   v_cache    : [num_phys_pages, Hkv, page_size, D] of kv_dtype
 *   page_table : [B, pt_stride] int32, logical page -> physical page
 *   ctx_lens   : [B] int32 (device) tokens per sequence
 *   o_part     : [B, Hq, num_splits, D] fp32   lse_part : [B, Hq, num_splits] fp32
 * Query head hq reads kv head hq / (Hq / Hkv). Scores are sm_scale * q.k.
 * Device data is clamped, never trusted: a negative ctx counts as 0, at most
 * pt_stride pages of a sequence are read, and a page id outside
 * [0, num_phys_pages) contributes no tokens. Token slots at or past ctx are
 * never used, whatever they hold. Supported: D = 128, page_size = 16,
 * Hq / Hkv in {1, 2, 4, 8}, kv_dtype f16 or bf16, num_splits in [1, 1024].
 */
mi_status mi_split_kv_partial(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* page_table, int32_t pt_stride,
                              const int32_t* ctx_lens, int32_t B, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t page_size, int64_t num_phys_pages,
                              int32_t num_splits, float sm_scale, mi_dtype kv_dtype,
                              float* o_part, float* lse_part, void* stream);

/*
 * Split-KV paged decode, both passes ("L3 hints: split-KV decode and LSE
 * merge", section 1): mi_split_kv_partial followed by the combine, i.e.
 * mi_merge_states over o_part viewed as [B*Hq, num_splits, 1, D], on `stream`.
 * o_part / lse_part are caller-owned fp32 workspaces (shapes as above) and are
 * left holding the partials. Outputs: o [B, Hq, D] of out_dtype, and
 * lse [B, Hq] fp32 base 2 (may be NULL). A sequence with ctx = 0 gets
 * o = 0, lse = -inf.
 */
mi_status mi_split_kv_decode(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* page_table, int32_t pt_stride, const int32_t* ctx_lens,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                             int64_t num_phys_pages, int32_t num_splits, float sm_scale,
                             mi_dtype kv_dtype, float* o_part, float* lse_part, void* o,
                             float* lse, mi_dtype out_dtype, void* stream);

/*
 * Split-KV paged decode in a single launch ("L3 hints: split-KV decode and LSE
 * merge", sections 1 and 3): pass 1 exactly as mi_split_kv_partial, after which
 * the last workgroup to finish for each (sequence, kv head) merges the splits
 * of that kv head's query heads and writes o and lse. Same results as
 * mi_split_kv_decode up to the order of rounding; saves the second launch.
 * Launch form: the single launch is used while the work items B * Hkv *
 * num_splits are at most twice the device's compute units; with more, the
 * per-workgroup hand-off costs more than a second launch (the same page,
 * section 6: more splits add intermediates), so pass 1 and the combine run as
 * the two launches of mi_split_kv_decode and the counters are not touched.
 *   counters : [B, Hkv] int32 device workspace used to find the last
 *              workgroup. It must be all zero before the first call; every call
 *              leaves it all zero again. Calls that share one counters buffer
 *              must not run concurrently (different streams race).
 * All other arguments, layouts and rules as mi_split_kv_decode; o_part and
 * lse_part are left holding the partials.
 */
mi_status mi_split_kv_decode_fused(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* page_table, int32_t pt_stride,
                                   const int32_t* ctx_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                   int32_t D, int32_t page_size, int64_t num_phys_pages,
                                   int32_t num_splits, float sm_scale, mi_dtype kv_dtype,
                                   float* o_part, float* lse_part, int32_t* counters, void* o,
                                   float* lse, mi_dtype out_dtype, void* stream);

/*
 * Per-sequence split counts for one decode step ("L3 hints: split-KV decode
 * and LSE merge", section 6: plan() can give sequences of different lengths
 * different numbers of splits). Host only; ctx_lens_host is a HOST array.
 * Rule (the uniform rule carried over to one page budget c per split): c is
 * the largest value in [8, longest sequence's page count] for which the work
 * items Hkv * sum_b max(1, ceil(pages_b / c)) still reach 2 * num_cus (8 if
 * none does); sequence b gets max(1, ceil(pages_b / c)) splits. Writes the
 * running sums to split_indptr_host[0 .. B] (split_indptr_host[0] = 0; the
 * last entry is the total). num_cus <= 0 asks the current HIP device.
 */
mi_status mi_plan_splits_varlen(int32_t B, int32_t Hkv, const int32_t* ctx_lens_host,
                                int32_t page_size, int32_t num_cus, int32_t* split_indptr_host);

/*
 * Split-KV paged decode with per-sequence split counts ("L3 hints", sections
 * 1-6). Sequence b is cut into n_b = split_indptr[b+1] - split_indptr[b]
 * splits, split k taking the page range of mi_split_range with n_b splits; one
 * workgroup per (kv head, split) over all sequences' splits.
 *   split_indptr : [B + 1] int32 (device), as written by mi_plan_splits_varlen:
 *                  split_indptr[0] = 0, n_b >= 1, last entry = total_splits
 *   o_part       : [total_splits, Hq, D] fp32   lse_part : [total_splits, Hq] fp32
 *                  caller-owned workspaces, left holding the partials (row
 *                  split_indptr[b] + k is split k of sequence b)
 *   counters     : [B, Hkv] int32 device workspace, or NULL. NULL: two
 *                  launches (pass 1, then mi_merge_states_varlen as the
 *                  combine). Given: one launch whose last workgroup per
 *                  (sequence, kv head) merges the splits, while the work items
 *                  total_splits * Hkv are at most twice the device's compute
 *                  units (two launches beyond, as for NULL); the counters must
 *                  be all zero before the first call and every call leaves them
 *                  zero; calls sharing them must not run concurrently.
 *   o            : [B, Hq, D] of out_dtype;  lse : [B, Hq] fp32 base 2 (may be NULL)
 * Other arguments, layouts, clamping of device data and supported sizes as in
 * mi_split_kv_partial; additionally B <= 4031 and total_splits <= 65535.
 * A sequence given no split (equal consecutive split_indptr entries) gets the
 * empty state o = 0, lse = -inf in both forms. split_indptr must be
 * non-decreasing; rows past split_indptr[B] (when total_splits is larger)
 * belong to no sequence: their partials are written as empty states and they
 * take no part in any combine. Inconsistent device data never leads to a
 * read or write outside the arguments' extents.
 */
mi_status mi_split_kv_decode_varlen(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* page_table, int32_t pt_stride,
                                    const int32_t* ctx_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                    int32_t D, int32_t page_size, int64_t num_phys_pages,
                                    const int32_t* split_indptr, int32_t total_splits,
                                    float sm_scale, mi_dtype kv_dtype, float* o_part,
                                    float* lse_part, int32_t* counters, void* o, float* lse,
                                    mi_dtype out_dtype, void* stream);

/*
 * Cascade level 0 ("F2 hints: merge_state, base-2 LSE merge", section 6): R
 * requests share one prefix; the prefix's K/V is read once and every request's
 * query heads attend to it together as dense matrix products on the matrix
 * cores. Produces each (request, query head)'s prefix state, to be merged with
 * its suffix state (mi_split_kv_decode*, then mi_merge_state).
 *   q            : [R, Hq, D] of kv_dtype
 *   k_cache,
 *   v_cache      : [num_phys_pages, Hkv, page_size, D] of kv_dtype
 *   prefix_pages : [ceil(prefix_len / page_size)] int32 (device), the prefix's
 *                  physical pages in order; ids outside [0, num_phys_pages)
 *                  contribute no tokens
 *   workspace    : fp32 device buffer of at least the size reported by
 *                  mi_prefix_attention_workspace (chunk partial states)
 *   v_out        : [R, Hq, D] of out_dtype;  s_out : [R, Hq] fp32 base 2 (may be NULL)
 * Query head hq uses kv head hq / (Hq / Hkv); scores are sm_scale * q.k.
 * prefix_len = 0 gives the empty state (0, -inf). Supported: D = 128,
 * page_size = 16, kv_dtype f16 or bf16. Two launches on `stream` (the chunked
 * contraction, then the merge of the chunk states).
 */
mi_status mi_prefix_attention(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* prefix_pages, int32_t prefix_len, int32_t R,
                              int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                              int64_t num_phys_pages, float sm_scale, mi_dtype kv_dtype,
                              float* workspace, size_t ws_bytes, void* v_out, float* s_out,
                              mi_dtype out_dtype, void* stream);

/*
 * Two-level cascade decode in two launches ("F2 hints: merge_state, base-2 LSE
 * merge", section 6; "L3 hints", sections 1-3): R requests share one prefix
 * (read once, on the matrix cores, as in mi_prefix_attention) and each has its
 * own suffix pages (split-KV decode as in mi_split_kv_decode_fused). The
 * suffix decode's combine merges each row's suffix splits together with that
 * row's prefix chunk states, so no separate merge launch follows.
 *   q               : [R, Hq, D] of kv_dtype
 *   k_cache,
 *   v_cache         : [num_phys_pages, Hkv, page_size, D] of kv_dtype (one pool
 *                     for prefix and suffix pages)
 *   prefix_pages    : [ceil(prefix_len / page_size)] int32 (device)
 *   suffix_table    : [R, suffix_stride] int32, suffix_lens : [R] int32 (device)
 *   workspace       : fp32 device buffer of at least mi_prefix_attention_workspace
 *                     bytes (prefix chunk states)
 *   o_part, lse_part: [R, Hq, suffix_splits, D] / [R, Hq, suffix_splits] fp32
 *   counters        : [R, Hkv] int32, all zero before the first call, left zero
 *   o               : [R, Hq, D] of out_dtype;  lse : [R, Hq] fp32 base 2 (may be NULL)
 * The result is attention over prefix followed by suffix for every (request,
 * query head). Supported sizes, clamping of device data and the rules for
 * counters as in mi_split_kv_decode_fused; calls sharing counters must not run
 * concurrently.
 */
mi_status mi_cascade_decode(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* prefix_pages, int32_t prefix_len,
                            const int32_t* suffix_table, int32_t suffix_stride,
                            const int32_t* suffix_lens, int32_t R, int32_t Hq, int32_t Hkv,
                            int32_t D, int32_t page_size, int64_t num_phys_pages,
                            int32_t suffix_splits, float sm_scale, mi_dtype kv_dtype,
                            float* workspace, size_t ws_bytes, float* o_part, float* lse_part,
                            int32_t* counters, void* o, float* lse, mi_dtype out_dtype,
                            void* stream);

/* Workspace bytes mi_prefix_attention needs for this shape (host only). */
mi_status mi_prefix_attention_workspace(int32_t R, int32_t Hq, int32_t Hkv, int32_t D,
                                        int32_t prefix_len, size_t* ws_bytes);

/*
 * Split-KV paged decode that allocates nothing, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same computation, arguments and rules as
 * mi_split_kv_decode without o_part / lse_part: the fp32 partials live in a
 * static device array of the library (one per GPU, held until the process
 * ends) and are not returned. Two launches on `stream` (one with a single
 * split); nothing is allocated, freed or synchronised.
 *   B * Hq * num_splits must not exceed MI_NOALLOC_MAX_PARTIAL_ROWS (the array
 *   holds that many partial rows of D = 128 floats plus their LSEs, about
 *   16.5 MB); larger work returns MI_ERR_SCRATCH without enqueuing anything.
 * All calls on one GPU share the array: calls that overlap on one GPU (other
 * streams, other threads) race on it and must be serialised by the caller.
 */
#define MI_NOALLOC_MAX_PARTIAL_ROWS 32768
mi_status mi_split_kv_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* page_table, int32_t pt_stride,
                                     const int32_t* ctx_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                     int32_t D, int32_t page_size, int64_t num_phys_pages,
                                     int32_t num_splits, float sm_scale, mi_dtype kv_dtype,
                                     void* o, float* lse, mi_dtype out_dtype, void* stream);

/*
 * Measurement aid, not a step of the method: one plain streaming read of a
 * buffer. It gives the practical HBM read rate of the device, the context in
 * which the other kernels' fractions of the peak are read.
 *   x       : bytes of device memory, 16-byte aligned; bytes a multiple of 16 (>= 0)
 *   xor_out : one uint32 on the device; *xor_out is XOR-ed with the XOR of all
 *             32-bit words of x, so a caller that zeroes it first gets that XOR
 *             (bytes = 0 leaves it unchanged and enqueues nothing)
 * Errors: MI_ERR_NULL (x or xor_out NULL with bytes > 0), MI_ERR_SHAPE (bytes
 * negative or not a multiple of 16), MI_ERR_UNSUPPORTED (alignment),
 * MI_ERR_ALIAS (xor_out inside x).
 */
mi_status mi_stream_read(const void* x, int64_t bytes, uint32_t* xor_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MI_H_ */

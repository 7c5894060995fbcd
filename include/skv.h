/*
 * skv.h — C ABI of libskv: paged split-KV decode/verify attention for MI355X
 * (gfx950).
 *
 * Sources, cited by page title and section:
 *   [PR]  sglang PR #39172, "[AMD] gfx950 assembly attention: length-aware
 *         split-KV for dynamic workload" — Motivation (the fixed split: one
 *         work-group per segment, sequence and KV head), Modifications (the
 *         length-aware planner, its work list and per-token segment counts,
 *         the segment kernel's work-list prologue, the split reduce).
 *   [RFC] vLLM RFC #59111, "NixlConnector: convert standard KV pages to ROCm
 *         AITER shuffled pages on the decode side" — Background (standard
 *         [H, N, 2D] pages and shuffled K [H, D/x, N, x] / V [H, N/x, D, x]
 *         planes, x = 16 / element bytes), Proposed Change §3 (a received
 *         standard block arrives as two byte halves in the K- and V-plane
 *         blocks) and §4 (converting the received blocks), Test plan (round
 *         trips).
 *
 * Conventions for every call:
 *   - Pointer arguments are DEVICE pointers owned by the caller (except the
 *     `stream`, a hipStream_t passed as void*; NULL is the null stream).
 *   - The library never allocates, frees or synchronizes; calls only enqueue
 *     work on `stream`. Its one piece of global state is the device array of
 *     skv_paged_decode_attn_static (a fixed-size __device__ array, looked up
 *     once per device). Grid sizes depend on the host integers alone and no
 *     device data is read back, so every call may be captured into a HIP
 *     graph.
 *   - Return value: SKV_OK, or an error code below; on error nothing was
 *     enqueued. Host-checkable argument errors are detected before any HIP
 *     call, so they can be tested without a GPU.
 *   - Device data must satisfy the stated contract (lengths, page ids,
 *     cu_seqlens_q); a violation is undefined behaviour and is not detected
 *     by these calls. skv_check_inputs checks it on request (a debug aid).
 *
 * Element types: KV is bf16 (IEEE binary32 upper half), OCP e4m3fn fp8
 * (kv_dtype 1) with per-tensor fp32 dequant scales, or IEEE binary16 fp16
 * (kv_dtype 2; the RFC's decoder scope is BF16/FP16). Q and the output are
 * fp16 with an fp16 cache and bf16 otherwise.
 * Supported geometry: head_dim 64, 128 or 256 for every entry point (the
 * attention runs 128 on kernels specialised for it, 64 and 256 on a
 * generic-width segment kernel); page_size 16 or 32 tokens for every
 * entry point (the RFC's decoder scope: 16- or 32-token pages; the split-KV
 * PR's kernels use 16); 1..4 query tokens per sequence,
 * (q_heads / kv_heads) * max_q <= 64.
 */
#ifndef SKV_H_
#define SKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum skv_status {
  SKV_OK = 0,
  SKV_EINVAL = 1,        /* NULL required pointer, bad size or relation   */
  SKV_EUNSUPPORTED = 2,  /* valid but outside the supported geometry      */
  SKV_ELAUNCH = 3        /* the HIP launch itself failed                  */
};

enum skv_layout { SKV_LAYOUT_STANDARD = 0, SKV_LAYOUT_SHUFFLED = 1 };
/* Flags of the attention entry points: 0 (the default, a fixed summation
 * order, bit-reproducible), SKV_ATTN_DETERMINISTIC (the same, stated
 * explicitly) or SKV_ATTN_CLAIM_UNITS (run-time claimed order, fp8 KV only;
 * see skv_paged_decode_attn). Both together are invalid. */
enum skv_attn_flags { SKV_ATTN_DETERMINISTIC = 1, SKV_ATTN_CLAIM_UNITS = 2 };

enum skv_kv_dtype { SKV_KV_BF16 = 0, SKV_KV_FP8_E4M3FN = 1, SKV_KV_FP16 = 2 };
enum skv_convert_dir { SKV_TO_SHUFFLED = 0, SKV_TO_STANDARD = 1 };
/* Device-data contract violations reported by skv_check_inputs (bits). */
enum skv_contract_violation {
  SKV_BAD_LEN_NEGATIVE = 1,   /* seq_lens[i] < 0                                  */
  SKV_BAD_LEN_TABLE = 2,      /* seq_lens[i] > pt_stride * page_size               */
  SKV_BAD_CU = 4,             /* cu[0] != 0, cu[i + 1] < cu[i] or cu[bs] != total_q */
  SKV_BAD_QLEN = 8,           /* cu[i + 1] - cu[i] > max_q                          */
  SKV_BAD_PAGE_ID = 16        /* a page-table entry the attention reads is not a
                                 block of the pool, i.e. outside [0, num_blocks)  */
};

/* Number of int32 words of a plan: 1 + max(num_cus / kv_heads, bs).
 * [PR, Modifications]: one word for the segment length, then the work list,
 * whose capacity covers both the per-kv-head CU budget and one segment per
 * sequence (the fallback when no segment length fits the budget).
 * Returns 0 if an argument is not positive. */
size_t skv_plan_words(int bs, int kv_heads, int num_cus);

/* Bytes of the partial-result workspace: part_o fp32 [total_q, q_heads,
 * seg_max, head_dim] followed by part_lse fp32 [total_q, q_heads, seg_max].
 * Returns 0 if an argument is not positive. */
size_t skv_workspace_bytes(int total_q, int q_heads, int head_dim, int seg_max);

/* Length-aware segment planner [PR, Modifications].
 *
 * In:  seq_lens int32 [bs] (KV tokens per sequence, the sequence's own query
 *      tokens included, 0 <= L); cu_seqlens_q int32 [bs + 1] (prefix sums of
 *      query tokens, cu[0] = 0, cu[bs] = total_q).
 * Out: plan int32 [skv_plan_words(bs, kv_heads, num_cus)]:
 *        plan[0] = T, pages per segment: the smallest T >= 1 for which
 *          sum_i ceil(ceil(L_i/P)/T) <= num_cus / kv_heads and
 *          max_i ceil(ceil(L_i/P)/T) <= seg_max; when no T qualifies, the
 *          longest sequence's page count (one segment per sequence);
 *        plan[1 + k] = (i << 16) | s for the k-th (sequence i, segment s),
 *          sequence-major with segments ascending, then -1 to the end.
 *      tok_nseg int32 [total_q]: for query token t of sequence i,
 *        ceil(visible_t / (T * page_size)) where visible_t is the number of
 *        keys t may see (causal: a sequence's q query tokens are its last q
 *        KV tokens, so query j sees L - q + j + 1 keys, clamped to [0, L];
 *        non-causal: L).
 * One single-work-group launch; integer arithmetic only.
 * Errors: EINVAL for NULL pointers, bs < 1, bs >= 32768, total_q < 1,
 * kv_heads < 1, num_cus < 1, seg_max outside [1, 65535]; EUNSUPPORTED for
 * page_size other than 16 or 32. */
int skv_plan_build(const int32_t* seq_lens, const int32_t* cu_seqlens_q, int bs,
                   int total_q, int kv_heads, int page_size, int num_cus,
                   int seg_max, int causal, int32_t* plan, int32_t* tok_nseg,
                   void* stream);

/* Paged decode/verify attention: the segment kernel, then the split reduce
 * [PR, Motivation and Modifications].
 *
 * q            [total_q, q_heads, head_dim], fp16 for SKV_KV_FP16, else bf16
 * kv_a, kv_b   layout STANDARD: kv_a = pages [num_blocks, kv_heads, page_size,
 *              2 * head_dim] (per token: K channels then V channels), kv_b NULL;
 *              layout SHUFFLED: kv_a = K plane [num_blocks, kv_heads,
 *              head_dim/x, page_size, x], kv_b = V plane [num_blocks, kv_heads,
 *              page_size/x, head_dim, x], x = 16 / element bytes [RFC, Background]
 * kv_dtype     SKV_KV_BF16, SKV_KV_FP8_E4M3FN or SKV_KV_FP16
 * page_table   int32 [bs, pt_stride]; entry [i, p] is the block holding tokens
 *              [p * page_size, (p + 1) * page_size) of sequence i; entries at
 *              p >= ceil(L_i / page_size) are never read
 * seq_lens, cu_seqlens_q, bs, total_q   as for skv_plan_build
 * max_q        an upper bound of the query tokens of any sequence (1..4)
 * q_heads, kv_heads   grouped-query heads: q head h reads kv head h / (q_heads/kv_heads)
 * k_scale, v_scale    device fp32 scalars: required for fp8 (dequantized value =
 *              code value * scale), NULL for bf16 and fp16
 * causal       1: bottom-right causal mask as in skv_plan_build; 0: all L keys
 * plan, tok_nseg      from skv_plan_build with the same bs, kv_heads, num_cus,
 *              seg_max, causal and page_size (planned split). plan NULL selects
 *              the FIXED split [PR, Motivation; Modifications: bs == 1 runs it
 *              without a plan]: every sequence gets S = max(1, min(seg_max,
 *              pow2floor(num_cus / (bs * kv_heads)))) segments of
 *              ceil(ceil(L_i/page_size) / S) pages (trailing ones empty when a sequence
 *              has fewer than S pages), one work-group per (sequence, segment,
 *              kv head); no plan launch is needed, and the segment kernel
 *              WRITES tok_nseg[t] = ceil(visible_t / segment tokens) for the
 *              reduce (tok_nseg is then an output; it is read otherwise)
 * part_o, part_lse    workspace of skv_workspace_bytes(): part_o fp32
 *              [total_q, q_heads, seg_max, head_dim] (each segment's
 *              softmax-normalized output), part_lse fp32 [total_q, q_heads,
 *              seg_max] (natural-log sum-exp); entries s >= tok_nseg[t] are
 *              unspecified
 * out          [total_q, q_heads, head_dim], the type of q, round to nearest even;
 *              a token that sees no key gets zeros
 * out_lse      fp32 [total_q, q_heads] or NULL; -inf where no key is visible
 * flags        0 or SKV_ATTN_DETERMINISTIC (the same): a fixed order (wave w
 *              of a work-group takes the segment's 32-token blocks w,
 *              w + waves, ...), so identical inputs give bit-identical
 *              results [PR, Accuracy Tests: a cached output must equal the
 *              uncached one bit for bit]. SKV_ATTN_CLAIM_UNITS (fp8 KV; a
 *              no-op for bf16 and fp16 KV): the waves take the blocks in the
 *              order they claim them at run time, so they finish together;
 *              each wave's fp32 sums then run in an order that depends on
 *              timing, and results for identical inputs agree to rounding,
 *              not bit for bit.
 * Scale: softmax(q.k / sqrt(head_dim)).
 * Errors: EINVAL for NULL required pointers, non-positive sizes, q_heads not a
 * multiple of kv_heads, bs >= 32768, seg_max outside [1, 65535], max_q < 1,
 * scales present for bf16/fp16 or missing for fp8, kv_b NULL for SHUFFLED or
 * non-NULL for STANDARD, pt_stride < 1, an unknown layout, dtype or flag,
 * both flags at once;
 * EUNSUPPORTED for head_dim not 64, 128 or 256, page_size other than 16 or 32, max_q > 4,
 * (q_heads/kv_heads) * max_q > 64. */
int skv_paged_decode_attn(const void* q, const void* kv_a, const void* kv_b,
                          int layout, int kv_dtype, const int32_t* page_table,
                          int pt_stride, const int32_t* seq_lens,
                          const int32_t* cu_seqlens_q, int bs, int total_q,
                          int max_q, int q_heads, int kv_heads, int head_dim,
                          int page_size, const float* k_scale,
                          const float* v_scale, int causal, const int32_t* plan,
                          int32_t* tok_nseg, int num_cus, int seg_max,
                          float* part_o, float* part_lse, void* out,
                          float* out_lse, int flags, void* stream);

/* The segment kernel of skv_paged_decode_attn alone: writes the partials
 * (part_o, part_lse) of every (token, q head, segment) that the plan lists
 * (with plan NULL: of the fixed split, and tok_nseg), without merging them. Arguments and errors as for skv_paged_decode_attn
 * (minus out and out_lse). skv_paged_decode_attn = this call followed by
 * skv_split_reduce on the same stream. Each call writes token t's partials at
 * segment indices 0 .. tok_nseg[t] - 1; partials of several calls over
 * disjoint key ranges (e.g. the shards of several GPUs) merge into attention
 * over their union when the caller places them side by side in one buffer of
 * the same layout (distinct segment indices, tok_nseg counting them all) and
 * runs skv_split_reduce on it. */
int skv_segment_attn(const void* q, const void* kv_a, const void* kv_b, int layout,
                     int kv_dtype, const int32_t* page_table, int pt_stride,
                     const int32_t* seq_lens, const int32_t* cu_seqlens_q, int bs,
                     int total_q, int max_q, int q_heads, int kv_heads, int head_dim,
                     int page_size, const float* k_scale, const float* v_scale,
                     int causal, const int32_t* plan, int32_t* tok_nseg,
                     int num_cus, int seg_max, float* part_o, float* part_lse,
                     int flags, void* stream);

/* Split reduce alone [PR, Modifications]: for every (t, h), merges the first
 * tok_nseg[t] partials by log-sum-exp: M = max_s lse_s,
 * lse = M + ln sum_s exp(lse_s - M), out = sum_s exp(lse_s - lse) * o_s.
 * A partial whose lse is -inf (a segment with no visible key) has weight 0;
 * tok_nseg[t] == 0, or only such partials, gives zeros and lse -inf. Values
 * of tok_nseg[t] above seg_max are clamped to seg_max.
 * Layouts as for skv_paged_decode_attn; out [total_q, q_heads, head_dim] of
 * out_dtype (SKV_KV_BF16: bf16, SKV_KV_FP16: fp16; round to nearest even);
 * out_lse may be NULL.
 * Errors: EINVAL for NULL required pointers, non-positive sizes, seg_max
 * outside [1, 65535], another out_dtype; EUNSUPPORTED for head_dim not 64, 128
 * or 256. */
int skv_split_reduce(const float* part_o, const float* part_lse,
                     const int32_t* tok_nseg, int total_q, int q_heads,
                     int head_dim, int seg_max, int out_dtype, void* out,
                     float* out_lse, void* stream);

/* Standard -> shuffled page repack [RFC, Background and Proposed Change §4].
 * For each listed block b (block_ids int32 [num_blocks]; NULL = blocks
 * 0..num_blocks-1) and head h:
 *   k_plane[b, h, c, n, i] = std_cache[b, h, n, c*x + i]
 *   v_plane[b, h, g, d, i] = std_cache[b, h, g*x + i, head_dim + d]
 * with x = 16 / elem_bytes. Pure byte movement, bit-exact. Out of place: the
 * source must not overlap the planes. Blocks not listed are left untouched.
 * Errors: EINVAL for NULL required pointers, num_blocks < 1, kv_heads < 1;
 * EUNSUPPORTED for head_dim not 64, 128 or 256, page_size not 16 or 32,
 * elem_bytes not 1 or 2. */
int skv_kv_page_shuffle(const void* std_cache, void* k_plane, void* v_plane,
                        const int32_t* block_ids, int num_blocks, int kv_heads,
                        int page_size, int head_dim, int elem_bytes,
                        void* stream);

/* In-place conversion of received blocks [RFC, Proposed Change §3 Descriptors
 * and §4 Convert] and its inverse [RFC, Test plan: round trips].
 * k_plane, v_plane: the decoder's planes, shaped like skv_kv_page_shuffle's
 * outputs ([blocks, H, D/x, N, x] and [blocks, H, N/x, D, x], H = kv_heads);
 * block b occupies S = kv_heads * page_size * head_dim * elem_bytes bytes at
 * offset b * S in each plane.
 *   SKV_TO_SHUFFLED: on entry K-plane block b holds the first S bytes of a
 *     standard block [H, N, 2D] and V-plane block b the last S bytes (what a
 *     transfer of the standard block as two half-block regions leaves); on
 *     return they hold its shuffled K and V, exactly as skv_kv_page_shuffle
 *     would write them. With an odd head count one head straddles the halves.
 *   SKV_TO_STANDARD: the inverse; a round trip restores the planes bit for bit.
 * block_ids int32 [num_blocks] lists DISTINCT blocks (NULL = blocks
 * 0..num_blocks-1); a block listed twice is rewritten by two work-groups at
 * once (undefined result). Blocks not listed are left untouched.
 * Errors: EINVAL for NULL planes, num_blocks < 1, kv_heads < 1, a direction
 * other than the two above; EUNSUPPORTED for head_dim not 64, 128 or 256,
 * page_size not 16 or 32, elem_bytes not 1 or 2, or a block (2 * S) above
 * 128 KiB (head dim 128 with 16-token pages: kv_heads > 16 for bf16, > 32 for
 * fp8; half that for 32-token pages or head dim 256, twice that for head dim
 * 64): the whole block is staged in on-chip memory. */
int skv_kv_page_convert(void* k_plane, void* v_plane, const int32_t* block_ids,
                        int num_blocks, int kv_heads, int page_size,
                        int head_dim, int elem_bytes, int direction,
                        void* stream);

/* Shuffled -> standard, out of place: the inverse of skv_kv_page_shuffle
 * [RFC, Background layouts; Test plan: round trips]. For each listed block b
 * and head h:
 *   std_cache[b, h, n, c*x + i]           = k_plane[b, h, c, n, i]
 *   std_cache[b, h, g*x + i, head_dim + d] = v_plane[b, h, g, d, i]
 * Bit-exact; the planes must not overlap std_cache; blocks not listed are left
 * untouched. Errors as for skv_kv_page_shuffle. */
int skv_kv_page_unshuffle(const void* k_plane, const void* v_plane,
                          void* std_cache, const int32_t* block_ids,
                          int num_blocks, int kv_heads, int page_size,
                          int head_dim, int elem_bytes, void* stream);

/* Cache writer into shuffled pages [RFC, Background and Proposed Change §4:
 * the shuffled backend's writer places each new token at its slot]. For each
 * token t with slot s = slot_mapping[t] in [0, num_blocks * page_size)
 * (block b = s / page_size, row n = s % page_size) and head h:
 *   k_plane[b, h, c / x, n, c % x] = K(key[t, h, c])
 *   v_plane[b, h, n / x, d, n % x] = V(value[t, h, d])
 * x = 16 / elem_bytes (the cache's element size). Negative slots (padding) and
 * slots past the cache are skipped. Slots must be distinct: two tokens at one
 * slot race.
 *   k_scale = v_scale = NULL: key, value hold element codes of the cache type
 *     (bf16 or fp8 e4m3fn) and K, V copy them unchanged (bit-exact).
 *   k_scale, v_scale = device fp32 scalars (fp8 cache only, elem_bytes 1): key,
 *     value are bf16 and K(v) = e4m3fn(v / k_scale), V(v) = e4m3fn(v / v_scale),
 *     the division in fp32, rounded to the nearest code with ties to even,
 *     magnitudes >= 448 saturating to +-448, NaN kept as NaN: the inverse of
 *     the attention path's value = code * scale.
 * Token t's [kv_heads, head_dim] input row starts key_stride (value_stride)
 * input elements after token t-1's; strides must be multiples of
 * 16 / (input element bytes) and at least kv_heads * head_dim; all pointers
 * 16-byte aligned.
 * Errors: EINVAL for NULL pointers, only one scale given, scales with
 * elem_bytes != 1, num_tokens < 1, num_blocks < 1, kv_heads < 1, a stride
 * below kv_heads * head_dim or not a multiple of the above; EUNSUPPORTED for
 * head_dim not 64, 128 or 256, page_size not 16 or 32, elem_bytes not 1 or
 * 2. */
int skv_kv_cache_write(const void* key, const void* value,
                       const int64_t* slot_mapping, int num_tokens,
                       long long key_stride, long long value_stride,
                       void* k_plane, void* v_plane, int num_blocks,
                       int kv_heads, int page_size, int head_dim,
                       int elem_bytes, const float* k_scale,
                       const float* v_scale, void* stream);

/* Bytes of the library's own device array that skv_paged_decode_attn_static
 * keeps its partials in (per GPU, for the life of the process). */
#define SKV_STATIC_SCRATCH_BYTES (64u << 20)

/* skv_paged_decode_attn without part_o / part_lse: for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The partials live in a fixed device array
 * of SKV_STATIC_SCRATCH_BYTES (64 MiB) that the library holds on every GPU it
 * runs on until the process ends; its address is looked up on the first call
 * made with that GPU current. This call allocates and frees nothing.
 * Arguments, results and the other errors are those of skv_paged_decode_attn
 * (same kernels, same summation order: identical outputs). Every call on one
 * GPU uses that GPU's one array, so calls that overlap on one GPU (several
 * streams or host threads at once) race and must be serialized by the caller.
 * Errors: EUNSUPPORTED when skv_workspace_bytes(total_q, q_heads, head_dim,
 * seg_max) exceeds SKV_STATIC_SCRATCH_BYTES (e.g. 55 query tokens x 32 heads x
 * 64 segments at head dim 128 need 58 MB and fit); ELAUNCH when the array's
 * device address cannot be obtained. */
int skv_paged_decode_attn_static(const void* q, const void* kv_a, const void* kv_b,
                                 int layout, int kv_dtype, const int32_t* page_table,
                                 int pt_stride, const int32_t* seq_lens,
                                 const int32_t* cu_seqlens_q, int bs, int total_q,
                                 int max_q, int q_heads, int kv_heads, int head_dim,
                                 int page_size, const float* k_scale,
                                 const float* v_scale, int causal, const int32_t* plan,
                                 int32_t* tok_nseg, int num_cus, int seg_max, void* out,
                                 float* out_lse, int flags, void* stream);

/* Static text for a status code. */
/* Debug check of the device data that skv_plan_build and the attention calls
 * take on trust (the contract stated with them; optional, never run by those
 * calls). One single-work-group launch reads seq_lens, cu_seqlens_q and the
 * page-table entries the attention reads (entries p < ceil(L_i / page_size)
 * of row i, at most pt_stride of them) and writes
 *   result[0] = the OR of the skv_contract_violation bits found (0: none),
 *   result[1] = the smallest sequence index with a violation (-1: none);
 * cu[0] != 0 counts against sequence 0 and cu[bs] != total_q against
 * sequence bs - 1; a sequence whose query count is negative (cu decreasing)
 * gets SKV_BAD_CU and no SKV_BAD_QLEN. The page ids are compared with
 * num_blocks, never dereferenced, so any input is safe to check.
 * result: device int32 [2], written on the stream (read it after a sync).
 * Errors: EINVAL for NULL pointers, bs outside [1, 32767], total_q < 1,
 * max_q < 1, pt_stride < 1, num_blocks < 1; EUNSUPPORTED for page_size other
 * than 16 or 32. */
int skv_check_inputs(const int32_t* page_table, int pt_stride, const int32_t* seq_lens,
                     const int32_t* cu_seqlens_q, int bs, int total_q, int max_q,
                     int page_size, int num_blocks, int32_t* result, void* stream);

const char* skv_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* SKV_H_ */

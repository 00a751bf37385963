/*
 * kvdecode.h -- C ABI of the MI355X (gfx950) paged Top-K decode-attention library.
 *
 * One decode step of one layer over a block-paged KV cache:
 *
 *   kv_block_meta_build   channel-wise min/max key of every KV page (the block index)
 *   kv_block_score_topk   Quest block score of every logical block, then Top-K blocks
 *   kv_block_mean_build   mean key of every KV page (the mean-key block index)
 *   kv_block_select       block scores from either index, then Top-K with the
 *                         blocks of the first / last tokens forced in
 *   kv_quantize_pages_fp8 K/V pages -> FP8 E4M3 cold pages with per-page scales
 *   kv_paged_decode_attn_fp8  decode attention over FP8 E4M3 cold pages
 *   kv_quantize_pages_int4 K/V pages -> INT4 cold pages with per-page scales
 *   kv_paged_decode_attn_int4 decode attention over INT4 cold pages
 *   kv_paged_decode_attn_tiered decode attention over hot 16-bit and cold code pages
 *   kv_paged_decode_attn_tiered_split the same as a hot launch and a cold launch
 *                         over the block lists split by tier
 *   kv_tier_plan          hot/cold tier policy: page heat from the step's selection,
 *                         demotions and promotions with a cooldown
 *   kv_cache_plan         GPU block cache: hits, misses and lookahead eviction
 *   kv_cache_fetch        copy only the missing blocks into their cache slots
 *   kv_cached_decode_attn decode attention over the cached blocks, with each
 *                         block's log-sum-exp for the next eviction
 *   kv_cache_fetch_codes, kv_cached_decode_attn_codes  the same over FP8 / INT4
 *                         code pools: the cache holds codes and scales
 *   kv_cached_decode_attn_fetch(_codes)  the delta fetch and the cached attention
 *                         in one launch
 *   kv_cache_slot_mass    eviction mass of every cache slot after a step
 *   kv_paged_decode_attn  split-K softmax decode attention, dense or over selected blocks
 *   kv_decode_combine     log-sum-exp merge of the split partials
 *   kv_append_token       store the new token's K/V and fold it into its page's meta
 *   kv_decode_select      kv_append_token followed by kv_block_select, in two launches
 *   kv_decode_score       kv_decode_select's append + score launch, without the Top-K
 *   kv_select_decode_attn the Top-K and the sparse attention over it, one launch for
 *                         rows of up to 2048 blocks (kv_auto_select_splits)
 *   kv_block_select_no_alloc  kv_block_select with its scores in a library-owned
 *                         device array, for callers that cannot allocate
 *   kv_check_tables       device-side check of the block table, lengths and selection
 *
 * The method is the select -> fetch -> compute decode step of the KVDrive paper
 * (§2.3, §4): a GPU-resident index picks the critical KV blocks, only those are
 * read, and attention runs over them.  The block index is Quest's (KVDrive
 * §2.2): per block the channel-wise minimum and maximum of the keys, and a
 * block score obtained by multiplying the query with them.  Dense decode (every
 * step reads all previous KV, Dual-Blade page, background section) is the same
 * attention call without a selection.  A KV pool may live in mapped pinned host
 * memory that the kernels read directly (the zero-copy KV manager of the
 * DirectKV review page, core method 4), so only the pages a call touches cross
 * the host link.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers are device addresses (or device-mapped host addresses from
 *   kv_host_alloc) unless stated otherwise; the caller owns every buffer.  No
 *   call allocates device memory; scratch comes in as a caller workspace.
 * - Every call is asynchronous and stream-ordered on `stream` (a hipStream_t;
 *   NULL = the default stream).  Nothing synchronises.
 * - Host-side validation runs before any launch and returns a status; the
 *   device is not touched when a call returns an error.  kv_last_error_message()
 *   gives the reason (thread-local).
 * - Device-side integer data (page ids, block tables, sequence lengths,
 *   selections) is trusted: it must satisfy the ranges stated below.
 *   kv_check_tables verifies them on the device when a caller cannot vouch
 *   for them.
 * - Head mapping: query head h reads KV head h / G, G = num_q_heads / num_kv_heads.
 * - Layouts (row-major, innermost last):
 *     q        [B, Hq, D]            dtype
 *     K, V     [P, Hkv, bs, D]       dtype   (page p, KV head j, slot s, channel c)
 *     kmeta    [P, Hkv, 2, D]        dtype   (index 0 = channel min, 1 = channel max)
 *     kmean    [P, Hkv, D]           fp32    (mean key of the page's valid slots)
 *     K8, V8   [P, Hkv, bs, D]       uint8   FP8 E4M3 codes of cold pages
 *     K4, V4   [P, Hkv, bs, D/2]     uint8   INT4 codes of cold pages, two per byte
 *     kv_scales [P, Hkv, 2]          fp32    (K scale, V scale) of each cold page
 *   GPU block cache with C = num_slots slots per (sequence, KV head):
 *     cache_k, cache_v [B * C, Hkv, bs, D]  dtype  page b*C + s: slot s of sequence b
 *     slot_block  int32 [B, Hkv, C]     block held by each slot, -1 free
 *     block_slot  int32 [B, Hkv, maxN]  slot of each resident block, -1 otherwise
 *     slot_mass   fp32  [B, Hkv, C]     eviction mass of each slot (latest step)
 *     sel_slots   int32 [B, Hkv, sel_stride]  slot of each list position
 *     fetch_block, fetch_slot int32 [B, Hkv, sel_stride]; fetch_count int32 [B, Hkv]
 *     block_lse   fp32  [B, Hq, sel_stride]   per list position
 *     block_table int32 [B, maxN]    logical block n of sequence b -> page
 *     seq_lens    int32 [B]          L_b >= 1 tokens, current token included,
 *                                    N_b = ceil(L_b / bs) <= maxN
 *     scores   fp32 [B, Hkv, maxN]   (-inf for n >= N_b)
 *     sel      int32 [B, Hkv, sel_stride] ascending logical block ids, -1 padded
 *     sel_count int32 [B, Hkv]
 *     part_o   fp32 [B, Hq, S, D]    per-split normalised output
 *     part_m, part_l fp32 [B, Hq, S] per-split max logit and sum of exp(logit - max)
 *     out      fp32 [B, Hq, D];  lse fp32 [B, Hq]
 * - Alignment: q, K, V, K8, V8, kmeta and kmean 16 bytes; part_o and out 16 bytes;
 *   kv_scales 8; the rest 4.
 */
#ifndef KVDECODE_H
#define KVDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KV_OK = 0,
  KV_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, inconsistent shape */
  KV_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim, block_size, group size, dtype */
  KV_ERR_ALIGNMENT = 3,   /* a pointer misses the alignment stated above */
  KV_ERR_WORKSPACE = 4,   /* workspace missing or smaller than the size query returned */
  KV_ERR_HIP = 5          /* the HIP runtime reported an error at launch */
} kv_status;

typedef enum { KV_F32 = 0, KV_F16 = 1, KV_BF16 = 2 } kv_dtype;

/* Block index kinds of kv_block_select. */
typedef enum {
  KV_INDEX_MINMAX = 0, /* kmeta: channel-wise min and max keys (Quest) */
  KV_INDEX_MEAN = 1    /* kmean: the mean key */
} kv_index_kind;

/* kv_shape.flags */
#define KV_FLAG_HOST_KV 0x1u /* K/V pools are device-mapped pinned host memory */

/* kv_host_alloc flags */
#define KV_HOST_COHERENT 0x0u    /* default mapped pinned memory */
#define KV_HOST_NONCOHERENT 0x1u /* mapped pinned memory the GPU may cache */

typedef struct {
  int32_t num_seqs;           /* B >= 1 */
  int32_t num_q_heads;        /* Hq, a multiple of Hkv */
  int32_t num_kv_heads;       /* Hkv >= 1; G = Hq / Hkv in {1, 2, 4, 8} */
  int32_t head_dim;           /* D in {64, 128} */
  int32_t block_size;         /* bs: tokens per page, 16 */
  int32_t max_blocks_per_seq; /* maxN >= 1: row length of block_table and scores */
  int32_t num_pages;          /* P >= 1: pages in the K/V pools */
  int32_t dtype;              /* kv_dtype of q, K, V and kmeta */
  uint32_t flags;             /* KV_FLAG_* */
} kv_shape;

/*
 * Block index build (KVDrive §2.2 and §2.3: a block is represented by the
 * channel-wise min and max of its keys; KVDrive §4: built at prefill).
 * For i < num_page_ids and every KV head j, writes
 *   kmeta[p, j, 0, c] = min_{s < v} K[p, j, s, c],  kmeta[p, j, 1, c] = max_{s < v} K[p, j, s, c]
 * with p = page_ids[i], v = page_valid_tokens[i] in [1, bs].  Exact (min and max
 * of representable values), so results are bit-identical to any exact reference
 * up to the sign of zero.  Pages not listed are not touched.  Page ids must be
 * distinct and in [0, P); any order is valid, and ascending page order reads
 * K and writes kmeta as sequential streams (the fastest order for a full build).
 */
kv_status kv_block_meta_build(const kv_shape* shape, const void* k_cache, const int32_t* page_ids,
                              const int32_t* page_valid_tokens, int32_t num_page_ids, void* kmeta,
                              void* stream);

/*
 * Mean-key block index (KVDrive §2.3: spatial blocking may represent a block by
 * the mean of its keys; §4: a page's mean key is its representative).
 * For i < num_page_ids and every KV head j, writes
 *   kmean[p, j, c] = (sum_{s < v} K[p, j, s, c]) / v     (fp32 [P, Hkv, D])
 * with p = page_ids[i], v = page_valid_tokens[i] in [1, bs].  The sum is taken
 * in fp64 in slot order and the quotient is rounded once to fp32; for fp16 and
 * bf16 keys the fp64 sum is exact, so kmean is the exact mean rounded to the
 * nearest fp32.  Pages not listed are not touched; ids as in kv_block_meta_build.
 */
kv_status kv_block_mean_build(const kv_shape* shape, const void* k_cache, const int32_t* page_ids,
                              const int32_t* page_valid_tokens, int32_t num_page_ids, float* kmean,
                              void* stream);

/*
 * Decode-step append (Dual-Blade background: a decode step stores the new K/V
 * pair after attending; DirectKV review, core method 4: the KV manager appends
 * at decode).  For every sequence b and KV head j, the new token sits at
 * position t = seq_lens[b] - 1 (seq_lens already counts it): page
 * p = block_table[b, t / bs], slot s = t mod bs.  Writes
 *   K[p, j, s, :] = k_new[b, j, :],  V[p, j, s, :] = v_new[b, j, :]
 * (k_new, v_new: [B, Hkv, D] in the storage dtype).  When kmeta is not NULL the
 * key is folded into the page's min/max rows: for s == 0 they become k_new (a
 * fresh page), otherwise the element-wise min / max with k_new; if kmeta held
 * the exact meta of slots 0..s-1, it then holds exactly what
 * kv_block_meta_build computes for slots 0..s.  When kmean is not NULL the
 * page's mean row is recomputed from slots 0..s with kv_block_mean_build's
 * arithmetic, so it equals a rebuild bit for bit.  Distinct sequences must own
 * distinct pages.
 */
kv_status kv_append_token(const kv_shape* shape, const void* k_new, const void* v_new,
                          const int32_t* block_table, const int32_t* seq_lens, void* k_cache,
                          void* v_cache, void* kmeta, float* kmean, void* stream);

/*
 * The decode step's append and selection in one call (Dual-Blade background
 * and DirectKV review, core method 4: the new K/V is stored at decode; KVDrive
 * §2.3: the index then picks the blocks).  Results are bit for bit those of
 * kv_append_token(shape, k_new, v_new, block_table, seq_lens, k_cache, v_cache,
 * kmeta, kmean) followed by kv_block_select(shape, index_kind, q, index, ...,
 * topk_blocks, sink_tokens, local_tokens, scores_out, sel_blocks, sel_count,
 * workspace, workspace_bytes), with index = kmeta for KV_INDEX_MINMAX and kmean
 * for KV_INDEX_MEAN (that one is required; the other may be NULL and is then
 * not maintained).  Arguments, layouts, ownership and errors are those of the
 * two calls.  It takes two launches instead of three: one extra workgroup per
 * (sequence, KV head) of the scoring launch appends the token and scores its
 * block from the updated index rows, while the other workgroups score the rest
 * of the blocks; the Top-K follows.
 */
kv_status kv_decode_select(const kv_shape* shape, int32_t index_kind, const void* q,
                           const void* k_new, const void* v_new, const int32_t* block_table,
                           const int32_t* seq_lens, void* k_cache, void* v_cache, void* kmeta,
                           float* kmean, int32_t topk_blocks, int32_t sink_tokens,
                           int32_t local_tokens, float* scores_out, int32_t* sel_blocks,
                           int32_t* sel_count, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * The decode step's append and scores in one launch: kv_decode_select without
 * its Top-K (Dual-Blade background: the step stores the new pair; KVDrive
 * §2.2-§2.3: the index scores every block).  Results are bit for bit those of
 * kv_append_token(shape, k_new, v_new, block_table, seq_lens, k_cache, v_cache,
 * kmeta, kmean) followed by the scores kv_block_select writes to scores_out
 * ([B, Hkv, maxN] fp32, -inf for n >= N_b) over index = kmeta
 * (KV_INDEX_MINMAX) or kmean (KV_INDEX_MEAN, which is then required).  The
 * selection and attention follow in kv_select_decode_attn.  Arguments,
 * layouts and errors are those of kv_decode_select; scores_out is required.
 */
kv_status kv_decode_score(const kv_shape* shape, int32_t index_kind, const void* q,
                          const void* k_new, const void* v_new, const int32_t* block_table,
                          const int32_t* seq_lens, void* k_cache, void* v_cache, void* kmeta,
                          float* kmean, float* scores_out, void* stream);

/*
 * Top-K selection and sparse split-K attention in one call (KVDrive §2.3: the
 * critical blocks are selected, then attention runs over them only).  Results
 * are bit for bit those of the Top-K of kv_block_select over `scores` (the
 * same topk_blocks, sink_tokens and local_tokens; written to sel_blocks
 * [B, Hkv, topk_blocks] and sel_count [B, Hkv]) followed by
 * kv_paged_decode_attn over that list with sel_stride = topk_blocks and the
 * same num_splits (part_o [B, Hq, S, D], part_m, part_l [B, Hq, S], merged by
 * kv_decode_combine).  scores: fp32 [B, Hkv, maxN], e.g. from kv_decode_score
 * or kv_block_select's scores_out.  For 16-bit K/V with G >= 2, maxN <= 2048
 * and at most 2048 list positions per four splits (4 * ceil(topk_blocks /
 * num_splits)) it is one launch: each workgroup repeats the row's Top-K
 * itself, keeps the positions of its four splits in LDS and attends them,
 * which saves the Top-K launch and the list's round trip through memory;
 * other calls (longer rows, where the repeated Top-K costs more than the
 * launch it saves) run the two launches.  Arguments and errors are those of
 * the two calls (KV_FLAG_HOST_KV pools included).
 */
kv_status kv_select_decode_attn(const kv_shape* shape, const float* scores,
                                const int32_t* block_table, const int32_t* seq_lens,
                                int32_t topk_blocks, int32_t sink_tokens, int32_t local_tokens,
                                const void* q, const void* k_cache, const void* v_cache,
                                float scale, int32_t num_splits, int32_t* sel_blocks,
                                int32_t* sel_count, float* part_o, float* part_m, float* part_l,
                                void* stream);

/*
 * Workspace bytes for kv_block_score_topk, kv_block_select and
 * kv_decode_select: the scores (B * Hkv * maxN fp32, rounded up to 256 bytes;
 * the least a call with scores_out NULL accepts) plus, for rows longer than
 * 16384 blocks where 2 * topk_blocks candidates per 4096-block chunk stay within
 * 16384 per row, the candidate storage of the two-level select (8 bytes per
 * candidate slot).  0 for an invalid shape.
 */
size_t kv_score_topk_workspace_size(const kv_shape* shape, int32_t topk_blocks);

/*
 * Quest block scoring and Top-K selection (KVDrive §2.2).
 * For every sequence b, query head h and logical block n < N_b:
 *   sigma[b,h,n] = sum_c max(q[b,h,c] * kmin[p,j,c], q[b,h,c] * kmax[p,j,c]),
 *   p = block_table[b,n], j = h / G   (fp32 accumulation; products are exact for
 *   fp16/bf16 inputs),
 * the group score S[b,j,n] = max over the G query heads of KV head j, and the
 * selection: the K_eff = min(topk_blocks, N_b) blocks of largest S (ties: lower
 * block index first), written ascending to sel_blocks[b, j, 0..K_eff) with -1
 * after, and K_eff to sel_count[b, j].  sel_blocks has row stride topk_blocks.
 * scores_out (nullable) receives S ([B, Hkv, maxN], -inf for n >= N_b); when it
 * is NULL the scores go to the head of `workspace`, which must hold at least
 * their bytes (see kv_score_topk_workspace_size).  Long rows (more than 16384
 * blocks): when the workspace also holds the candidate storage (after the
 * scores, or from its head when scores_out is given), the select runs in two
 * launches -- each 4096-block chunk's forced blocks and best topk_blocks
 * competing blocks, then the select among those -- which return the same
 * list; otherwise one workgroup per row selects.  topk_blocks >= 1; maxN <=
 * 65536 (a 1M-token context of 16-token blocks).
 */
kv_status kv_block_score_topk(const kv_shape* shape, const void* q, const void* kmeta,
                              const int32_t* block_table, const int32_t* seq_lens,
                              int32_t topk_blocks, float* scores_out, int32_t* sel_blocks,
                              int32_t* sel_count, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Upper bound of the blocks kv_block_select forces in for any sequence length:
 * ceil(sink / bs) + (local > 0 ? ceil((local - 1) / bs) + 1 : 0).  -1 for an
 * invalid shape or a negative count.
 */
int32_t kv_max_forced_blocks(const kv_shape* shape, int32_t sink_tokens, int32_t local_tokens);

/*
 * Block scoring from either index, then Top-K with forced tokens.
 * index_kind KV_INDEX_MINMAX: `index` is kmeta and the head score is Quest's,
 * as in kv_block_score_topk.  KV_INDEX_MEAN: `index` is kmean and the head
 * score is sigma[b,h,n] = q[b,h] . kmean[p, j] (fp32 accumulation).  Group score
 * and ranking as in kv_block_score_topk, except that every block holding one of
 * the first sink_tokens tokens (n * bs < sink_tokens) or one of the last
 * local_tokens tokens ((n + 1) * bs > L_b - local_tokens) is always selected
 * and counts against the budget (KVDrive §9.1: the sparse systems keep the
 * first 4 and the last 64 tokens); the other min(topk_blocks, N_b) - #forced
 * places go to the best of the remaining blocks (ties: lower index).  scores_out
 * holds the unforced scores.  Requires kv_max_forced_blocks() <= topk_blocks;
 * workspace as in kv_block_score_topk.  With KV_INDEX_MINMAX and
 * sink_tokens = local_tokens = 0 this is kv_block_score_topk.
 */
kv_status kv_block_select(const kv_shape* shape, int32_t index_kind, const void* q,
                          const void* index, const int32_t* block_table, const int32_t* seq_lens,
                          int32_t topk_blocks, int32_t sink_tokens, int32_t local_tokens,
                          float* scores_out, int32_t* sel_blocks, int32_t* sel_count,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * kv_block_select for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same selection, written to the same sel_blocks / sel_count, without a
 * scores buffer or workspace.  The scores are kept in device memory of the
 * library itself, a 4 MiB array that each GPU it runs on holds until the
 * process ends; its address on the current device is looked up (never
 * allocated) on the first call on that device.  The call itself allocates
 * nothing.  Limit: num_seqs * num_kv_heads * max_blocks_per_seq <= 1048576
 * scores (for example 16 sequences of 8 KV heads and 8192 blocks), else
 * KV_ERR_WORKSPACE before any launch.  Rows longer than 16384 blocks take the
 * two-level select (see kv_block_score_topk) when its candidates fit in the
 * array after the scores.  Every call on one GPU shares that array: calls that
 * overlap on one GPU (other streams, other threads) race and may select from
 * each other's scores; calls ordered on one stream do not.  Arguments, checks
 * and errors are otherwise those of kv_block_select.
 */
kv_status kv_block_select_no_alloc(const kv_shape* shape, int32_t index_kind, const void* q,
                                   const void* index, const int32_t* block_table,
                                   const int32_t* seq_lens, int32_t topk_blocks,
                                   int32_t sink_tokens, int32_t local_tokens, int32_t* sel_blocks,
                                   int32_t* sel_count, void* stream);

/*
 * Number of splits the library would pick for kv_paged_decode_attn (and the
 * cached attention) with `blocks_per_unit` blocks per (sequence, KV head)
 * (maxN for dense calls, the list length for sparse ones): about 6 waves per
 * compute unit on the matrix-core path (16-bit, G >= 2), 4 on the vector path,
 * at least 2 blocks per split (8 with KV_FLAG_HOST_KV).  Always >= 1.
 */
int32_t kv_auto_num_splits(const kv_shape* shape, int32_t blocks_per_unit);

/*
 * Number of splits for kv_select_decode_attn with topk_blocks: where the call
 * is one launch, four splits (one workgroup) per compute unit over the
 * (sequence, KV head) rows, at most 4 * ceil(topk_blocks / 4); elsewhere
 * kv_auto_num_splits(shape, topk_blocks).  Always >= 1.
 */
int32_t kv_auto_select_splits(const kv_shape* shape, int32_t topk_blocks);

/* The same for kv_paged_decode_attn_fp8: about 8 waves per compute unit. */
int32_t kv_auto_num_splits_fp8(const kv_shape* shape, int32_t blocks_per_unit);

/* The same for kv_paged_decode_attn_tiered: about 12 waves per compute unit. */
int32_t kv_auto_num_splits_tiered(const kv_shape* shape, int32_t blocks_per_unit);

/*
 * Split-K decode attention (Dual-Blade background: a decode step attends over
 * all previous KV; KVDrive §2.3 step 3: sparse attention over the selected
 * blocks; DirectKV review, core method 2/3: the query and the running output
 * stay in registers and each KV tile is read once, with a streaming softmax).
 * For query head h of sequence b, the block list is 0..N_b-1 when sel_blocks is
 * NULL, else sel_blocks[b, h/G, 0..sel_count[b, h/G]) (ascending, distinct,
 * < N_b; row stride sel_stride).  Split s covers list positions
 * [s*c, min((s+1)*c, n)) with c = ceil(n / num_splits); over its tokens t < L_b:
 *   z_t = scale * (q . k_t),  m = max z_t,  l = sum exp(z_t - m),
 *   part_o = sum exp(z_t - m) v_t / l,  part_m = m,  part_l = l
 * (fp32 accumulation).  An empty split writes m = -inf, l = 0, o = 0.
 * num_splits >= 1 (see kv_auto_num_splits).  With num_splits = 1 (and a
 * non-empty list) part_o, read as [B, Hq, D], already is the attention output
 * and part_m + ln(part_l) its log-sum-exp, so the merge launch may be skipped.
 * With KV_FLAG_HOST_KV the K/V pointers may be device pointers of
 * kv_host_alloc memory.
 */
kv_status kv_paged_decode_attn(const kv_shape* shape, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* sel_blocks,
                               const int32_t* sel_count, int32_t sel_stride, float scale,
                               int32_t num_splits, float* part_o, float* part_m, float* part_l,
                               void* stream);

/*
 * Exact log-sum-exp merge of split partials (the streaming-softmax rescale of
 * the DirectKV review, core method 3, applied across splits):
 *   M = max_s m_s,  w_s = l_s * exp(m_s - M) (0 for an empty split),
 *   out = sum_s w_s o_s / sum_s w_s,  lse = M + ln(sum_s w_s).
 * lse_out is nullable.  Every row needs at least one non-empty split.
 */
kv_status kv_decode_combine(const kv_shape* shape, int32_t num_splits, const float* part_o,
                            const float* part_m, const float* part_l, float* out, float* lse_out,
                            void* stream);

/*
 * FP8 cold pages (KVDrive §11: cold blocks stored with aggressive quantisation
 * while hot blocks keep high precision; DirectKV review, assumption stress
 * test: FP8 KV).  The format is OCP FP8 E4M3 (bias 7, no infinities, largest
 * finite value 448).  For i < num_page_ids, every KV head j and tensor
 * X in {K, V}, with p = page_ids[i] and v = page_valid_tokens[i] in [1, bs]:
 *   amax = max_{s < v, c} |X[p, j, s, c]|
 *   kv_scales[p, j, t] = amax / 448 (fp32, correctly rounded; 1 if amax == 0),
 *                        t = 0 for K, 1 for V
 *   X8[p, j, s, c] = E4M3 code of X[p, j, s, c] / scale (fp32, correctly
 *                    rounded), rounded to nearest with ties to the even code,
 *                    saturated to +-448;  0 for s >= v.
 * The codes are a deterministic function of the stored values (amax ignores
 * NaNs; the code of a NaN value is an E4M3 NaN, 0x7f with either sign bit).
 * K/V keep the layout of the source pools with one byte per channel.  Pages not listed are
 * not touched; ids as in kv_block_meta_build, except that a negative id is a
 * skipped entry (so a -1-padded list such as kv_tier_plan's demote rows can be
 * passed whole).  page_valid_tokens may be NULL: every listed page is full
 * (v = bs).  The block index (kmeta, kmean) is built from the high-precision
 * keys and is not affected.
 */
kv_status kv_quantize_pages_fp8(const kv_shape* shape, const void* k_cache, const void* v_cache,
                                const int32_t* page_ids, const int32_t* page_valid_tokens,
                                int32_t num_page_ids, uint8_t* k_fp8, uint8_t* v_fp8,
                                float* kv_scales, void* stream);

/*
 * kv_paged_decode_attn over FP8 E4M3 cold pages: every K and V value is
 * decode(code) * scale of its (page, KV head), and the call computes exactly
 * what kv_paged_decode_attn computes over those values (fp32 accumulation;
 * the decoded codes are exact in the 16-bit MFMA operands, the K scale
 * multiplies the logits and the V scale the softmax weights).  q keeps
 * shape->dtype.  kv_scales must be device memory; with KV_FLAG_HOST_KV the code
 * pools may be device pointers of kv_host_alloc memory.
 */
kv_status kv_paged_decode_attn_fp8(const kv_shape* shape, const void* q, const uint8_t* k_fp8,
                                   const uint8_t* v_fp8, const float* kv_scales,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   const int32_t* sel_blocks, const int32_t* sel_count,
                                   int32_t sel_stride, float scale, int32_t num_splits,
                                   float* part_o, float* part_m, float* part_l, void* stream);

/*
 * INT4 cold pages (KVDrive §11 names INT4 for the cold blocks of its
 * mixed-precision tiering; DirectKV review, assumption stress test: FP8/INT4
 * KV).  The pages fix no format; this one is symmetric with one scale per tile.
 * For i < num_page_ids, every KV head j and tensor X in {K, V}, with
 * p = page_ids[i] and v = page_valid_tokens[i] in [1, bs]:
 *   amax = max_{s < v, c} |X[p, j, s, c]|
 *   kv_scales[p, j, t] = amax / 7 (fp32, correctly rounded; 1 if amax == 0),
 *                        t = 0 for K, 1 for V
 *   n[p, j, s, c] = X[p, j, s, c] / scale (fp32, correctly rounded), rounded to
 *                   nearest with ties to even, clamped to [-7, 7];  0 for s >= v
 *   X4[p, j, s, c / 2] holds n of channel c in bits 4 * (c mod 2) .. +3, as
 *                   4-bit two's complement (the even channel in the low nibble).
 * The value a code stands for is n * scale; amax ignores NaNs, and the code
 * of a NaN value is not specified.  fp16 and bf16 pools only
 * (KV_ERR_UNSUPPORTED for fp32).  Pages not listed are not touched; negative
 * ids are skipped and a NULL page_valid_tokens means full pages, as for
 * kv_quantize_pages_fp8; the block index is not affected.
 */
kv_status kv_quantize_pages_int4(const kv_shape* shape, const void* k_cache, const void* v_cache,
                                 const int32_t* page_ids, const int32_t* page_valid_tokens,
                                 int32_t num_page_ids, uint8_t* k_int4, uint8_t* v_int4,
                                 float* kv_scales, void* stream);

/*
 * kv_paged_decode_attn over INT4 cold pages: every K and V value is n * scale
 * of its (page, KV head), and the call computes exactly what
 * kv_paged_decode_attn computes over those values (fp32 accumulation; the
 * codes are exact in the 16-bit operands, the K scale multiplies the logits
 * and the V scale the softmax weights).  q keeps shape->dtype (fp16 or bf16).
 * kv_scales must be device memory; with KV_FLAG_HOST_KV the code pools may be
 * device pointers of kv_host_alloc memory.  kv_auto_num_splits_fp8 serves
 * these pages too.
 */
kv_status kv_paged_decode_attn_int4(const kv_shape* shape, const void* q, const uint8_t* k_int4,
                                    const uint8_t* v_int4, const float* kv_scales,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* sel_blocks, const int32_t* sel_count,
                                    int32_t sel_stride, float scale, int32_t num_splits,
                                    float* part_o, float* part_m, float* part_l, void* stream);

/* Cold-page formats of kv_paged_decode_attn_tiered. */
#define KV_COLD_FP8 8  /* the pages of kv_quantize_pages_fp8 */
#define KV_COLD_INT4 4 /* the pages of kv_quantize_pages_int4 */

/*
 * Decode attention over tiered pools (KVDrive §11: hot blocks keep high
 * precision in HBM while cold blocks are stored with aggressive quantisation,
 * chosen per block from what the cache manager knows of hot and cold).  Page
 * p is read from k_cache / v_cache (shape->dtype) when page_tier[p] == 0, and
 * from the code pools k_cold / v_cold in cold_format, with kv_scales[p], when
 * page_tier[p] != 0 (uint8 [P], device memory).  The result is exactly what
 * kv_paged_decode_attn computes over the pools whose cold pages hold their
 * decoded values (code * scale); the other arguments, layouts and errors are
 * those of kv_paged_decode_attn.  The cold pools have the layouts of
 * kv_quantize_pages_fp8 / _int4 and may be device pointers of kv_host_alloc
 * memory.  fp16 or bf16 with G >= 2 (KV_ERR_UNSUPPORTED otherwise).
 */
kv_status kv_paged_decode_attn_tiered(const kv_shape* shape, const void* q, const void* k_cache,
                                      const void* v_cache, const uint8_t* k_cold,
                                      const uint8_t* v_cold, const float* kv_scales,
                                      int32_t cold_format, const uint8_t* page_tier,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      const int32_t* sel_blocks, const int32_t* sel_count,
                                      int32_t sel_stride, float scale, int32_t num_splits,
                                      float* part_o, float* part_m, float* part_l, void* stream);

/*
 * Tiered pools as two launches: the list (sel_blocks, or every block of the
 * sequence when sel_blocks is NULL) of each (b, KV head) is split by page_tier
 * into a hot list and a cold list (order kept) in the workspace, then the
 * hot blocks are attended by the 16-bit kernel in num_splits_hot splits and
 * the cold ones by the code-page kernel in num_splits_cold splits, each
 * launch with the register budget of its own page format.  The partials hold
 * S = num_splits_hot + num_splits_cold splits per row ([B, Hq, S, D] and
 * [B, Hq, S]): columns [0, num_splits_hot) cover the hot list, the others the
 * cold list, each list chunked as kv_paged_decode_attn chunks a list, and
 * kv_decode_combine with S merges them.  The merged result is what
 * kv_paged_decode_attn_tiered computes (up to the order of the fp32 sums).
 * The pools, formats and errors are those of kv_paged_decode_attn_tiered,
 * except that any dtype and group size the two kernels serve is accepted
 * (INT4 needs fp16 or bf16).  The workspace holds the lists:
 * kv_tiered_split_workspace_size(shape, sel_stride) bytes (sel_stride 0 for
 * dense lists), 4-byte aligned, else KV_ERR_WORKSPACE.
 */
size_t kv_tiered_split_workspace_size(const kv_shape* shape, int32_t sel_stride);
kv_status kv_paged_decode_attn_tiered_split(
    const kv_shape* shape, const void* q, const void* k_cache, const void* v_cache,
    const uint8_t* k_cold, const uint8_t* v_cold, const float* kv_scales, int32_t cold_format,
    const uint8_t* page_tier, const int32_t* block_table, const int32_t* seq_lens,
    const int32_t* sel_blocks, const int32_t* sel_count, int32_t sel_stride, float scale,
    int32_t num_splits_hot, int32_t num_splits_cold, float* part_o, float* part_m,
    float* part_l, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Hot/cold tier policy, one decode step (the tiered-offload blog, page
 * replacement: pages whose heat has fallen move down a tier, and a cooldown
 * after a demotion keeps a page from moving straight back up; KVDrive §11:
 * hot blocks keep full precision, cold blocks are stored quantised).  For each
 * sequence b and block n < N_b = ceil(seq_lens[b] / bs), page p =
 * block_table[b, n]:
 *   hit  = n is in sel_blocks[b, j, 0..sel_count[b, j]) for some KV head j
 *          (sel_blocks is [B, Hkv, sel_stride] int32 and is read whole, the
 *          entries past a count included; a count above sel_stride counts as
 *          sel_stride; the lists of kv_block_select or kv_select_decode_attn)
 *   page_heat[p] = hit ? fma(decay, h, 1 - decay) : decay * h      (fp32, h the
 *          heat before the call)
 *   recent = the block holds one of the last recent_tokens tokens of b
 *   a hot page (page_tier[p] == 0) that is not recent turns cold when
 *     page_heat[p] < cold_below: page_tier[p] = 1, page_stamp[p] = step;
 *   a cold page (page_tier[p] != 0) turns hot (page_tier[p] = 0) when it is
 *     recent, or when page_heat[p] > hot_above and
 *     step - page_stamp[p] >= cooldown_steps.
 * demote / promote [B, maxN] receive, per sequence and in block order, the
 * pages that turned cold / hot, -1 after the last; demote_count /
 * promote_count [B] their numbers.  page_heat (fp32), page_tier (uint8, the
 * array kv_paged_decode_attn_tiered reads) and page_stamp (int32) are [P] and
 * are updated in place; pages that no sequence references, and block_table
 * entries outside [0, P), are left alone.  Each page may be referenced by at
 * most one (sequence, block), as in any block table of distinct pages.
 * recent_tokens >= 1 keeps the page being appended to hot (kv_append_token
 * writes the 16-bit pools), so every demoted page is full: passing the demote
 * rows whole (B * maxN ids) to kv_quantize_pages_fp8 / _int4 with
 * page_valid_tokens NULL writes their cold codes; do that on the same stream
 * before the next tiered attention call reads page_tier.  A promoted page is
 * read from the 16-bit pools again, which this library never frees.
 * Errors: KV_ERR_INVALID_ARG for a NULL array, sel_stride < 1 or
 * sel_stride * num_kv_heads > 2^30, decay outside
 * [0, 1], a NaN threshold, recent_tokens < 1, cooldown_steps < 0 or
 * max_blocks_per_seq > 262144; KV_ERR_ALIGNMENT for an int32 / fp32 array
 * that is not 4-byte aligned.  All arrays are device memory.
 */
kv_status kv_tier_plan(const kv_shape* shape, const int32_t* sel_blocks, const int32_t* sel_count,
                       int32_t sel_stride, const int32_t* block_table, const int32_t* seq_lens,
                       float decay, float hot_above, float cold_below, int32_t recent_tokens,
                       int32_t cooldown_steps, int32_t step, float* page_heat,
                       uint8_t* page_tier, int32_t* page_stamp, int32_t* demote,
                       int32_t* demote_count, int32_t* promote, int32_t* promote_count,
                       void* stream);

/*
 * GPU-resident block cache with lookahead eviction (KVDrive §5.1: a window of
 * critical KV entries stays in GPU memory; each decode step fetches the new
 * critical entries from host memory and drops the entries that received the
 * least attention in the latest step, so host-to-GPU traffic is the set
 * difference between consecutive selections).  Each (sequence, KV head) owns
 * C = num_slots >= sel_stride slots of one 16-token K/V tile each.  A step is
 *   kv_block_score_topk / kv_block_select -> kv_cache_plan -> kv_cache_fetch
 *   -> kv_cached_decode_attn -> kv_decode_combine -> kv_cache_slot_mass.
 * The caller initialises slot_block and block_slot to -1 and slot_mass to 0.
 *
 * kv_cache_plan: for every (b, j), with the step's list sel_blocks[b, j, 0..n)
 * (distinct blocks, n = sel_count[b, j] <= sel_stride <= num_slots):
 *   - a resident block (block_slot >= 0) keeps its slot;
 *   - for the m missing blocks the reused slots are the first m of: the free
 *     slots in slot order, then the slots whose block is not in the list, by
 *     increasing slot_mass (ties: lower slot);
 *   - the missing blocks, in list order, take the reused slots in increasing
 *     slot order; an evicted block's block_slot becomes -1.
 * Writes sel_slots (-1 past n), the fetch list fetch_block / fetch_slot (the m
 * missing blocks and their slots, in list order, -1 padded to sel_stride) and
 * fetch_count = m, and updates slot_block / block_slot in place.  One
 * workgroup per (b, j); num_slots <= 8192.
 */
kv_status kv_cache_plan(const kv_shape* shape, int32_t num_slots, const int32_t* sel_blocks,
                        const int32_t* sel_count, int32_t sel_stride, int32_t* slot_block,
                        int32_t* block_slot, const float* slot_mass, int32_t* sel_slots,
                        int32_t* fetch_block, int32_t* fetch_slot, int32_t* fetch_count,
                        void* stream);

/*
 * Delta fetch: for k < fetch_count[b, j], copies the K and V tiles of block
 * n = fetch_block[b, j, k] (pool page block_table[b, n], KV head j) into cache
 * page b * num_slots + fetch_slot[b, j, k], KV head j.  With KV_FLAG_HOST_KV the
 * pools are kv_host_alloc memory, read directly by the kernel (only the missing
 * blocks cross the host link); the cache pools are device memory.
 */
kv_status kv_cache_fetch(const kv_shape* shape, int32_t num_slots, const void* k_cache,
                         const void* v_cache, const int32_t* block_table,
                         const int32_t* fetch_block, const int32_t* fetch_slot,
                         const int32_t* fetch_count, int32_t fetch_stride, void* cache_k,
                         void* cache_v, void* stream);

/*
 * kv_paged_decode_attn over the list sel_blocks with every block read from
 * cache page b * num_slots + sel_slots[b, j, pos] (the block index n still sets
 * the token positions and the valid count).  When block_lse is not NULL it
 * also receives, per query head and list position,
 *   block_lse[b, h, pos] = ln sum_{t in block} exp(scale * (q . k_t)),
 * so exp(block_lse - lse) is the block's attention weight in the step.
 */
kv_status kv_cached_decode_attn(const kv_shape* shape, int32_t num_slots, const void* q,
                                const void* cache_k, const void* cache_v,
                                const int32_t* seq_lens, const int32_t* sel_blocks,
                                const int32_t* sel_count, const int32_t* sel_slots,
                                int32_t sel_stride, float scale, int32_t num_splits,
                                float* part_o, float* part_m, float* part_l, float* block_lse,
                                void* stream);

/*
 * The block cache over code pools (KVDrive §5.1's GPU window combined with
 * §11's quantised cold blocks: the host pool holds FP8 or INT4 pages, so the
 * delta fetch moves a quarter or an eighth of the 16-bit bytes).  The cache
 * pools keep the pool's format: cache_k / cache_v [B * C, Hkv, 16, D] bytes of
 * E4M3 codes (code_format KV_COLD_FP8) or [B * C, Hkv, 16, D / 2] INT4 bytes
 * (KV_COLD_INT4), and cache_scales fp32 [B * C, Hkv, 2] beside them.
 *
 * kv_cache_fetch_codes: kv_cache_fetch over the code pools k_codes / v_codes
 * (the layouts of kv_quantize_pages_fp8 / _int4, device memory or kv_host_alloc
 * memory with KV_FLAG_HOST_KV); each fetched tile's scale pair
 * kv_scales[page, j, 0..1] (device or kv_host_alloc memory) is copied to
 * cache_scales[b * C + slot, j, 0..1].
 *
 * kv_cached_decode_attn_codes: kv_cached_decode_attn over the code cache; the
 * result is what kv_paged_decode_attn_fp8 / _int4 compute with the same list,
 * splits and codes (each block read from its cache page and scales).  INT4
 * needs fp16 or bf16 (KV_ERR_UNSUPPORTED for fp32); an unknown code_format is
 * KV_ERR_INVALID_ARG.
 */
kv_status kv_cache_fetch_codes(const kv_shape* shape, int32_t num_slots, int32_t code_format,
                               const uint8_t* k_codes, const uint8_t* v_codes,
                               const float* kv_scales, const int32_t* block_table,
                               const int32_t* fetch_block, const int32_t* fetch_slot,
                               const int32_t* fetch_count, int32_t fetch_stride,
                               uint8_t* cache_k, uint8_t* cache_v, float* cache_scales,
                               void* stream);
kv_status kv_cached_decode_attn_codes(const kv_shape* shape, int32_t num_slots,
                                      int32_t code_format, const void* q, const uint8_t* cache_k,
                                      const uint8_t* cache_v, const float* cache_scales,
                                      const int32_t* seq_lens, const int32_t* sel_blocks,
                                      const int32_t* sel_count, const int32_t* sel_slots,
                                      int32_t sel_stride, float scale, int32_t num_splits,
                                      float* part_o, float* part_m, float* part_l,
                                      float* block_lse, void* stream);

/*
 * The delta fetch fused into the cached attention (KVDrive §6 overlaps the
 * fetch of the missing entries with computation; here both are one launch, so
 * the waves whose blocks are cached compute while the others read theirs over
 * the host link, and a fetched tile is read once instead of written to the
 * cache and read back).  kv_cached_decode_attn_fetch computes exactly what
 * kv_cache_fetch(shape, num_slots, k_pool, v_pool, block_table, *, fetch_slot,
 * fetch_count, sel_stride, cache_k, cache_v) followed by kv_cached_decode_attn
 * computes, outputs and cache contents alike: a list position whose slot is
 * among fetch_slot[b, j, 0 .. fetch_count[b, j]) (rows of sel_stride, as
 * kv_cache_plan writes them; every such slot is in this step's list) reads
 * block n's tiles from pool page block_table[b, n] and stores them into its
 * cache page; the others read the cache.  The pools may be device pointers of
 * kv_host_alloc memory (KV_FLAG_HOST_KV); the cache pools must not overlap
 * them.  kv_cached_decode_attn_fetch_codes does the same over FP8 / INT4 code
 * pools (the layouts of kv_cache_fetch_codes) and also copies each fetched
 * block's scale pair from kv_scales to cache_scales.
 */
kv_status kv_cached_decode_attn_fetch(const kv_shape* shape, int32_t num_slots, const void* q,
                                      const void* k_pool, const void* v_pool,
                                      const int32_t* block_table, const int32_t* fetch_slot,
                                      const int32_t* fetch_count, void* cache_k, void* cache_v,
                                      const int32_t* seq_lens, const int32_t* sel_blocks,
                                      const int32_t* sel_count, const int32_t* sel_slots,
                                      int32_t sel_stride, float scale, int32_t num_splits,
                                      float* part_o, float* part_m, float* part_l,
                                      float* block_lse, void* stream);
kv_status kv_cached_decode_attn_fetch_codes(
    const kv_shape* shape, int32_t num_slots, int32_t code_format, const void* q,
    const uint8_t* k_codes, const uint8_t* v_codes, const float* kv_scales,
    const int32_t* block_table, const int32_t* fetch_slot, const int32_t* fetch_count,
    uint8_t* cache_k, uint8_t* cache_v, float* cache_scales, const int32_t* seq_lens,
    const int32_t* sel_blocks, const int32_t* sel_count, const int32_t* sel_slots,
    int32_t sel_stride, float scale, int32_t num_splits, float* part_o, float* part_m,
    float* part_l, float* block_lse, void* stream);

/*
 * Eviction mass after a step: slot_mass[b, j, :] = 0, then for every list
 * position pos < sel_count[b, j]:
 *   slot_mass[b, j, sel_slots[b, j, pos]] = max over the G query heads h of
 *                                           group j of exp(block_lse[b, h, pos] - lse[b, h])
 * (lse from kv_decode_combine of the same step).
 */
kv_status kv_cache_slot_mass(const kv_shape* shape, int32_t num_slots, const float* block_lse,
                             const float* lse, const int32_t* sel_count,
                             const int32_t* sel_slots, int32_t sel_stride, float* slot_mass,
                             void* stream);

/*
 * Check of the device-side tables the other calls trust (block_table,
 * seq_lens and, when sel_blocks is not NULL, a selection with row stride
 * sel_stride).  For every sequence b it writes result[b] (uint32, device
 * memory, B words) as the OR of:
 *   KV_CHECK_BAD_SEQ_LEN    L_b < 1 or L_b > maxN * bs (nothing else of b is checked)
 *   KV_CHECK_BAD_PAGE_ID    block_table[b, n] outside [0, P) for some n < N_b
 *   KV_CHECK_BAD_SEL_COUNT  sel_count[b, j] outside [0, min(sel_stride, N_b)] for some j
 *   KV_CHECK_BAD_SEL_BLOCK  a listed block outside [0, N_b), or a list not
 *                           strictly ascending
 * and 0 when the tables of b are fit for every call.  It reads only the
 * tables, at indexes bounded by the shape, so it is safe on any contents.
 * The selection of kv_cache_plan's callers and of kv_paged_decode_attn obeys
 * these same rules.
 */
#define KV_CHECK_BAD_SEQ_LEN 0x1u
#define KV_CHECK_BAD_PAGE_ID 0x2u
#define KV_CHECK_BAD_SEL_COUNT 0x4u
#define KV_CHECK_BAD_SEL_BLOCK 0x8u
kv_status kv_check_tables(const kv_shape* shape, const int32_t* block_table,
                          const int32_t* seq_lens, const int32_t* sel_blocks,
                          const int32_t* sel_count, int32_t sel_stride, uint32_t* result,
                          void* stream);

/*
 * Read-ceiling probes, for measurement: they read bytes as the path does and
 * compute nothing, so the path's kernels can be reported against what the
 * memory system delivers for the same access pattern on the same GPU.
 * kv_probe_stream_read reads `bytes` (a positive multiple of 16) of `buf`
 * front to back with 16-byte non-temporal loads; buf may be device memory or
 * a kv_host_alloc device pointer (the kernel-side host-read rate).  sink:
 * 4096 uint32 words.  kv_probe_gather_read performs exactly the loads of
 * dense kv_paged_decode_attn with `num_splits` splits on 16-bit pools (the
 * matrix-core kernel's lane layout, one page ahead); sink: B * Hkv * num_splits
 * words.
 */
kv_status kv_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
kv_status kv_probe_gather_read(const kv_shape* shape, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               int32_t num_splits, uint32_t* sink, void* stream);

/*
 * Instruction probe behind the bf16 quantizers' E4M3 codes (see
 * kv_quantize_pages_fp8): every one of the 2^32 fp32 bit patterns goes through
 * the GPU's fp32 -> E4M3 conversion instruction, in both of its operand
 * slots, and is compared with the codes' rounding rule (round to nearest
 * even, subnormals kept, saturating to 448, NaN to 0x7f | sign).  counts
 * (device, 4 uint64) receives the mismatches per class of input magnitude:
 * [0] finite below 464 (the only range the quantizers convert), [1] finite
 * from 464 up, [2] infinity, [3] NaN; first (device, 4 uint32) the smallest
 * mismatching bit pattern of each class (0xffffffff for none).  Both arrays
 * are overwritten; the call takes well under a second.
 */
kv_status kv_probe_fp8_convert(uint64_t* counts, uint32_t* first, void* stream);

/*
 * Pinned, device-mapped host memory for a zero-copy K/V pool (DirectKV review,
 * core method 4: KV kept in pinned host memory behind a device-visible pointer).
 * *host_ptr is the CPU address, *dev_ptr the address to pass to the kernels.
 * flags: KV_HOST_COHERENT or KV_HOST_NONCOHERENT.  Free with kv_host_free.
 */
kv_status kv_host_alloc(size_t bytes, uint32_t flags, void** host_ptr, void** dev_ptr);
kv_status kv_host_free(void* host_ptr);

/* Static description of a status code: the name of a kv_status value, or
 * "unknown kv_status" for any other int (the code is taken as an int so that
 * any value a caller holds may be passed). */
const char* kv_status_string(int32_t status);

/* Message of the last failing call on this thread ("" if none). */
const char* kv_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* KVDECODE_H */

// C ABI of the paged Top-K decode library: host-side validation, then one
// launcher call per entry point.  Every check runs before any device work, so
// an error status means the device was not touched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/kvdecode.h"
#include "kvd_launch.hpp"

// Split heuristic knobs (build macros): target waves per compute unit of each
// attention path (measured on the 128k and 32k GQA and the OPT MHA workloads:
// the bf16 MFMA kernel is fastest at 6, the FP8 code path at 8, the VALU
// kernel at 4; odd targets leave the 2-wave workgroups unevenly spread over the
// compute units), and the fewest pages a split should own (4: in the sparse
// decode step of the 128k and 32k GQA workloads, 64 and 32 splits of four
// selected blocks beat 128 and 48 splits of two, since the merge then reads
// fewer partials: 31.0 against 31.4 us and 30.5 against 31.7 us per step).
#ifndef KVD_SPLIT_WAVES_PER_CU
#define KVD_SPLIT_WAVES_PER_CU 6
#endif
#ifndef KVD_SPLIT_WAVES_PER_CU_FP8
#define KVD_SPLIT_WAVES_PER_CU_FP8 8
#endif
#ifndef KVD_SPLIT_WAVES_PER_CU_TIERED
#define KVD_SPLIT_WAVES_PER_CU_TIERED 12   // tiered pools: cold pages want more waves
#endif
#ifndef KVD_SPLIT_WAVES_PER_CU_VALU
#define KVD_SPLIT_WAVES_PER_CU_VALU 4
#endif
#ifndef KVD_SPLIT_MIN_BLOCKS
#define KVD_SPLIT_MIN_BLOCKS 4
#endif

namespace {

thread_local std::string g_last_error;

kv_status fail(kv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

kv_status ok() {
  g_last_error.clear();
  return KV_OK;
}

kv_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(KV_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t dtype_bytes(int dt) { return dt == KV_F32 ? 4 : 2; }

// Checks shared by every call that takes a shape.
kv_status check_shape(const kv_shape* s) {
  if (!s) return fail(KV_ERR_INVALID_ARG, "shape is NULL");
  if (s->num_seqs < 1 || s->num_seqs > 65535)
    return fail(KV_ERR_INVALID_ARG, "num_seqs=%d must be in [1, 65535]", s->num_seqs);
  if (s->num_kv_heads < 1 || s->num_kv_heads > 65535)
    return fail(KV_ERR_INVALID_ARG, "num_kv_heads=%d must be in [1, 65535]", s->num_kv_heads);
  if (s->num_q_heads < 1 || s->num_q_heads % s->num_kv_heads != 0)
    return fail(KV_ERR_INVALID_ARG, "num_q_heads=%d must be a positive multiple of num_kv_heads=%d",
                s->num_q_heads, s->num_kv_heads);
  const int G = s->num_q_heads / s->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(KV_ERR_UNSUPPORTED, "group size %d not built (1, 2, 4, 8)", G);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(KV_ERR_UNSUPPORTED, "head_dim=%d not built (64, 128)", s->head_dim);
  if (s->block_size != 16)
    return fail(KV_ERR_UNSUPPORTED, "block_size=%d not built (16)", s->block_size);
  if (s->max_blocks_per_seq < 1)
    return fail(KV_ERR_INVALID_ARG, "max_blocks_per_seq=%d must be >= 1", s->max_blocks_per_seq);
  if (s->num_pages < 1) return fail(KV_ERR_INVALID_ARG, "num_pages=%d must be >= 1", s->num_pages);
  if ((long)s->num_pages * s->num_kv_heads > 0x7fffffffL)
    return fail(KV_ERR_INVALID_ARG, "num_pages * num_kv_heads must fit in int32");
  if (s->dtype != KV_F32 && s->dtype != KV_F16 && s->dtype != KV_BF16)
    return fail(KV_ERR_UNSUPPORTED, "dtype=%d unknown", s->dtype);
  if (s->flags & ~KV_FLAG_HOST_KV) return fail(KV_ERR_INVALID_ARG, "unknown flags 0x%x", s->flags);
  return KV_OK;
}

size_t scores_bytes(const kv_shape* s) {
  return (size_t)s->num_seqs * s->num_kv_heads * s->max_blocks_per_seq * sizeof(float);
}

// The scores' part of a Top-K workspace (256-byte rounded), and the candidate
// storage of the two-level select of long rows (0 where it does not apply).
size_t scores_region(const kv_shape* s) { return (scores_bytes(s) + 255) & ~(size_t)255; }
size_t topk_candidates(const kv_shape* s, int32_t topk_blocks) {
  return kvd::topk_candidate_bytes(s->num_seqs, s->num_kv_heads, s->max_blocks_per_seq,
                                   topk_blocks);
}

// Where the scores and the Top-K candidates go: scores_out, else the head of
// the workspace (at least the scores' bytes, else KV_ERR_WORKSPACE); the
// candidates after them when the workspace also holds those (with scores_out
// given: at the head of a workspace that holds them), else nowhere and the
// select runs in one level.
kv_status topk_buffers(const kv_shape* shape, int32_t topk_blocks, float* scores_out,
                       void* workspace, size_t workspace_bytes, float** scores, void** cand) {
  const size_t sb = scores_region(shape), cb = topk_candidates(shape, topk_blocks);
  *scores = scores_out;
  *cand = nullptr;
  if (!scores_out) {
    if (!workspace || workspace_bytes < sb)
      return fail(KV_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", sb,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 4)) return fail(KV_ERR_ALIGNMENT, "workspace must be 4-byte aligned");
    *scores = static_cast<float*>(workspace);
    if (cb && workspace_bytes >= sb + cb) *cand = static_cast<char*>(workspace) + sb;
  } else if (cb && workspace && workspace_bytes >= cb && aligned(workspace, 4)) {
    *cand = workspace;
  }
  return KV_OK;
}

// Bytes of one (page, KV head) tile of a code pool; 0 for an unknown format.
int code_tile_bytes(const kv_shape* shape, int32_t code_format) {
  const int tile = shape->block_size * shape->head_dim;
  return code_format == KV_COLD_FP8 ? tile : (code_format == KV_COLD_INT4 ? tile / 2 : 0);
}

kv_status check_code_format(const kv_shape* shape, int32_t code_format) {
  if (code_format != KV_COLD_FP8 && code_format != KV_COLD_INT4)
    return fail(KV_ERR_INVALID_ARG, "code_format=%d must be KV_COLD_FP8 or KV_COLD_INT4",
                code_format);
  if (code_format == KV_COLD_INT4 && shape->dtype == KV_F32)
    return fail(KV_ERR_UNSUPPORTED, "INT4 pages are read with fp16 or bf16 queries");
  return KV_OK;
}

// Validation and launch shared by the 16-bit/fp32 pools (kvq 0) and the code
// pools (kvq 8: E4M3, kvq 4: INT4; kv_scales != nullptr).
// Pointer, list and scale checks shared by the attention entry points.
kv_status check_attn_args(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* seq_lens,
                          const int32_t* sel_blocks, const int32_t* sel_count, int32_t sel_stride,
                          float scale, const float* part_o, const float* part_m,
                          const float* part_l) {
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !part_o || !part_m || !part_l)
    return fail(KV_ERR_INVALID_ARG, "q, k_cache, v_cache, block_table, seq_lens and partials are required");
  if ((sel_blocks == nullptr) != (sel_count == nullptr))
    return fail(KV_ERR_INVALID_ARG, "sel_blocks and sel_count go together");
  if (sel_blocks && sel_stride < 1)
    return fail(KV_ERR_INVALID_ARG, "sel_stride=%d must be >= 1", sel_stride);
  if (!(scale > 0.0f) || !(scale < INFINITY))
    return fail(KV_ERR_INVALID_ARG, "scale must be finite and positive");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(part_o, 16))
    return fail(KV_ERR_ALIGNMENT, "q, k_cache, v_cache and part_o must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(part_m, 4) ||
      !aligned(part_l, 4) || (sel_blocks && (!aligned(sel_blocks, 4) || !aligned(sel_count, 4))))
    return fail(KV_ERR_ALIGNMENT, "integer and partial arrays must be 4-byte aligned");
  return KV_OK;
}

kv_status attn_common(const kv_shape* shape, int kvq, const void* q, const void* k_cache,
                      const void* v_cache, const float* kv_scales, const int32_t* block_table,
                      const int32_t* seq_lens, const int32_t* sel_blocks,
                      const int32_t* sel_count, int32_t sel_stride, float scale,
                      int32_t num_splits, float* part_o, float* part_m, float* part_l,
                      void* stream, int cold = 0, const void* k_cold = nullptr,
                      const void* v_cold = nullptr, const uint8_t* page_tier = nullptr) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (num_splits < 1 || num_splits > 65535 * 4)
    return fail(KV_ERR_INVALID_ARG, "num_splits=%d must be in [1, 262140]", num_splits);
  if ((st = check_attn_args(q, k_cache, v_cache, block_table, seq_lens, sel_blocks, sel_count,
                            sel_stride, scale, part_o, part_m, part_l)) != KV_OK)
    return st;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  return hip_status(
      kvd::launch_paged_attn(shape->dtype, shape->head_dim, G, kvq, q, k_cache, v_cache,
                             kv_scales, block_table, seq_lens, sel_blocks, sel_count, sel_stride,
                             nullptr, 0, shape->num_seqs, shape->num_q_heads, shape->num_kv_heads,
                             shape->max_blocks_per_seq, num_splits, scale, part_o, part_m, part_l,
                             nullptr, (hipStream_t)stream, cold, k_cold, v_cold, page_tier),
      cold ? "kv_paged_decode_attn_tiered launch"
           : (kvq == 8 ? "kv_paged_decode_attn_fp8 launch"
                       : (kvq == 4 ? "kv_paged_decode_attn_int4 launch"
                                   : "kv_paged_decode_attn launch")));
}

}  // namespace

extern "C" {

const char* kv_status_string(int32_t status) {
  switch (status) {
    case KV_OK: return "KV_OK";
    case KV_ERR_INVALID_ARG: return "KV_ERR_INVALID_ARG";
    case KV_ERR_UNSUPPORTED: return "KV_ERR_UNSUPPORTED";
    case KV_ERR_ALIGNMENT: return "KV_ERR_ALIGNMENT";
    case KV_ERR_WORKSPACE: return "KV_ERR_WORKSPACE";
    case KV_ERR_HIP: return "KV_ERR_HIP";
  }
  return "unknown kv_status";
}

const char* kv_last_error_message(void) { return g_last_error.c_str(); }

kv_status kv_block_meta_build(const kv_shape* shape, const void* k_cache, const int32_t* page_ids,
                              const int32_t* page_valid_tokens, int32_t num_page_ids, void* kmeta,
                              void* stream) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (num_page_ids < 0) return fail(KV_ERR_INVALID_ARG, "num_page_ids=%d < 0", num_page_ids);
  if (num_page_ids == 0) return ok();
  if (!k_cache || !page_ids || !page_valid_tokens || !kmeta)
    return fail(KV_ERR_INVALID_ARG, "k_cache, page_ids, page_valid_tokens and kmeta are required");
  if ((long)num_page_ids * shape->num_kv_heads > 0x7fffffffL)
    return fail(KV_ERR_INVALID_ARG, "num_page_ids * num_kv_heads overflows int32");
  if (!aligned(k_cache, 16) || !aligned(kmeta, 16))
    return fail(KV_ERR_ALIGNMENT, "k_cache and kmeta must be 16-byte aligned");
  if (!aligned(page_ids, 4) || !aligned(page_valid_tokens, 4))
    return fail(KV_ERR_ALIGNMENT, "page_ids and page_valid_tokens must be 4-byte aligned");
  return hip_status(kvd::launch_block_meta(shape->dtype, shape->head_dim, k_cache, page_ids,
                                           page_valid_tokens, num_page_ids, shape->num_kv_heads,
                                           kmeta, (hipStream_t)stream),
                    "kv_block_meta_build launch");
}

kv_status kv_block_mean_build(const kv_shape* shape, const void* k_cache, const int32_t* page_ids,
                              const int32_t* page_valid_tokens, int32_t num_page_ids, float* kmean,
                              void* stream) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (num_page_ids < 0) return fail(KV_ERR_INVALID_ARG, "num_page_ids=%d < 0", num_page_ids);
  if (num_page_ids == 0) return ok();
  if (!k_cache || !page_ids || !page_valid_tokens || !kmean)
    return fail(KV_ERR_INVALID_ARG, "k_cache, page_ids, page_valid_tokens and kmean are required");
  if ((long)num_page_ids * shape->num_kv_heads > 0x7fffffffL)
    return fail(KV_ERR_INVALID_ARG, "num_page_ids * num_kv_heads overflows int32");
  if (!aligned(k_cache, 16) || !aligned(kmean, 16))
    return fail(KV_ERR_ALIGNMENT, "k_cache and kmean must be 16-byte aligned");
  if (!aligned(page_ids, 4) || !aligned(page_valid_tokens, 4))
    return fail(KV_ERR_ALIGNMENT, "page_ids and page_valid_tokens must be 4-byte aligned");
  return hip_status(kvd::launch_block_mean(shape->dtype, shape->head_dim, k_cache, page_ids,
                                           page_valid_tokens, num_page_ids, shape->num_kv_heads,
                                           kmean, (hipStream_t)stream),
                    "kv_block_mean_build launch");
}

kv_status kv_decode_select(const kv_shape* shape, int32_t index_kind, const void* q,
                           const void* k_new, const void* v_new, const int32_t* block_table,
                           const int32_t* seq_lens, void* k_cache, void* v_cache, void* kmeta,
                           float* kmean, int32_t topk_blocks, int32_t sink_tokens,
                           int32_t local_tokens, float* scores_out, int32_t* sel_blocks,
                           int32_t* sel_count, void* workspace, size_t workspace_bytes,
                           void* stream) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (index_kind != KV_INDEX_MINMAX && index_kind != KV_INDEX_MEAN)
    return fail(KV_ERR_INVALID_ARG, "index_kind=%d unknown", index_kind);
  const void* index = index_kind == KV_INDEX_MINMAX ? kmeta : static_cast<const void*>(kmean);
  if (!index)
    return fail(KV_ERR_INVALID_ARG, "the index selected by index_kind (%s) is required",
                index_kind == KV_INDEX_MINMAX ? "kmeta" : "kmean");
  if (topk_blocks < 1) return fail(KV_ERR_INVALID_ARG, "topk_blocks=%d must be >= 1", topk_blocks);
  if (sink_tokens < 0 || local_tokens < 0)
    return fail(KV_ERR_INVALID_ARG, "sink_tokens=%d and local_tokens=%d must be >= 0", sink_tokens,
                local_tokens);
  const int32_t forced = kv_max_forced_blocks(shape, sink_tokens, local_tokens);
  if (forced > topk_blocks)
    return fail(KV_ERR_INVALID_ARG,
                "sink_tokens=%d and local_tokens=%d can force %d blocks, more than topk_blocks=%d",
                sink_tokens, local_tokens, forced, topk_blocks);
  if (shape->max_blocks_per_seq > kvd::kTopkMaxBlocks)
    return fail(KV_ERR_UNSUPPORTED, "max_blocks_per_seq=%d above the Top-K limit %d",
                shape->max_blocks_per_seq, kvd::kTopkMaxBlocks);
  if (!q || !k_new || !v_new || !block_table || !seq_lens || !k_cache || !v_cache || !sel_blocks ||
      !sel_count)
    return fail(KV_ERR_INVALID_ARG,
                "q, k_new, v_new, block_table, seq_lens, k_cache, v_cache, sel_blocks and "
                "sel_count are required");
  if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || (kmeta && !aligned(kmeta, 16)) || (kmean && !aligned(kmean, 16)))
    return fail(KV_ERR_ALIGNMENT,
                "q, k_new, v_new, k_cache, v_cache, kmeta and kmean must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(sel_blocks, 4) ||
      !aligned(sel_count, 4) || (scores_out && !aligned(scores_out, 4)))
    return fail(KV_ERR_ALIGNMENT, "integer and score arrays must be 4-byte aligned");
  float* scores = nullptr;
  void* cand = nullptr;
  if ((st = topk_buffers(shape, topk_blocks, scores_out, workspace, workspace_bytes, &scores,
                         &cand)) != KV_OK)
    return st;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  hipStream_t s = (hipStream_t)stream;
  // the scorer's extra workgroups append the token and score its block from the
  // updated index rows; the other blocks' index rows are not touched by it
  hipError_t e = kvd::launch_block_score(shape->dtype, shape->head_dim, G, index_kind, q, index,
                                         block_table, seq_lens, shape->num_seqs,
                                         shape->num_q_heads, shape->num_kv_heads,
                                         shape->max_blocks_per_seq, scores, s, k_new, v_new,
                                         k_cache, v_cache, kmeta, kmean);
  if (e != hipSuccess) return hip_status(e, "append + block score launch");
  return hip_status(kvd::launch_topk(scores, seq_lens, shape->num_seqs, shape->num_kv_heads,
                                     shape->max_blocks_per_seq, topk_blocks, sink_tokens,
                                     local_tokens, sel_blocks, sel_count, s, cand),
                    "top-k launch");
}

kv_status kv_decode_score(const kv_shape* shape, int32_t index_kind, const void* q,
                          const void* k_new, const void* v_new, const int32_t* block_table,
                          const int32_t* seq_lens, void* k_cache, void* v_cache, void* kmeta,
                          float* kmean, float* scores_out, void* stream) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (index_kind != KV_INDEX_MINMAX && index_kind != KV_INDEX_MEAN)
    return fail(KV_ERR_INVALID_ARG, "index_kind=%d unknown", index_kind);
  const void* index = index_kind == KV_INDEX_MINMAX ? kmeta : static_cast<const void*>(kmean);
  if (!index)
    return fail(KV_ERR_INVALID_ARG, "the index selected by index_kind (%s) is required",
                index_kind == KV_INDEX_MINMAX ? "kmeta" : "kmean");
  if (!q || !k_new || !v_new || !block_table || !seq_lens || !k_cache || !v_cache || !scores_out)
    return fail(KV_ERR_INVALID_ARG,
                "q, k_new, v_new, block_table, seq_lens, k_cache, v_cache and scores_out are "
                "required");
  if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || (kmeta && !aligned(kmeta, 16)) || (kmean && !aligned(kmean, 16)))
    return fail(KV_ERR_ALIGNMENT,
                "q, k_new, v_new, k_cache, v_cache, kmeta and kmean must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(scores_out, 4))
    return fail(KV_ERR_ALIGNMENT, "integer and score arrays must be 4-byte aligned");
  const int G = shape->num_q_heads / shape->num_kv_heads;
  return hip_status(kvd::launch_block_score(shape->dtype, shape->head_dim, G, index_kind, q, index,
                                            block_table, seq_lens, shape->num_seqs,
                                            shape->num_q_heads, shape->num_kv_heads,
                                            shape->max_blocks_per_seq, scores_out,
                                            (hipStream_t)stream, k_new, v_new, k_cache, v_cache,
                                            kmeta, kmean),
                    "kv_decode_score launch");
}

kv_status kv_select_decode_attn(const kv_shape* shape, const float* scores,
                                const int32_t* block_table, const int32_t* seq_lens,
                                int32_t topk_blocks, int32_t sink_tokens, int32_t local_tokens,
                                const void* q, const void* k_cache, const void* v_cache,
                                float scale, int32_t num_splits, int32_t* sel_blocks,
                                int32_t* sel_count, float* part_o, float* part_m, float* part_l,
                                void* stream) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (topk_blocks < 1) return fail(KV_ERR_INVALID_ARG, "topk_blocks=%d must be >= 1", topk_blocks);
  if (sink_tokens < 0 || local_tokens < 0)
    return fail(KV_ERR_INVALID_ARG, "sink_tokens=%d and local_tokens=%d must be >= 0", sink_tokens,
                local_tokens);
  const int32_t forced = kv_max_forced_blocks(shape, sink_tokens, local_tokens);
  if (forced > topk_blocks)
    return fail(KV_ERR_INVALID_ARG,
                "sink_tokens=%d and local_tokens=%d can force %d blocks, more than topk_blocks=%d",
                sink_tokens, local_tokens, forced, topk_blocks);
  if (shape->max_blocks_per_seq > kvd::kTopkMaxBlocks)
    return fail(KV_ERR_UNSUPPORTED, "max_blocks_per_seq=%d above the Top-K limit %d",
                shape->max_blocks_per_seq, kvd::kTopkMaxBlocks);
  if (num_splits < 1 || num_splits > 65535 * 4)
    return fail(KV_ERR_INVALID_ARG, "num_splits=%d must be in [1, 262140]", num_splits);
  if (!scores || !sel_blocks || !sel_count)
    return fail(KV_ERR_INVALID_ARG, "scores, sel_blocks and sel_count are required");
  if (!aligned(scores, 4))
    return fail(KV_ERR_ALIGNMENT, "scores must be 4-byte aligned");
  if ((st = check_attn_args(q, k_cache, v_cache, block_table, seq_lens, sel_blocks, sel_count,
                            topk_blocks, scale, part_o, part_m, part_l)) != KV_OK)
    return st;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  hipStream_t s = (hipStream_t)stream;
  if (kvd::select_attn_fusable(shape->dtype, G, shape->max_blocks_per_seq, topk_blocks,
                               num_splits))
    return hip_status(
        kvd::launch_select_attn(shape->dtype, shape->head_dim, G, scores, topk_blocks, sink_tokens,
                                local_tokens, sel_blocks, sel_count, q, k_cache, v_cache,
                                block_table, seq_lens, shape->num_seqs, shape->num_q_heads,
                                shape->num_kv_heads, shape->max_blocks_per_seq, num_splits, scale,
                                part_o, part_m, part_l, s),
        "kv_select_decode_attn launch");
  // the same two steps as separate launches (same lists, same partials)
  hipError_t e = kvd::launch_topk(scores, seq_lens, shape->num_seqs, shape->num_kv_heads,
                                  shape->max_blocks_per_seq, topk_blocks, sink_tokens,
                                  local_tokens, sel_blocks, sel_count, s);
  if (e != hipSuccess) return hip_status(e, "kv_select_decode_attn top-k launch");
  return hip_status(
      kvd::launch_paged_attn(shape->dtype, shape->head_dim, G, 0, q, k_cache, v_cache, nullptr,
                             block_table, seq_lens, sel_blocks, sel_count, topk_blocks, nullptr, 0,
                             shape->num_seqs, shape->num_q_heads, shape->num_kv_heads,
                             shape->max_blocks_per_seq, num_splits, scale, part_o, part_m, part_l,
                             nullptr, s, 0, nullptr, nullptr, nullptr),
      "kv_select_decode_attn attention launch");
}

kv_status kv_append_token(const kv_shape* shape, const void* k_new, const void* v_new,
                          const int32_t* block_table, const int32_t* seq_lens, void* k_cache,
                          void* v_cache, void* kmeta, float* kmean, void* stream) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (!k_new || !v_new || !block_table || !seq_lens || !k_cache || !v_cache)
    return fail(KV_ERR_INVALID_ARG, "k_new, v_new, block_table, seq_lens, k_cache and v_cache are required");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      (kmeta && !aligned(kmeta, 16)) || (kmean && !aligned(kmean, 16)))
    return fail(KV_ERR_ALIGNMENT,
                "k_new, v_new, k_cache, v_cache, kmeta and kmean must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4))
    return fail(KV_ERR_ALIGNMENT, "block_table and seq_lens must be 4-byte aligned");
  return hip_status(kvd::launch_append_token(shape->dtype, shape->head_dim, k_new, v_new,
                                             block_table, seq_lens, shape->num_seqs,
                                             shape->num_kv_heads, shape->max_blocks_per_seq,
                                             k_cache, v_cache, kmeta, kmean, (hipStream_t)stream),
                    "kv_append_token launch");
}

size_t kv_score_topk_workspace_size(const kv_shape* shape, int32_t topk_blocks) {
  if (check_shape(shape) != KV_OK) return 0;
  return scores_region(shape) + topk_candidates(shape, topk_blocks);
}

int32_t kv_max_forced_blocks(const kv_shape* shape, int32_t sink_tokens, int32_t local_tokens) {
  if (check_shape(shape) != KV_OK || sink_tokens < 0 || local_tokens < 0) return -1;
  const long bs = shape->block_size;
  // the first sink tokens fill ceil(sink / bs) blocks; local consecutive tokens
  // touch at most ceil((local - 1) / bs) + 1 blocks
  long n = (sink_tokens + bs - 1) / bs;
  if (local_tokens > 0) n += (local_tokens - 1 + bs - 1) / bs + 1;
  return (int32_t)std::min<long>(n, 0x7fffffffL);
}

}  // extern "C"

namespace {
// Argument checks of the selection calls; scores_out may be NULL (the caller
// then supplies the score buffer).
kv_status check_select(const kv_shape* shape, int32_t index_kind, const void* q, const void* index,
                       const int32_t* block_table, const int32_t* seq_lens, int32_t topk_blocks,
                       int32_t sink_tokens, int32_t local_tokens, const float* scores_out,
                       const int32_t* sel_blocks, const int32_t* sel_count) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (index_kind != KV_INDEX_MINMAX && index_kind != KV_INDEX_MEAN)
    return fail(KV_ERR_INVALID_ARG, "index_kind=%d unknown", index_kind);
  if (topk_blocks < 1) return fail(KV_ERR_INVALID_ARG, "topk_blocks=%d must be >= 1", topk_blocks);
  if (sink_tokens < 0 || local_tokens < 0)
    return fail(KV_ERR_INVALID_ARG, "sink_tokens=%d and local_tokens=%d must be >= 0", sink_tokens,
                local_tokens);
  const int32_t forced = kv_max_forced_blocks(shape, sink_tokens, local_tokens);
  if (forced > topk_blocks)
    return fail(KV_ERR_INVALID_ARG,
                "sink_tokens=%d and local_tokens=%d can force %d blocks, more than topk_blocks=%d",
                sink_tokens, local_tokens, forced, topk_blocks);
  if (shape->max_blocks_per_seq > kvd::kTopkMaxBlocks)
    return fail(KV_ERR_UNSUPPORTED, "max_blocks_per_seq=%d above the Top-K limit %d",
                shape->max_blocks_per_seq, kvd::kTopkMaxBlocks);
  if (!q || !index || !block_table || !seq_lens || !sel_blocks || !sel_count)
    return fail(KV_ERR_INVALID_ARG, "q, index, block_table, seq_lens, sel_blocks, sel_count are required");
  if (!aligned(q, 16) || !aligned(index, 16))
    return fail(KV_ERR_ALIGNMENT, "q and the index must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(sel_blocks, 4) ||
      !aligned(sel_count, 4) || (scores_out && !aligned(scores_out, 4)))
    return fail(KV_ERR_ALIGNMENT, "integer and score arrays must be 4-byte aligned");
  return KV_OK;
}

// Score + Top-K launches into a checked score buffer.
kv_status launch_select(const kv_shape* shape, int32_t index_kind, const void* q,
                        const void* index, const int32_t* block_table, const int32_t* seq_lens,
                        int32_t topk_blocks, int32_t sink_tokens, int32_t local_tokens,
                        float* scores, int32_t* sel_blocks, int32_t* sel_count, void* stream,
                        void* cand) {
  const int G = shape->num_q_heads / shape->num_kv_heads;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = kvd::launch_block_score(shape->dtype, shape->head_dim, G, index_kind, q, index,
                                         block_table, seq_lens, shape->num_seqs,
                                         shape->num_q_heads, shape->num_kv_heads,
                                         shape->max_blocks_per_seq, scores, s);
  if (e != hipSuccess) return hip_status(e, "block score launch");
  return hip_status(kvd::launch_topk(scores, seq_lens, shape->num_seqs, shape->num_kv_heads,
                                     shape->max_blocks_per_seq, topk_blocks, sink_tokens,
                                     local_tokens, sel_blocks, sel_count, s, cand),
                    "top-k launch");
}

// The score buffer of kv_block_select_no_alloc: device memory of the library
// itself (a copy per GPU, held until the process ends), so the call allocates
// nothing.  Host code reaches it only through the address hipGetSymbolAddress
// gives on each device (the name is a host-side stand-in there).
constexpr size_t kNoAllocScores = (size_t)1 << 20;   // floats: B * Hkv * maxN at most (4 MiB)
static __device__ __align__(256) float scratch[kNoAllocScores];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call on
// that device (with it current) and kept.
kv_status scratch_scores(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KV_ERR_UNSUPPORTED, "device %d above the %d devices the scratch table holds", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    g_scratch[dev] = static_cast<float*>(p);
  }
  *out = g_scratch[dev];
  return KV_OK;
}
}  // namespace

extern "C" {

kv_status kv_block_select(const kv_shape* shape, int32_t index_kind, const void* q,
                          const void* index, const int32_t* block_table, const int32_t* seq_lens,
                          int32_t topk_blocks, int32_t sink_tokens, int32_t local_tokens,
                          float* scores_out, int32_t* sel_blocks, int32_t* sel_count,
                          void* workspace, size_t workspace_bytes, void* stream) {
  kv_status st = check_select(shape, index_kind, q, index, block_table, seq_lens, topk_blocks,
                              sink_tokens, local_tokens, scores_out, sel_blocks, sel_count);
  if (st != KV_OK) return st;
  float* scores = nullptr;
  void* cand = nullptr;
  if ((st = topk_buffers(shape, topk_blocks, scores_out, workspace, workspace_bytes, &scores,
                         &cand)) != KV_OK)
    return st;
  return launch_select(shape, index_kind, q, index, block_table, seq_lens, topk_blocks,
                       sink_tokens, local_tokens, scores, sel_blocks, sel_count, stream, cand);
}

kv_status kv_block_select_no_alloc(const kv_shape* shape, int32_t index_kind, const void* q,
                                   const void* index, const int32_t* block_table,
                                   const int32_t* seq_lens, int32_t topk_blocks,
                                   int32_t sink_tokens, int32_t local_tokens, int32_t* sel_blocks,
                                   int32_t* sel_count, void* stream) {
  kv_status st = check_select(shape, index_kind, q, index, block_table, seq_lens, topk_blocks,
                              sink_tokens, local_tokens, nullptr, sel_blocks, sel_count);
  if (st != KV_OK) return st;
  const size_t n = (size_t)shape->num_seqs * shape->num_kv_heads * shape->max_blocks_per_seq;
  if (n > kNoAllocScores)
    return fail(KV_ERR_WORKSPACE,
                "num_seqs * num_kv_heads * max_blocks_per_seq = %zu scores, above the %zu the "
                "library's scratch holds", n, kNoAllocScores);
  float* scores = nullptr;
  st = scratch_scores(&scores);
  if (st != KV_OK) return st;
  // the two-level select's candidates go after the scores when the array
  // holds both; every candidate slot a call reads is written in that call
  void* cand = nullptr;
  const size_t sb = scores_region(shape), cb = topk_candidates(shape, topk_blocks);
  if (cb && sb + cb <= kNoAllocScores * sizeof(float))
    cand = reinterpret_cast<char*>(scores) + sb;
  // the score launch writes every one of the n scores, so nothing is cleared
  return launch_select(shape, index_kind, q, index, block_table, seq_lens, topk_blocks,
                       sink_tokens, local_tokens, scores, sel_blocks, sel_count, stream, cand);
}

kv_status kv_block_score_topk(const kv_shape* shape, const void* q, const void* kmeta,
                              const int32_t* block_table, const int32_t* seq_lens,
                              int32_t topk_blocks, float* scores_out, int32_t* sel_blocks,
                              int32_t* sel_count, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return kv_block_select(shape, KV_INDEX_MINMAX, q, kmeta, block_table, seq_lens, topk_blocks, 0,
                         0, scores_out, sel_blocks, sel_count, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {
int32_t auto_splits(const kv_shape* shape, int32_t blocks_per_unit, long waves_per_cu) {
  if (check_shape(shape) != KV_OK || blocks_per_unit < 1) return 1;
  const long units = (long)shape->num_seqs * shape->num_kv_heads;
  const long target_waves = (long)kvd::device_cu_count() * waves_per_cu;
  long s = (target_waves + units - 1) / units;
  // pages read over the host link favour fewer, longer splits
  const long min_blocks = (shape->flags & KV_FLAG_HOST_KV) ? 8 : KVD_SPLIT_MIN_BLOCKS;
  s = std::min<long>(s, (blocks_per_unit + min_blocks - 1) / min_blocks);
  return (int32_t)std::max<long>(1, std::min<long>(s, 65535L * 4));
}

bool mfma_path(const kv_shape* s) {
  return s->dtype != KV_F32 && s->num_q_heads / std::max(1, s->num_kv_heads) >= 2;
}
}  // namespace

extern "C" {

int32_t kv_auto_num_splits(const kv_shape* shape, int32_t blocks_per_unit) {
  if (!shape) return 1;
  return auto_splits(shape, blocks_per_unit,
                     mfma_path(shape) ? KVD_SPLIT_WAVES_PER_CU : KVD_SPLIT_WAVES_PER_CU_VALU);
}

int32_t kv_auto_select_splits(const kv_shape* shape, int32_t topk_blocks) {
  if (!shape || check_shape(shape) != KV_OK || topk_blocks < 1) return 1;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  // one workgroup of kSelAttnWaves splits per compute unit
  const long units = (long)shape->num_seqs * shape->num_kv_heads;
  const long wgs = std::max<long>(1, kvd::device_cu_count() / units);
  const long cap = ((long)topk_blocks + kvd::kSelAttnWaves - 1) / kvd::kSelAttnWaves;
  const int32_t s = (int32_t)(kvd::kSelAttnWaves * std::min(wgs, cap));
  if (kvd::select_attn_fusable(shape->dtype, G, shape->max_blocks_per_seq, topk_blocks, s))
    return s;
  return kv_auto_num_splits(shape, topk_blocks);
}

int32_t kv_auto_num_splits_fp8(const kv_shape* shape, int32_t blocks_per_unit) {
  if (!shape) return 1;
  return auto_splits(shape, blocks_per_unit, KVD_SPLIT_WAVES_PER_CU_FP8);
}

int32_t kv_auto_num_splits_tiered(const kv_shape* shape, int32_t blocks_per_unit) {
  if (!shape) return 1;
  return auto_splits(shape, blocks_per_unit, KVD_SPLIT_WAVES_PER_CU_TIERED);
}

kv_status kv_paged_decode_attn(const kv_shape* shape, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* sel_blocks,
                               const int32_t* sel_count, int32_t sel_stride, float scale,
                               int32_t num_splits, float* part_o, float* part_m, float* part_l,
                               void* stream) {
  return attn_common(shape, 0, q, k_cache, v_cache, nullptr, block_table, seq_lens, sel_blocks,
                     sel_count, sel_stride, scale, num_splits, part_o, part_m, part_l, stream);
}

}  // extern "C"

namespace {
kv_status quantize_common(const kv_shape* shape, int fmt, const void* k_cache, const void* v_cache,
                          const int32_t* page_ids, const int32_t* page_valid_tokens,
                          int32_t num_page_ids, uint8_t* k_codes, uint8_t* v_codes,
                          float* kv_scales, void* stream, const char* name) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (fmt == 4 && shape->dtype == KV_F32)
    return fail(KV_ERR_UNSUPPORTED, "%s: INT4 pages are made from fp16 or bf16 pools", name);
  if (num_page_ids < 0) return fail(KV_ERR_INVALID_ARG, "num_page_ids=%d < 0", num_page_ids);
  if (num_page_ids == 0) return ok();
  if (!k_cache || !v_cache || !page_ids || !k_codes || !v_codes || !kv_scales)
    return fail(KV_ERR_INVALID_ARG,
                "%s: k_cache, v_cache, page_ids, the code pools and kv_scales are required", name);
  if ((long)num_page_ids * shape->num_kv_heads > 0x7fffffffL)
    return fail(KV_ERR_INVALID_ARG, "num_page_ids * num_kv_heads overflows int32");
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(k_codes, 16) ||
      !aligned(v_codes, 16))
    return fail(KV_ERR_ALIGNMENT, "k_cache, v_cache and the code pools must be 16-byte aligned");
  if (!aligned(page_ids, 4) || (page_valid_tokens && !aligned(page_valid_tokens, 4)) ||
      !aligned(kv_scales, 8))
    return fail(KV_ERR_ALIGNMENT,
                "page_ids and page_valid_tokens must be 4-byte aligned, kv_scales 8-byte aligned");
  std::string what = std::string(name) + " launch";
  return hip_status(kvd::launch_quantize(fmt, shape->dtype, shape->head_dim, k_cache, v_cache,
                                         page_ids, page_valid_tokens, num_page_ids,
                                         shape->num_kv_heads, k_codes, v_codes, kv_scales,
                                         (hipStream_t)stream),
                    what.c_str());
}
}  // namespace

extern "C" {

kv_status kv_quantize_pages_fp8(const kv_shape* shape, const void* k_cache, const void* v_cache,
                                const int32_t* page_ids, const int32_t* page_valid_tokens,
                                int32_t num_page_ids, uint8_t* k_fp8, uint8_t* v_fp8,
                                float* kv_scales, void* stream) {
  return quantize_common(shape, 8, k_cache, v_cache, page_ids, page_valid_tokens, num_page_ids,
                         k_fp8, v_fp8, kv_scales, stream, "kv_quantize_pages_fp8");
}

kv_status kv_quantize_pages_int4(const kv_shape* shape, const void* k_cache, const void* v_cache,
                                 const int32_t* page_ids, const int32_t* page_valid_tokens,
                                 int32_t num_page_ids, uint8_t* k_int4, uint8_t* v_int4,
                                 float* kv_scales, void* stream) {
  return quantize_common(shape, 4, k_cache, v_cache, page_ids, page_valid_tokens, num_page_ids,
                         k_int4, v_int4, kv_scales, stream, "kv_quantize_pages_int4");
}

kv_status kv_paged_decode_attn_fp8(const kv_shape* shape, const void* q, const uint8_t* k_fp8,
                                   const uint8_t* v_fp8, const float* kv_scales,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   const int32_t* sel_blocks, const int32_t* sel_count,
                                   int32_t sel_stride, float scale, int32_t num_splits,
                                   float* part_o, float* part_m, float* part_l, void* stream) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (!kv_scales) return fail(KV_ERR_INVALID_ARG, "kv_scales is required");
  if (!aligned(kv_scales, 8)) return fail(KV_ERR_ALIGNMENT, "kv_scales must be 8-byte aligned");
  return attn_common(shape, 8, q, k_fp8, v_fp8, kv_scales, block_table, seq_lens, sel_blocks,
                     sel_count, sel_stride, scale, num_splits, part_o, part_m, part_l, stream);
}

kv_status kv_paged_decode_attn_int4(const kv_shape* shape, const void* q, const uint8_t* k_int4,
                                    const uint8_t* v_int4, const float* kv_scales,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* sel_blocks, const int32_t* sel_count,
                                    int32_t sel_stride, float scale, int32_t num_splits,
                                    float* part_o, float* part_m, float* part_l, void* stream) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (shape->dtype == KV_F32)
    return fail(KV_ERR_UNSUPPORTED, "INT4 pages are read with fp16 or bf16 queries");
  if (!kv_scales) return fail(KV_ERR_INVALID_ARG, "kv_scales is required");
  if (!aligned(kv_scales, 8)) return fail(KV_ERR_ALIGNMENT, "kv_scales must be 8-byte aligned");
  return attn_common(shape, 4, q, k_int4, v_int4, kv_scales, block_table, seq_lens, sel_blocks,
                     sel_count, sel_stride, scale, num_splits, part_o, part_m, part_l, stream);
}

kv_status kv_paged_decode_attn_tiered(const kv_shape* shape, const void* q, const void* k_cache,
                                      const void* v_cache, const uint8_t* k_cold,
                                      const uint8_t* v_cold, const float* kv_scales,
                                      int32_t cold_format, const uint8_t* page_tier,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      const int32_t* sel_blocks, const int32_t* sel_count,
                                      int32_t sel_stride, float scale, int32_t num_splits,
                                      float* part_o, float* part_m, float* part_l,
                                      void* stream) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (!mfma_path(shape))
    return fail(KV_ERR_UNSUPPORTED,
                "tiered pools need fp16 or bf16 and a GQA group of 2 or more query heads");
  if (cold_format != KV_COLD_FP8 && cold_format != KV_COLD_INT4)
    return fail(KV_ERR_INVALID_ARG, "cold_format=%d must be KV_COLD_FP8 or KV_COLD_INT4",
                cold_format);
  if (!k_cold || !v_cold || !kv_scales || !page_tier)
    return fail(KV_ERR_INVALID_ARG, "k_cold, v_cold, kv_scales and page_tier are required");
  if (!aligned(k_cold, 16) || !aligned(v_cold, 16) || !aligned(kv_scales, 8))
    return fail(KV_ERR_ALIGNMENT, "the cold pools must be 16-byte aligned, kv_scales 8-byte");
  return attn_common(shape, 0, q, k_cache, v_cache, kv_scales, block_table, seq_lens, sel_blocks,
                     sel_count, sel_stride, scale, num_splits, part_o, part_m, part_l, stream,
                     cold_format, k_cold, v_cold, page_tier);
}

size_t kv_tiered_split_workspace_size(const kv_shape* shape, int32_t sel_stride) {
  if (!shape || check_shape(shape) != KV_OK || sel_stride < 0) return 0;
  const int stride = sel_stride > 0 ? sel_stride : shape->max_blocks_per_seq;
  const size_t rows = (size_t)shape->num_seqs * shape->num_kv_heads;
  const size_t chunks = (size_t)kvd::tier_chunks(stride);
  // hot and cold lists and counts, then the tier flags and per-chunk counts
  return rows * ((2 * (size_t)stride + 2 + chunks) * sizeof(int32_t) +
                 chunks * kvd::kTierChunkPositions);
}

kv_status kv_paged_decode_attn_tiered_split(
    const kv_shape* shape, const void* q, const void* k_cache, const void* v_cache,
    const uint8_t* k_cold, const uint8_t* v_cold, const float* kv_scales, int32_t cold_format,
    const uint8_t* page_tier, const int32_t* block_table, const int32_t* seq_lens,
    const int32_t* sel_blocks, const int32_t* sel_count, int32_t sel_stride, float scale,
    int32_t num_splits_hot, int32_t num_splits_cold, float* part_o, float* part_m,
    float* part_l, void* workspace, size_t workspace_bytes, void* stream) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if ((st = check_code_format(shape, cold_format)) != KV_OK) return st;
  if (num_splits_hot < 1 || num_splits_cold < 1 ||
      (long)num_splits_hot + num_splits_cold > 65535L * 4)
    return fail(KV_ERR_INVALID_ARG, "num_splits_hot=%d and num_splits_cold=%d must be >= 1 "
                "with a sum of at most 262140", num_splits_hot, num_splits_cold);
  if (!k_cold || !v_cold || !kv_scales || !page_tier)
    return fail(KV_ERR_INVALID_ARG, "k_cold, v_cold, kv_scales and page_tier are required");
  if (!aligned(k_cold, 16) || !aligned(v_cold, 16) || !aligned(kv_scales, 8))
    return fail(KV_ERR_ALIGNMENT, "the cold pools must be 16-byte aligned, kv_scales 8-byte");
  if ((st = check_attn_args(q, k_cache, v_cache, block_table, seq_lens, sel_blocks, sel_count,
                            sel_stride, scale, part_o, part_m, part_l)) != KV_OK)
    return st;
  const size_t need = kv_tiered_split_workspace_size(shape, sel_blocks ? sel_stride : 0);
  if (!workspace || workspace_bytes < need)
    return fail(KV_ERR_WORKSPACE, "the workspace needs %zu bytes", need);
  if (!aligned(workspace, 4)) return fail(KV_ERR_ALIGNMENT, "the workspace must be 4-byte aligned");
  const int stride = sel_blocks ? sel_stride : shape->max_blocks_per_seq;
  const size_t rows = (size_t)shape->num_seqs * shape->num_kv_heads;
  int32_t* ws = static_cast<int32_t*>(workspace);
  int32_t* hot = ws;
  int32_t* cold = hot + rows * stride;
  int32_t* hot_n = cold + rows * stride;
  int32_t* cold_n = hot_n + rows;
  int32_t* chunk_cold = cold_n + rows;
  uint8_t* flags = reinterpret_cast<uint8_t*>(chunk_cold + rows * kvd::tier_chunks(stride));
  hipStream_t s = (hipStream_t)stream;
  const int G = shape->num_q_heads / shape->num_kv_heads;
  const int S = num_splits_hot + num_splits_cold;
  hipError_t e = kvd::launch_tier_lists(sel_blocks, sel_count, sel_stride, block_table, seq_lens,
                                        page_tier, shape->num_seqs, shape->num_kv_heads,
                                        shape->max_blocks_per_seq, stride, hot, hot_n, cold,
                                        cold_n, flags, chunk_cold, s);
  if (e == hipSuccess)     // hot pages: columns [0, num_splits_hot) of the partials
    e = kvd::launch_paged_attn(shape->dtype, shape->head_dim, G, 0, q, k_cache, v_cache, nullptr,
                               block_table, seq_lens, hot, hot_n, stride, nullptr, 0,
                               shape->num_seqs, shape->num_q_heads, shape->num_kv_heads,
                               shape->max_blocks_per_seq, num_splits_hot, scale, part_o, part_m,
                               part_l, nullptr, s, 0, nullptr, nullptr, nullptr, nullptr, S);
  if (e == hipSuccess)     // cold pages: the columns after them
    e = kvd::launch_paged_attn(shape->dtype, shape->head_dim, G, cold_format, q, k_cold, v_cold,
                               kv_scales, block_table, seq_lens, cold, cold_n, stride, nullptr, 0,
                               shape->num_seqs, shape->num_q_heads, shape->num_kv_heads,
                               shape->max_blocks_per_seq, num_splits_cold, scale,
                               part_o + (size_t)num_splits_hot * shape->head_dim,
                               part_m + num_splits_hot, part_l + num_splits_hot, nullptr, s, 0,
                               nullptr, nullptr, nullptr, nullptr, S);
  return hip_status(e, "kv_paged_decode_attn_tiered_split launch");
}

kv_status kv_decode_combine(const kv_shape* shape, int32_t num_splits, const float* part_o,
                            const float* part_m, const float* part_l, float* out, float* lse_out,
                            void* stream) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (num_splits < 1) return fail(KV_ERR_INVALID_ARG, "num_splits=%d must be >= 1", num_splits);
  if (!part_o || !part_m || !part_l || !out)
    return fail(KV_ERR_INVALID_ARG, "partials and out are required");
  if (!aligned(part_o, 16) || !aligned(out, 16))
    return fail(KV_ERR_ALIGNMENT, "part_o and out must be 16-byte aligned");
  if (!aligned(part_m, 4) || !aligned(part_l, 4) || (lse_out && !aligned(lse_out, 4)))
    return fail(KV_ERR_ALIGNMENT, "part_m, part_l and lse must be 4-byte aligned");
  const long rows = (long)shape->num_seqs * shape->num_q_heads;
  if (rows > 0x7fffffffL) return fail(KV_ERR_INVALID_ARG, "too many rows");
  return hip_status(kvd::launch_combine(shape->head_dim, part_o, part_m, part_l, (int)rows,
                                        num_splits, out, lse_out, (hipStream_t)stream),
                    "kv_decode_combine launch");
}

static kv_status check_cache(const kv_shape* shape, int32_t num_slots, int32_t sel_stride) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (num_slots < 1 || num_slots > kvd::kCacheMaxSlots)
    return fail(KV_ERR_INVALID_ARG, "num_slots=%d must be in [1, %d]", num_slots,
                kvd::kCacheMaxSlots);
  if (sel_stride < 1 || sel_stride > num_slots)
    return fail(KV_ERR_INVALID_ARG, "sel_stride=%d must be in [1, num_slots=%d]", sel_stride,
                num_slots);
  if ((long)shape->num_seqs * num_slots * shape->num_kv_heads > 0x7fffffffL)
    return fail(KV_ERR_INVALID_ARG, "num_seqs * num_slots * num_kv_heads must fit in int32");
  return KV_OK;
}

kv_status kv_cache_plan(const kv_shape* shape, int32_t num_slots, const int32_t* sel_blocks,
                        const int32_t* sel_count, int32_t sel_stride, int32_t* slot_block,
                        int32_t* block_slot, const float* slot_mass, int32_t* sel_slots,
                        int32_t* fetch_block, int32_t* fetch_slot, int32_t* fetch_count,
                        void* stream) {
  kv_status st = check_cache(shape, num_slots, sel_stride);
  if (st != KV_OK) return st;
  if (!sel_blocks || !sel_count || !slot_block || !block_slot || !slot_mass || !sel_slots ||
      !fetch_block || !fetch_slot || !fetch_count)
    return fail(KV_ERR_INVALID_ARG, "every array of kv_cache_plan is required");
  const void* ptrs[] = {sel_blocks, sel_count, slot_block, block_slot, slot_mass, sel_slots,
                        fetch_block, fetch_slot, fetch_count};
  for (const void* p : ptrs)
    if (!aligned(p, 4)) return fail(KV_ERR_ALIGNMENT, "cache arrays must be 4-byte aligned");
  return hip_status(kvd::launch_cache_plan(sel_blocks, sel_count, sel_stride, shape->num_seqs,
                                           shape->num_kv_heads, shape->max_blocks_per_seq,
                                           num_slots, slot_block, block_slot, slot_mass,
                                           sel_slots, fetch_block, fetch_slot, fetch_count,
                                           (hipStream_t)stream),
                    "kv_cache_plan launch");
}

kv_status kv_tier_plan(const kv_shape* shape, const int32_t* sel_blocks, const int32_t* sel_count,
                       int32_t sel_stride, const int32_t* block_table, const int32_t* seq_lens,
                       float decay, float hot_above, float cold_below, int32_t recent_tokens,
                       int32_t cooldown_steps, int32_t step, float* page_heat,
                       uint8_t* page_tier, int32_t* page_stamp, int32_t* demote,
                       int32_t* demote_count, int32_t* promote, int32_t* promote_count,
                       void* stream) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (shape->max_blocks_per_seq > kvd::kTierPlanMaxBlocks)
    return fail(KV_ERR_INVALID_ARG, "kv_tier_plan: max_blocks_per_seq=%d exceeds %d",
                shape->max_blocks_per_seq, kvd::kTierPlanMaxBlocks);
  if (sel_stride < 1 || (long)sel_stride * shape->num_kv_heads > (1L << 30))
    return fail(KV_ERR_INVALID_ARG,
                "sel_stride=%d must be >= 1, and sel_stride * num_kv_heads at most 2^30",
                sel_stride);
  if (!(decay >= 0.0f && decay <= 1.0f))
    return fail(KV_ERR_INVALID_ARG, "decay=%g must be in [0, 1]", (double)decay);
  if (hot_above != hot_above || cold_below != cold_below)
    return fail(KV_ERR_INVALID_ARG, "hot_above and cold_below must not be NaN");
  if (recent_tokens < 1)
    return fail(KV_ERR_INVALID_ARG,
                "recent_tokens=%d must be >= 1 (the page being appended to stays hot)",
                recent_tokens);
  if (cooldown_steps < 0)
    return fail(KV_ERR_INVALID_ARG, "cooldown_steps=%d must be >= 0", cooldown_steps);
  if (!sel_blocks || !sel_count || !block_table || !seq_lens || !page_heat || !page_tier ||
      !page_stamp || !demote || !demote_count || !promote || !promote_count)
    return fail(KV_ERR_INVALID_ARG, "every array of kv_tier_plan is required");
  const void* ptrs[] = {sel_blocks, sel_count, block_table, seq_lens, page_heat, page_stamp,
                        demote, demote_count, promote, promote_count};
  for (const void* p : ptrs)
    if (!aligned(p, 4))
      return fail(KV_ERR_ALIGNMENT, "kv_tier_plan: arrays other than page_tier must be 4-byte aligned");
  const kvd::TierPolicy pol{decay, hot_above, cold_below, recent_tokens, cooldown_steps};
  return hip_status(kvd::launch_tier_plan(sel_blocks, sel_count, sel_stride, block_table,
                                          seq_lens, shape->num_seqs, shape->num_kv_heads,
                                          shape->max_blocks_per_seq, shape->num_pages, pol, step,
                                          page_heat, page_tier, page_stamp, demote, demote_count,
                                          promote, promote_count, (hipStream_t)stream),
                    "kv_tier_plan launch");
}

}  // extern "C"

namespace {

// Delta fetch of tiles of tile_bytes (16-bit / fp32 pools, or code pools with
// their scales: kv_scales != nullptr).
kv_status fetch_common(const kv_shape* shape, int32_t num_slots, int tile_bytes,
                       const void* k_pool, const void* v_pool, const float* kv_scales,
                       const int32_t* block_table, const int32_t* fetch_block,
                       const int32_t* fetch_slot, const int32_t* fetch_count,
                       int32_t fetch_stride, void* cache_k, void* cache_v, float* cache_scales,
                       void* stream, const char* name) {
  if (!k_pool || !v_pool || !block_table || !fetch_block || !fetch_slot || !fetch_count ||
      !cache_k || !cache_v)
    return fail(KV_ERR_INVALID_ARG, "every array of %s is required", name);
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(cache_k, 16) ||
      !aligned(cache_v, 16))
    return fail(KV_ERR_ALIGNMENT, "the pools and the cache pools must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(fetch_block, 4) || !aligned(fetch_slot, 4) ||
      !aligned(fetch_count, 4))
    return fail(KV_ERR_ALIGNMENT, "integer arrays must be 4-byte aligned");
  return hip_status(kvd::launch_cache_fetch(tile_bytes, k_pool, v_pool, kv_scales, block_table,
                                            fetch_block, fetch_slot, fetch_count, fetch_stride,
                                            shape->num_seqs, shape->num_kv_heads,
                                            shape->max_blocks_per_seq, num_slots, cache_k,
                                            cache_v, cache_scales, (hipStream_t)stream),
                    name);
}

// Attention over the cached blocks: kvq 0 (16-bit / fp32 cache pools) or a
// code format with the cache's scales.
kv_status cached_attn_common(const kv_shape* shape, int32_t num_slots, int kvq, const void* q,
                             const void* cache_k, const void* cache_v, const float* cache_scales,
                             const int32_t* seq_lens, const int32_t* sel_blocks,
                             const int32_t* sel_count, const int32_t* sel_slots,
                             int32_t sel_stride, float scale, int32_t num_splits, float* part_o,
                             float* part_m, float* part_l, float* block_lse, void* stream,
                             const char* name, const int32_t* block_table = nullptr,
                             const kvd::FetchArgs* fetch = nullptr) {
  if (!sel_blocks || !sel_count || !sel_slots)
    return fail(KV_ERR_INVALID_ARG, "sel_blocks, sel_count and sel_slots are required");
  if (!aligned(sel_slots, 4) || (block_lse && !aligned(block_lse, 4)))
    return fail(KV_ERR_ALIGNMENT, "sel_slots and block_lse must be 4-byte aligned");
  if (num_splits < 1 || num_splits > 65535 * 4)
    return fail(KV_ERR_INVALID_ARG, "num_splits=%d must be in [1, 262140]", num_splits);
  if (!q || !cache_k || !cache_v || !seq_lens || !part_o || !part_m || !part_l)
    return fail(KV_ERR_INVALID_ARG, "q, cache_k, cache_v, seq_lens and partials are required");
  if (!(scale > 0.0f) || !(scale < INFINITY))
    return fail(KV_ERR_INVALID_ARG, "scale must be finite and positive");
  if (!aligned(q, 16) || !aligned(cache_k, 16) || !aligned(cache_v, 16) || !aligned(part_o, 16))
    return fail(KV_ERR_ALIGNMENT, "q, cache_k, cache_v and part_o must be 16-byte aligned");
  if (!aligned(seq_lens, 4) || !aligned(part_m, 4) || !aligned(part_l, 4) ||
      !aligned(sel_blocks, 4) || !aligned(sel_count, 4))
    return fail(KV_ERR_ALIGNMENT, "integer and partial arrays must be 4-byte aligned");
  // the cache pools hold num_seqs * num_slots pages and are device memory
  const int G = shape->num_q_heads / shape->num_kv_heads;
  return hip_status(
      kvd::launch_paged_attn(shape->dtype, shape->head_dim, G, kvq, q, cache_k, cache_v,
                             cache_scales, block_table, seq_lens, sel_blocks, sel_count,
                             sel_stride, sel_slots, num_slots, shape->num_seqs,
                             shape->num_q_heads, shape->num_kv_heads, shape->max_blocks_per_seq,
                             num_splits, scale, part_o, part_m, part_l, block_lse,
                             (hipStream_t)stream, 0, nullptr, nullptr, nullptr, fetch),
      name);
}

}  // namespace

extern "C" {

kv_status kv_cache_fetch(const kv_shape* shape, int32_t num_slots, const void* k_cache,
                         const void* v_cache, const int32_t* block_table,
                         const int32_t* fetch_block, const int32_t* fetch_slot,
                         const int32_t* fetch_count, int32_t fetch_stride, void* cache_k,
                         void* cache_v, void* stream) {
  kv_status st = check_cache(shape, num_slots, fetch_stride);
  if (st != KV_OK) return st;
  const int tile = shape->block_size * shape->head_dim * (shape->dtype == KV_F32 ? 4 : 2);
  return fetch_common(shape, num_slots, tile, k_cache, v_cache, nullptr, block_table,
                      fetch_block, fetch_slot, fetch_count, fetch_stride, cache_k, cache_v,
                      nullptr, stream, "kv_cache_fetch launch");
}

kv_status kv_cache_fetch_codes(const kv_shape* shape, int32_t num_slots, int32_t code_format,
                               const uint8_t* k_codes, const uint8_t* v_codes,
                               const float* kv_scales, const int32_t* block_table,
                               const int32_t* fetch_block, const int32_t* fetch_slot,
                               const int32_t* fetch_count, int32_t fetch_stride,
                               uint8_t* cache_k, uint8_t* cache_v, float* cache_scales,
                               void* stream) {
  kv_status st = check_cache(shape, num_slots, fetch_stride);
  if (st != KV_OK) return st;
  if ((st = check_code_format(shape, code_format)) != KV_OK) return st;
  if (!kv_scales || !cache_scales)
    return fail(KV_ERR_INVALID_ARG, "kv_scales and cache_scales are required");
  if (!aligned(kv_scales, 8) || !aligned(cache_scales, 8))
    return fail(KV_ERR_ALIGNMENT, "kv_scales and cache_scales must be 8-byte aligned");
  return fetch_common(shape, num_slots, code_tile_bytes(shape, code_format), k_codes, v_codes,
                      kv_scales, block_table, fetch_block, fetch_slot, fetch_count, fetch_stride,
                      cache_k, cache_v, cache_scales, stream, "kv_cache_fetch_codes launch");
}

kv_status kv_cached_decode_attn(const kv_shape* shape, int32_t num_slots, const void* q,
                                const void* cache_k, const void* cache_v,
                                const int32_t* seq_lens, const int32_t* sel_blocks,
                                const int32_t* sel_count, const int32_t* sel_slots,
                                int32_t sel_stride, float scale, int32_t num_splits,
                                float* part_o, float* part_m, float* part_l, float* block_lse,
                                void* stream) {
  kv_status st = check_cache(shape, num_slots, sel_stride);
  if (st != KV_OK) return st;
  return cached_attn_common(shape, num_slots, 0, q, cache_k, cache_v, nullptr, seq_lens,
                            sel_blocks, sel_count, sel_slots, sel_stride, scale, num_splits,
                            part_o, part_m, part_l, block_lse, stream,
                            "kv_cached_decode_attn launch");
}

kv_status kv_cached_decode_attn_codes(const kv_shape* shape, int32_t num_slots,
                                      int32_t code_format, const void* q, const uint8_t* cache_k,
                                      const uint8_t* cache_v, const float* cache_scales,
                                      const int32_t* seq_lens, const int32_t* sel_blocks,
                                      const int32_t* sel_count, const int32_t* sel_slots,
                                      int32_t sel_stride, float scale, int32_t num_splits,
                                      float* part_o, float* part_m, float* part_l,
                                      float* block_lse, void* stream) {
  kv_status st = check_cache(shape, num_slots, sel_stride);
  if (st != KV_OK) return st;
  if ((st = check_code_format(shape, code_format)) != KV_OK) return st;
  if (!cache_scales) return fail(KV_ERR_INVALID_ARG, "cache_scales is required");
  if (!aligned(cache_scales, 8))
    return fail(KV_ERR_ALIGNMENT, "cache_scales must be 8-byte aligned");
  return cached_attn_common(shape, num_slots, code_format, q, cache_k, cache_v, cache_scales,
                            seq_lens, sel_blocks, sel_count, sel_slots, sel_stride, scale,
                            num_splits, part_o, part_m, part_l, block_lse, stream,
                            "kv_cached_decode_attn_codes launch");
}

}  // extern "C"

namespace {
// Arguments of the fused fetch shared by both entry points.
kv_status check_fetch(const void* k_pool, const void* v_pool, const int32_t* block_table,
                      const int32_t* fetch_slot, const int32_t* fetch_count) {
  if (!k_pool || !v_pool || !block_table || !fetch_slot || !fetch_count)
    return fail(KV_ERR_INVALID_ARG, "the pools, block_table, fetch_slot and fetch_count are required");
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16))
    return fail(KV_ERR_ALIGNMENT, "the pools must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(fetch_slot, 4) || !aligned(fetch_count, 4))
    return fail(KV_ERR_ALIGNMENT, "integer arrays must be 4-byte aligned");
  return KV_OK;
}
}  // namespace

extern "C" {

kv_status kv_cached_decode_attn_fetch(const kv_shape* shape, int32_t num_slots, const void* q,
                                      const void* k_pool, const void* v_pool,
                                      const int32_t* block_table, const int32_t* fetch_slot,
                                      const int32_t* fetch_count, void* cache_k, void* cache_v,
                                      const int32_t* seq_lens, const int32_t* sel_blocks,
                                      const int32_t* sel_count, const int32_t* sel_slots,
                                      int32_t sel_stride, float scale, int32_t num_splits,
                                      float* part_o, float* part_m, float* part_l,
                                      float* block_lse, void* stream) {
  kv_status st = check_cache(shape, num_slots, sel_stride);
  if (st != KV_OK) return st;
  if ((st = check_fetch(k_pool, v_pool, block_table, fetch_slot, fetch_count)) != KV_OK) return st;
  const kvd::FetchArgs fa{k_pool, v_pool, nullptr, nullptr, fetch_slot, fetch_count};
  return cached_attn_common(shape, num_slots, 0, q, cache_k, cache_v, nullptr, seq_lens,
                            sel_blocks, sel_count, sel_slots, sel_stride, scale, num_splits,
                            part_o, part_m, part_l, block_lse, stream,
                            "kv_cached_decode_attn_fetch launch", block_table, &fa);
}

kv_status kv_cached_decode_attn_fetch_codes(
    const kv_shape* shape, int32_t num_slots, int32_t code_format, const void* q,
    const uint8_t* k_codes, const uint8_t* v_codes, const float* kv_scales,
    const int32_t* block_table, const int32_t* fetch_slot, const int32_t* fetch_count,
    uint8_t* cache_k, uint8_t* cache_v, float* cache_scales, const int32_t* seq_lens,
    const int32_t* sel_blocks, const int32_t* sel_count, const int32_t* sel_slots,
    int32_t sel_stride, float scale, int32_t num_splits, float* part_o, float* part_m,
    float* part_l, float* block_lse, void* stream) {
  kv_status st = check_cache(shape, num_slots, sel_stride);
  if (st != KV_OK) return st;
  if ((st = check_code_format(shape, code_format)) != KV_OK) return st;
  if ((st = check_fetch(k_codes, v_codes, block_table, fetch_slot, fetch_count)) != KV_OK)
    return st;
  if (!kv_scales || !cache_scales)
    return fail(KV_ERR_INVALID_ARG, "kv_scales and cache_scales are required");
  if (!aligned(kv_scales, 8) || !aligned(cache_scales, 8))
    return fail(KV_ERR_ALIGNMENT, "kv_scales and cache_scales must be 8-byte aligned");
  const kvd::FetchArgs fa{k_codes, v_codes, kv_scales, cache_scales, fetch_slot, fetch_count};
  return cached_attn_common(shape, num_slots, code_format, q, cache_k, cache_v, cache_scales,
                            seq_lens, sel_blocks, sel_count, sel_slots, sel_stride, scale,
                            num_splits, part_o, part_m, part_l, block_lse, stream,
                            "kv_cached_decode_attn_fetch_codes launch", block_table, &fa);
}

kv_status kv_cache_slot_mass(const kv_shape* shape, int32_t num_slots, const float* block_lse,
                             const float* lse, const int32_t* sel_count,
                             const int32_t* sel_slots, int32_t sel_stride, float* slot_mass,
                             void* stream) {
  kv_status st = check_cache(shape, num_slots, sel_stride);
  if (st != KV_OK) return st;
  if (!block_lse || !lse || !sel_count || !sel_slots || !slot_mass)
    return fail(KV_ERR_INVALID_ARG, "every array of kv_cache_slot_mass is required");
  const void* ptrs[] = {block_lse, lse, sel_count, sel_slots, slot_mass};
  for (const void* p : ptrs)
    if (!aligned(p, 4)) return fail(KV_ERR_ALIGNMENT, "arrays must be 4-byte aligned");
  return hip_status(kvd::launch_slot_mass(block_lse, lse, sel_count, sel_slots, sel_stride,
                                          shape->num_seqs, shape->num_q_heads,
                                          shape->num_kv_heads, num_slots, slot_mass,
                                          (hipStream_t)stream),
                    "kv_cache_slot_mass launch");
}

kv_status kv_check_tables(const kv_shape* shape, const int32_t* block_table,
                          const int32_t* seq_lens, const int32_t* sel_blocks,
                          const int32_t* sel_count, int32_t sel_stride, uint32_t* result,
                          void* stream) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (!block_table || !seq_lens || !result)
    return fail(KV_ERR_INVALID_ARG, "block_table, seq_lens and result are required");
  if ((sel_blocks == nullptr) != (sel_count == nullptr))
    return fail(KV_ERR_INVALID_ARG, "sel_blocks and sel_count go together");
  if (sel_blocks && sel_stride < 1)
    return fail(KV_ERR_INVALID_ARG, "sel_stride=%d must be >= 1", sel_stride);
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(result, 4) ||
      (sel_blocks && (!aligned(sel_blocks, 4) || !aligned(sel_count, 4))))
    return fail(KV_ERR_ALIGNMENT, "the tables and result must be 4-byte aligned");
  return hip_status(kvd::launch_check_tables(block_table, seq_lens, sel_blocks, sel_count,
                                             sel_blocks ? sel_stride : 0, shape->num_seqs,
                                             shape->num_kv_heads, shape->max_blocks_per_seq,
                                             shape->num_pages, result, (hipStream_t)stream),
                    "kv_check_tables launch");
}

kv_status kv_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return fail(KV_ERR_INVALID_ARG, "buf and sink are required");
  if (bytes == 0 || bytes % 16) return fail(KV_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if (!aligned(buf, 16) || !aligned(sink, 4))
    return fail(KV_ERR_ALIGNMENT, "buf must be 16-byte aligned, sink 4-byte aligned");
  return hip_status(kvd::launch_stream_read(buf, bytes, sink, kvd::kProbeSinkWords,
                                            (hipStream_t)stream),
                    "kv_probe_stream_read launch");
}

kv_status kv_probe_gather_read(const kv_shape* shape, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* seq_lens,
                               int32_t num_splits, uint32_t* sink, void* stream) {
  kv_status st = check_shape(shape);
  if (st != KV_OK) return st;
  if (shape->dtype == KV_F32) return fail(KV_ERR_UNSUPPORTED, "the gather probe models 16-bit pools");
  if (num_splits < 1 || num_splits > 65535 * 2)
    return fail(KV_ERR_INVALID_ARG, "num_splits=%d out of range", num_splits);
  if (!k_cache || !v_cache || !block_table || !seq_lens || !sink)
    return fail(KV_ERR_INVALID_ARG, "every array of kv_probe_gather_read is required");
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_table, 4) ||
      !aligned(seq_lens, 4) || !aligned(sink, 4))
    return fail(KV_ERR_ALIGNMENT, "pools 16-byte aligned, integer arrays 4-byte aligned");
  return hip_status(kvd::launch_gather_read(shape->dtype, shape->head_dim, k_cache, v_cache,
                                            block_table, seq_lens, shape->num_seqs,
                                            shape->num_kv_heads, shape->max_blocks_per_seq,
                                            num_splits, sink, (hipStream_t)stream),
                    "kv_probe_gather_read launch");
}

kv_status kv_probe_fp8_convert(uint64_t* counts, uint32_t* first, void* stream) {
  if (!counts || !first) return fail(KV_ERR_INVALID_ARG, "counts and first are required");
  if (!aligned(counts, 8) || !aligned(first, 4))
    return fail(KV_ERR_ALIGNMENT, "counts must be 8-byte aligned, first 4-byte aligned");
  return hip_status(kvd::launch_fp8_convert(reinterpret_cast<unsigned long long*>(counts), first,
                                            (hipStream_t)stream),
                    "kv_probe_fp8_convert launch");
}

kv_status kv_host_alloc(size_t bytes, uint32_t flags, void** host_ptr, void** dev_ptr) {
  if (!host_ptr || !dev_ptr) return fail(KV_ERR_INVALID_ARG, "host_ptr and dev_ptr are required");
  *host_ptr = nullptr;
  *dev_ptr = nullptr;
  if (bytes == 0) return fail(KV_ERR_INVALID_ARG, "bytes must be > 0");
  if (flags & ~KV_HOST_NONCOHERENT) return fail(KV_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  unsigned hf = hipHostMallocMapped;
  hf |= (flags & KV_HOST_NONCOHERENT) ? hipHostMallocNonCoherent : hipHostMallocCoherent;
  void* h = nullptr;
  hipError_t e = hipHostMalloc(&h, bytes, hf);
  if (e != hipSuccess) return hip_status(e, "kv_host_alloc hipHostMalloc");
  void* d = nullptr;
  e = hipHostGetDevicePointer(&d, h, 0);
  if (e != hipSuccess) {
    (void)hipHostFree(h);
    return hip_status(e, "kv_host_alloc hipHostGetDevicePointer");
  }
  *host_ptr = h;
  *dev_ptr = d;
  return ok();
}

kv_status kv_host_free(void* host_ptr) {
  if (!host_ptr) return ok();
  return hip_status(hipHostFree(host_ptr), "kv_host_free");
}

}  // extern "C"

// Internal launchers: one per kernel family, dispatching on (dtype, head_dim,
// group size) to the template instances.  Shapes are validated by the C ABI
// layer before these run; the launchers only size grids.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>


namespace kvd {

hipError_t launch_block_meta(int dtype, int D, const void* k_cache, const int32_t* page_ids,
                             const int32_t* valid_tokens, int n_ids, int Hkv, void* kmeta,
                             hipStream_t stream);

hipError_t launch_block_mean(int dtype, int D, const void* k_cache, const int32_t* page_ids,
                             const int32_t* valid_tokens, int n_ids, int Hkv, float* kmean,
                             hipStream_t stream);

hipError_t launch_append_token(int dtype, int D, const void* k_new, const void* v_new,
                               const int32_t* block_table, const int32_t* seq_lens, int B,
                               int Hkv, int maxN, void* k_cache, void* v_cache, void* kmeta,
                               float* kmean, hipStream_t stream);

// index_kind: 0 = channel min/max rows in the K dtype, 1 = fp32 mean rows
hipError_t launch_block_score(int dtype, int D, int G, int index_kind, const void* q,
                              const void* index, const int32_t* block_table,
                              const int32_t* seq_lens, int B, int Hq, int Hkv, int maxN,
                              float* scores, hipStream_t stream, const void* k_new = nullptr,
                              const void* v_new = nullptr, void* k_cache = nullptr,
                              void* v_cache = nullptr, void* kmeta = nullptr,
                              float* kmean = nullptr);

// cand (nullable): candidate storage of topk_candidate_bytes(B, Hkv, maxN, K)
// bytes; with it, rows longer than kTopkTwoLevelMin blocks take the two-level
// select where topk_candidates_per_row allows (the same lists either way).
hipError_t launch_topk(const float* scores, const int32_t* seq_lens, int B, int Hkv, int maxN,
                       int K, int sink, int local, int32_t* sel, int32_t* sel_count,
                       hipStream_t stream, void* cand = nullptr);

// kv_scales == nullptr: K/V pools in `dtype`; otherwise E4M3 code pools with
// fp32 (k, v) scales per (page, KV head)
// sel_slots (with sel): the list's blocks live in cache page b*num_slots + slot;
// block_lse (with sel, nullable): ln of each list block's summed exp-logits per query head
// kvq: 0 = pools of the storage dtype, 8 = FP8 E4M3 code pools, 4 = INT4 code
// pools (16-bit dtypes); code pools need kv_scales.  cold = 8 / 4 (with kvq 0):
// tiered pools, page p read from k_cold / v_cold in that format when
// page_tier[p] != 0 (16-bit dtypes, G >= 2)
// The step's delta fetch inside a cached attention launch: the list positions
// whose cache slot is among fetch_slot[b, j, 0 .. fetch_count[b, j]) (rows of
// sel_stride) read their block from the pools (page block_table[b, n]) instead
// of the cache, and store it into that slot; with code pools the pools' scale
// pair of the block goes to cache_scales too.
struct FetchArgs {
  const void* k_pool;
  const void* v_pool;
  const float* pool_scales;
  float* cache_scales;
  const int32_t* fetch_slot;
  const int32_t* fetch_count;
};

// part_stride: splits per row of the partial arrays (0: S).  With part_o,
// part_m and part_l offset by s0 columns, a launch fills columns
// [s0, s0 + S) of a wider partial set that one merge reads whole.
hipError_t launch_paged_attn(int dtype, int D, int G, int kvq, const void* q,
                             const void* k_cache, const void* v_cache, const float* kv_scales,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* sel, const int32_t* sel_count, int sel_stride,
                             const int32_t* sel_slots, int num_slots, int B, int Hq, int Hkv,
                             int maxN, int S, float scale, float* part_o, float* part_m,
                             float* part_l, float* block_lse, hipStream_t stream, int cold = 0,
                             const void* k_cold = nullptr, const void* v_cold = nullptr,
                             const uint8_t* page_tier = nullptr, const FetchArgs* fetch = nullptr,
                             int part_stride = 0);

// Per (sequence, KV head): the list (sel, or every block of the sequence when
// sel is null) split by page tier into the hot (tier 0) and cold lists, both
// in list order, rows of out_stride entries.  Scratch: flags (B * Hkv rows of
// out_stride bytes, rounded up to whole chunks) and chunk_cold (B * Hkv rows
// of tier_chunks(out_stride) ints).
constexpr int kTierChunkPositions = 1024;
inline int tier_chunks(int out_stride) {
  return (out_stride + kTierChunkPositions - 1) / kTierChunkPositions;
}
hipError_t launch_tier_lists(const int32_t* sel, const int32_t* sel_count, int sel_stride,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const uint8_t* page_tier, int B, int Hkv, int maxN, int out_stride,
                             int32_t* hot, int32_t* hot_count, int32_t* cold, int32_t* cold_count,
                             uint8_t* flags, int32_t* chunk_cold, hipStream_t stream);

// Hot/cold tier policy of kv_tier_plan.
struct TierPolicy {
  float decay, hot_above, cold_below;
  int recent, cooldown;
};
constexpr int kTierPlanMaxBlocks = 1 << 18;       // blocks per sequence (64 passes of the list compaction)

hipError_t launch_tier_plan(const int32_t* sel, const int32_t* sel_count, int sel_stride,
                            const int32_t* block_table, const int32_t* seq_lens, int B, int Hkv,
                            int maxN, int num_pages, const TierPolicy& pol, int step, float* heat,
                            uint8_t* tier, int32_t* stamp, int32_t* demote, int32_t* demote_count,
                            int32_t* promote, int32_t* promote_count, hipStream_t stream);

hipError_t launch_cache_plan(const int32_t* sel, const int32_t* sel_count, int sel_stride, int B,
                             int Hkv, int maxN, int C, int32_t* slot_block, int32_t* block_slot,
                             const float* slot_mass, int32_t* sel_slots, int32_t* fetch_block,
                             int32_t* fetch_slot, int32_t* fetch_count, hipStream_t stream);

// tile_bytes: one (page, KV head) tile of the pools (512 .. 8192); with
// kv_scales (code pools) each fetched tile's scale pair goes to cache_scales.
hipError_t launch_cache_fetch(int tile_bytes, const void* k_pool, const void* v_pool,
                              const float* kv_scales, const int32_t* block_table,
                              const int32_t* fetch_block, const int32_t* fetch_slot,
                              const int32_t* fetch_count, int fetch_stride, int B, int Hkv,
                              int maxN, int C, void* cache_k, void* cache_v, float* cache_scales,
                              hipStream_t stream);

hipError_t launch_slot_mass(const float* block_lse, const float* lse, const int32_t* sel_count,
                            const int32_t* sel_slots, int sel_stride, int B, int Hq, int Hkv,
                            int C, float* slot_mass, hipStream_t stream);

// Result bits of the table check (one word per sequence).
constexpr uint32_t kCheckBadSeqLen = 0x1u, kCheckBadPageId = 0x2u, kCheckBadSelCount = 0x4u,
                   kCheckBadSelBlock = 0x8u;

hipError_t launch_check_tables(const int32_t* block_table, const int32_t* seq_lens,
                               const int32_t* sel, const int32_t* sel_count, int sel_stride,
                               int B, int Hkv, int maxN, int num_pages, uint32_t* result,
                               hipStream_t stream);

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int sink_words,
                              hipStream_t stream);

hipError_t launch_gather_read(int dtype, int D, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, int B, int Hkv,
                              int maxN, int S, uint32_t* sink, hipStream_t stream);

// Words of the stream-read probe's sink (one per workgroup).
constexpr int kProbeSinkWords = 4096;

// Classes of kv_probe_fp8_convert's counts; the launch writes them all.
constexpr int kProbeFp8Classes = 4;
hipError_t launch_fp8_convert(unsigned long long* counts, uint32_t* first, hipStream_t stream);

// Largest cache (slots per sequence and KV head) the plan kernel holds.
constexpr int kCacheMaxSlots = 8192;

// fmt 8: FP8 E4M3 pages; fmt 4: INT4 pages (16-bit sources only)
hipError_t launch_quantize(int fmt, int dtype, int D, const void* k_cache, const void* v_cache,
                           const int32_t* page_ids, const int32_t* valid_tokens, int n_ids,
                           int Hkv, uint8_t* k8, uint8_t* v8, float* scales, hipStream_t stream);

hipError_t launch_combine(int D, const float* part_o, const float* part_m, const float* part_l,
                          int rows, int S, float* out, float* lse, hipStream_t stream);

// Compute units of the current device (queried once).
inline int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
  }
  return n;
}

inline int device_cu_count() { return cu_count(); }

// Largest maxN of the Top-K (1024 threads x 64 keys; past 32 keys per thread
// the keys live in LDS).
constexpr int kTopkMaxBlocks = 65536;

// Two-level select of long rows: each chunk of kTopkChunk blocks passes its
// forced blocks and its best K competing blocks (the candidates, in ascending
// block order), and a second launch selects among a row's candidates.  It is
// used for rows longer than kTopkTwoLevelMin blocks while a row's candidate
// slots (chunks x 2K, enough for K + the forced blocks the host check allows)
// stay within kTopkMaxCandidates.
#ifndef KVD_TOPK_CHUNK_THREADS
#define KVD_TOPK_CHUNK_THREADS 1024   // threads of a chunk's workgroup
#endif
#ifndef KVD_TOPK_CHUNK
#define KVD_TOPK_CHUNK 4096           // blocks per chunk
#endif
constexpr int kTopkChunk = KVD_TOPK_CHUNK;
constexpr int kTopkTwoLevelMin = 16384;
constexpr int kTopkMaxCandidates = 16384;
inline int topk_candidates_per_row(int maxN, int K) {
  if (maxN <= kTopkTwoLevelMin || K < 1) return 0;
  const long slots = (long)((maxN + kTopkChunk - 1) / kTopkChunk) * 2 * K;
  return slots <= kTopkMaxCandidates ? (int)slots : 0;
}
inline size_t topk_candidate_bytes(int B, int Hkv, int maxN, int K) {
  return (size_t)B * Hkv * topk_candidates_per_row(maxN, K) * 8;   // uint32 key + int32 block
}

// Top-K + sparse attention in one launch: waves (= splits) per workgroup, the
// list positions a workgroup keeps in LDS, and the longest row it takes (every
// workgroup of a row repeats the row's Top-K; past 2048 blocks that costs more
// than the Top-K launch it saves).
#ifndef KVD_SEL_ATTN_WAVES
#define KVD_SEL_ATTN_WAVES 4   // a multiple of 4 (the row select's scans)
#endif
constexpr int kSelAttnWaves = KVD_SEL_ATTN_WAVES;
constexpr int kSelAttnListMax = 2048;
constexpr int kSelAttnMaxBlocks = 2048;

// Whether launch_select_attn takes this call (16-bit keys, G >= 2, maxN <=
// kSelAttnMaxBlocks, the workgroup's share of the list fits in LDS); other
// calls run the Top-K and attention launches, with the same results.
bool select_attn_fusable(int dtype, int G, int maxN, int K, int S);

hipError_t launch_select_attn(int dtype, int D, int G, const float* scores, int K, int sink,
                              int local, int32_t* sel, int32_t* sel_count, const void* q,
                              const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, int B, int Hq,
                              int Hkv, int maxN, int S, float scale, float* part_o, float* part_m,
                              float* part_l, hipStream_t stream);


}  // namespace kvd

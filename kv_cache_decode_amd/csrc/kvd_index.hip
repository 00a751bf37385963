// gfx950 kernels that build and query the block index of the paged KV cache.
//
//   block_meta_kernel   channel-wise min/max key per (page, KV head)      KVDrive §2.2, §2.3
//   block_mean_kernel   mean key per (page, KV head)                      KVDrive §2.3, §4
//   append_token_kernel store a decode token's K/V and refresh its page's index rows
//   block_score_kernel  Quest (or mean-key) score per logical block, max over
//                       the GQA group                                     KVDrive §2.2, §2.3
//   topk_kernel         exact Top-K of the block scores, ascending output, with
//                       the blocks of the first / last tokens forced in    KVDrive §9.1
//
// All three are HBM- or latency-bound; rows of D channels move as coalesced
// 16-byte chunks (RowGeom in kvd_device.hpp).
#include <math.h>

#include "kvd_device.hpp"
#include "kvd_dispatch.hpp"
#include "kvd_launch.hpp"
#include "kvd_topk.hpp"

// Launch-shape knobs (build macros): most workgroups per compute unit of the
// meta build (the grid strides over wave steps beyond that); 16-byte steps per
// wave of the scorer.
#ifndef KVD_META_WGS_PER_CU
#define KVD_META_WGS_PER_CU 16
#endif
#ifndef KVD_META_WAVES
#define KVD_META_WAVES 4
#endif
#ifndef KVD_SCORE_STEPS
#define KVD_SCORE_STEPS 2
#endif
#ifndef KVD_SCORE_WAVES
#define KVD_SCORE_WAVES 4
#endif
// waves per workgroup of the matrix-core scorer (16 blocks per wave)
#ifndef KVD_SCORE_MFMA_WAVES
#define KVD_SCORE_MFMA_WAVES 4
#endif

namespace kvd {

// ============================================================== block meta
//
// Lane (us, c) of a wave owns channel chunk c (E channels, 16 bytes) of unit
// slot us: a wave step covers UPS = 64 / LPR consecutive (page, KV head) units
// u = i*Hkv + j (i indexes page_ids).  Each lane walks the 16 token rows of
// its unit with one 16-byte load per row -- a load instruction reads UPS full
// row segments of D*eb bytes -- and keeps the running min and max of its
// chunk in registers, so no cross-lane reduction is needed.  It then writes
// its chunk of the min row and of the max row.  min/max of representable
// values is exact, so the narrowing back to the storage dtype is exact too.
// Wave steps are spread grid-stride; with page_ids in ascending order a step
// reads UPS*16*D*eb contiguous bytes.

template <typename DT, int D, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void block_meta_kernel(
    const void* __restrict__ k_cache, const int32_t* __restrict__ page_ids,
    const int32_t* __restrict__ valid_tokens, int n_ids, int Hkv, void* __restrict__ kmeta) {
  using G_ = RowGeom<DT, D>;
  using St = typename DT::storage;
  constexpr int E = G_::E, LPR = G_::LPR;
  constexpr int UPS = kWave / LPR;  // units per wave step
  const int lane = threadIdx.x & (kWave - 1);
  const int us = lane / LPR, c = lane % LPR;
  const long units = (long)n_ids * Hkv;
  const long steps = (units + UPS - 1) / UPS;
  const long nwaves = (long)gridDim.x * WAVES;

  for (long step = (long)blockIdx.x * WAVES + (threadIdx.x >> 6); step < steps; step += nwaves) {
    const long u = step * UPS + us;
    if (u >= units) continue;                      // tail lanes of the last step
    const int i = (int)(u / Hkv);
    const int j = (int)(u - (long)i * Hkv);
    const size_t tile = (size_t)page_ids[i] * Hkv + j;
    const int nv = valid_tokens[i];
    const St* src = static_cast<const St*>(k_cache) + tile * kBlockSize * D + (size_t)c * E;
    uint4 w[kBlockSize];
#pragma unroll
    for (int t = 0; t < kBlockSize; ++t) w[t] = load16_stream(src + (size_t)t * D);
    float mn[E], mx[E];
    DT::widen(w[0], mn);                           // slot 0 is always valid
#pragma unroll
    for (int e = 0; e < E; ++e) mx[e] = mn[e];
#pragma unroll
    for (int t = 1; t < kBlockSize; ++t) {
      if (t < nv) {
        float f[E];
        DT::widen(w[t], f);
#pragma unroll
        for (int e = 0; e < E; ++e) { mn[e] = fminf(mn[e], f[e]); mx[e] = fmaxf(mx[e], f[e]); }
      }
    }
    St* dst = static_cast<St*>(kmeta) + tile * 2 * D + (size_t)c * E;
    store16(dst, DT::narrow_exact(mn));
    store16(dst + D, DT::narrow_exact(mx));
  }
}

// ============================================================== block mean
//
// Same lane layout and wave steps as the meta build.  Each lane sums its chunk
// of the valid token rows in fp64, in slot order, divides by the valid count
// in fp64 and rounds once to fp32: for fp16 / bf16 keys (and fp32 keys whose
// exponents lie within 29 binades of each other) the fp64 sum is exact, so the
// stored row is the exact mean rounded to nearest fp32.

template <int E>
__device__ inline void store_f32_chunk(float* dst, const float (&v)[E]) {
#pragma unroll
  for (int i = 0; i < E; i += 4)
    store16(dst + i, make_uint4(__float_as_uint(v[i]), __float_as_uint(v[i + 1]),
                                __float_as_uint(v[i + 2]), __float_as_uint(v[i + 3])));
}

template <typename DT, int D, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void block_mean_kernel(
    const void* __restrict__ k_cache, const int32_t* __restrict__ page_ids,
    const int32_t* __restrict__ valid_tokens, int n_ids, int Hkv, float* __restrict__ kmean) {
  using G_ = RowGeom<DT, D>;
  using St = typename DT::storage;
  constexpr int E = G_::E, LPR = G_::LPR;
  constexpr int UPS = kWave / LPR;
  const int lane = threadIdx.x & (kWave - 1);
  const int us = lane / LPR, c = lane % LPR;
  const long units = (long)n_ids * Hkv;
  const long steps = (units + UPS - 1) / UPS;
  const long nwaves = (long)gridDim.x * WAVES;

  for (long step = (long)blockIdx.x * WAVES + (threadIdx.x >> 6); step < steps; step += nwaves) {
    const long u = step * UPS + us;
    if (u >= units) continue;
    const int i = (int)(u / Hkv);
    const int j = (int)(u - (long)i * Hkv);
    const size_t tile = (size_t)page_ids[i] * Hkv + j;
    const int nv = valid_tokens[i];
    const St* src = static_cast<const St*>(k_cache) + tile * kBlockSize * D + (size_t)c * E;
    uint4 w[kBlockSize];
#pragma unroll
    for (int t = 0; t < kBlockSize; ++t) w[t] = load16_stream(src + (size_t)t * D);
    double acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0;
#pragma unroll
    for (int t = 0; t < kBlockSize; ++t) {
      if (t < nv) {
        float f[E];
        DT::widen(w[t], f);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += (double)f[e];
      }
    }
    float m[E];
#pragma unroll
    for (int e = 0; e < E; ++e) m[e] = (float)(acc[e] / (double)nv);
    store_f32_chunk<E>(kmean + tile * D + (size_t)c * E, m);
  }
}

// ============================================================== decode-step append
//
// One wave per (sequence, KV head); lane c < LPR owns channel chunk c
// (append_lane, shared with the fused append + select kernel).  The new key
// and value rows are stored into their slot, and the key is folded into the
// page's min/max rows (a fresh page, slot 0, starts them over).  The page's
// mean row is recomputed from slots 0..s with the mean build's exact
// arithmetic (fp64 sum in slot order, one rounding), so it equals a rebuild.
// The lane returns its chunk of the updated rows.

template <typename DT, int D, int E = RowGeom<DT, D>::E>
__device__ inline void append_lane(const void* __restrict__ k_new, const void* __restrict__ v_new,
                                   const int32_t* __restrict__ block_table,
                                   const int32_t* __restrict__ seq_lens, int Hkv, int maxN, int j,
                                   int b, int c, void* __restrict__ k_cache,
                                   void* __restrict__ v_cache, void* __restrict__ kmeta,
                                   float* __restrict__ kmean, float (&mn)[E], float (&mx)[E],
                                   float (&mv)[E]) {
  using St = typename DT::storage;
  const int t = seq_lens[b] - 1;
  const int s = t % kBlockSize;
  const size_t tile = (size_t)block_table[(size_t)b * maxN + t / kBlockSize] * Hkv + j;
  const size_t src = ((size_t)b * Hkv + j) * D + (size_t)c * E;
  const size_t dst = (tile * kBlockSize + s) * D + (size_t)c * E;
  const uint4 kw = load16(static_cast<const St*>(k_new) + src);
  store16(static_cast<St*>(k_cache) + dst, kw);
  store16(static_cast<St*>(v_cache) + dst, load16(static_cast<const St*>(v_new) + src));
  if (kmeta) {
    St* m = static_cast<St*>(kmeta) + tile * 2 * D + (size_t)c * E;
    if (s == 0) {
      store16(m, kw);
      store16(m + D, kw);
      DT::widen(kw, mn);
#pragma unroll
      for (int e = 0; e < E; ++e) mx[e] = mn[e];
    } else {
      float f[E];
      DT::widen(kw, f);
      DT::widen(load16(m), mn);
      DT::widen(load16(m + D), mx);
#pragma unroll
      for (int e = 0; e < E; ++e) { mn[e] = fminf(mn[e], f[e]); mx[e] = fmaxf(mx[e], f[e]); }
      store16(m, DT::narrow_exact(mn));
      store16(m + D, DT::narrow_exact(mx));
    }
  }
  if (kmean) {
    // slots before s come from the cache (this lane wrote none of them), slot s
    // is the new key; rows are loaded half a page at a time (rows past s unused)
    // and summed in slot order
    const St* rows = static_cast<const St*>(k_cache) + tile * kBlockSize * D + (size_t)c * E;
    double acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0;
    constexpr int kHalf = kBlockSize / 2;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 w[kHalf];
#pragma unroll
      for (int r = 0; r < kHalf; ++r) {
        const int t = h * kHalf + r;
        w[r] = (t < s) ? load16(rows + (size_t)t * D) : kw;
      }
#pragma unroll
      for (int r = 0; r < kHalf; ++r) {
        if (h * kHalf + r <= s) {
          float f[E];
          DT::widen(w[r], f);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] += (double)f[e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) mv[e] = (float)(acc[e] / (double)(s + 1));
    store_f32_chunk<E>(kmean + tile * D + (size_t)c * E, mv);
  }
}

template <typename DT, int D>
__global__ __launch_bounds__(kWave) void append_token_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int Hkv,
    int maxN, void* __restrict__ k_cache, void* __restrict__ v_cache, void* __restrict__ kmeta,
    float* __restrict__ kmean) {
  constexpr int E = RowGeom<DT, D>::E, LPR = RowGeom<DT, D>::LPR;
  const int c = threadIdx.x;
  if (c >= LPR) return;
  float mn[E], mx[E], mv[E];
  append_lane<DT, D>(k_new, v_new, block_table, seq_lens, Hkv, maxN, blockIdx.x, blockIdx.y, c,
                     k_cache, v_cache, kmeta, kmean, mn, mx, mv);
}

// ============================================================== block score
//
// sigma_h = sum_c max(q_hc kmin_c, q_hc kmax_c) = sum_c (q+_hc kmax_c + q-_hc kmin_c)
// with q+ = max(q, 0), q- = min(q, 0): for each channel one of the two products
// is an exact zero, so the fused multiply-adds accumulate exactly the max term.
// With the mean-key index (IDX = kIndexMean) the score is q_h . kmean, the
// fp32 mean row read as E floats per lane.
// A wave owns STEPS * TPI consecutive logical blocks of one (sequence, KV
// head); lane (rg, c) handles channels [c*E, c*E+E) of block n0 + step*TPI + rg.
// All index loads of the wave are issued before any arithmetic.

constexpr int kIndexMinMax = 0, kIndexMean = 1;

// Where the scorer's append workgroups store the new token (kernel argument).
struct AppendArgs {
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  void* kmeta;
  float* kmean;
};

// One lane's query chunk as the score uses it: q+ and q- for min/max, q and 0
// for the mean index.
template <int E, int IDX>
__device__ inline void split_query(const float (&f)[E], float (&qp)[E], float (&qn)[E]) {
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if constexpr (IDX == kIndexMinMax) {
      qp[e] = fmaxf(f[e], 0.0f);
      qn[e] = fminf(f[e], 0.0f);
    } else {
      qp[e] = f[e];
      qn[e] = 0.0f;
    }
  }
}

// One head's block score from the LPR lanes of an aligned lane group, lane c
// holding channels [c*E, c*E+E): ka / kb are the kmin / kmax chunks (ka the
// mean chunk for the mean index).  Every lane of the wave must take part; each
// lane of the group ends with the group's sum.
template <int E, int LPR, int IDX>
__device__ inline float head_score_lane(const float (&qp)[E], const float (&qn)[E],
                                        const float (&ka)[E], const float (&kb)[E]) {
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if constexpr (IDX == kIndexMinMax) {
      acc = fmaf(qp[e], kb[e], acc);
      acc = fmaf(qn[e], ka[e], acc);
    } else {
      acc = fmaf(qp[e], ka[e], acc);
    }
  }
  return group_reduce<LPR, OpSum>(acc);
}

template <typename DT, int D, int G, int WAVES, int STEPS, int IDX, bool APPEND>
__global__ __launch_bounds__(WAVES * kWave) void block_score_kernel(
    const void* __restrict__ q, const void* __restrict__ kmeta,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int Hq,
    int Hkv, int maxN, float* __restrict__ scores, AppendArgs ap) {
  using G_ = RowGeom<DT, D>;
  using St = typename DT::storage;
  constexpr int E = G_::E, LPR = G_::LPR, TPI = G_::TPI;
  const int lane = threadIdx.x & (kWave - 1);
  const int rg = lane / LPR, c = lane % LPR;
  const int j = blockIdx.y, b = blockIdx.z;
  // with APPEND, the first workgroup of every (b, j) row (dispatched first, so
  // its dependent loads overlap the scoring) appends the new token and scores
  // its block from the updated rows; the others skip that block
  int nskip = -1;
  if constexpr (APPEND) {
    nskip = (seq_lens[b] - 1) / kBlockSize;
    if (blockIdx.x == 0) {
      if (threadIdx.x >= kWave) return;                  // wave 0 only
      const bool mine = lane < LPR;
      float qp[G][E], qn[G][E];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float f[E];
        DT::widen(mine ? load16(static_cast<const St*>(q) + ((size_t)b * Hq + j * G + g) * D +
                                lane * E)
                       : make_uint4(0, 0, 0, 0),
                  f);
        split_query<E, IDX>(f, qp[g], qn[g]);
      }
      float mn[E], mx[E], mv[E];
#pragma unroll
      for (int e = 0; e < E; ++e) mn[e] = mx[e] = mv[e] = 0.0f;
      if (mine)
        append_lane<DT, D>(ap.k_new, ap.v_new, block_table, seq_lens, Hkv, maxN, j, b, lane,
                           ap.k_cache, ap.v_cache, ap.kmeta, ap.kmean, mn, mx, mv);
      float best = -INFINITY;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if constexpr (IDX == kIndexMinMax)
          best = fmaxf(best, head_score_lane<E, LPR, IDX>(qp[g], qn[g], mn, mx));
        else
          best = fmaxf(best, head_score_lane<E, LPR, IDX>(qp[g], qn[g], mv, mv));
      }
      if (lane == 0) scores[((size_t)b * Hkv + j) * maxN + nskip] = best;
      return;
    }
  }
  const int wg = APPEND ? (int)blockIdx.x - 1 : (int)blockIdx.x;
  const int n0 = (wg * WAVES + (threadIdx.x >> 6)) * (STEPS * TPI);
  if (n0 >= maxN) return;
  // the wave's block-table entries are read beside the sequence length (every
  // entry of the row is readable), so the index loads wait for one round trip
  const int32_t* bt_row = block_table + (size_t)b * maxN;
  int32_t pg[STEPS];
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int n = n0 + st * TPI + rg;
    pg[st] = n < maxN ? bt_row[n] : 0;
  }
  const int nb = (seq_lens[b] + kBlockSize - 1) / kBlockSize;

  // 16-byte index loads per block and lane: the min and max chunks, or the
  // E floats of the mean chunk
  constexpr int NL = (IDX == kIndexMinMax) ? 2 : E / 4;
  uint4 w[STEPS][NL];
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int n = n0 + st * TPI + rg;
    if (n < nb) {
      const size_t p = (size_t)pg[st];
      if constexpr (IDX == kIndexMinMax) {
        const St* src = static_cast<const St*>(kmeta) + (p * Hkv + j) * 2 * D + c * E;
        w[st][0] = load16(src);
        w[st][1] = load16(src + D);
      } else {
        const float* src = static_cast<const float*>(kmeta) + (p * Hkv + j) * D + c * E;
#pragma unroll
        for (int i = 0; i < NL; ++i) w[st][i] = load16(src + 4 * i);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NL; ++i) w[st][i] = make_uint4(0, 0, 0, 0);
    }
  }

  float qp[G][E], qn[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float f[E];
    DT::widen(load16(static_cast<const St*>(q) + ((size_t)b * Hq + j * G + g) * D + c * E), f);
    split_query<E, IDX>(f, qp[g], qn[g]);
  }

  float* out = scores + ((size_t)b * Hkv + j) * maxN;
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int n = n0 + st * TPI + rg;
    float ka[E], kb[E];   // minmax: kmin, kmax; mean: the mean row
    if constexpr (IDX == kIndexMinMax) {
      DT::widen(w[st][0], ka);
      DT::widen(w[st][1], kb);
    } else {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        ka[4 * i + 0] = __uint_as_float(w[st][i].x);
        ka[4 * i + 1] = __uint_as_float(w[st][i].y);
        ka[4 * i + 2] = __uint_as_float(w[st][i].z);
        ka[4 * i + 3] = __uint_as_float(w[st][i].w);
      }
    }
    float best = -INFINITY;
#pragma unroll
    for (int g = 0; g < G; ++g) best = fmaxf(best, head_score_lane<E, LPR, IDX>(qp[g], qn[g], ka, kb));
    if (c == 0 && n < maxN && n != nskip) out[n] = (n < nb) ? best : -INFINITY;
  }
}

// ============================================================== block score on the matrix cores
//
// With 16-bit min/max index rows the scores of one (sequence, KV head) are a
// small dense contraction: S[n, h] = [kmin_n | kmax_n] . [q-_h | q+_h] over the
// 2D channels of the row pair, q- = min(q, 0) against kmin and q+ = max(q, 0)
// against kmax (for each channel one of the two products is an exact zero,
// and products of 16-bit values are exact in fp32).  A wave takes 16
// consecutive logical blocks as the 16 rows of the MFMA A operand, read
// straight from the index rows (lane l: block l % 16, channels
// 32 st + 8 (l / 16) .. + 8 of step st), and the G query heads of the group as
// the first G columns of B (the other columns are zero).  A block's group
// score is the max over those G columns of its output row.  Each output
// element depends on its own A row and B column only, so a block scores the
// same bits wherever it sits in a tile.

// Lane l's B operand: column l % 16 (head j*G + l % 16 when l % 16 < G) at
// channels 32 st + 8 (l / 16) .. + 8 of [q- | q+] (16-bit sign masks, exact).
template <typename DT, int D, int G>
__device__ inline void score_query_operand(const void* __restrict__ q, size_t head0, int lane,
                                           uint4 (&qB)[2 * D / 32]) {
  using St = typename DT::storage;
  const int r = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int st = 0; st < 2 * D / 32; ++st) {
    const int k0 = 32 * st + 8 * kg;
    const bool pos = k0 >= D;            // the q+ half pairs with kmax
    uint4 w = r < G ? load16(static_cast<const St*>(q) + (head0 + r) * D + (pos ? k0 - D : k0))
                    : make_uint4(0, 0, 0, 0);
    auto keep = [pos](uint32_t x) {
      const uint32_t neg = ((x >> 15) & 0x00010001u) * 0xFFFFu;   // per 16-bit half: sign set
      return x & (pos ? ~neg : neg);
    };
    qB[st] = make_uint4(keep(w.x), keep(w.y), keep(w.z), keep(w.w));
  }
}

// Group score of the tile's rows 4 (l / 16) + i from the accumulators: the max
// over the G head columns of each row (aligned groups of G lanes).
template <int G>
__device__ inline void group_max_columns(f32x4_v& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = group_reduce<G, OpMax>(acc[i]);
}

// MEAN: the append also refreshes a mean-key index (its registers are kept
// out of the instances that have none to refresh).
template <typename DT, int D, int G, int WAVES, bool APPEND, bool MEAN = false>
__global__ __launch_bounds__(WAVES * kWave) void block_score_mfma_kernel(
    const void* __restrict__ q, const void* __restrict__ kmeta,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int Hq,
    int Hkv, int maxN, float* __restrict__ scores, AppendArgs ap) {
  static_assert(G >= 1 && G <= 8, "the group fills 1..8 of the 16 B columns");
  using St = typename DT::storage;
  constexpr int KS = 2 * D / 32;              // MFMA steps over a row pair
  const int lane = threadIdx.x & (kWave - 1);
  const int r = lane & 15, kg = lane >> 4;
  const int j = blockIdx.y, b = blockIdx.z;
  const size_t head0 = (size_t)b * Hq + (size_t)j * G;
  float* out = scores + ((size_t)b * Hkv + j) * maxN;
  int nskip = -1;
  if constexpr (APPEND) {
    // the first workgroup of each (b, j) row appends the new token (lanes
    // c < LPR of wave 0) and scores its block from the updated rows, staged in
    // LDS as row 0 of a tile; the other workgroups skip that block
    nskip = (seq_lens[b] - 1) / kBlockSize;
    if (blockIdx.x == 0) {
      if (threadIdx.x >= kWave) return;                  // wave 0 only
      constexpr int E = RowGeom<DT, D>::E, LPR = RowGeom<DT, D>::LPR;
      static_assert(2 * LPR == KS * 4, "row-pair chunks");
      __shared__ uint4 pair[2 * LPR];                    // kmin chunks, then kmax chunks
      uint4 qB[KS];
      score_query_operand<DT, D, G>(q, head0, lane, qB);
      float mn[E], mx[E], mv[E];
      if (lane < LPR) {
        append_lane<DT, D>(ap.k_new, ap.v_new, block_table, seq_lens, Hkv, maxN, j, b, lane,
                           ap.k_cache, ap.v_cache, ap.kmeta, MEAN ? ap.kmean : nullptr, mn, mx,
                           mv);
        pair[lane] = DT::narrow_exact(mn);
        pair[LPR + lane] = DT::narrow_exact(mx);
      }
      // one wave: its LDS writes complete before its later LDS reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      f32x4_v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st)
        acc = mfma_16x16x32<DT>(r == 0 ? pair[4 * st + kg] : make_uint4(0, 0, 0, 0), qB[st], acc);
      group_max_columns<G>(acc);
      if (lane == 0) out[nskip] = acc[0];
      return;
    }
  }
  const int wg = APPEND ? (int)blockIdx.x - 1 : (int)blockIdx.x;
  const int n0 = (wg * WAVES + (threadIdx.x >> 6)) * 16;
  if (n0 >= maxN) return;
  // the table entry is read beside the length (the whole row is readable)
  const int n = n0 + r;
  const int pg = n < maxN ? block_table[(size_t)b * maxN + n] : 0;
  const int nb = (seq_lens[b] + kBlockSize - 1) / kBlockSize;
  uint4 qB[KS];
  score_query_operand<DT, D, G>(q, head0, lane, qB);
  uint4 a[KS];
  const St* src = static_cast<const St*>(kmeta) + ((size_t)pg * Hkv + j) * 2 * D + 8 * kg;
#pragma unroll
  for (int st = 0; st < KS; ++st) a[st] = n < nb ? load16(src + 32 * st) : make_uint4(0, 0, 0, 0);
  f32x4_v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < KS; ++st) acc = mfma_16x16x32<DT>(a[st], qB[st], acc);
  group_max_columns<G>(acc);
  if (r == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = n0 + 4 * kg + i;
      if (m < maxN && m != nskip) out[m] = m < nb ? acc[i] : -INFINITY;
    }
  }
}

// ============================================================== Top-K
//
// The row select (topk_row) is in kvd_topk.hpp.

template <int NT, int EPT>
__global__ __launch_bounds__(NT) void topk_kernel(const float* __restrict__ scores,
                                                    const int32_t* __restrict__ seq_lens,
                                                    int Hkv, int maxN, int K, int sink,
                                                    int local, int32_t* __restrict__ sel,
                                                    int32_t* __restrict__ sel_count) {
  __shared__ TopkSmemFor<NT, EPT> sm;
  const int j = blockIdx.x, b = blockIdx.y;
  const size_t u = (size_t)b * Hkv + j;
  int32_t* out = sel + u * K;
  topk_row<NT, EPT>(scores + u * maxN, maxN, seq_lens[b], K, sink, local, out, sel_count + u, sm,
                    [out](int pos, int n) { out[pos] = n; });
}

// Two-level select of a long row.  topk_chunk_kernel: one workgroup per
// (chunk of kTopkChunk blocks, KV head, sequence) selects the chunk's forced
// blocks and its best min(K, #competing) competing blocks -- the one-level
// select's rule applied to the chunk -- and writes them, ascending, to the
// chunk's capc candidate slots (the score's key, 0 for a forced block, and
// the block; block -1 in unused slots).  Every block of the row's Top-K is
// among its chunk's candidates, and the candidate slots run in ascending
// block order, so topk_merge_kernel, the select over a row's candidate slots
// with each slot standing for its block, returns the one-level list exactly.

template <int NT, int EPT>
__global__ __launch_bounds__(NT) void topk_chunk_kernel(const float* __restrict__ scores,
                                                          const int32_t* __restrict__ seq_lens,
                                                          int Hkv, int maxN, int K, int sink,
                                                          int local, int capc,
                                                          uint32_t* __restrict__ cand_key,
                                                          int32_t* __restrict__ cand_block) {
  static_assert(NT * EPT == kTopkChunk, "one chunk per workgroup");
  __shared__ TopkSmemFor<NT, EPT> sm;
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int nch = gridDim.x;
  const size_t u = (size_t)b * Hkv + j;
  const int c0 = c * kTopkChunk;
  const int npos = min(kTopkChunk, maxN - c0);
  const float* row = scores + u * maxN + c0;
  uint32_t* ck = cand_key + (u * nch + c) * capc;
  int32_t* cb = cand_block + (u * nch + c) * capc;
  const int L = seq_lens[b];
  // the chunk's K_eff: its forced blocks (the one-level select's token tests,
  // counted as ranges) plus min(K, its competing blocks)
  auto keff_of = [&]() {
    const int nb = (L + kBlockSize - 1) / kBlockSize;
    const int a = c0, e = min(nb, c0 + npos);
    if (e <= a) return 0;
    const int sb = (sink + kBlockSize - 1) / kBlockSize;          // blocks below hold sink tokens
    const int t = L - local;
    const int lb = local > 0 ? (t > 0 ? t / kBlockSize : 0) : 0x7fffffff;   // first local block
    const int competing = max(0, min(e, lb) - max(a, sb));
    return (e - a) - competing + min(K, competing);
  };
  topk_select<NT, EPT, false>(row, npos, L, sink, local, c0, nullptr, keff_of, cb, nullptr, capc,
                              sm, [&](int pos, int n, uint32_t key) {
                                ck[pos] = key;
                                cb[pos] = n;
                              });
}

template <int NT, int EPT>
__global__ __launch_bounds__(NT) void topk_merge_kernel(const uint32_t* __restrict__ cand_key,
                                                          const int32_t* __restrict__ cand_block,
                                                          const int32_t* __restrict__ seq_lens,
                                                          int Hkv, int ncand, int K, int sink,
                                                          int local, int32_t* __restrict__ sel,
                                                          int32_t* __restrict__ sel_count) {
  __shared__ TopkSmemFor<NT, EPT> sm;
  const int j = blockIdx.x, b = blockIdx.y;
  const size_t u = (size_t)b * Hkv + j;
  const int L = seq_lens[b];
  int32_t* out = sel + u * K;
  topk_select<NT, EPT, true>(reinterpret_cast<const float*>(cand_key + u * ncand), ncand, L, sink,
                             local, 0, cand_block + u * ncand,
                             [&]() { return min(K, (L + kBlockSize - 1) / kBlockSize); }, out,
                             sel_count + u, K, sm, [&](int pos, int n, uint32_t) { out[pos] = n; });
}

// ============================================================== launchers


hipError_t launch_block_meta(int dtype, int D, const void* k_cache, const int32_t* page_ids,
                             const int32_t* valid_tokens, int n_ids, int Hkv, void* kmeta,
                             hipStream_t stream) {
  if (n_ids <= 0) return hipSuccess;
  return with_dtype(dtype, [&](auto dt) {
    return with_dim(D, [&](auto d) {
      using DT = decltype(dt);
      constexpr int DD = decltype(d)::value;
      constexpr int WAVES = KVD_META_WAVES;
      constexpr int UPS = kWave / RowGeom<DT, DD>::LPR;
      const long steps = ((long)n_ids * Hkv + UPS - 1) / UPS;
      const long want = (steps + WAVES - 1) / WAVES;
      const int grid = (int)std::min<long>(want, (long)cu_count() * KVD_META_WGS_PER_CU);
      hipLaunchKernelGGL((block_meta_kernel<DT, DD, WAVES>), dim3(grid), dim3(WAVES * kWave), 0,
                         stream, k_cache, page_ids, valid_tokens, n_ids, Hkv, kmeta);
      return hipGetLastError();
    });
  });
}

hipError_t launch_block_mean(int dtype, int D, const void* k_cache, const int32_t* page_ids,
                             const int32_t* valid_tokens, int n_ids, int Hkv, float* kmean,
                             hipStream_t stream) {
  if (n_ids <= 0) return hipSuccess;
  return with_dtype(dtype, [&](auto dt) {
    return with_dim(D, [&](auto d) {
      using DT = decltype(dt);
      constexpr int DD = decltype(d)::value;
      constexpr int WAVES = KVD_META_WAVES;
      constexpr int UPS = kWave / RowGeom<DT, DD>::LPR;
      const long steps = ((long)n_ids * Hkv + UPS - 1) / UPS;
      const long want = (steps + WAVES - 1) / WAVES;
      const int grid = (int)std::min<long>(want, (long)cu_count() * KVD_META_WGS_PER_CU);
      hipLaunchKernelGGL((block_mean_kernel<DT, DD, WAVES>), dim3(grid), dim3(WAVES * kWave), 0,
                         stream, k_cache, page_ids, valid_tokens, n_ids, Hkv, kmean);
      return hipGetLastError();
    });
  });
}

hipError_t launch_append_token(int dtype, int D, const void* k_new, const void* v_new,
                               const int32_t* block_table, const int32_t* seq_lens, int B,
                               int Hkv, int maxN, void* k_cache, void* v_cache, void* kmeta,
                               float* kmean, hipStream_t stream) {
  return with_dtype(dtype, [&](auto dt) {
    return with_dim(D, [&](auto d) {
      hipLaunchKernelGGL((append_token_kernel<decltype(dt), decltype(d)::value>), dim3(Hkv, B),
                         dim3(kWave), 0, stream, k_new, v_new, block_table, seq_lens, Hkv, maxN,
                         k_cache, v_cache, kmeta, kmean);
      return hipGetLastError();
    });
  });
}

hipError_t launch_block_score(int dtype, int D, int G, int index_kind, const void* q,
                              const void* index, const int32_t* block_table,
                              const int32_t* seq_lens, int B, int Hq, int Hkv, int maxN,
                              float* scores, hipStream_t stream, const void* k_new,
                              const void* v_new, void* k_cache, void* v_cache, void* kmeta,
                              float* kmean) {
  const AppendArgs ap{k_new, v_new, k_cache, v_cache, kmeta, kmean};
  const bool append = k_new != nullptr;
  return with_dtype(dtype, [&](auto dt) {
    return with_dim(D, [&](auto d) {
      return with_group(G, [&](auto g) {
        using DT = decltype(dt);
        constexpr int DD = decltype(d)::value;
        constexpr int GG = decltype(g)::value;
        if constexpr (!std::is_same<DT, F32>::value) {
          if (index_kind == kIndexMinMax) {     // 16-bit min/max rows: the matrix cores
            constexpr int W = KVD_SCORE_MFMA_WAVES;
            const dim3 grid_m((maxN + 16 * W - 1) / (16 * W) + (append ? 1 : 0), Hkv, B);
            if (append && kmean)
              hipLaunchKernelGGL((block_score_mfma_kernel<DT, DD, GG, W, true, true>), grid_m,
                                 dim3(W * kWave), 0, stream, q, index, block_table, seq_lens, Hq,
                                 Hkv, maxN, scores, ap);
            else if (append)
              hipLaunchKernelGGL((block_score_mfma_kernel<DT, DD, GG, W, true, false>), grid_m,
                                 dim3(W * kWave), 0, stream, q, index, block_table, seq_lens, Hq,
                                 Hkv, maxN, scores, ap);
            else
              hipLaunchKernelGGL((block_score_mfma_kernel<DT, DD, GG, W, false>), grid_m,
                                 dim3(W * kWave), 0, stream, q, index, block_table, seq_lens, Hq,
                                 Hkv, maxN, scores, ap);
            return hipGetLastError();
          }
        }
        constexpr int WAVES = KVD_SCORE_WAVES, STEPS = KVD_SCORE_STEPS;
        constexpr int per_wg = WAVES * STEPS * RowGeom<DT, DD>::TPI;
        // one more workgroup per row does the append
        const dim3 grid((maxN + per_wg - 1) / per_wg + (append ? 1 : 0), Hkv, B);
#define KVD_SCORE(IDX, APP)                                                                     \
  hipLaunchKernelGGL((block_score_kernel<DT, DD, GG, WAVES, STEPS, IDX, APP>), grid,           \
                     dim3(WAVES * kWave), 0, stream, q, index, block_table, seq_lens, Hq, Hkv, \
                     maxN, scores, ap)
        if (index_kind == kIndexMean) {
          if (append) KVD_SCORE(kIndexMean, true);
          else KVD_SCORE(kIndexMean, false);
        } else {
          if (append) KVD_SCORE(kIndexMinMax, true);
          else KVD_SCORE(kIndexMinMax, false);
        }
#undef KVD_SCORE
        return hipGetLastError();
      });
    });
  });
}

hipError_t launch_topk(const float* scores, const int32_t* seq_lens, int B, int Hkv, int maxN,
                       int K, int sink, int local, int32_t* sel, int32_t* sel_count,
                       hipStream_t stream, void* cand) {
  const int slots = topk_candidates_per_row(maxN, K);
  if (cand && slots > 0) {
    // candidate slots per chunk: K + the most blocks the tokens can force
    const int forced = (sink + kBlockSize - 1) / kBlockSize +
                       (local > 0 ? (local - 1 + kBlockSize - 1) / kBlockSize + 1 : 0);
    const int nch = (maxN + kTopkChunk - 1) / kTopkChunk;
    const int capc = K + min(forced, K);
    const int ncand = nch * capc;                      // <= slots
    uint32_t* ck = static_cast<uint32_t*>(cand);
    int32_t* cb = reinterpret_cast<int32_t*>(ck + (size_t)B * Hkv * slots);
    constexpr int CT = KVD_TOPK_CHUNK_THREADS;
    hipLaunchKernelGGL((topk_chunk_kernel<CT, kTopkChunk / CT>), dim3(nch, Hkv, B), dim3(CT), 0,
                       stream, scores, seq_lens, Hkv, maxN, K, sink, local, capc, ck, cb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 gm(Hkv, B);
    const int ept = (ncand + 1023) / 1024;
#define KVD_TOPK_MERGE(N)                                                                      \
  hipLaunchKernelGGL((topk_merge_kernel<1024, N>), gm, dim3(1024), 0, stream, ck, cb, seq_lens, \
                     Hkv, ncand, K, sink, local, sel, sel_count)
    if (ept <= 1) KVD_TOPK_MERGE(1);
    else if (ept <= 2) KVD_TOPK_MERGE(2);
    else if (ept <= 4) KVD_TOPK_MERGE(4);
    else if (ept <= 8) KVD_TOPK_MERGE(8);
    else if (ept <= 16) KVD_TOPK_MERGE(16);
    else return hipErrorInvalidValue;
#undef KVD_TOPK_MERGE
    return hipGetLastError();
  }
  const dim3 grid(Hkv, B);
  const int ept = (maxN + 1023) / 1024;
#define KVD_TOPK(N)                                                                          \
  hipLaunchKernelGGL((topk_kernel<1024, N>), grid, dim3(1024), 0, stream, scores, seq_lens, Hkv, \
                     maxN, K, sink, local, sel, sel_count)
  if (ept <= 1) KVD_TOPK(1);
  else if (ept <= 2) KVD_TOPK(2);
  else if (ept <= 4) KVD_TOPK(4);
  else if (ept <= 8) KVD_TOPK(8);
  else if (ept <= 16) KVD_TOPK(16);
  else if (ept <= 32) KVD_TOPK(32);
  else if (ept <= 64) KVD_TOPK(64);
  else return hipErrorInvalidValue;
#undef KVD_TOPK
  return hipGetLastError();
}

}  // namespace kvd

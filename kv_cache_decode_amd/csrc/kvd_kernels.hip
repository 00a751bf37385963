// gfx950 kernels of the paged Top-K decode step.
//
//   block_meta_kernel   channel-wise min/max key per (page, KV head)      KVDrive §2.2, §2.3
//   block_score_kernel  Quest score per logical block, max over the GQA group   KVDrive §2.2
//   topk_kernel         exact Top-K of the block scores, ascending output
//   paged_attn_kernel   split-K streaming-softmax decode attention      DirectKV review, core
//                       method 2-3; Dual-Blade background; KVDrive §2.3
//   combine_kernel      log-sum-exp merge of the split partials
//
// Data movement is HBM-bound everywhere, so the kernels are built around
// coalesced 16-byte loads: a token row (or a meta row) of D channels is spread
// over LPR = D / E lanes (E channels per 16-byte chunk), and one wave64 load
// instruction covers TPI = 64 / LPR consecutive rows, i.e. 1 KiB of contiguous
// memory.  Each K/V byte is read exactly once; nothing is re-read from another
// workgroup, so the blockIdx -> XCD placement carries no L2 reuse to exploit.
#include <math.h>

#include "kvd_device.hpp"
#include "kvd_launch.hpp"

namespace kvd {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Lane geometry of a row of D channels in 16-byte chunks.
template <typename DT, int D>
struct RowGeom {
  static constexpr int E = DT::E;                  // channels per chunk
  static constexpr int LPR = D / E;                // lanes per row
  static constexpr int TPI = kWave / LPR;          // rows per load instruction
  static constexpr int NI = kBlockSize / TPI;      // instructions per 16-row page
  static_assert(LPR >= 8 && LPR <= 32 && TPI * LPR == kWave && NI >= 1, "row geometry");
};

// ============================================================== block meta
//
// One wave per (page, KV head) unit: NI loads cover the 16 x D key tile, each
// lane folds the slots it holds (slot it*TPI + rg) into a running min and max,
// the row groups are merged across lanes, and row group 0 writes the min row,
// row group 1 the max row.  min/max of representable values is exact, so the
// narrowing back to the storage dtype is exact too.

template <typename DT, int D, int WAVES, int UNROLL>
__global__ __launch_bounds__(WAVES * kWave) void block_meta_kernel(
    const void* __restrict__ k_cache, const int32_t* __restrict__ page_ids,
    const int32_t* __restrict__ valid_tokens, int n_ids, int Hkv, void* __restrict__ kmeta) {
  using G_ = RowGeom<DT, D>;
  using St = typename DT::storage;
  constexpr int E = G_::E, LPR = G_::LPR, TPI = G_::TPI, NI = G_::NI;
  const int lane = threadIdx.x & (kWave - 1);
  const int rg = lane / LPR, c = lane % LPR;
  const int nwaves = gridDim.x * WAVES;
  const int units = n_ids * Hkv;

  for (int u0 = blockIdx.x * WAVES + (threadIdx.x >> 6); u0 < units; u0 += nwaves * UNROLL) {
    uint4 w[UNROLL][NI];
    int page[UNROLL], nv[UNROLL], head[UNROLL];
#pragma unroll
    for (int x = 0; x < UNROLL; ++x) {
      const int u = u0 + x * nwaves;
      page[x] = -1;
      if (u < units) {
        const int i = u / Hkv;
        head[x] = u - i * Hkv;
        page[x] = page_ids[i];
        nv[x] = valid_tokens[i];
        const St* src = static_cast<const St*>(k_cache) +
                        (((size_t)page[x] * Hkv + head[x]) * kBlockSize + rg) * D + c * E;
#pragma unroll
        for (int it = 0; it < NI; ++it) w[x][it] = load16(src + (size_t)it * TPI * D);
      }
    }
#pragma unroll
    for (int x = 0; x < UNROLL; ++x) {
      if (page[x] < 0) break;  // wave-uniform
      float mn[E], mx[E];
#pragma unroll
      for (int e = 0; e < E; ++e) { mn[e] = INFINITY; mx[e] = -INFINITY; }
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        if (it * TPI + rg < nv[x]) {
          float f[E];
          DT::widen(w[x][it], f);
#pragma unroll
          for (int e = 0; e < E; ++e) { mn[e] = fminf(mn[e], f[e]); mx[e] = fmaxf(mx[e], f[e]); }
        }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        mn[e] = cross_group_reduce<LPR, OpMin>(mn[e]);
        mx[e] = cross_group_reduce<LPR, OpMax>(mx[e]);
      }
      St* dst = static_cast<St*>(kmeta) + ((size_t)page[x] * Hkv + head[x]) * 2 * D + c * E;
      if (rg == 0) store16(dst, DT::narrow_exact(mn));
      if (rg == 1) store16(dst + D, DT::narrow_exact(mx));
    }
  }
}

// ============================================================== block score
//
// sigma_h = sum_c max(q_hc kmin_c, q_hc kmax_c) = sum_c (q+_hc kmax_c + q-_hc kmin_c)
// with q+ = max(q, 0), q- = min(q, 0): for each channel one of the two products
// is an exact zero, so the fused multiply-adds accumulate exactly the max term.
// A wave owns STEPS * TPI consecutive logical blocks of one (sequence, KV
// head); lane (rg, c) handles channels [c*E, c*E+E) of block n0 + step*TPI + rg.
// All meta loads of the wave are issued before any arithmetic.

template <typename DT, int D, int G, int WAVES, int STEPS>
__global__ __launch_bounds__(WAVES * kWave) void block_score_kernel(
    const void* __restrict__ q, const void* __restrict__ kmeta,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int Hq,
    int Hkv, int maxN, float* __restrict__ scores) {
  using G_ = RowGeom<DT, D>;
  using St = typename DT::storage;
  constexpr int E = G_::E, LPR = G_::LPR, TPI = G_::TPI;
  const int lane = threadIdx.x & (kWave - 1);
  const int rg = lane / LPR, c = lane % LPR;
  const int j = blockIdx.y, b = blockIdx.z;
  const int n0 = (blockIdx.x * WAVES + (threadIdx.x >> 6)) * (STEPS * TPI);
  if (n0 >= maxN) return;
  const int nb = (seq_lens[b] + kBlockSize - 1) / kBlockSize;

  const int32_t* bt_row = block_table + (size_t)b * maxN;
  uint4 wmin[STEPS], wmax[STEPS];
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int n = n0 + st * TPI + rg;
    if (n < nb) {
      const size_t p = (size_t)bt_row[n];
      const St* src = static_cast<const St*>(kmeta) + (p * Hkv + j) * 2 * D + c * E;
      wmin[st] = load16(src);
      wmax[st] = load16(src + D);
    } else {
      wmin[st] = make_uint4(0, 0, 0, 0);
      wmax[st] = make_uint4(0, 0, 0, 0);
    }
  }

  float qp[G][E], qn[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float f[E];
    DT::widen(load16(static_cast<const St*>(q) + ((size_t)b * Hq + j * G + g) * D + c * E), f);
#pragma unroll
    for (int e = 0; e < E; ++e) { qp[g][e] = fmaxf(f[e], 0.0f); qn[g][e] = fminf(f[e], 0.0f); }
  }

  float* out = scores + ((size_t)b * Hkv + j) * maxN;
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int n = n0 + st * TPI + rg;
    float kmn[E], kmx[E];
    DT::widen(wmin[st], kmn);
    DT::widen(wmax[st], kmx);
    float best = -INFINITY;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float acc = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        acc = fmaf(qp[g][e], kmx[e], acc);
        acc = fmaf(qn[g][e], kmn[e], acc);
      }
      acc = group_reduce<LPR, OpSum>(acc);
      best = fmaxf(best, acc);
    }
    if (c == 0 && n < maxN) out[n] = (n < nb) ? best : -INFINITY;
  }
}

// ============================================================== Top-K
//
// One 1024-thread workgroup per (sequence, KV head).  Scores become monotone
// uint32 keys (larger score -> larger key; -0 folded onto +0 so equal scores
// give equal keys); thread t keeps the keys of blocks [t*EPT, t*EPT+EPT) in
// registers.  The K_eff-th largest key T is found by a radix select: the bits
// above the highest bit where the smallest and largest valid keys differ are
// fixed at once, then 8-bit digits below them are resolved from the top, each
// pass building one private LDS histogram per wave (no atomic traffic between
// waves) that wave 0 merges and scans.  A block is selected if its key is
// above T, or equal to T and among the first K_eff - #{key > T} equal keys in
// index order; one exclusive scan of packed (#greater, #equal) counts gives
// every selected block its output position, so the list comes out ascending.

__device__ inline uint32_t score_key(float f) {
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v = min(v, (uint32_t)__shfl_xor((int)v, off, kWave));
  return v;
}
__device__ inline uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, kWave));
  return v;
}
__device__ inline uint32_t wave_inclusive_scan(uint32_t v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

template <int NWAVES>
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* buf) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) buf[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave; ++w) before += buf[w];
  return before + inc - v;
}

template <int EPT>
__global__ __launch_bounds__(1024) void topk_kernel(const float* __restrict__ scores,
                                                    const int32_t* __restrict__ seq_lens,
                                                    int Hkv, int maxN, int K,
                                                    int32_t* __restrict__ sel,
                                                    int32_t* __restrict__ sel_count) {
  constexpr int NW = 1024 / kWave;
  __shared__ __align__(16) uint32_t hist[NW][256];
  __shared__ uint32_t buf_a[NW], buf_b[NW], buf_c[NW];
  __shared__ uint32_t state[2];
  const int j = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int nb = (seq_lens[b] + kBlockSize - 1) / kBlockSize;
  const int keff = min(K, nb);
  int32_t* out = sel + ((size_t)b * Hkv + j) * K;
  if (tid == 0) sel_count[(size_t)b * Hkv + j] = max(keff, 0);
  for (int i = max(keff, 0) + tid; i < K; i += 1024) out[i] = -1;
  if (keff <= 0) return;  // workgroup-uniform
  const float* row = scores + ((size_t)b * Hkv + j) * maxN;

  uint32_t key[EPT];
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
  for (int r = 0; r < EPT; ++r) {
    const int n = tid * EPT + r;
    key[r] = 0u;
    if (n < nb) {
      key[r] = score_key(row[n]);  // valid keys are >= key(-inf) > 0
      kmn = min(kmn, key[r]);
      kmx = max(kmx, key[r]);
    }
  }
  kmn = wave_min_u32(kmn);
  kmx = wave_max_u32(kmx);
  if (lane == 0) { buf_a[wave] = kmn; buf_b[wave] = kmx; }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) { kmn = min(kmn, buf_a[w]); kmx = max(kmx, buf_b[w]); }

  // bits [lo, 32) of T are known; resolve the rest 8 bits at a time
  const uint32_t diff = kmn ^ kmx;
  int lo = diff ? 32 - __clz(diff) : 0;
  uint32_t prefix = (lo >= 32) ? 0u : (kmx >> lo) << lo;
  uint32_t krem = (uint32_t)keff;
  while (lo > 0) {
    const int width = min(8, lo);
    const int shift = lo - width;
    const uint32_t dmask = (1u << width) - 1u;
    uint32_t* h = hist[wave];
#pragma unroll
    for (int i = lane; i < 256; i += kWave) h[i] = 0u;
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      const bool match = key[r] != 0u && (lo >= 32 || (key[r] >> lo) == (prefix >> lo));
      if (match) atomicAdd(&h[(key[r] >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane L owns digits 255-4L .. 252-4L (descending)
      const int base = 252 - 4 * lane;
      uint32_t c3 = 0, c2 = 0, c1 = 0, c0 = 0;  // c3 = digit base+3 (largest)
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const uint4 v = *reinterpret_cast<const uint4*>(&hist[w][base]);
        c0 += v.x; c1 += v.y; c2 += v.z; c3 += v.w;
      }
      const uint32_t mine = c0 + c1 + c2 + c3;
      uint32_t above = wave_inclusive_scan(mine) - mine;   // keys in larger digits
      const uint32_t cs[4] = {c3, c2, c1, c0};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (above < krem && above + cs[q] >= krem) {
          state[0] = (uint32_t)(base + 3 - q);
          state[1] = krem - above;
        }
        above += cs[q];
      }
    }
    __syncthreads();
    prefix |= state[0] << shift;
    krem = state[1];
    lo = shift;
  }
  const uint32_t T = prefix;   // the K_eff-th largest key; krem of its copies are taken

  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int r = 0; r < EPT; ++r) {
    n_gt += key[r] > T;
    n_eq += key[r] == T;
  }
  // own buffer: with no radix pass, slower waves may still read buf_a / buf_b
  const uint32_t ex = block_exclusive_scan<NW>((n_gt << 16) | n_eq, buf_c);
  uint32_t gt_before = ex >> 16, eq_before = ex & 0xFFFFu;
#pragma unroll
  for (int r = 0; r < EPT; ++r) {
    const int n = tid * EPT + r;
    if (key[r] > T) {
      out[gt_before + min(eq_before, krem)] = n;
      ++gt_before;
    } else if (key[r] == T) {
      if (eq_before < krem) out[gt_before + eq_before] = n;
      ++eq_before;
    }
  }
}

// ============================================================== decode attention
//
// A wave owns one split of one (sequence, KV head) and all G query heads of
// that group: each K/V tile is read once and serves the whole group, and the
// queries, running max, running sum and output accumulators stay in registers
// for the whole split.  Per 16-token page: NI coalesced 16-byte loads of K and
// of V (issued one page ahead), fp32 partial dot products over the lane's E
// channels, an all-reduce over the LPR lanes of the token row, a wave max per
// head, a rescale of the accumulators only when some head's max grows, then
// p = 2^(z*log2e - m) and o += p v.  The page ids of up to 64 blocks of the
// split are fetched once (one per lane) and broadcast with readlane, so the
// K/V loads never wait on a table lookup.

template <typename DT, int D, int G, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void paged_attn_kernel(
    const void* __restrict__ q, const void* __restrict__ k_cache, const void* __restrict__ v_cache,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int sel_stride,
    int Hq, int Hkv, int maxN, int S, float qscale, float* __restrict__ part_o,
    float* __restrict__ part_m, float* __restrict__ part_l) {
  using G_ = RowGeom<DT, D>;
  using St = typename DT::storage;
  constexpr int E = G_::E, LPR = G_::LPR, TPI = G_::TPI, NI = G_::NI;
  const int lane = threadIdx.x & (kWave - 1);
  const int s = blockIdx.x * WAVES + (threadIdx.x >> 6);
  if (s >= S) return;
  const int j = blockIdx.y, b = blockIdx.z;
  const int rg = lane / LPR, c = lane % LPR;

  const int L = seq_lens[b];
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  const int n_list = sel ? sel_count[(size_t)b * Hkv + j] : nb;
  const int chunk = (n_list + S - 1) / S;
  const int p0 = min(s * chunk, n_list);
  const int p1 = min(p0 + chunk, n_list);
  const size_t row0 = (size_t)b * Hq + (size_t)j * G;

  float qf[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    DT::widen(load16(static_cast<const St*>(q) + (row0 + g) * D + c * E), qf[g]);
#pragma unroll
    for (int e = 0; e < E; ++e) qf[g][e] *= qscale;
  }
  float m[G], lsum[G], acc[G][E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    lsum[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = 0.0f;
  }

  const size_t page_stride = (size_t)Hkv * kBlockSize * D;
  const size_t lane_off = ((size_t)j * kBlockSize + rg) * D + (size_t)c * E;
  const St* kb = static_cast<const St*>(k_cache) + lane_off;
  const St* vb = static_cast<const St*>(v_cache) + lane_off;
  const int32_t* sel_row = sel ? sel + ((size_t)b * Hkv + j) * sel_stride : nullptr;
  const int32_t* bt_row = block_table + (size_t)b * maxN;

  for (int base = p0; base < p1; base += kWave) {
    const int cnt = min(kWave, p1 - base);
    int my_page = 0, my_valid = 0;
    if (lane < cnt) {
      const int n = sel_row ? sel_row[base + lane] : base + lane;
      my_page = bt_row[n];
      my_valid = min(kBlockSize, L - n * kBlockSize);
    }
    uint4 kc[NI], vc[NI];
    {
      const size_t off = (size_t)readlane(my_page, 0) * page_stride;
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        kc[it] = load16(kb + off + (size_t)it * TPI * D);
        vc[it] = load16(vb + off + (size_t)it * TPI * D);
      }
    }
    for (int i = 0; i < cnt; ++i) {
      uint4 kn[NI], vn[NI];
      if (i + 1 < cnt) {
        const size_t off = (size_t)readlane(my_page, i + 1) * page_stride;
#pragma unroll
        for (int it = 0; it < NI; ++it) {
          kn[it] = load16(kb + off + (size_t)it * TPI * D);
          vn[it] = load16(vb + off + (size_t)it * TPI * D);
        }
      }
      const int valid = readlane(my_valid, i);

      // logits (log2 units) of the lane's NI tokens for every head
      float z[NI][G];
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        float kf[E];
        DT::widen(kc[it], kf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float a = 0.0f;
#pragma unroll
          for (int e = 0; e < E; ++e) a = fmaf(qf[g][e], kf[e], a);
          z[it][g] = group_reduce<LPR, OpSum>(a);
        }
        if (it * TPI + rg >= valid) {
#pragma unroll
          for (int g = 0; g < G; ++g) z[it][g] = -INFINITY;
        }
      }
      // running max per head; rescale only when it grows (wave-uniform test)
      bool grow = false;
      float bm[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float v = z[0][g];
#pragma unroll
        for (int it = 1; it < NI; ++it) v = fmaxf(v, z[it][g]);
        bm[g] = cross_group_reduce<LPR, OpMax>(v);
        grow |= bm[g] > m[g];
      }
      if (grow) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float mn = fmaxf(m[g], bm[g]);
          const float alpha = fast_exp2(m[g] - mn);
          m[g] = mn;
          lsum[g] *= alpha;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[g][e] *= alpha;
        }
      }
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        float vf[E];
        DT::widen(vc[it], vf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p = fast_exp2(z[it][g] - m[g]);
          lsum[g] += p;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e]);
        }
      }
#pragma unroll
      for (int it = 0; it < NI; ++it) { kc[it] = kn[it]; vc[it] = vn[it]; }
    }
  }

  // merge the row groups (each saw a disjoint set of tokens) and write the split
#pragma unroll
  for (int g = 0; g < G; ++g) {
    lsum[g] = cross_group_reduce<LPR, OpSum>(lsum[g]);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = cross_group_reduce<LPR, OpSum>(acc[g][e]);
  }
  if (rg == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float inv = lsum[g] > 0.0f ? 1.0f / lsum[g] : 0.0f;
      float* dst = part_o + ((row0 + g) * S + s) * D + c * E;
#pragma unroll
      for (int e4 = 0; e4 < E; e4 += 4)
        *reinterpret_cast<float4*>(dst + e4) =
            make_float4(acc[g][e4] * inv, acc[g][e4 + 1] * inv, acc[g][e4 + 2] * inv,
                        acc[g][e4 + 3] * inv);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      part_m[(row0 + g) * S + s] = m[g] * kLn2;
      part_l[(row0 + g) * S + s] = lsum[g];
    }
  }
}

// ============================================================== combine
//
// One 256-thread workgroup per (row, 32-channel chunk), row = (sequence, query
// head).  Pass 1: the max M of the split maxima.  Pass 2: 32 split slots of 8
// threads (a float4 each) walk the splits with stride 32 and accumulate
// w_s * o_s and w_s, w_s = l_s exp(m_s - M) (0 for an empty split, whose o is
// 0); the loop body has no branch, so the loads of several splits are in
// flight together.  The 32 slots are then summed through LDS.

constexpr int kCombineChunk = 32;

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_m,
                                                      const float* __restrict__ part_l, int S,
                                                      int D, float* __restrict__ out,
                                                      float* __restrict__ lse) {
  constexpr int TPS = kCombineChunk / 4;   // threads per split slot
  constexpr int SLOTS = 256 / TPS;
  __shared__ float red[256 / kWave];
  __shared__ float4 acc_s[SLOTS][TPS];
  __shared__ float w_s[SLOTS];
  const size_t row = blockIdx.x;
  const int d0 = blockIdx.y * kCombineChunk;
  const int tid = threadIdx.x;
  const float* pm = part_m + row * S;
  const float* pl = part_l + row * S;

  float M = -INFINITY;
  for (int s = tid; s < S; s += 256) M = fmaxf(M, pm[s]);
  M = group_reduce<kWave, OpMax>(M);
  if ((tid & (kWave - 1)) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  const int slot = tid / TPS, q4 = tid % TPS;
  const float* po = part_o + (row * S) * D + d0 + q4 * 4;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  float W = 0.0f;
#pragma unroll 4
  for (int s = slot; s < S; s += SLOTS) {
    const float ms = pm[s];
    const float w = (ms == -INFINITY) ? 0.0f : pl[s] * expf(ms - M);
    const float4 o = *reinterpret_cast<const float4*>(po + (size_t)s * D);
    W += w;
    a.x = fmaf(w, o.x, a.x);
    a.y = fmaf(w, o.y, a.y);
    a.z = fmaf(w, o.z, a.z);
    a.w = fmaf(w, o.w, a.w);
  }
  acc_s[slot][q4] = a;
  if (q4 == 0) w_s[slot] = W;
  __syncthreads();
  if (tid < TPS) {
    float4 t = acc_s[0][tid];
    float wt = w_s[0];
#pragma unroll
    for (int k = 1; k < SLOTS; ++k) {
      const float4 u = acc_s[k][tid];
      t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
      wt += w_s[k];
    }
    const float inv = 1.0f / wt;
    *reinterpret_cast<float4*>(out + row * D + d0 + tid * 4) =
        make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
    if (lse && tid == 0 && blockIdx.y == 0) lse[row] = M + logf(wt);
  }
}

// ============================================================== launchers

namespace {

template <typename F>
hipError_t with_dtype(int dtype, F&& f) {
  switch (dtype) {
    case 0: return f(F32{});
    case 1: return f(F16{});
    case 2: return f(BF16{});
  }
  return hipErrorInvalidValue;
}

template <typename F>
hipError_t with_dim(int D, F&& f) {
  switch (D) {
    case 64: return f(std::integral_constant<int, 64>{});
    case 128: return f(std::integral_constant<int, 128>{});
  }
  return hipErrorInvalidValue;
}

template <typename F>
hipError_t with_group(int G, F&& f) {
  switch (G) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 8: return f(std::integral_constant<int, 8>{});
  }
  return hipErrorInvalidValue;
}

int cu_count() {
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

}  // namespace

hipError_t launch_block_meta(int dtype, int D, const void* k_cache, const int32_t* page_ids,
                             const int32_t* valid_tokens, int n_ids, int Hkv, void* kmeta,
                             hipStream_t stream) {
  if (n_ids <= 0) return hipSuccess;
  return with_dtype(dtype, [&](auto dt) {
    return with_dim(D, [&](auto d) {
      using DT = decltype(dt);
      constexpr int WAVES = 4, UNROLL = 2;
      const long units = (long)n_ids * Hkv;
      const long want = (units + WAVES * UNROLL - 1) / (WAVES * UNROLL);
      const int grid = (int)std::min<long>(want, (long)cu_count() * 16);
      hipLaunchKernelGGL((block_meta_kernel<DT, decltype(d)::value, WAVES, UNROLL>), dim3(grid),
                         dim3(WAVES * kWave), 0, stream, k_cache, page_ids, valid_tokens, n_ids,
                         Hkv, kmeta);
      return hipGetLastError();
    });
  });
}

hipError_t launch_block_score(int dtype, int D, int G, const void* q, const void* kmeta,
                              const int32_t* block_table, const int32_t* seq_lens, int B, int Hq,
                              int Hkv, int maxN, float* scores, hipStream_t stream) {
  return with_dtype(dtype, [&](auto dt) {
    return with_dim(D, [&](auto d) {
      return with_group(G, [&](auto g) {
        using DT = decltype(dt);
        constexpr int DD = decltype(d)::value;
        constexpr int WAVES = 4, STEPS = 8;
        constexpr int per_wg = WAVES * STEPS * RowGeom<DT, DD>::TPI;
        const dim3 grid((maxN + per_wg - 1) / per_wg, Hkv, B);
        hipLaunchKernelGGL((block_score_kernel<DT, DD, decltype(g)::value, WAVES, STEPS>), grid,
                           dim3(WAVES * kWave), 0, stream, q, kmeta, block_table, seq_lens, Hq,
                           Hkv, maxN, scores);
        return hipGetLastError();
      });
    });
  });
}

hipError_t launch_topk(const float* scores, const int32_t* seq_lens, int B, int Hkv, int maxN,
                       int K, int32_t* sel, int32_t* sel_count, hipStream_t stream) {
  const dim3 grid(Hkv, B);
  const int ept = (maxN + 1023) / 1024;
#define KVD_TOPK(N)                                                                          \
  hipLaunchKernelGGL((topk_kernel<N>), grid, dim3(1024), 0, stream, scores, seq_lens, Hkv, \
                     maxN, K, sel, sel_count)
  if (ept <= 1) KVD_TOPK(1);
  else if (ept <= 2) KVD_TOPK(2);
  else if (ept <= 4) KVD_TOPK(4);
  else if (ept <= 8) KVD_TOPK(8);
  else if (ept <= 16) KVD_TOPK(16);
  else if (ept <= 32) KVD_TOPK(32);
  else return hipErrorInvalidValue;
#undef KVD_TOPK
  return hipGetLastError();
}

hipError_t launch_paged_attn(int dtype, int D, int G, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* sel,
                             const int32_t* sel_count, int sel_stride, int B, int Hq, int Hkv,
                             int maxN, int S, float scale, float* part_o, float* part_m,
                             float* part_l, hipStream_t stream) {
  return with_dtype(dtype, [&](auto dt) {
    return with_dim(D, [&](auto d) {
      return with_group(G, [&](auto g) {
        using DT = decltype(dt);
        constexpr int WAVES = 4;
        const dim3 grid((S + WAVES - 1) / WAVES, Hkv, B);
        hipLaunchKernelGGL(
            (paged_attn_kernel<DT, decltype(d)::value, decltype(g)::value, WAVES>), grid,
            dim3(WAVES * kWave), 0, stream, q, k_cache, v_cache, block_table, seq_lens, sel,
            sel_count, sel_stride, Hq, Hkv, maxN, S, scale * kLog2e, part_o, part_m, part_l);
        return hipGetLastError();
      });
    });
  });
}

hipError_t launch_combine(int D, const float* part_o, const float* part_m, const float* part_l,
                          int rows, int S, float* out, float* lse, hipStream_t stream) {
  if (D % kCombineChunk) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_kernel, dim3(rows, D / kCombineChunk), dim3(256), 0, stream, part_o,
                     part_m, part_l, S, D, out, lse);
  return hipGetLastError();
}

int device_cu_count() { return cu_count(); }

}  // namespace kvd

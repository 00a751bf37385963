// Top-K of one row of block scores by one workgroup (the selection step of
// kv_block_score_topk / kv_block_select, and of the fused select + attention
// launch).  KVDrive §2.2: the Top-K blocks by Quest score; ties go to the
// lower block index, the list is ascending.
#pragma once

#include "kvd_device.hpp"

namespace kvd {

// One workgroup of NT threads per (sequence, KV head) row (1024 in the Top-K
// launch).  Scores become monotone
// uint32 keys (larger score -> larger key; -0 folded onto +0 so equal scores
// give equal keys); thread t keeps the keys of blocks [t*EPT, t*EPT+EPT) in
// registers.  The K_eff-th largest key T is found by a radix select: the bits
// above the highest bit where the smallest and largest valid keys differ are
// fixed at once; the next log2(4 NT) bits (4 NT digits) are resolved by one pass
// over a shared LDS histogram and a block scan.  If at most kTopkCandMax keys
// share the bits known so far, they are gathered in LDS and each is ranked
// against the others, which gives T directly; otherwise 8-bit digits are
// resolved from the top, each pass building one private LDS histogram per
// wave that wave 0 merges and scans.  A block is selected if its key is
// above T, or equal to T and among the first K_eff - #{key > T} equal keys in
// index order; one exclusive scan of packed (#greater, #equal) counts gives
// every selected block its output position, so the list comes out ascending.
// A block holding one of the first `sink` or the last `local` tokens is forced:
// it is kept out of the radix select (its key slot is 0, like a block past
// N_b, and a bit of the thread's forced mask records it), the select looks for
// the (K_eff - #forced)-th largest key among the other blocks, and in the
// output scan a forced block counts like a key above the threshold.  The
// caller keeps #forced <= K, so #forced <= K_eff.

// monotone key of a score: larger score -> larger key; f + 0 turns -0 into +0
// so equal scores give equal keys; negative scores flip every bit, the
// others only the sign bit
__device__ inline uint32_t score_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ inline uint32_t wave_inclusive_scan(uint32_t v) { return wave_scan_add_u32(v); }

// buf: NWAVES words, 16-byte aligned
template <int NWAVES>
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* buf) {
  static_assert(NWAVES % 4 == 0, "wave totals are read 4 at a time");
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) buf[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < NWAVES; w += 4) {
    const uint4 t = *reinterpret_cast<const uint4*>(buf + w);
    before += (w < wave ? t.x : 0u) + (w + 1 < wave ? t.y : 0u) + (w + 2 < wave ? t.z : 0u) +
              (w + 3 < wave ? t.w : 0u);
  }
  return before + inc - v;
}

// Top-K of one row by the NT threads of a workgroup (all of them call it);
// EPT keys per thread, NT * EPT >= maxN.  The per-key work is written without
// branches (selects, unconditional LDS adds, one candidate reservation per
// wave): with 16 waves sharing a compute unit's 4 SIMDs, per-key exec-mask
// branches cost more time than the row's loads.
// Most keys the rank count after the wide pass resolves (else 8-bit passes go on).
#ifndef KVD_TOPK_CAND_MAX
#define KVD_TOPK_CAND_MAX 512
#endif
constexpr int kTopkCandMax = KVD_TOPK_CAND_MAX;

// Keys a thread keeps in registers.  Rows of more than 32 keys per thread
// (EPT 64: up to 65536 blocks) keep keys 32 .. EPT-1 in LDS instead, one word
// per thread per key, lane-strided (thread t's key 32 + i at xkeys[i * NT + t],
// so a wave's accesses fall on distinct banks): at 1024 threads a thread has
// 128 VGPRs, and 64 keys in registers spilled to scratch memory.
constexpr int kTopkRegKeys = 32;
template <int EPT>
constexpr int topk_lds_keys() { return EPT > kTopkRegKeys ? EPT - kTopkRegKeys : 0; }

template <int NT, int XK = 0>
struct TopkSmem {
  static constexpr int NW = NT / kWave;
  static_assert(NW % 4 == 0, "wave partials are read 4 at a time");
  // per-wave 256-bin histograms of the 8-bit passes; the wide first pass uses
  // the same words as one shared histogram of NT * 4 bins
  alignas(16) uint32_t hist[NW][256];
  // per-wave partials of the first pass: min and max key, #forced, min of the
  // keys of scores >= +0, max of the others, #keys of scores >= +0
  alignas(16) uint32_t part[6][NW];
  alignas(16) uint32_t scan_a[NW];
  alignas(16) uint32_t scan_c[NW];
  alignas(16) uint32_t scan_d[NW];
  uint32_t state[3];
  uint32_t cand_n;
  // candidates of the rank count, and four key-0 pads after the last one
  alignas(16) uint32_t cand_key[kTopkCandMax + 4];
  alignas(16) int32_t cand_idx[kTopkCandMax + 4];
  uint32_t cand_gt[kTopkCandMax], cand_rank[kTopkCandMax];   // partial counts summed over waves
  alignas(16) uint32_t xkeys[XK > 0 ? XK * NT : 1];
};
template <int NT, int EPT>
using TopkSmemFor = TopkSmem<NT, topk_lds_keys<EPT>()>;

// Row select over npos positions of `row`.  Without IDX, row holds scores and
// position p stands for global block nbase + p.  With IDX, row holds keys
// (score_key values, as emitted by an earlier select) and position p stands
// for block bidx[p] (-1: no block).  A position is live when its block is in
// [0, N_b), N_b = ceil(L / bs), and the forced-token tests apply to its block.
// Ranking is by (key descending, position ascending), so positions must run
// in ascending block order for the lower-block tie rule.  keff_of() gives
// K_eff once the loads are issued (it may read only scalars).  The selected
// blocks go to emit(position in the ascending list, block, key; 0 for a
// forced block); when out is not null, K_eff goes to *count_out (if not null)
// and -1 to out[K_eff..out_len).
template <int NT, int EPT, bool IDX, typename KeffOf, typename Emit>
__device__ inline void topk_select(const float* __restrict__ row, int npos, int L, int sink,
                                   int local, int nbase, const int32_t* __restrict__ bidx,
                                   KeffOf&& keff_of, int32_t* __restrict__ out,
                                   int32_t* __restrict__ count_out, int out_len,
                                   TopkSmemFor<NT, EPT>& sm, Emit&& emit) {
  constexpr int NW = NT / kWave;
  constexpr int FW = (EPT + 31) / 32;   // words of the forced mask
  constexpr int ER = EPT - topk_lds_keys<EPT>();   // keys held in registers
  auto& hist = sm.hist;
  auto& state = sm.state;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int n0 = tid * EPT;
  const int maxN = npos;
  // key r of the thread (r is a compile-time index in every unrolled loop)
  uint32_t key[ER];
  uint32_t* xk = sm.xkeys + tid;
  auto kget = [&](int r) -> uint32_t { return r < ER ? key[r < ER ? r : 0] : xk[(r - ER) * NT]; };
  auto kset = [&](int r, uint32_t v) {
    if (r < ER) key[r < ER ? r : 0] = v;
    else xk[(r - ER) * NT] = v;
  };
  // the scores (and block indexes) are read first: the row is readable up to
  // npos whatever the length, so the loads need not wait for it (the keys hold
  // the score bits)
  if constexpr (EPT % 4 == 0) {
    // 16-byte loads of the thread's contiguous scores when the row allows it
    if ((reinterpret_cast<uintptr_t>(row) & 15u) == 0 && n0 + EPT <= maxN) {
#pragma unroll
      for (int r = 0; r < EPT; r += 4) {
        const uint4 v = load16(row + n0 + r);
        kset(r, v.x); kset(r + 1, v.y); kset(r + 2, v.z); kset(r + 3, v.w);
      }
    } else {
#pragma unroll
      for (int r = 0; r < EPT; ++r) kset(r, (n0 + r < maxN) ? __float_as_uint(row[n0 + r]) : 0u);
    }
  } else {
#pragma unroll
    for (int r = 0; r < EPT; ++r) kset(r, (n0 + r < maxN) ? __float_as_uint(row[n0 + r]) : 0u);
  }
  // the block of each of the thread's positions: with IDX from the index
  // array, read beside the scores (-1 past npos); else nbase + position (a
  // position past npos lies past the row, so past N_b)
  constexpr int EB = IDX ? EPT : 1;
  int32_t blkr[EB];
  if constexpr (IDX) {
#pragma unroll
    for (int r = 0; r < EPT; ++r) blkr[r] = (n0 + r < maxN) ? bidx[n0 + r] : -1;
  }
  auto blk = [&](int r) -> int {
    if constexpr (IDX) return blkr[r];
    else return nbase + n0 + r;
  };
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  const int keff = keff_of();
  const int local_from = local > 0 ? L - local : 0x7fffffff;  // first forced local token
  if (out) {
    if (count_out && tid == 0) *count_out = max(keff, 0);
    for (int i = max(keff, 0) + tid; i < out_len; i += NT) out[i] = -1;
  }
  if (keff <= 0) return;  // workgroup-uniform

  // keys: valid competing blocks get monotone keys (> 0); blocks past N_b and
  // forced blocks get 0, and a forced block sets its bit of fm
  const bool forcing = sink > 0 || local > 0;   // workgroup-uniform
  uint32_t fm[FW];
#pragma unroll
  for (int w = 0; w < FW; ++w) fm[w] = 0u;
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u, nf = 0u;
  auto convert = [&](auto with_forcing) {
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      const int n = blk(r);
      bool live = (n >= 0) & (n < nb);
      if constexpr (decltype(with_forcing)::value) {
        const bool forced = live & ((n * kBlockSize < sink) | ((n + 1) * kBlockSize > local_from));
        fm[r / 32] |= (uint32_t)forced << (r % 32);
        nf += (uint32_t)forced;
        live &= !forced;
      }
      uint32_t k = kget(r);
      if constexpr (!IDX) k = score_key(__uint_as_float(k));
      k = live ? k : 0u;
      kset(r, k);
      kmn = min(kmn, live ? k : 0xFFFFFFFFu);
      kmx = max(kmx, k);
    }
  };
  if (forcing) convert(std::true_type{});
  else convert(std::false_type{});
  kmn = wave_reduce_u32(kmn, MinU32());
  kmx = wave_reduce_u32(kmx, MaxU32());
  if (forcing) nf = wave_reduce_u32(nf, AddU32());
  if (lane == 0) {
    sm.part[0][wave] = kmn;
    sm.part[1][wave] = kmx;
    sm.part[2][wave] = nf;
  }
  if (tid == 0) sm.cand_n = 0u;
  // the wide pass's shared histogram is cleared under the same barrier
#pragma unroll
  for (int i = 0; i < 4; ++i) (&hist[0][0])[tid + i * NT] = 0u;
  __syncthreads();
  nf = 0u;
#pragma unroll
  for (int w = 0; w < NW; w += 4) {
    const uint4 a = *reinterpret_cast<const uint4*>(&sm.part[0][w]);
    const uint4 x = *reinterpret_cast<const uint4*>(&sm.part[1][w]);
    const uint4 f = *reinterpret_cast<const uint4*>(&sm.part[2][w]);
    kmn = min(min(kmn, min(a.x, a.y)), min(a.z, a.w));
    kmx = max(max(kmx, max(x.x, x.y)), max(x.z, x.w));
    nf += (f.x + f.y) + (f.z + f.w);
  }

  // places left for the blocks that compete; with none, T is above every key
  uint32_t krem = (uint32_t)keff - nf;
  // keys of both signs (workgroup-uniform): the count of keys of scores >= +0
  // says on which side of zero T lies, so the select starts inside that half
  // (its top bit is then known); this pass runs only for such rows
  const bool split = krem != 0u && ((kmn ^ kmx) >> 31);
  if (split) {
    uint32_t kmn_pos = 0xFFFFFFFFu, kmx_neg = 0u, npos = 0u;
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      const uint32_t kr = kget(r);
      const bool pos = (kr >> 31) != 0u;
      kmn_pos = min(kmn_pos, pos ? kr : 0xFFFFFFFFu);
      kmx_neg = max(kmx_neg, pos ? 0u : kr);
      npos += (uint32_t)pos;
    }
    kmn_pos = wave_reduce_u32(kmn_pos, MinU32());
    kmx_neg = wave_reduce_u32(kmx_neg, MaxU32());
    npos = wave_reduce_u32(npos, AddU32());
    if (lane == 0) {
      sm.part[3][wave] = kmn_pos;
      sm.part[4][wave] = kmx_neg;
      sm.part[5][wave] = npos;
    }
    __syncthreads();
    npos = 0u;
#pragma unroll
    for (int w = 0; w < NW; w += 4) {
      const uint4 mp = *reinterpret_cast<const uint4*>(&sm.part[3][w]);
      const uint4 xn = *reinterpret_cast<const uint4*>(&sm.part[4][w]);
      const uint4 np = *reinterpret_cast<const uint4*>(&sm.part[5][w]);
      kmn_pos = min(min(kmn_pos, min(mp.x, mp.y)), min(mp.z, mp.w));
      kmx_neg = max(max(kmx_neg, max(xn.x, xn.y)), max(xn.z, xn.w));
      npos += (np.x + np.y) + (np.z + np.w);
    }
    if (npos >= krem) {
      kmn = kmn_pos;
    } else {
      krem -= npos;             // every key of a score >= +0 ranks above T
      kmx = kmx_neg;
    }
  }
  // bits [lo, 32) of T are known; resolve the rest
  const uint32_t diff = kmn ^ kmx;
  int lo = (krem == 0u) ? 0 : (diff ? 32 - __clz(diff) : 0);
  uint32_t prefix = (krem == 0u) ? 0xFFFFFFFFu : ((lo >= 32) ? 0u : (kmx >> lo) << lo);
  // does key k share the known bits [lo, 32) of T? (key 0 never does)
  auto known = [&](uint32_t k) {
    return (k != 0u) & ((lo >= 32) | ((k >> (lo & 31)) == (prefix >> (lo & 31))));
  };
  if (lo > 0) {
    // one wide digit first: a shared histogram of NB = NT * 4 bins (thread t
    // owns digits NB-1-4t .. NB-4-4t, top down) and one block scan over them
    constexpr int NB = NT * 4;
    constexpr int WB = 31 - __builtin_clz(NB);
    const int width = min(WB, lo);
    const int shift = lo - width;
    const uint32_t dmask = (1u << width) - 1u;
    uint32_t* hs = &hist[0][0];
    static_assert(sizeof(sm.hist) == NB * sizeof(uint32_t), "shared histogram size");
    // without the sign split every valid key lies in [kmn, kmx] and so
    // shares the known bits
    if (split) {
#pragma unroll
      for (int r = 0; r < EPT; ++r) {
        const uint32_t kr = kget(r);
        atomicAdd(&hs[(kr >> shift) & dmask], (uint32_t)known(kr));
      }
    } else {
#pragma unroll
      for (int r = 0; r < EPT; ++r) {
        const uint32_t kr = kget(r);
        atomicAdd(&hs[(kr >> shift) & dmask], (uint32_t)(kr != 0u));
      }
    }
    __syncthreads();
    const uint4 v4 = *reinterpret_cast<const uint4*>(&hs[NB - 4 - 4 * tid]);
    const uint32_t cs[4] = {v4.w, v4.z, v4.y, v4.x};   // digits NB-1-4t down to NB-4-4t
    uint32_t above = block_exclusive_scan<NW>(v4.x + v4.y + v4.z + v4.w, sm.scan_a);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (above < krem && above + cs[q] >= krem) {
        state[0] = (uint32_t)(NB - 1 - 4 * tid - q);
        state[1] = krem - above;
        state[2] = cs[q];
      }
      above += cs[q];
    }
    __syncthreads();
    prefix |= state[0] << shift;
    krem = state[1];
    lo = shift;
    const uint32_t nc = state[2];
    if (lo > 0 && nc <= (uint32_t)kTopkCandMax) {
      // few keys share the known bits: gather them (one reservation per wave)
      // and rank each against the others by (key descending, index
      // ascending); the key ranked krem-1 is T
      if (tid < 4) sm.cand_key[nc + tid] = 0u;   // pads: rank below every candidate
      const bool spread = nc > (uint32_t)kWave;    // more than one wave's candidates
      if (spread) {
        for (int i = tid; i < (int)nc; i += NT) {
          sm.cand_gt[i] = 0u;
          sm.cand_rank[i] = 0u;
        }
      }
      uint32_t mine = 0u;
#pragma unroll
      for (int r = 0; r < EPT; ++r) mine += (uint32_t)known(kget(r));
      const uint32_t incl = wave_scan_add_u32(mine);
      uint32_t wbase = 0u;
      if (lane == kWave - 1 && incl != 0u) wbase = atomicAdd(&sm.cand_n, incl);
      uint32_t pos = (uint32_t)__builtin_amdgcn_readlane((int)wbase, kWave - 1) + incl - mine;
#pragma unroll
      for (int r = 0; r < EPT; ++r) {
        const uint32_t kr = kget(r);
        if (known(kr)) {
          sm.cand_key[pos] = kr;
          sm.cand_idx[pos] = n0 + r;
          ++pos;
        }
      }
      __syncthreads();
      // candidates are ranked by (key descending, index ascending) against
      // all others, four at a time: every lane reads the same 16 bytes of keys
      // and of indexes (an LDS broadcast), so the compares wait on no scalar
      // round trip; the key-0 pads past nc never count.  Up to 64 candidates
      // wave 0 ranks them all.  Beyond that, each block of 64 candidates (one
      // per lane) is compared by NW / blocks waves, each over its own range of
      // candidates, and the partial counts are summed in LDS.
      if (spread) {
        const int nblk = ((int)nc + kWave - 1) / kWave;
        const int parts = max(1, NW / nblk);
        const int nc4 = ((int)nc + 3) & ~3;
        const int len = (((nc4 + parts - 1) / parts) + 3) & ~3;
        for (int wv = wave; wv < nblk * parts; wv += NW) {
          const int cb = wv / parts, pt = wv - cb * parts;
          const int i = cb * kWave + lane;
          const bool own = i < (int)nc;
          const uint32_t ki = own ? sm.cand_key[i] : 0u;
          const int ii = own ? sm.cand_idx[i] : 0;
          uint32_t gt = 0, rank = 0;
          const int c1 = min(nc4, (pt + 1) * len);
#pragma unroll 2
          for (int c = pt * len; c < c1; c += 4) {
            const uint4 kc = *reinterpret_cast<const uint4*>(&sm.cand_key[c]);
            const int4 ic = *reinterpret_cast<const int4*>(&sm.cand_idx[c]);
            const uint32_t k4[4] = {kc.x, kc.y, kc.z, kc.w};
            const int i4[4] = {ic.x, ic.y, ic.z, ic.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              gt += k4[q] > ki;
              rank += k4[q] > ki || (k4[q] == ki && i4[q] < ii);
            }
          }
          if (own) {
            atomicAdd(&sm.cand_gt[i], gt);
            atomicAdd(&sm.cand_rank[i], rank);
          }
        }
        __syncthreads();
        for (int i = tid; i < (int)nc; i += NT) {
          if (sm.cand_rank[i] == krem - 1u) {
            state[0] = sm.cand_key[i];
            state[1] = krem - sm.cand_gt[i];
          }
        }
      }
      for (int cw = wave; !spread && cw * kWave < (int)nc; cw += NW) {
        const int i = cw * kWave + lane;
        const bool own = i < (int)nc;
        const uint32_t ki = own ? sm.cand_key[i] : 0u;
        const int ii = own ? sm.cand_idx[i] : 0;
        uint32_t gt = 0, rank = 0;
#pragma unroll 2
        for (int c = 0; c < (int)nc; c += 4) {
          const uint4 kc = *reinterpret_cast<const uint4*>(&sm.cand_key[c]);
          const int4 ic = *reinterpret_cast<const int4*>(&sm.cand_idx[c]);
          const uint32_t k4[4] = {kc.x, kc.y, kc.z, kc.w};
          const int i4[4] = {ic.x, ic.y, ic.z, ic.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gt += k4[q] > ki;
            rank += k4[q] > ki || (k4[q] == ki && i4[q] < ii);
          }
        }
        if (own && rank == krem - 1u) {
          state[0] = ki;
          state[1] = krem - gt;
        }
      }
      __syncthreads();
      prefix = state[0];
      krem = state[1];
      lo = 0;
    }
  }
  while (lo > 0) {
    const int width = min(8, lo);
    const int shift = lo - width;
    const uint32_t dmask = (1u << width) - 1u;
    uint32_t* h = hist[wave];
#pragma unroll
    for (int i = lane; i < 256; i += kWave) h[i] = 0u;
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      const uint32_t kr = kget(r);
      atomicAdd(&h[(kr >> shift) & dmask], (uint32_t)known(kr));
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
  const uint32_t T = prefix;   // the (K_eff - #forced)-th largest competing key; krem of its copies are taken

  // forced blocks rank with the keys above T (key slot 0 never equals T > 0)
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int r = 0; r < EPT; ++r) {
    const uint32_t kr = kget(r);
    n_gt += ((fm[r / 32] >> (r % 32)) & 1u) | (uint32_t)(kr > T);
    n_eq += (uint32_t)(kr == T);
  }
  // the scans use their own buffers: with no radix pass, slower waves may
  // still read the partials, and a wide pass's readers the first scan buffer
  uint32_t gt_before, eq_before;
  if constexpr ((long)NT * EPT < 65536) {
    const uint32_t ex = block_exclusive_scan<NW>((n_gt << 16) | n_eq, sm.scan_c);
    gt_before = ex >> 16;
    eq_before = ex & 0xFFFFu;
  } else {   // a count can reach 65536: one scan per count
    gt_before = block_exclusive_scan<NW>(n_gt, sm.scan_c);
    eq_before = block_exclusive_scan<NW>(n_eq, sm.scan_d);
  }
#pragma unroll
  for (int r = 0; r < EPT; ++r) {
    const uint32_t kr = kget(r);
    const bool gt = (((fm[r / 32] >> (r % 32)) & 1u) != 0u) | (kr > T);
    const bool eq = kr == T;
    if (gt | (eq & (eq_before < krem))) emit((int)(gt_before + min(eq_before, krem)), blk(r), kr);
    gt_before += (uint32_t)gt;
    eq_before += (uint32_t)eq;
  }
}

// Top-K of one full row of maxN block scores (blocks 0..maxN-1); when out is
// not null, K_eff goes to *count_out and -1 to out[K_eff..K).
template <int NT, int EPT, typename Emit>
__device__ inline void topk_row(const float* __restrict__ row, int maxN, int L, int K, int sink,
                                int local, int32_t* __restrict__ out,
                                int32_t* __restrict__ count_out, TopkSmemFor<NT, EPT>& sm,
                                Emit&& emit) {
  topk_select<NT, EPT, false>(row, maxN, L, sink, local, 0, nullptr,
                              [&]() { return min(K, (L + kBlockSize - 1) / kBlockSize); }, out,
                              count_out, K, sm, [&](int pos, int n, uint32_t) { emit(pos, n); });
}

}  // namespace kvd

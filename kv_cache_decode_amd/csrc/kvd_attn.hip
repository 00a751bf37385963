// gfx950 kernels of split-K paged decode attention.
//
//   paged_attn_kernel   split-K streaming-softmax decode attention      DirectKV review, core
//                       method 2-3; Dual-Blade background; KVDrive §2.3
//   paged_attn_mfma_kernel  the same on the matrix cores (16-bit q, G >= 2)
//   combine_kernel      log-sum-exp merge of the split partials
//
// Both attention kernels also read quantised cold pages (KVQ = 8: FP8 E4M3,
// one code byte per channel; KVQ = 4: INT4, two codes per byte) with one fp32
// scale per (page, KV head) and tensor (KVDrive §11; DirectKV review,
// assumption stress test).  Codes are decoded in registers; the K scale
// multiplies the page's logits and the V scale its softmax weights.
//
// Each K/V byte is read exactly once; nothing is re-read from another
// workgroup, so the blockIdx -> XCD placement carries no L2 reuse to exploit.
#include <math.h>

#include "kvd_device.hpp"
#include "kvd_dispatch.hpp"
#include "kvd_launch.hpp"
#include "kvd_topk.hpp"

// Launch-shape knobs (build macros): waves (= splits) per workgroup, and a
// lower bound on waves per SIMD for the MFMA kernel (0 = the compiler's
// choice), which caps its register allocation: 3 fits in 142 VGPRs without
// spilling, where the unconstrained allocation gave 180 registers (2 waves).
#ifndef KVD_ATTN_WAVES
#define KVD_ATTN_WAVES 2
#endif
#ifndef KVD_MFMA_WAVES_PER_EU
#define KVD_MFMA_WAVES_PER_EU 3
#endif
#if KVD_MFMA_WAVES_PER_EU > 0
#define KVD_MFMA_OCCUPANCY __attribute__((amdgpu_waves_per_eu(KVD_MFMA_WAVES_PER_EU)))
// tiered instances carry both page paths; 3 waves per SIMD caps them at 168
// VGPRs (registers go in granules of 8, so 169 would leave room for 2 waves).
// With INT4 cold pages that cap spills a few dozen bytes to scratch; the
// selected-list (sparse) instances, which give each compute unit few waves
// anyway, take 2 waves per SIMD and no spill (the 128k tier-policy step 43.0
// -> 40.9 us), while the dense ones keep 3 (at 2 they took 63 against 50.5 us).
#ifndef KVD_MFMA_TIER_WAVES_PER_EU
#define KVD_MFMA_TIER_WAVES_PER_EU 3
#endif
#ifndef KVD_MFMA_TIER_INT4_SPARSE_WAVES_PER_EU
#define KVD_MFMA_TIER_INT4_SPARSE_WAVES_PER_EU 2
#endif
#define KVD_MFMA_OCCUPANCY_T(cold, sparse)                                                   \
  __attribute__((amdgpu_waves_per_eu(                                                      \
      (cold) ? (((cold) == 4 && (sparse)) ? KVD_MFMA_TIER_INT4_SPARSE_WAVES_PER_EU         \
                                          : KVD_MFMA_TIER_WAVES_PER_EU)                    \
             : KVD_MFMA_WAVES_PER_EU)))
#else
#define KVD_MFMA_OCCUPANCY
#define KVD_MFMA_OCCUPANCY_T(cold, sparse)
#endif

namespace kvd {

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

// Bytes of x channels of a pool row: the storage dtype, or code bytes (KVQ 8:
// one per channel; KVQ 4: one per two channels -- x is always even there).
template <typename DT, int KVQ>
__host__ __device__ constexpr size_t kv_bytes(size_t x) {
  return KVQ == 0 ? x * sizeof(typename DT::storage) : (KVQ == 8 ? x : x / 2);
}

// A lane's chunk of one K or V row: E channels as 16 bytes of the storage
// dtype, or E codes (KVQ 8: E bytes; KVQ 4: E/2 bytes, 16-bit dtypes only).
template <typename DT, int KVQ>
struct KVChunk {
  using raw = uint4;
  __device__ static inline raw load(const uint8_t* p) { return load16_stream(p); }
  __device__ static inline void store(uint8_t* p, const raw& w) { store16(p, w); }
  __device__ static inline void widen(const raw& w, float* f) { DT::widen(w, f); }
};
template <typename DT>
struct KVChunk<DT, 4> {
  static_assert(DT::E == 8, "INT4 pages hold 16-bit channels");
  using raw = uint32_t;
  __device__ static inline raw load(const uint8_t* p) { return load4_stream(p); }
  __device__ static inline void store(uint8_t* p, const raw& w) { store4(p, w); }
  __device__ static inline void widen(const raw& w, float* f) { int4x8_to_f32(w, f); }
};
template <typename DT>
struct KVChunk<DT, 8> {
  static constexpr int E = DT::E;
  using raw = typename std::conditional<E == 8, uint2, uint32_t>::type;
  __device__ static inline raw load(const uint8_t* p) {
    if constexpr (E == 8) return load8_stream(p);
    else return load4_stream(p);
  }
  __device__ static inline void store(uint8_t* p, const raw& w) {
    if constexpr (E == 8) store8(p, w);
    else store4(p, w);
  }
  __device__ static inline void widen(const raw& w, float* f) {
    if constexpr (E == 8) {
      fp8x4_to_f32(w.x, f);
      fp8x4_to_f32(w.y, f + 4);
    } else {
      fp8x4_to_f32(w, f);
    }
  }
};

__device__ inline float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// The cache slots of (b, j) that this step fetches, as a bitmap in LDS built
// by the whole workgroup (all waves of a workgroup serve the same (b, j)).
// Slots lie below num_slots <= kCacheMaxSlots.
template <int NT>
__device__ inline const uint32_t* fetched_slot_bits(const FetchArgs& fa, int b, int j, int Hkv,
                                                   int stride, int num_slots) {
  __shared__ uint32_t bits[kCacheMaxSlots / 32];
  const size_t u = (size_t)b * Hkv + j;
  const int words = (num_slots + 31) >> 5;
  for (int w = threadIdx.x; w < words; w += NT) bits[w] = 0u;
  __syncthreads();
  const int fc = fa.fetch_count[u];
  for (int k = threadIdx.x; k < fc; k += NT) {
    const int sl = fa.fetch_slot[u * stride + k];
    atomicOr(&bits[sl >> 5], 1u << (sl & 31));
  }
  __syncthreads();
  return bits;
}

// The first 64 entries of split s's share of a selected list (and their cache
// slots), loaded before the list's count arrives, on the guess that the list
// fills its row of sel_stride entries (a Top-K selection of a long sequence
// does).  The split's chunk is ceil(count / S); the preloaded entries stand in
// for its first loads only when the guessed chunk ceil(sel_stride / S) equals
// it, so the split covers the same positions either way.  Loads stay inside
// the row.
struct ListHead {
  int n = 0, slot = 0, chunk = -1;
};

__device__ inline ListHead list_head(const int32_t* __restrict__ sel,
                                     const int32_t* __restrict__ sel_slots, size_t row,
                                     int sel_stride, int S, int s, int lane) {
  ListHead h;
  h.chunk = (sel_stride + S - 1) / S;
  const int pos = s * h.chunk + lane;
  if (lane < h.chunk && pos < sel_stride) {
    h.n = sel[row * sel_stride + pos];
    if (sel_slots) h.slot = sel_slots[row * sel_stride + pos];
  }
  return h;
}

template <typename DT, int D, int G, int WAVES, bool SPARSE, int KVQ, bool FETCH = false>
__global__ __launch_bounds__(WAVES * kWave) void paged_attn_kernel(
    const void* __restrict__ q, const void* __restrict__ k_cache, const void* __restrict__ v_cache,
    const float* __restrict__ kv_scales, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ sel_count, int sel_stride, const int32_t* __restrict__ sel_slots,
    int num_slots, int Hq, int Hkv, int maxN, int S, int PS, float qscale,
    float* __restrict__ part_o,
    float* __restrict__ part_m, float* __restrict__ part_l, float* __restrict__ block_lse,
    FetchArgs fa) {
  static_assert(!FETCH || SPARSE, "the fused fetch serves cached lists");
  using G_ = RowGeom<DT, D>;
  using St = typename DT::storage;
  using KC = KVChunk<DT, KVQ>;
  constexpr int E = G_::E, LPR = G_::LPR, TPI = G_::TPI, NI = G_::NI;
  const int lane = threadIdx.x & (kWave - 1);
  const int s = blockIdx.x * WAVES + (threadIdx.x >> 6);
  const int j = blockIdx.y, b = blockIdx.z;
  [[maybe_unused]] const uint32_t* fetched = nullptr;
  if constexpr (FETCH) fetched = fetched_slot_bits<WAVES * kWave>(fa, b, j, Hkv, sel_stride, num_slots);
  if (s >= S) return;
  const int rg = lane / LPR, c = lane % LPR;

  const int L = seq_lens[b];
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  const ListHead pre = SPARSE ? list_head(sel, sel_slots, (size_t)b * Hkv + j, sel_stride, S, s, lane)
                             : ListHead{};
  const int n_list = SPARSE ? sel_count[(size_t)b * Hkv + j] : nb;
  const int chunk = (n_list + S - 1) / S;
  const bool pre_ok = SPARSE && pre.chunk == chunk;
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

  // byte addressing (code pages: fewer bytes per channel)
  const size_t page_stride = kv_bytes<DT, KVQ>((size_t)Hkv * kBlockSize * D);
  const size_t lane_off = kv_bytes<DT, KVQ>(((size_t)j * kBlockSize + rg) * D + (size_t)c * E);
  const size_t row_step = kv_bytes<DT, KVQ>((size_t)TPI * D);
  const uint8_t* kb = static_cast<const uint8_t*>(k_cache) + lane_off;
  const uint8_t* vb = static_cast<const uint8_t*>(v_cache) + lane_off;
  const uint8_t* kbp = FETCH ? static_cast<const uint8_t*>(fa.k_pool) + lane_off : nullptr;
  const uint8_t* vbp = FETCH ? static_cast<const uint8_t*>(fa.v_pool) + lane_off : nullptr;
  uint8_t* kbw = FETCH ? static_cast<uint8_t*>(const_cast<void*>(k_cache)) + lane_off : nullptr;
  uint8_t* vbw = FETCH ? static_cast<uint8_t*>(const_cast<void*>(v_cache)) + lane_off : nullptr;
  const int32_t* sel_row = SPARSE ? sel + ((size_t)b * Hkv + j) * sel_stride : nullptr;
  const int32_t* slots_row = (SPARSE && sel_slots) ? sel_slots + ((size_t)b * Hkv + j) * sel_stride
                                                   : nullptr;
  const int32_t* bt_row = block_table ? block_table + (size_t)b * maxN : nullptr;

  for (int base = p0; base < p1; base += kWave) {
    const int cnt = min(kWave, p1 - base);
    int my_page = 0, my_valid = 0, my_pool = -1;
    float my_sk = 1.0f, my_sv = 1.0f;
    if (lane < cnt) {
      const bool use_pre = pre_ok && base == p0;
      const int n = SPARSE ? (use_pre ? pre.n : sel_row[base + lane]) : base + lane;
      // cached list: the block sits in slot sel_slots[.] of cache page b*C + slot
      const int slot = slots_row ? (use_pre ? pre.slot : slots_row[base + lane]) : 0;
      my_page = slots_row ? b * num_slots + slot : bt_row[n];
      if constexpr (FETCH) {   // fetched this step: read from the pool page
        if ((fetched[slot >> 5] >> (slot & 31)) & 1u) my_pool = bt_row[n];
      }
      my_valid = min(kBlockSize, L - n * kBlockSize);
      if constexpr (KVQ != 0) {
        const float* sp = kv_scales + ((size_t)my_page * Hkv + j) * 2;
        if constexpr (FETCH) {
          if (my_pool >= 0) sp = fa.pool_scales + ((size_t)my_pool * Hkv + j) * 2;
        }
        const float2 sc = *reinterpret_cast<const float2*>(sp);
        my_sk = sc.x;
        my_sv = sc.y;
        if constexpr (FETCH) {
          if (my_pool >= 0)
            *reinterpret_cast<float2*>(fa.cache_scales + ((size_t)my_page * Hkv + j) * 2) = sc;
        }
      }
    }
    struct PageRegs {
      typename KC::raw k[NI], v[NI];
    };
    auto load_page = [&](PageRegs& r, int idx) {
      const uint8_t* kb_ = kb;
      const uint8_t* vb_ = vb;
      size_t off = (size_t)readlane(my_page, idx) * page_stride;
      if constexpr (FETCH) {
        const int pp = readlane(my_pool, idx);   // wave-uniform
        if (pp >= 0) {
          kb_ = kbp;
          vb_ = vbp;
          off = (size_t)pp * page_stride;
        }
      }
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        r.k[it] = KC::load(kb_ + off + it * row_step);
        r.v[it] = KC::load(vb_ + off + it * row_step);
      }
    };
    auto process = [&](const PageRegs& cur, int i) {
      if constexpr (FETCH) {   // a page read from the pool goes to its cache page
        if (readlane(my_pool, i) >= 0) {
          const size_t off = (size_t)readlane(my_page, i) * page_stride;
#pragma unroll
          for (int it = 0; it < NI; ++it) {
            KC::store(kbw + off + it * row_step, cur.k[it]);
            KC::store(vbw + off + it * row_step, cur.v[it]);
          }
        }
      }
      const typename KC::raw* kc = cur.k;
      const typename KC::raw* vc = cur.v;
      const int valid = readlane(my_valid, i);
      const float sk = KVQ ? readlane_f(my_sk, i) : 1.0f;
      const float sv = KVQ ? readlane_f(my_sv, i) : 1.0f;

      // logits (log2 units) of the lane's NI tokens for every head
      float z[NI][G];
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        float kf[E];
        KC::widen(kc[it], kf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float a = 0.0f;
#pragma unroll
          for (int e = 0; e < E; ++e) a = fmaf(qf[g][e], kf[e], a);
          z[it][g] = group_reduce<LPR, OpSum>(a);
          if constexpr (KVQ != 0) z[it][g] *= sk;
        }
        if (it * TPI + rg >= valid) {
#pragma unroll
          for (int g = 0; g < G; ++g) z[it][g] = -INFINITY;
        }
      }
      // running max per head; rescale only when it grows (wave-uniform test)
      bool grow = false;
      float bm[G], psum[G];
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
      for (int g = 0; g < G; ++g) psum[g] = 0.0f;
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        float vf[E];
        KC::widen(vc[it], vf);
        if (it * TPI + rg >= valid) {  // slots past the sequence end may hold anything
#pragma unroll
          for (int e = 0; e < E; ++e) vf[e] = 0.0f;
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p = fast_exp2(z[it][g] - m[g]);
          lsum[g] += p;
          if constexpr (SPARSE) psum[g] += p;
          const float pv = KVQ ? p * sv : p;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[g][e] = fmaf(pv, vf[e], acc[g][e]);
        }
      }
      if (SPARSE && block_lse) {   // ln of the page's summed exp-logits per head (its
                                   // attention weight is exp(block_lse - lse)); lists only
#pragma unroll
        for (int g = 0; g < G; ++g) {
          // every lane of a token row holds that token's p: sum over the row groups
          const float t = cross_group_reduce<LPR, OpSum>(psum[g]);
          if (lane == 0)
            block_lse[(row0 + g) * sel_stride + base + i] = (m[g] + __log2f(t)) * kLn2;
        }
      }
    };
    // page i+1 loads while page i is computed; the last page of the group is
    // peeled off so that every load in the loop is unconditional
    PageRegs cur, nxt;
    load_page(cur, 0);
    for (int i = 0; i + 1 < cnt; ++i) {
      load_page(nxt, i + 1);
      process(cur, i);
      cur = nxt;
    }
    process(cur, cnt - 1);
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
      float* dst = part_o + ((row0 + g) * PS + s) * D + c * E;
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
      part_m[(row0 + g) * PS + s] = m[g] * kLn2;
      part_l[(row0 + g) * PS + s] = lsum[g];
    }
  }
}

// ============================================================== decode attention, MFMA path
//
// For 16-bit K/V and a GQA group of G = 2..8 query heads the two contractions
// of a page are small dense products, so they run on the matrix cores:
//
//   S^T[16 tok x 16] = K[16 tok x D] . Q^T[D x 16]       v_mfma_f32_16x16x32 (D/32 steps)
//   O[16 x D]       += P[16 x 16 tok] . V[16 tok x D]     v_mfma_f32_16x16x16 (D/16 tiles)
//
// (INT4 pages go two at a time, with one v_mfma_f32_16x16x32 per tile over the
// 32 tokens of both pages: see process2.)
//
// with the G heads padded to the 16 MFMA columns of S^T (columns >= G are zero
// queries) and to the 16 rows of O.  Lane l = 16*grp + col:
//   * K is the A operand read straight from the page: lane l holds token col,
//     channels 8*(4*st + grp) .. +8 of step st;
//   * Q^T is the B operand, loaded once: head col, the same channels;
//   * the S^T result gives lane l the logits of head col for tokens 4*grp + i,
//     i = 0..3 -- exactly the A-operand layout of P for the second product, so
//     P never moves between lanes;
//   * V rows load coalesced (lane l: token 4*grp + i, channels D/16*col ..),
//     and v_perm repacks them into the B operand (4 tokens x 1 channel per
//     lane and tile);
//   * lane l accumulates O[4*grp + i][D/16*col + n] in tile n.
// The softmax state of head col lives in every lane of that column; the rows
// of O are rescaled only when some head's running max grows.  P is fed to the
// 16-bit product as a hi + lo pair (p = hi + lo exactly up to 2^-17 relative),
// so the weights keep close to fp32 precision: rows h < G of P carry hi, rows
// G + h (otherwise padding) carry lo, and the two row sums of O are added after
// the last page, so both halves cost one product per tile.

typedef _Float16 f16x4_v __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef short s16x4_v __attribute__((ext_vector_type(4)));

template <typename DT>
struct MfmaOps;

template <>
struct MfmaOps<BF16> {
  __device__ static inline f32x4_v qk(const uint4& a, const uint4& b, f32x4_v c) {
    return mfma_16x16x32<BF16>(a, b, c);
  }
  __device__ static inline f32x4_v pv(const uint2& a, const uint2& b, f32x4_v c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_v, a),
                                                     __builtin_bit_cast(s16x4_v, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack(float lo, float hi) {  // round to nearest even
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{lo, hi}, bf16x2_v));
  }
  __device__ static inline float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static inline float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
};

template <>
struct MfmaOps<F16> {
  __device__ static inline f32x4_v qk(const uint4& a, const uint4& b, f32x4_v c) {
    return mfma_16x16x32<F16>(a, b, c);
  }
  __device__ static inline f32x4_v pv(const uint2& a, const uint2& b, f32x4_v c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_v, a),
                                                 __builtin_bit_cast(f16x4_v, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_v{lo, hi}, f16x2_v));
  }
  __device__ static inline float lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
  }
  __device__ static inline float hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
};

// The P.V operand A of a page with P = phi + plo (the weights' 16-bit high
// part and its rounding residue), for G heads in the 16 MFMA rows: rows h < G
// take phi of head h (the lane's own), rows G + h the residue plo of head h,
// moved up G lanes within each 16-lane row.  One 16x16x16 product per output
// tile then takes both halves; rows h and G + h are added once, after the
// split's last page (add_residue_rows).  Rows from 2G on carry finite values
// nothing reads.
template <int G>
__device__ inline uint2 pv_rows_hi_lo(const uint2& phi, const uint2& plo, int col) {
  static_assert(2 * G <= 16, "phi and plo rows share the 16 MFMA rows");
  // row_shr:G; lanes col < G keep phi, so what the shift leaves there is unused
  const uint32_t sx = (uint32_t)__builtin_amdgcn_mov_dpp((int)plo.x, 0x110 + G, 0xF, 0xF, true);
  const uint32_t sy = (uint32_t)__builtin_amdgcn_mov_dpp((int)plo.y, 0x110 + G, 0xF, 0xF, true);
  return make_uint2(col < G ? phi.x : sx, col < G ? phi.y : sy);
}
// Row r of an MFMA output tile sits in element r % 4 of lane group r / 4: add
// row G + h into row h (G = 2: the same lanes; G = 4 / 8: 16 / 32 lanes on).
template <int G>
__device__ inline void add_residue_rows(f32x4_v& t) {
  static_assert(G == 2 || G == 4 || G == 8, "the dispatched group sizes");
  if constexpr (G == 2) {
    t[0] += t[2];
    t[1] += t[3];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] += (G == 4) ? xor16(t[i]) : xor32(t[i]);
  }
}

// Four E4M3 codes (one dword) as four 16-bit values (two dwords), exact:
// gfx950's scaled conversion with scale 1 turns two codes straight into a
// 16-bit pair (word_sel picks codes 0-1 or 2-3).  Every E4M3 value is exact in
// bf16 and in f16 (an in-bounds probe compared all non-NaN codes with the
// fp32 route on the GPU).
template <typename DT>
__device__ inline uint2 fp8x4_to_16(uint32_t w);
template <>
__device__ inline uint2 fp8x4_to_16<BF16>(uint32_t w) {
  return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)));
}
template <>
__device__ inline uint2 fp8x4_to_16<F16>(uint32_t w) {
  return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)));
}

// NDW dwords (2*NDW 16-bit channels) of one token row, as one vector load.
template <int NDW>
struct RowWords {
  uint32_t w[NDW];
  __device__ inline void load(const void* p) {
    if constexpr (NDW == 4) {
      const uint4 v = load16_stream(p);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
      static_assert(NDW == 2, "64 or 128 channels");
      const uint2 v = load8_stream(p);
      w[0] = v.x; w[1] = v.y;
    }
  }
  __device__ inline void store(void* p) const {
    if constexpr (NDW == 4) store16(p, make_uint4(w[0], w[1], w[2], w[3]));
    else store8(p, make_uint2(w[0], w[1]));
  }
};

// INT4 codes as 16-bit MFMA operand words.  With u = n + 8 (the code's
// nibble with its sign bit flipped, 0..15) in the low four bits, the 16-bit
// pattern kExp | u is the number 2^p + u exactly (bf16: 128 + u, f16: 1024 +
// u).  f16 words then take one packed f16 subtraction of 1032, which leaves
// the code n exactly.  gfx950 has no packed bf16 arithmetic, so bf16 words
// keep the value n + kOffset (136): the kernel starts each logit sum at
// -136 * sum(q) and takes 136 * (the page's summed softmax weights) off the
// P.V sums (see the kernel).  Either way the operands are integers, exact in
// the 16-bit format, and the products are exact in fp32.
template <typename DT>
struct Int4Words;
template <>
struct Int4Words<BF16> {
  static constexpr uint32_t kExp = 0x43004300u;
  static constexpr float kOffset = 136.0f;
  __device__ static inline uint32_t fix(uint32_t w) { return w; }
};
template <>
struct Int4Words<F16> {
  static constexpr uint32_t kExp = 0x64006400u;
  static constexpr float kOffset = 0.0f;
  __device__ static inline uint32_t fix(uint32_t w) {
    const f16x2_v v = __builtin_bit_cast(f16x2_v, w) - f16x2_v{(_Float16)1032.0f, (_Float16)1032.0f};
    return __builtin_bit_cast(uint32_t, v);
  }
};
// perm selector: byte d of src1 into byte 0, byte d of src0 into byte 2, zeros
// elsewhere
__device__ constexpr uint32_t pair_sel(int d) {
  return (0x0Cu << 24) | ((4u + (uint32_t)d) << 16) | (0x0Cu << 8) | (uint32_t)d;
}
// One dword of eight K codes (channel c in nibble c) as four words holding
// the channel pairs (0, 4), (1, 5), (2, 6), (3, 7): nibbles c and c + 4 sit
// 16 bits apart, so each word is one shift and one and-or.  q's B operand
// takes the same channel order (int4_q_order).
// The nibbles at bits 0-3 and 16-19 of x as one word of two 16-bit operands:
// (nibble ^ 8) | kExp in each half, as one and + xor (kExp has no bits under
// the mask, so its or and the xor with 8 fold into one constant).
template <typename DT>
__device__ inline uint32_t int4_word(uint32_t x) {
  using W = Int4Words<DT>;
  return W::fix((x & 0x000F000Fu) ^ (W::kExp | 0x00080008u));
}
template <typename DT>
__device__ inline uint4 int4_k_words(uint32_t w) {
  return make_uint4(int4_word<DT>(w), int4_word<DT>(w >> 4), int4_word<DT>(w >> 8),
                    int4_word<DT>(w >> 12));
}
// Eight consecutive 16-bit q values (channel pairs (0, 1) .. (6, 7)) in the
// order of int4_k_words.
__device__ inline uint4 int4_q_order(const uint4& q) {
  return make_uint4(__builtin_amdgcn_perm(q.z, q.x, 0x05040100u),
                    __builtin_amdgcn_perm(q.z, q.x, 0x07060302u),
                    __builtin_amdgcn_perm(q.w, q.y, 0x05040100u),
                    __builtin_amdgcn_perm(q.w, q.y, 0x07060302u));
}
// The V codes of the lane's four tokens (v[i]: 2*NDW channels of token 4*grp+i,
// channel c in nibble c) straight into the B operands of P.V: vB[2k] holds
// channel 2k and vB[2k+1] channel 2k+1 of tokens (0, 1) in .x and (2, 3) in .y.
template <typename DT, int NDW>
__device__ inline void int4_v_operands(const uint32_t (&v)[4], uint2 (&vB)[2 * NDW]) {
#pragma unroll
  for (int k = 0; k < NDW; ++k) {
    const uint32_t t01 = __builtin_amdgcn_perm(v[1], v[0], pair_sel(k));
    const uint32_t t23 = __builtin_amdgcn_perm(v[3], v[2], pair_sel(k));
    vB[2 * k].x = int4_word<DT>(t01);
    vB[2 * k].y = int4_word<DT>(t23);
    vB[2 * k + 1].x = int4_word<DT>(t01 >> 4);
    vB[2 * k + 1].y = int4_word<DT>(t23 >> 4);
  }
}

// With FP8 code pages (KVQ 8) lane (col, grp) reads 16 K codes at a time:
// channels 64*sp + 16*grp .. +16 of token col feed QK steps 2*sp (first 8) and
// 2*sp+1 (next 8).  With INT4 pages (KVQ 4) it reads its quarter of the row at
// once: channels D/4*grp .. +D/4, eight per QK step.  The QK sum runs over all
// channels in any order, so q's B operand simply uses the same channel
// assignment.  V codes come as D/16 codes per token and decode into the 16-bit
// words the repack expects.
template <int KVQ, int D>
__device__ inline int qk_channel(int st, int grp) {
  return KVQ == 8 ? 64 * (st >> 1) + 16 * grp + 8 * (st & 1)
                  : (KVQ == 4 ? D / 4 * grp + 8 * st : 8 * (4 * st + grp));
}

// The raw page registers of format F (0: 16-bit rows, 8: E4M3, 4: INT4).
template <int F, typename R16, typename R8, typename R4>
struct PageRegsOf {
  using type = typename std::conditional<F == 8, R8,
                                         typename std::conditional<F == 4, R4, R16>::type>::type;
};

// Tiered pools (COLD = 8 or 4, with KVQ = 0): page p is read from the 16-bit
// pools when page_tier[p] == 0 (hot) and from the code pools k_cold / v_cold
// in format COLD when page_tier[p] != 0 (cold, scales in kv_scales).  Each
// group of 64 list positions runs its hot pages, then its cold pages, in two
// loops, each compiled for one page format: a cold page is read and decoded
// exactly as a code-page call reads its pages (its own lane layout, and a
// second copy of q's B operand in that layout).
// Split s of (sequence b, KV head j) by the calling wave: the body of
// paged_attn_mfma_kernel, and of the fused select + attention kernel, which
// passes its list (LDS_LIST: the list count and a pointer that indexes the
// list by position) instead of sel / sel_count.
template <typename DT, int D, int G, bool SPARSE, int KVQ, int COLD, bool FETCH, bool LDS_LIST>
__device__ __forceinline__ void mfma_attn_split(
    const void* __restrict__ q, const void* __restrict__ k_cache, const void* __restrict__ v_cache,
    const float* __restrict__ kv_scales, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ sel_count, int sel_stride, const int32_t* __restrict__ sel_slots,
    int num_slots, int Hq, int Hkv, int maxN, int S, int PS, float qscale,
    float* __restrict__ part_o,
    float* __restrict__ part_m, float* __restrict__ part_l, float* __restrict__ block_lse,
    const void* __restrict__ k_cold, const void* __restrict__ v_cold,
    const uint8_t* __restrict__ page_tier, const FetchArgs& fa, const uint32_t* fetched, int s,
    int j, int b, int list_count, const int32_t* list, int list_first) {
  static_assert(G >= 2 && G <= 8, "the group fills 2..8 of the 16 MFMA rows");
  static_assert(COLD == 0 || KVQ == 0, "tiered pools pair 16-bit hot pages with code pages");
  static_assert(!FETCH || (SPARSE && COLD == 0), "the fused fetch serves cached lists");
  static_assert(!LDS_LIST || (SPARSE && !FETCH && COLD == 0), "a given list is a plain selection");
  using St = typename DT::storage;
  using Ops = MfmaOps<DT>;
  constexpr int KS = D / 32;   // QK steps of 32 channels
  constexpr int NT = D / 16;   // PV tiles of 16 output channels
  constexpr int NDW = D / 32;  // dwords of V per lane and token (D/16 channels)
  const int lane = threadIdx.x & (kWave - 1);
  if (s >= S) return;
  const int col = lane & 15, grp = lane >> 4;

  const int L = seq_lens[b];
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  const ListHead pre = (SPARSE && !LDS_LIST)
                           ? list_head(sel, sel_slots, (size_t)b * Hkv + j, sel_stride, S, s, lane)
                           : ListHead{};
  const int n_list = LDS_LIST ? list_count : (SPARSE ? sel_count[(size_t)b * Hkv + j] : nb);
  const int chunk = (n_list + S - 1) / S;
  const bool pre_ok = SPARSE && !LDS_LIST && pre.chunk == chunk;
  const int p0 = min(s * chunk, n_list);
  const int p1 = min(p0 + chunk, n_list);
  const size_t row0 = (size_t)b * Hq + (size_t)j * G;

  // q's B operand for pages of format F (0: 16-bit rows, 8: E4M3, 4: INT4), in
  // the channel order that format's K loads give each lane
  using FmtP = std::integral_constant<int, KVQ>;    // the pools k_cache / v_cache
  using FmtC = std::integral_constant<int, COLD>;   // tiered calls' cold pools
  auto load_qB = [&](uint4 (&qb)[KS], auto fmt) {
    constexpr int F = decltype(fmt)::value;
#pragma unroll
    for (int st = 0; st < KS; ++st)
      qb[st] = col < G ? load16(static_cast<const St*>(q) + (row0 + col) * D + qk_channel<F, D>(st, grp))
                       : make_uint4(0, 0, 0, 0);
    if constexpr (F == 4) {
#pragma unroll
      for (int st = 0; st < KS; ++st) qb[st] = int4_q_order(qb[st]);
    }
  };
  uint4 qB[KS], qBc[KS];
  load_qB(qB, FmtP{});
  if constexpr (COLD != 0) load_qB(qBc, FmtC{});
  // bf16 INT4 pages give operands of code + 136 (Int4Words): a page's logit
  // sums start at -136 * sum_c q_c of their head (the lane's column; the sum is
  // the same in any channel order), and vcorr accumulates P times a row of
  // ones (each head's summed weights) beside o, so o - 136 * vcorr is the sum
  // over the codes.  vcorr is folded into o every eight pages, which keeps o's
  // magnitude (and so its rounding) near that of the true sum.
  constexpr bool kInt4Off = std::is_same<DT, BF16>::value && (KVQ == 4 || COLD == 4);
  float qcorr = 0.0f;
  if constexpr (kInt4Off) {
    float t = 0.0f;
#pragma unroll
    for (int st = 0; st < KS; ++st)
      t += ((Ops::lo(qB[st].x) + Ops::hi(qB[st].x)) + (Ops::lo(qB[st].y) + Ops::hi(qB[st].y))) +
           ((Ops::lo(qB[st].z) + Ops::hi(qB[st].z)) + (Ops::lo(qB[st].w) + Ops::hi(qB[st].w)));
    t += xor16(t);
    t += xor32(t);
    qcorr = -Int4Words<DT>::kOffset * t;
  }
  f32x4_v vcorr = {0.f, 0.f, 0.f, 0.f};


  f32x4_v o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.0f;
  auto fold_vcorr = [&]() {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[n][i] = fmaf(-Int4Words<DT>::kOffset, vcorr[i], o[n][i]);
    vcorr = f32x4_v{0.f, 0.f, 0.f, 0.f};
  };

  // byte addressing per page format (code pages: fewer bytes per channel): the
  // lane's K and V offsets inside a page of KV head j, and the page stride
  struct Lanes {
    size_t k, v, stride;
  };
  auto lanes = [&](auto fmt) {
    constexpr int F = decltype(fmt)::value;
    constexpr int KCH = F == 8 ? 16 : (F == 4 ? D / 4 : 8);   // K channels a lane starts at, per grp
    return Lanes{kv_bytes<DT, F>((size_t)j * kBlockSize * D + (size_t)col * D + KCH * grp),
                 kv_bytes<DT, F>((size_t)j * kBlockSize * D + (size_t)(4 * grp) * D + 2 * NDW * col),
                 kv_bytes<DT, F>((size_t)Hkv * kBlockSize * D)};
  };
  const Lanes lp = lanes(FmtP{});
  const size_t page_stride = lp.stride, k_lane = lp.k, v_lane = lp.v;
  const uint8_t* kb = static_cast<const uint8_t*>(k_cache) + k_lane;
  const uint8_t* vb = static_cast<const uint8_t*>(v_cache) + v_lane;
  // fused fetch: the pools a fetched block is read from, and the cache pages
  // it is stored to (the same lane offsets: pools and cache share the layout)
  const uint8_t* kbp = FETCH ? static_cast<const uint8_t*>(fa.k_pool) + k_lane : nullptr;
  const uint8_t* vbp = FETCH ? static_cast<const uint8_t*>(fa.v_pool) + v_lane : nullptr;
  uint8_t* kbw = FETCH ? static_cast<uint8_t*>(const_cast<void*>(k_cache)) + k_lane : nullptr;
  uint8_t* vbw = FETCH ? static_cast<uint8_t*>(const_cast<void*>(v_cache)) + v_lane : nullptr;
  // the cold pools of tiered calls, in the code format's own lane layout
  const Lanes lc = lanes(FmtC{});
  const size_t page_stride_c = lc.stride;
  const uint8_t* kbc = COLD ? static_cast<const uint8_t*>(k_cold) + lc.k : nullptr;
  const uint8_t* vbc = COLD ? static_cast<const uint8_t*>(v_cold) + lc.v : nullptr;
  const int32_t* sel_row = LDS_LIST ? list : (SPARSE ? sel + ((size_t)b * Hkv + j) * sel_stride : nullptr);
  const int32_t* slots_row = (SPARSE && sel_slots) ? sel_slots + ((size_t)b * Hkv + j) * sel_stride
                                                   : nullptr;
  const int32_t* bt_row = block_table ? block_table + (size_t)b * maxN : nullptr;

  for (int base = p0; base < p1; base += kWave) {
    const int cnt = min(kWave, p1 - base);
    int my_page = 0, my_valid = 0, my_tier = 0, my_pool = -1;
    float my_sk = 1.0f, my_sv = 1.0f;
    if (lane < cnt) {
      const bool use_pre = pre_ok && base == p0;
      // a given list holds positions list_first.. (the caller's share of it)
      const int n = SPARSE ? (use_pre ? pre.n : sel_row[base + lane - (LDS_LIST ? list_first : 0)])
                           : base + lane;
      // cached list: the block sits in slot sel_slots[.] of cache page b*C + slot
      const int slot = slots_row ? (use_pre ? pre.slot : slots_row[base + lane]) : 0;
      my_page = slots_row ? b * num_slots + slot : bt_row[n];
      if constexpr (FETCH) {   // fetched this step: read from the pool page
        if ((fetched[slot >> 5] >> (slot & 31)) & 1u) my_pool = bt_row[n];
      }
      my_valid = min(kBlockSize, L - n * kBlockSize);
      if constexpr (KVQ != 0 || COLD != 0) {
        const float* sp = kv_scales + ((size_t)my_page * Hkv + j) * 2;
        if constexpr (FETCH) {
          if (my_pool >= 0) sp = fa.pool_scales + ((size_t)my_pool * Hkv + j) * 2;
        }
        const float2 sc = *reinterpret_cast<const float2*>(sp);
        my_sk = sc.x;
        my_sv = sc.y;
        if constexpr (FETCH) {
          if (my_pool >= 0)
            *reinterpret_cast<float2*>(fa.cache_scales + ((size_t)my_page * Hkv + j) * 2) = sc;
        }
      }
      if constexpr (COLD != 0) my_tier = page_tier[my_page];
    }
    // raw registers of one page: 16-bit rows, E4M3 codes (K: 16 per load,
    // V: D/16 per token row, NDW/2 dwords), or INT4 codes (K: D/4 per lane in
    // one load, one dword per QK step; V: D/16 per token row in 4 or 2 bytes)
    struct PageRegs16 {
      uint4 k[KS];
      RowWords<NDW> v[4];
    };
    struct PageRegs8 {
      uint4 k[KS / 2];
      uint32_t v[4][NDW / 2];
    };
    struct PageRegs4 {
      uint32_t k[KS];
      uint32_t v[4];
    };
    using PageRegs = typename PageRegsOf<KVQ, PageRegs16, PageRegs8, PageRegs4>::type;
    // fmt (std::integral_constant<int, F>): the format of page idx, known at
    // compile time in each page loop; a tiered call's cold pages (F = COLD)
    // come from the cold pools
    auto load_page = [&](auto& r, int idx, auto fmt) {
      constexpr int F = decltype(fmt)::value;
      constexpr bool kCold = COLD != 0 && F == COLD;
      const uint8_t* kb_ = kCold ? kbc : kb;
      const uint8_t* vb_ = kCold ? vbc : vb;
      size_t off = (size_t)readlane(my_page, idx) * (kCold ? page_stride_c : page_stride);
      if constexpr (FETCH) {
        const int pp = readlane(my_pool, idx);   // wave-uniform
        if (pp >= 0) {
          kb_ = kbp;
          vb_ = vbp;
          off = (size_t)pp * page_stride;
        }
      }
      if constexpr (F == 4) {
        if constexpr (KS == 4) {
          const uint4 t = load16_stream(kb_ + off);
          r.k[0] = t.x; r.k[1] = t.y; r.k[2] = t.z; r.k[3] = t.w;
        } else {
          const uint2 t = load8_stream(kb_ + off);
          r.k[0] = t.x; r.k[1] = t.y;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (NDW == 4) r.v[i] = load4_stream(vb_ + off + (size_t)i * (D / 2));
          else r.v[i] = load2_stream(vb_ + off + (size_t)i * (D / 2));
        }
      } else if constexpr (F == 8) {
#pragma unroll
        for (int sp = 0; sp < KS / 2; ++sp) r.k[sp] = load16_stream(kb_ + off + 64 * sp);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (NDW / 2 == 2) {
            const uint2 t = load8_stream(vb_ + off + (size_t)i * D);
            r.v[i][0] = t.x;
            r.v[i][1] = t.y;
          } else {
            r.v[i][0] = load4_stream(vb_ + off + (size_t)i * D);
          }
        }
      } else {
#pragma unroll
        for (int st = 0; st < KS; ++st) r.k[st] = load16_stream(kb_ + off + kv_bytes<DT, 0>(32 * st));
#pragma unroll
        for (int i = 0; i < 4; ++i) r.v[i].load(vb_ + off + kv_bytes<DT, 0>((size_t)i * D));
      }
    };
    // fused fetch: a page read from the pool goes to its cache page, from the
    // same registers and lane offsets it was loaded with
    auto store_page = [&](const auto& r, size_t off) {
      if constexpr (KVQ == 4) {
        if constexpr (KS == 4) store16(kbw + off, make_uint4(r.k[0], r.k[1], r.k[2], r.k[3]));
        else store8(kbw + off, make_uint2(r.k[0], r.k[1]));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (NDW == 4) store4(vbw + off + (size_t)i * (D / 2), r.v[i]);
          else store2(vbw + off + (size_t)i * (D / 2), r.v[i]);
        }
      } else if constexpr (KVQ == 8) {
#pragma unroll
        for (int sp = 0; sp < KS / 2; ++sp) store16(kbw + off + 64 * sp, r.k[sp]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (NDW / 2 == 2) store8(vbw + off + (size_t)i * D, make_uint2(r.v[i][0], r.v[i][1]));
          else store4(vbw + off + (size_t)i * D, r.v[i][0]);
        }
      } else {
#pragma unroll
        for (int st = 0; st < KS; ++st) store16(kbw + off + kv_bytes<DT, 0>(32 * st), r.k[st]);
#pragma unroll
        for (int i = 0; i < 4; ++i) r.v[i].store(vbw + off + kv_bytes<DT, 0>((size_t)i * D));
      }
    };
    // raise the running max of each head to the page's (or pair's) max bm where
    // it grows, rescaling the sums (the test is wave-uniform)
    auto grow_max = [&](float bm) {
      if (__builtin_amdgcn_ballot_w64(col < G && bm > m)) {
        const float mn = fmaxf(m, bm);
        const float alpha = fast_exp2(m - mn);
        m = mn;
        lsum *= alpha;
        float ar[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, (4 * grp + i) & (G - 1), kWave);
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[n][i] *= ar[i];
        if constexpr (kInt4Off) {   // (vcorr is zero between the INT4 pages of a tiered call)
#pragma unroll
          for (int i = 0; i < 4; ++i) vcorr[i] *= ar[i];
        }
      }
    };
    // one page of compute; `cur` holds page `it` of the group
    auto process = [&](const auto& cur, int it, auto fmt) {
      constexpr int F = decltype(fmt)::value;
      constexpr bool kCold = COLD != 0 && F == COLD;
      if constexpr (FETCH) {
        if (readlane(my_pool, it) >= 0) store_page(cur, (size_t)readlane(my_page, it) * page_stride);
      }
      const int valid = readlane(my_valid, it);
      const float sk = F ? readlane_f(my_sk, it) : 1.0f;
      const float sv = F ? readlane_f(my_sv, it) : 1.0f;

      // 16-bit operands of the page: K words kA, and V rows vr that become the
      // P.V operands below (INT4 V codes are decoded straight into them there,
      // after the softmax, when fewer registers are live)
      uint4 kA[KS];
      RowWords<NDW> vr[4];
      if constexpr (F == 4) {
#pragma unroll
        for (int st = 0; st < KS; ++st) kA[st] = int4_k_words<DT>(cur.k[st]);
      } else if constexpr (F == 8) {
#pragma unroll
        for (int sp = 0; sp < KS / 2; ++sp) {
          const uint2 a0 = fp8x4_to_16<DT>(cur.k[sp].x), a1 = fp8x4_to_16<DT>(cur.k[sp].y);
          const uint2 b0 = fp8x4_to_16<DT>(cur.k[sp].z), b1 = fp8x4_to_16<DT>(cur.k[sp].w);
          kA[2 * sp] = make_uint4(a0.x, a0.y, a1.x, a1.y);
          kA[2 * sp + 1] = make_uint4(b0.x, b0.y, b1.x, b1.y);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int k = 0; k < NDW / 2; ++k) {
            const uint2 t = fp8x4_to_16<DT>(cur.v[i][k]);
            vr[i].w[2 * k] = t.x;
            vr[i].w[2 * k + 1] = t.y;
          }
      } else {
#pragma unroll
        for (int st = 0; st < KS; ++st) kA[st] = cur.k[st];
#pragma unroll
        for (int i = 0; i < 4; ++i) vr[i] = cur.v[i];
      }

      f32x4_v sacc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (kInt4Off && F == 4) {
        sacc = f32x4_v{qcorr, qcorr, qcorr, qcorr};
      }
#pragma unroll
      for (int st = 0; st < KS; ++st) sacc = Ops::qk(kA[st], kCold ? qBc[st] : qB[st], sacc);
      const float zs = qscale * sk;
      float z[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = sacc[i] * zs;
      if (valid < kBlockSize) {   // wave-uniform: only a sequence's last page is partial
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = (4 * grp + i < valid) ? z[i] : -INFINITY;
      }
      grow_max(rows_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]))));
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(z[i] - m);
      lsum += (p[0] + p[1]) + (p[2] + p[3]);
      if (SPARSE && block_lse) {   // ln of the page's summed exp-logits per head; lists only
        float ps = (p[0] + p[1]) + (p[2] + p[3]);
        ps += xor16(ps);
        ps += xor32(ps);
        if (grp == 0 && col < G)
          block_lse[(row0 + col) * sel_stride + base + it] = (m + __log2f(ps)) * kLn2;
      }
      if constexpr (F != 0) {    // the page's V scale rides on its weights
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] *= sv;
      }
      uint2 phi, plo;
      phi.x = Ops::pack(p[0], p[1]);
      phi.y = Ops::pack(p[2], p[3]);
      plo.x = Ops::pack(p[0] - Ops::lo(phi.x), p[1] - Ops::hi(phi.x));
      plo.y = Ops::pack(p[2] - Ops::lo(phi.y), p[3] - Ops::hi(phi.y));

      uint2 vB[NT];
      if constexpr (F == 4) {
        int4_v_operands<DT, NDW>(cur.v, vB);
      } else {
        if (valid < kBlockSize) {  // slots past the sequence end may hold anything
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * grp + i >= valid)
#pragma unroll
              for (int k = 0; k < NDW; ++k) vr[i].w[k] = 0u;
        }
#pragma unroll
        for (int k = 0; k < NDW; ++k) {
          vB[2 * k].x = __builtin_amdgcn_perm(vr[1].w[k], vr[0].w[k], 0x05040100u);
          vB[2 * k].y = __builtin_amdgcn_perm(vr[3].w[k], vr[2].w[k], 0x05040100u);
          vB[2 * k + 1].x = __builtin_amdgcn_perm(vr[1].w[k], vr[0].w[k], 0x07060302u);
          vB[2 * k + 1].y = __builtin_amdgcn_perm(vr[3].w[k], vr[2].w[k], 0x07060302u);
        }
      }
      // (INT4 operands of slots past the sequence end are finite and meet
      // weights of exactly 0)
      const uint2 pa = pv_rows_hi_lo<G>(phi, plo, col);
#pragma unroll
      for (int n = 0; n < NT; ++n) o[n] = Ops::pv(pa, vB[n], o[n]);
      if constexpr (kInt4Off && F == 4) {
        const uint2 ones = make_uint2(0x3F803F80u, 0x3F803F80u);   // bf16 1.0 pairs
        vcorr = Ops::pv(pa, ones, vcorr);
        if ((it & 7) == 7) fold_vcorr();
      }

    };
    // Two INT4 pages (ia, ib) of the pools at once.  The P.V products take the
    // 32 tokens of both pages per 16x16x32 product: in lane group g, k slots
    // 0-3 hold page a's tokens 4g..4g+3 and slots 4-7 page b's, in P's operand
    // (rows h < G: hi, rows G + h: lo, as pv_rows_hi_lo) and in V's alike.
    // That is half the products of one page at a time, and the running max is
    // raised once per pair.
    // K operand words of QK step st, and the P.V B operands (vB[n]: output
    // tile n), of a code page of format F (8 or 4); V rows of tokens past a
    // partial page's end are zeroed first (E4M3 slots there may hold NaN codes;
    // INT4 codes are always finite and meet weights of exactly 0)
    auto code_k_words = [&](const auto& cur, int st, auto fmt) -> uint4 {
      if constexpr (decltype(fmt)::value == 4) {
        return int4_k_words<DT>(cur.k[st]);
      } else {
        const uint4 w = cur.k[st >> 1];
        const uint2 a0 = fp8x4_to_16<DT>((st & 1) ? w.z : w.x);
        const uint2 a1 = fp8x4_to_16<DT>((st & 1) ? w.w : w.y);
        return make_uint4(a0.x, a0.y, a1.x, a1.y);
      }
    };
    auto code_v_operands = [&](const auto& cur, int valid, uint2 (&vB)[NT], auto fmt) {
      if constexpr (decltype(fmt)::value == 4) {
        int4_v_operands<DT, NDW>(cur.v, vB);
      } else {
        RowWords<NDW> vr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int k = 0; k < NDW / 2; ++k) {
            const uint2 t = fp8x4_to_16<DT>(cur.v[i][k]);
            vr[i].w[2 * k] = t.x;
            vr[i].w[2 * k + 1] = t.y;
          }
        if (valid < kBlockSize) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * grp + i >= valid)
#pragma unroll
              for (int k = 0; k < NDW; ++k) vr[i].w[k] = 0u;
        }
#pragma unroll
        for (int k = 0; k < NDW; ++k) {
          vB[2 * k].x = __builtin_amdgcn_perm(vr[1].w[k], vr[0].w[k], 0x05040100u);
          vB[2 * k].y = __builtin_amdgcn_perm(vr[3].w[k], vr[2].w[k], 0x05040100u);
          vB[2 * k + 1].x = __builtin_amdgcn_perm(vr[1].w[k], vr[0].w[k], 0x07060302u);
          vB[2 * k + 1].y = __builtin_amdgcn_perm(vr[3].w[k], vr[2].w[k], 0x07060302u);
        }
      }
    };
    auto process2 = [&](const auto& ca, const auto& cb, int ia, int ib, auto fmt) {
      constexpr int F = decltype(fmt)::value;
      static_assert(F == 4 || F == 8, "pairs of code pages");
      constexpr bool kCold = COLD != 0 && F == COLD;
      if constexpr (FETCH) {   // pages read from the pool go to their cache pages
        if (readlane(my_pool, ia) >= 0) store_page(ca, (size_t)readlane(my_page, ia) * page_stride);
        if (readlane(my_pool, ib) >= 0) store_page(cb, (size_t)readlane(my_page, ib) * page_stride);
      }
      const int vla = readlane(my_valid, ia), vlb = readlane(my_valid, ib);
      const float zsa = qscale * readlane_f(my_sk, ia), zsb = qscale * readlane_f(my_sk, ib);
      const float sva = readlane_f(my_sv, ia), svb = readlane_f(my_sv, ib);
      f32x4_v sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
      if constexpr (kInt4Off && F == 4) {
        sa = f32x4_v{qcorr, qcorr, qcorr, qcorr};
        sb = sa;
      }
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        sa = Ops::qk(code_k_words(ca, st, fmt), kCold ? qBc[st] : qB[st], sa);
        sb = Ops::qk(code_k_words(cb, st, fmt), kCold ? qBc[st] : qB[st], sb);
      }
      float z[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = sa[i] * zsa;
        z[4 + i] = sb[i] * zsb;
      }
      if (vla < kBlockSize) {   // wave-uniform: partial last pages only
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = (4 * grp + i < vla) ? z[i] : -INFINITY;
      }
      if (vlb < kBlockSize) {
#pragma unroll
        for (int i = 0; i < 4; ++i) z[4 + i] = (4 * grp + i < vlb) ? z[4 + i] : -INFINITY;
      }
      grow_max(rows_max(fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])),
                              fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])))));
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = fast_exp2(z[i] - m);
      const float psa = (p[0] + p[1]) + (p[2] + p[3]), psb = (p[4] + p[5]) + (p[6] + p[7]);
      lsum += psa + psb;
      if (SPARSE && block_lse) {   // ln of each page's summed exp-logits per head; lists only
        float ta = psa, tb = psb;
        ta += xor16(ta);
        ta += xor32(ta);
        tb += xor16(tb);
        tb += xor32(tb);
        if (grp == 0 && col < G) {
          block_lse[(row0 + col) * sel_stride + base + ia] = (m + __log2f(ta)) * kLn2;
          block_lse[(row0 + col) * sel_stride + base + ib] = (m + __log2f(tb)) * kLn2;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // each page's V scale rides on its weights
        p[i] *= sva;
        p[4 + i] *= svb;
      }
      uint2 ph[2], pl[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        ph[h].x = Ops::pack(p[4 * h], p[4 * h + 1]);
        ph[h].y = Ops::pack(p[4 * h + 2], p[4 * h + 3]);
        pl[h].x = Ops::pack(p[4 * h] - Ops::lo(ph[h].x), p[4 * h + 1] - Ops::hi(ph[h].x));
        pl[h].y = Ops::pack(p[4 * h + 2] - Ops::lo(ph[h].y), p[4 * h + 3] - Ops::hi(ph[h].y));
      }
      const uint2 xa = pv_rows_hi_lo<G>(ph[0], pl[0], col), xb = pv_rows_hi_lo<G>(ph[1], pl[1], col);
      const uint4 pa = make_uint4(xa.x, xa.y, xb.x, xb.y);
      uint2 va[NT], vb2[NT];
      code_v_operands(ca, vla, va, fmt);
      code_v_operands(cb, vlb, vb2, fmt);
#pragma unroll
      for (int n = 0; n < NT; ++n)
        o[n] = mfma_16x16x32<DT>(pa, make_uint4(va[n].x, va[n].y, vb2[n].x, vb2[n].y), o[n]);
      if constexpr (kInt4Off && F == 4) {
        const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
        vcorr = mfma_16x16x32<DT>(pa, ones, vcorr);
        if ((ib & 7) == 7) fold_vcorr();
      }
    };
    // page it+1 loads while page it is computed; the group's last page is
    // peeled off so every load in the loop is unconditional.  (With a
    // conditional prefetch the compiler waited for every outstanding load, the
    // prefetch included, before using a page.)
    if constexpr (COLD != 0) {
      // Tiered calls: the group's hot pages, then its cold pages, each in a
      // loop of its own, so a loop carries one page path and the two paths'
      // registers are not live at once.  The masks are wave-uniform.
      const uint64_t live = cnt >= kWave ? ~0ull : ((1ull << cnt) - 1ull);
      const uint64_t cold_mask = __builtin_amdgcn_ballot_w64(my_tier != 0) & live;
      auto run = [&](uint64_t mask, auto fmt) {
        if (mask == 0) return;
        using Regs = typename PageRegsOf<decltype(fmt)::value, PageRegs16, PageRegs8, PageRegs4>::type;
        int idx = __builtin_ctzll(mask);
        mask &= mask - 1;
        Regs cur, nxt;
        load_page(cur, idx, fmt);
        while (mask != 0) {
          const int nx = __builtin_ctzll(mask);
          mask &= mask - 1;
          load_page(nxt, nx, fmt);
          process(cur, idx, fmt);
          cur = nxt;
          idx = nx;
        }
        process(cur, idx, fmt);
      };
      run(live & ~cold_mask, std::integral_constant<int, 0>{});
      run(cold_mask, FmtC{});
    } else if constexpr (KVQ == 4) {
      // INT4 pools: pages two at a time (process2), the next pair loading
      // while the current one is computed; an odd last page takes process.
      // (FP8 pools measured slower in pairs, 48.1 against 46.5 us for the 128k
      // dense call, also with their two-codes-per-instruction conversion.)
      // (Two register sets used in turn, two pairs per trip, measured slower
      // for INT4 pages: the compiler then needs more registers than three
      // waves per SIMD allow.  Tiered calls keep one page at a time: their
      // instances carry both page paths and have no registers to spare.  The
      // fused-fetch instances pair pages too, so a fetch inside the attention
      // gives the same sums as the fetch before it.)
      PageRegs ra, rb, na, nb;
      int it = 0;
      if (cnt >= 2) {
        load_page(ra, 0, FmtP{});
        load_page(rb, 1, FmtP{});
        for (; it + 3 < cnt; it += 2) {
          load_page(na, it + 2, FmtP{});
          load_page(nb, it + 3, FmtP{});
          process2(ra, rb, it, it + 1, FmtP{});
          ra = na;
          rb = nb;
        }
        if (it + 2 < cnt) load_page(na, it + 2, FmtP{});
        process2(ra, rb, it, it + 1, FmtP{});
        it += 2;
      } else {
        load_page(na, 0, FmtP{});
      }
      if (it < cnt) process(na, it, FmtP{});
    } else {
      PageRegs cur, nxt;
      load_page(cur, 0, FmtP{});
      for (int it = 0; it + 1 < cnt; ++it) {
        load_page(nxt, it + 1, FmtP{});
        process(cur, it, FmtP{});
        cur = nxt;
      }
      process(cur, cnt - 1, FmtP{});
    }
  }

  if constexpr (kInt4Off) fold_vcorr();
#pragma unroll
  for (int n = 0; n < NT; ++n) add_residue_rows<G>(o[n]);
  // totals per head (the four k-groups of a column saw disjoint tokens)
  lsum += xor16(lsum);
  lsum += xor32(lsum);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = 4 * grp + i;                  // output row held in o[.][i]
    const float lt = __shfl(lsum, g & 15, kWave);
    if (g < G) {
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
      float* dst = part_o + ((row0 + g) * PS + s) * D + 2 * NDW * col;
#pragma unroll
      for (int n4 = 0; n4 < NT; n4 += 4)
        *reinterpret_cast<float4*>(dst + n4) =
            make_float4(o[n4][i] * inv, o[n4 + 1][i] * inv, o[n4 + 2][i] * inv,
                        o[n4 + 3][i] * inv);
    }
  }
  if (grp == 0 && col < G) {
    part_m[(row0 + col) * PS + s] = m * kLn2;
    part_l[(row0 + col) * PS + s] = lsum;
  }
}

template <typename DT, int D, int G, int WAVES, bool SPARSE, int KVQ, int COLD = 0, bool FETCH = false>
__global__ __launch_bounds__(WAVES * kWave) KVD_MFMA_OCCUPANCY_T(COLD, SPARSE) void paged_attn_mfma_kernel(
    const void* __restrict__ q, const void* __restrict__ k_cache, const void* __restrict__ v_cache,
    const float* __restrict__ kv_scales, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ sel_count, int sel_stride, const int32_t* __restrict__ sel_slots,
    int num_slots, int Hq, int Hkv, int maxN, int S, int PS, float qscale,
    float* __restrict__ part_o,
    float* __restrict__ part_m, float* __restrict__ part_l, float* __restrict__ block_lse,
    const void* __restrict__ k_cold, const void* __restrict__ v_cold,
    const uint8_t* __restrict__ page_tier, FetchArgs fa) {
  const int s = blockIdx.x * WAVES + (threadIdx.x >> 6);
  const int j = blockIdx.y, b = blockIdx.z;
  [[maybe_unused]] const uint32_t* fetched = nullptr;
  if constexpr (FETCH) fetched = fetched_slot_bits<WAVES * kWave>(fa, b, j, Hkv, sel_stride, num_slots);
  mfma_attn_split<DT, D, G, SPARSE, KVQ, COLD, FETCH, false>(
      q, k_cache, v_cache, kv_scales, block_table, seq_lens, sel, sel_count, sel_stride, sel_slots,
      num_slots, Hq, Hkv, maxN, S, PS, qscale, part_o, part_m, part_l, block_lse, k_cold, v_cold,
      page_tier, fa, fetched, s, j, b, 0, nullptr, 0);
}

// ============================================================== select + attention in one launch
//
// KVDrive §2.3 selects the critical blocks, then computes attention over them.
// Here the Top-K and the sparse attention of a (sequence, KV head) row share
// one launch: each workgroup of kSelAttnWaves waves takes that many
// consecutive splits of the row's selected list.  It first runs the row's
// Top-K itself (topk_row: the Top-K launch's algorithm, so the list is the
// same bit for bit; the workgroups of a row repeat it side by side), keeps
// the list positions of its own splits in LDS, and then each wave attends its
// split from that list (mfma_attn_split: the attention launch's code and
// partition, so the partials are the same bit for bit).  Workgroup 0 of each
// row writes the list and its count.  This saves the Top-K launch's fixed
// cost and the list's round trip through memory; it pays while the repeated
// Top-K is short (rows of at most kSelAttnMaxBlocks blocks) and each compute
// unit holds about one such workgroup (kv_auto_select_splits).

template <typename DT, int D, int G, int EPT>
__global__ __launch_bounds__(kSelAttnWaves * kWave) KVD_MFMA_OCCUPANCY void select_attn_mfma_kernel(
    const float* __restrict__ scores, int K, int sink, int local, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_count, const void* __restrict__ q,
    const void* __restrict__ k_cache, const void* __restrict__ v_cache,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int Hq,
    int Hkv, int maxN, int S, float qscale, float* __restrict__ part_o,
    float* __restrict__ part_m, float* __restrict__ part_l) {
  constexpr int W = kSelAttnWaves, NT = W * kWave;
  __shared__ TopkSmemFor<NT, EPT> sm;
  __shared__ int32_t lst[kSelAttnListMax];
  const int j = blockIdx.y, b = blockIdx.z;
  const size_t u = (size_t)b * Hkv + j;
  const int L = seq_lens[b];
  const int keff = min(K, (L + kBlockSize - 1) / kBlockSize);
  const int chunk = (keff + S - 1) / S;        // the attention launch's partition
  const int first = min((int)blockIdx.x * W * chunk, keff);
  const int last = min(first + W * chunk, keff);
  int32_t* out = blockIdx.x == 0 ? sel + u * K : nullptr;
  topk_row<NT, EPT>(scores + u * maxN, maxN, L, K, sink, local, out, sel_count + u, sm,
                    [&](int pos, int n) {
                      if (pos >= first && pos < last) lst[pos - first] = n;
                      if (out) out[pos] = n;
                    });
  __syncthreads();
  mfma_attn_split<DT, D, G, true, 0, 0, false, true>(
      q, k_cache, v_cache, nullptr, block_table, seq_lens, nullptr, nullptr, K, nullptr, 0, Hq,
      Hkv, maxN, S, S, qscale, part_o, part_m, part_l, nullptr, nullptr, nullptr, nullptr,
      FetchArgs{}, nullptr, (int)blockIdx.x * W + (int)(threadIdx.x >> 6), j, b, keff, lst, first);
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

// R > 0: S <= R * SLOTS, and each thread issues the loads of all its split
// slots (m, l and its four o channels) before the first reduction, so the
// partials arrive in one memory round trip; R = 0 loops for larger S, with
// the m loads first and the o loads after the maximum.
template <int R>
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

  const int slot = tid / TPS, q4 = tid % TPS;
  const float* po = part_o + (row * S) * D + d0 + q4 * 4;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  float W = 0.0f;
  float M = -INFINITY;
  if constexpr (R > 0) {
    float ms[R], ls[R];
    float4 os[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int s = slot + r * SLOTS;
      ms[r] = -INFINITY;
      ls[r] = 0.0f;
      os[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s < S) {
        ms[r] = pm[s];
        ls[r] = pl[s];
        os[r] = *reinterpret_cast<const float4*>(po + (size_t)s * D);
      }
      M = fmaxf(M, ms[r]);
    }
    M = group_reduce<kWave, OpMax>(M);
    if ((tid & (kWave - 1)) == 0) red[tid >> 6] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float w = (ms[r] == -INFINITY) ? 0.0f : ls[r] * expf(ms[r] - M);
      W += w;
      a.x = fmaf(w, os[r].x, a.x);
      a.y = fmaf(w, os[r].y, a.y);
      a.z = fmaf(w, os[r].z, a.z);
      a.w = fmaf(w, os[r].w, a.w);
    }
  } else {
    for (int s = tid; s < S; s += 256) M = fmaxf(M, pm[s]);
    M = group_reduce<kWave, OpMax>(M);
    if ((tid & (kWave - 1)) == 0) red[tid >> 6] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
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

// Few splits (S <= kCombineFew): one thread per (row, float4 of channels)
// walks all S splits, issuing every load before the first reduction; a row's
// D/4 threads read the same m and l.  The sums run in split order, each term
// rounded on its own as in the workgroup kernel's slots.  This keeps the
// grid at rows * D / 1024 workgroups instead of rows * D / 32, which matters
// when a single split is the whole list (one fully occupied launch of
// short-context rows).
constexpr int kCombineFew = 8;

__global__ __launch_bounds__(256) void combine_few_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_m,
                                                          const float* __restrict__ part_l,
                                                          int rows, int S, int D,
                                                          float* __restrict__ out,
                                                          float* __restrict__ lse) {
  const int q4n = D / 4;
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (size_t)rows * q4n) return;
  const size_t row = gid / q4n;
  const int c = (int)(gid % q4n) * 4;
  float ms[kCombineFew], ls[kCombineFew];
  float4 os[kCombineFew];
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kCombineFew; ++s) {
    ms[s] = -INFINITY;
    ls[s] = 0.0f;
    os[s] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (s < S) {
      ms[s] = part_m[row * S + s];
      ls[s] = part_l[row * S + s];
      os[s] = *reinterpret_cast<const float4*>(part_o + (row * S + s) * D + c);
    }
    M = fmaxf(M, ms[s]);
  }
  float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
  float wt = 0.0f;
#pragma unroll
  for (int s = 0; s < kCombineFew; ++s) {
    if (s < S) {
      const float w = (ms[s] == -INFINITY) ? 0.0f : ls[s] * expf(ms[s] - M);
      t.x += fmaf(w, os[s].x, 0.0f);
      t.y += fmaf(w, os[s].y, 0.0f);
      t.z += fmaf(w, os[s].z, 0.0f);
      t.w += fmaf(w, os[s].w, 0.0f);
      wt += w;
    }
  }
  const float inv = 1.0f / wt;
  *reinterpret_cast<float4*>(out + row * D + c) = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
  if (lse && c == 0) lse[row] = M + logf(wt);
}

// ============================================================== tier lists
//
// Two passes over chunks of kTierChunk list positions, so that a long list is
// spread over many compute units (its page-tier lookups are scattered byte
// loads).  tier_flags_kernel: per chunk, each position's tier as a byte, and
// the chunk's cold count.  tier_write_kernel: per chunk, the hot / cold
// entries before it from the counts of the chunks before, then one block
// scan places the chunk's entries in the hot and the cold list, order kept;
// the chunk holding the list's last entry writes the two counts.
constexpr int kTierThreads = 256;
constexpr int kTierEPT = 4;
constexpr int kTierChunk = kTierThreads * kTierEPT;
static_assert(kTierChunk == kTierChunkPositions, "the launcher sizes chunks by this");

__global__ __launch_bounds__(kTierThreads) void tier_flags_kernel(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int sel_stride,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const uint8_t* __restrict__ page_tier, int Hkv, int maxN, int out_stride, int n_chunks,
    uint8_t* __restrict__ flags, int32_t* __restrict__ chunk_cold) {
  __shared__ uint32_t wsum[kTierThreads / kWave];
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const size_t u = (size_t)b * Hkv + j;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int n = sel ? sel_count[u] : (seq_lens[b] + kBlockSize - 1) / kBlockSize;
  const int c0 = c * kTierChunk;
  if (c0 >= n) return;                             // workgroup-uniform
  const int32_t* list = sel ? sel + u * sel_stride : nullptr;
  const int32_t* bt = block_table + (size_t)b * maxN;
  uint32_t nc = 0;
  uint32_t f = 0;
#pragma unroll
  for (int r = 0; r < kTierEPT; ++r) {
    const int pos = c0 + tid * kTierEPT + r;
    if (pos < n) {
      const int blk = list ? list[pos] : pos;
      const uint32_t t = page_tier[bt[blk]] != 0 ? 1u : 0u;
      f |= t << (8 * r);
      nc += t;
    }
  }
  // the thread's 4 flags as one word (positions past n stay 0 and are never read)
  *reinterpret_cast<uint32_t*>(flags + u * (size_t)n_chunks * kTierChunk + c0 + tid * kTierEPT) = f;
  nc = wave_reduce_u32(nc, AddU32());
  if (lane == 0) wsum[wave] = nc;
  __syncthreads();
  if (tid == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kTierThreads / kWave; ++w) t += wsum[w];
    chunk_cold[u * n_chunks + c] = (int32_t)t;
  }
}

__global__ __launch_bounds__(kTierThreads) void tier_write_kernel(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int sel_stride,
    const int32_t* __restrict__ seq_lens, int Hkv, int out_stride, int n_chunks,
    const uint8_t* __restrict__ flags, const int32_t* __restrict__ chunk_cold,
    int32_t* __restrict__ hot, int32_t* __restrict__ hot_count, int32_t* __restrict__ cold,
    int32_t* __restrict__ cold_count) {
  __shared__ uint32_t wsum[kTierThreads / kWave];
  const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const size_t u = (size_t)b * Hkv + j;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
  const int n = sel ? sel_count[u] : (seq_lens[b] + kBlockSize - 1) / kBlockSize;
  const int c0 = c * kTierChunk;
  const int last = n > 0 ? (n - 1) / kTierChunk : 0;
  if (c > last) return;                            // workgroup-uniform
  // cold entries before this chunk (every chunk before it is full)
  uint32_t cold_before = 0;
  for (int k = lane; k < c; k += kWave) cold_before += (uint32_t)chunk_cold[u * n_chunks + k];
  cold_before = wave_reduce_u32(cold_before, AddU32());
  const uint32_t hot_before = (uint32_t)c0 - cold_before;
  const int32_t* list = sel ? sel + u * sel_stride : nullptr;
  uint32_t f = 0;
  int valid = 0;
  int blk[kTierEPT];
  if (c0 < n) {
    f = *reinterpret_cast<const uint32_t*>(flags + u * (size_t)n_chunks * kTierChunk + c0 +
                                           tid * kTierEPT);
    valid = min(kTierEPT, max(0, n - (c0 + tid * kTierEPT)));
  }
#pragma unroll
  for (int r = 0; r < kTierEPT; ++r) {
    const int pos = c0 + tid * kTierEPT + r;
    blk[r] = r < valid ? (list ? list[pos] : pos) : -1;
  }
  uint32_t nc = 0;
#pragma unroll
  for (int r = 0; r < kTierEPT; ++r) nc += r < valid ? ((f >> (8 * r)) & 1u) : 0u;
  const uint32_t packed = (((uint32_t)valid - nc) << 16) | nc;   // (hot, cold) in 16 bits each
  const uint32_t incl = wave_scan_add_u32(packed);
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kTierThreads / kWave; ++w) {
    if (w < wave) before += wsum[w];
    total += wsum[w];
  }
  const uint32_t ex = before + incl - packed;
  uint32_t h = hot_before + (ex >> 16), cl = cold_before + (ex & 0xFFFFu);
  int32_t* hot_row = hot + u * out_stride;
  int32_t* cold_row = cold + u * out_stride;
#pragma unroll
  for (int r = 0; r < kTierEPT; ++r) {
    if (r < valid) {
      if ((f >> (8 * r)) & 1u) cold_row[cl++] = blk[r];
      else hot_row[h++] = blk[r];
    }
  }
  if (c == last && tid == 0) {
    hot_count[u] = (int)(hot_before + (total >> 16));
    cold_count[u] = (int)(cold_before + (total & 0xFFFFu));
  }
}

// ============================================================== launchers


hipError_t launch_paged_attn(int dtype, int D, int G, int kvq, const void* q,
                             const void* k_cache, const void* v_cache, const float* kv_scales,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* sel, const int32_t* sel_count, int sel_stride,
                             const int32_t* sel_slots, int num_slots, int B, int Hq, int Hkv,
                             int maxN, int S, float scale, float* part_o, float* part_m,
                             float* part_l, float* block_lse, hipStream_t stream, int cold,
                             const void* k_cold, const void* v_cold, const uint8_t* page_tier,
                             const FetchArgs* fetch, int part_stride) {
  constexpr int WAVES = KVD_ATTN_WAVES;
  const int PS = part_stride > 0 ? part_stride : S;
  const FetchArgs fa = fetch ? *fetch : FetchArgs{};
  const dim3 grid((S + WAVES - 1) / WAVES, Hkv, B);
  const float qscale = scale * kLog2e;
  return with_dtype(dtype, [&](auto dt) {
    return with_dim(D, [&](auto d) {
      return with_group(G, [&](auto g) {
        using DT = decltype(dt);
        constexpr int DD = decltype(d)::value, GG = decltype(g)::value;
        auto go = [&](auto sparse, auto fmt, auto coldc, auto fetchc) {
          constexpr bool SP = decltype(sparse)::value, FE = decltype(fetchc)::value;
          constexpr int KQ = decltype(fmt)::value, CQ = decltype(coldc)::value;
          if constexpr (KQ == 4 && std::is_same_v<DT, F32>) {
            return;                           // INT4 pages: 16-bit dtypes only
          } else if constexpr (!std::is_same_v<DT, F32> && GG >= 2) {
            hipLaunchKernelGGL((paged_attn_mfma_kernel<DT, DD, GG, WAVES, SP, KQ, CQ, FE>), grid,
                               dim3(WAVES * kWave), 0, stream, q, k_cache, v_cache, kv_scales,
                               block_table, seq_lens, sel, sel_count, sel_stride, sel_slots,
                               num_slots, Hq, Hkv, maxN, S, PS, qscale, part_o, part_m, part_l,
                               block_lse, k_cold, v_cold, page_tier, fa);
          } else if constexpr (CQ == 0) {
            hipLaunchKernelGGL((paged_attn_kernel<DT, DD, GG, WAVES, SP, KQ, FE>), grid,
                               dim3(WAVES * kWave), 0, stream, q, k_cache, v_cache, kv_scales,
                               block_table, seq_lens, sel, sel_count, sel_stride, sel_slots,
                               num_slots, Hq, Hkv, maxN, S, PS, qscale, part_o, part_m, part_l,
                               block_lse, fa);
          }
        };
        using C0 = std::integral_constant<int, 0>;
        using C8 = std::integral_constant<int, 8>;
        using C4 = std::integral_constant<int, 4>;
        using T = std::true_type;
        using F = std::false_type;
        if (kvq == 4 && std::is_same_v<DT, F32>) return hipErrorInvalidValue;
        if (fetch) {
          // fused delta fetch: cached lists only
          if (!sel || !sel_slots || !block_table || cold != 0) return hipErrorInvalidValue;
          if (kvq == 8) go(T{}, C8{}, C0{}, T{});
          else if (kvq == 4) go(T{}, C4{}, C0{}, T{});
          else go(T{}, C0{}, C0{}, T{});
        } else if (cold != 0) {
          // tiered pools: 16-bit hot pages on the matrix-core path only
          if (kvq != 0 || std::is_same_v<DT, F32> || GG < 2) return hipErrorInvalidValue;
          if (sel) {
            if (cold == 8) go(T{}, C0{}, C8{}, F{});
            else go(T{}, C0{}, C4{}, F{});
          } else {
            if (cold == 8) go(F{}, C0{}, C8{}, F{});
            else go(F{}, C0{}, C4{}, F{});
          }
        } else if (sel) {
          if (kvq == 8) go(T{}, C8{}, C0{}, F{});
          else if (kvq == 4) go(T{}, C4{}, C0{}, F{});
          else go(T{}, C0{}, C0{}, F{});
        } else {
          if (kvq == 8) go(F{}, C8{}, C0{}, F{});
          else if (kvq == 4) go(F{}, C4{}, C0{}, F{});
          else go(F{}, C0{}, C0{}, F{});
        }
        return hipGetLastError();
      });
    });
  });
}

hipError_t launch_tier_lists(const int32_t* sel, const int32_t* sel_count, int sel_stride,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const uint8_t* page_tier, int B, int Hkv, int maxN, int out_stride,
                             int32_t* hot, int32_t* hot_count, int32_t* cold, int32_t* cold_count,
                             uint8_t* flags, int32_t* chunk_cold, hipStream_t stream) {
  const int n_chunks = tier_chunks(out_stride);
  const dim3 grid(n_chunks, Hkv, B);
  hipLaunchKernelGGL(tier_flags_kernel, grid, dim3(kTierThreads), 0, stream, sel, sel_count,
                     sel_stride, block_table, seq_lens, page_tier, Hkv, maxN, out_stride,
                     n_chunks, flags, chunk_cold);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tier_write_kernel, grid, dim3(kTierThreads), 0, stream, sel, sel_count,
                     sel_stride, seq_lens, Hkv, out_stride, n_chunks, flags, chunk_cold, hot,
                     hot_count, cold, cold_count);
  return hipGetLastError();
}

hipError_t launch_combine(int D, const float* part_o, const float* part_m, const float* part_l,
                          int rows, int S, float* out, float* lse, hipStream_t stream) {
  if (D % kCombineChunk) return hipErrorInvalidValue;
  if (S <= kCombineFew) {
    const size_t threads = (size_t)rows * (D / 4);
    hipLaunchKernelGGL(combine_few_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, part_o, part_m, part_l, rows, S, D, out, lse);
    return hipGetLastError();
  }
  constexpr int SLOTS = 256 / (kCombineChunk / 4);
  const dim3 grid(rows, D / kCombineChunk);
  auto go = [&](auto r) {
    hipLaunchKernelGGL((combine_kernel<decltype(r)::value>), grid, dim3(256), 0, stream, part_o,
                       part_m, part_l, S, D, out, lse);
  };
  if (S <= SLOTS) go(std::integral_constant<int, 1>{});
  else if (S <= 2 * SLOTS) go(std::integral_constant<int, 2>{});
  else if (S <= 4 * SLOTS) go(std::integral_constant<int, 4>{});
  else if (S <= 8 * SLOTS) go(std::integral_constant<int, 8>{});
  else go(std::integral_constant<int, 0>{});
  return hipGetLastError();
}

bool select_attn_fusable(int dtype, int G, int maxN, int K, int S) {
  const long per_wg = (long)kSelAttnWaves * ((K + S - 1) / S);   // list positions per workgroup
  return dtype != 0 && G >= 2 && maxN <= kSelAttnMaxBlocks && per_wg <= kSelAttnListMax;
}

hipError_t launch_select_attn(int dtype, int D, int G, const float* scores, int K, int sink,
                              int local, int32_t* sel, int32_t* sel_count, const void* q,
                              const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, int B, int Hq,
                              int Hkv, int maxN, int S, float scale, float* part_o, float* part_m,
                              float* part_l, hipStream_t stream) {
  if (!select_attn_fusable(dtype, G, maxN, K, S)) return hipErrorInvalidValue;
  constexpr int NT = kSelAttnWaves * kWave;
  const dim3 grid((S + kSelAttnWaves - 1) / kSelAttnWaves, Hkv, B);
  const float qscale = scale * kLog2e;
  constexpr int EPT = (kSelAttnMaxBlocks + NT - 1) / NT;   // keys per thread of the row select
  return with_dtype(dtype, [&](auto dt) {
    return with_dim(D, [&](auto d) {
      return with_group(G, [&](auto g) {
        using DT = decltype(dt);
        constexpr int DD = decltype(d)::value, GG = decltype(g)::value;
        if constexpr (!std::is_same_v<DT, F32> && GG >= 2) {
          hipLaunchKernelGGL((select_attn_mfma_kernel<DT, DD, GG, EPT>), grid, dim3(NT), 0, stream,
                             scores, K, sink, local, sel, sel_count, q, k_cache, v_cache,
                             block_table, seq_lens, Hq, Hkv, maxN, S, qscale, part_o, part_m,
                             part_l);
          return hipGetLastError();
        } else {
          return hipErrorInvalidValue;
        }
      });
    });
  });
}

}  // namespace kvd

// gfx950 kernels of the GPU-resident block cache (KVDrive §5.1: a window of
// critical KV entries stays on the GPU; each step fetches the new critical
// entries from host memory and drops the entries that received the least
// attention in the latest step).
//
//   cache_plan_kernel   per (sequence, KV head): hits keep their slots; the m
//                       missing blocks reuse the first m of [free slots by
//                       index, then unselected slots by increasing mass (ties:
//                       lower slot)], taken in increasing slot order
//   cache_fetch_kernel  copies only the missing K/V tiles (16-bit, fp32 or code
//                       pages) from the (host) pool into their cache slots: the
//                       delta fetch (the attention kernels can also do it
//                       themselves, in the same launch)
//   slot_mass_kernel    eviction mass of every slot from the step's attention:
//                       max over the group's heads of exp(block_lse - lse), 0
//                       for slots the step did not attend
//
// The cache pools are [B * C, Hkv, bs, D] (code pools: D or D/2 bytes per
// row, with fp32 (k, v) scales [B * C, Hkv, 2]): page b*C + s holds slot s of
// every KV head of sequence b (each head's slot s caches its own block).
#include <math.h>

#include "kvd_device.hpp"
#include "kvd_dispatch.hpp"
#include "kvd_launch.hpp"

namespace kvd {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;

// Exclusive prefix over threads (in thread order) of v; buf holds kPlanWaves.
// With total, also the sum over the block (same two barriers).
__device__ inline uint32_t block_exclusive_u32(uint32_t v, uint32_t* buf,
                                               uint32_t* total = nullptr) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t o = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += o;
  }
  __syncthreads();
  if (lane == kWave - 1) buf[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    if (w < wave) before += buf[w];
    all += buf[w];
  }
  if (total) *total = all;
  return before + inc - v;
}

// EPT consecutive slots per thread (C <= 1024 * EPT); PPT consecutive list
// positions per thread (sel_stride <= 1024 * PPT).
template <int EPT, int PPT>
__global__ __launch_bounds__(kPlanThreads) void cache_plan_kernel(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int sel_stride,
    int Hkv, int maxN, int C, int32_t* __restrict__ slot_block, int32_t* __restrict__ block_slot,
    const float* __restrict__ slot_mass, int32_t* __restrict__ sel_slots,
    int32_t* __restrict__ fetch_block, int32_t* __restrict__ fetch_slot,
    int32_t* __restrict__ fetch_count) {
  __shared__ uint8_t in_use[kPlanThreads * EPT];
  __shared__ int32_t reused[kPlanThreads * EPT];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t buf[kPlanWaves];
  __shared__ uint32_t state[2];
  const int tid = threadIdx.x;
  const size_t u = (size_t)blockIdx.y * Hkv + blockIdx.x;
  const int cnt = sel_count[u];
  const int32_t* list = sel + u * sel_stride;
  int32_t* sb = slot_block + u * C;
  int32_t* bsl = block_slot + u * maxN;
  const float* mass = slot_mass + u * C;
  int32_t* out_slots = sel_slots + u * sel_stride;
  int32_t* fb = fetch_block + u * sel_stride;
  int32_t* fs = fetch_slot + u * sel_stride;

  // slot states first: they do not depend on the list (a slot's entry is
  // rewritten below only by the one thread that reuses it, after these reads)
  int32_t sbv[EPT];
  float mv[EPT];
#pragma unroll
  for (int r = 0; r < EPT; ++r) {
    const int c = tid * EPT + r;
    sbv[r] = c < C ? sb[c] : 0;
    mv[r] = c < C ? mass[c] : 0.0f;
  }
  for (int c = tid; c < C; c += kPlanThreads) in_use[c] = 0;
  __syncthreads();
  // hits keep their slots; count the misses of this thread's positions
  int pslot[PPT];
  uint32_t my_miss = 0;
#pragma unroll
  for (int r = 0; r < PPT; ++r) {
    const int pos = tid * PPT + r;
    pslot[r] = -1;
    if (pos < cnt) {
      pslot[r] = bsl[list[pos]];
      if (pslot[r] >= 0) in_use[pslot[r]] = 1;
      else ++my_miss;
    }
  }
  uint32_t m;
  const uint32_t miss_before = block_exclusive_u32(my_miss, buf, &m);   // also orders in_use

  // slot states
  uint32_t key[EPT];
  uint32_t free_mask = 0, elig_mask = 0;
#pragma unroll
  for (int r = 0; r < EPT; ++r) {
    const int c = tid * EPT + r;
    key[r] = 0u;
    if (c < C) {
      if (sbv[r] < 0) free_mask |= 1u << r;
      else if (!in_use[c]) {
        elig_mask |= 1u << r;
        key[r] = __float_as_uint(fmaxf(mv[r], 0.0f));   // monotone for masses >= 0
      }
    }
  }
  uint32_t n_free;
  const uint32_t free_before = block_exclusive_u32((uint32_t)__popc(free_mask), buf, &n_free);

  // reused: the first min(m, n_free) free slots, then the m - n_free smallest
  // (mass, slot) among the eligible slots (radix select from the top byte)
  uint32_t reuse_mask = 0;
  {
    uint32_t fr = free_before;
#pragma unroll
    for (int r = 0; r < EPT; ++r)
      if ((free_mask >> r) & 1u) {
        if (fr < m) reuse_mask |= 1u << r;
        ++fr;
      }
  }
  uint32_t need = m > n_free ? m - n_free : 0u;          // uniform
  if (need > 0) {
    uint32_t prefix = 0u, krem = need;
    for (int shift = 24; shift >= 0; shift -= 8) {
      const uint32_t hi_mask = shift == 24 ? 0u : (0xffffffffu << (shift + 8));
      for (int i = tid; i < 256; i += kPlanThreads) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int r = 0; r < EPT; ++r)
        if (((elig_mask >> r) & 1u) && ((key[r] ^ prefix) & hi_mask) == 0u)
          atomicAdd(&hist[(key[r] >> shift) & 255u], 1u);
      __syncthreads();
      if (tid < kWave) {
        // lane L owns digits 4L .. 4L+3 (ascending)
        const uint32_t c0 = hist[4 * tid], c1 = hist[4 * tid + 1], c2 = hist[4 * tid + 2],
                       c3 = hist[4 * tid + 3];
        const uint32_t mine = c0 + c1 + c2 + c3;
        uint32_t inc = mine;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
          const uint32_t o = __shfl_up(inc, off, kWave);
          if (tid >= off) inc += o;
        }
        uint32_t below = inc - mine;
        const uint32_t cs[4] = {c0, c1, c2, c3};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (below < krem && below + cs[q] >= krem) {
            state[0] = (uint32_t)(4 * tid + q);
            state[1] = krem - below;
          }
          below += cs[q];
        }
      }
      __syncthreads();
      prefix |= state[0] << shift;
      krem = state[1];
      __syncthreads();                                    // state is rewritten next pass
    }
    const uint32_t T = prefix;                            // the need-th smallest key
    uint32_t n_eq = 0;
#pragma unroll
    for (int r = 0; r < EPT; ++r) n_eq += ((elig_mask >> r) & 1u) && key[r] == T;
    uint32_t eq_before = block_exclusive_u32(n_eq, buf);
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      if (!((elig_mask >> r) & 1u)) continue;
      if (key[r] < T) reuse_mask |= 1u << r;
      else if (key[r] == T) {
        if (eq_before < krem) reuse_mask |= 1u << r;
        ++eq_before;
      }
    }
  }
  // reused slots in slot order
  {
    uint32_t rk = block_exclusive_u32((uint32_t)__popc(reuse_mask), buf);
#pragma unroll
    for (int r = 0; r < EPT; ++r)
      if ((reuse_mask >> r) & 1u) reused[rk++] = tid * EPT + r;
  }
  __syncthreads();
  // misses take them in list order; a reused slot is written by one thread
  {
    uint32_t mr = miss_before;
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
      const int pos = tid * PPT + r;
      if (pos < cnt && pslot[r] < 0) {
        const int s = reused[mr];
        const int n = list[pos];
        const int old = sb[s];
        if (old >= 0) bsl[old] = -1;
        sb[s] = n;
        bsl[n] = s;
        pslot[r] = s;
        fb[mr] = n;
        fs[mr] = s;
        ++mr;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < PPT; ++r) {
    const int pos = tid * PPT + r;
    if (pos < sel_stride) {
      out_slots[pos] = pos < cnt ? pslot[r] : -1;
      if (pos >= (int)m) { fb[pos] = -1; fs[pos] = -1; }
    }
  }
  if (tid == 0) fetch_count[u] = (int)m;
}

// One wave per (fetch k, KV head j, sequence b): copies the K and V tiles of
// block fetch_block[b, j, k] from the pool page block_table[b, n] into cache
// page b*C + fetch_slot[b, j, k].  Source bytes are read once (non-temporal;
// they may be mapped host memory), the cache tile is read by the attention
// right after and is stored normally.  TILE is the tile's size in the pools'
// format: 16 * D elements of a 16-bit or fp32 pool, or the codes of a code
// pool (16 * D bytes of E4M3, 16 * D / 2 of INT4); a code pool's tile also
// brings its (k, v) scale pair along.
template <int TILE>
__global__ __launch_bounds__(kWave) void cache_fetch_kernel(
    const void* __restrict__ k_pool, const void* __restrict__ v_pool,
    const float* __restrict__ kv_scales, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ fetch_block, const int32_t* __restrict__ fetch_slot,
    const int32_t* __restrict__ fetch_count, int fetch_stride, int Hkv, int maxN, int C,
    void* __restrict__ cache_k, void* __restrict__ cache_v, float* __restrict__ cache_scales) {
  constexpr int ITER = (TILE + 16 * kWave - 1) / (16 * kWave);
  constexpr bool FULL = TILE % (16 * kWave) == 0;   // else the last load is partial
  static_assert(TILE % 16 == 0, "tiles are whole 16-byte chunks");
  const int k = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const size_t u = (size_t)b * Hkv + j;
  if (k >= fetch_count[u]) return;
  const int n = fetch_block[u * fetch_stride + k];
  const int s = fetch_slot[u * fetch_stride + k];
  const size_t src_unit = (size_t)block_table[(size_t)b * maxN + n] * Hkv + j;
  const size_t dst_unit = ((size_t)b * C + s) * Hkv + j;
  const size_t src = src_unit * TILE, dst = dst_unit * TILE;
  const int lane = threadIdx.x;
  uint4 kw[ITER], vw[ITER];
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const size_t off = (size_t)(i * kWave + lane) * 16;
    if (FULL || off < TILE) {
      kw[i] = load16_stream(static_cast<const uint8_t*>(k_pool) + src + off);
      vw[i] = load16_stream(static_cast<const uint8_t*>(v_pool) + src + off);
    }
  }
  float2 sc = make_float2(0.0f, 0.0f);
  if (kv_scales && lane == 0) sc = *reinterpret_cast<const float2*>(kv_scales + src_unit * 2);
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const size_t off = (size_t)(i * kWave + lane) * 16;
    if (FULL || off < TILE) {
      store16(static_cast<uint8_t*>(cache_k) + dst + off, kw[i]);
      store16(static_cast<uint8_t*>(cache_v) + dst + off, vw[i]);
    }
  }
  if (kv_scales && lane == 0) *reinterpret_cast<float2*>(cache_scales + dst_unit * 2) = sc;
}

// One 256-thread workgroup per (sequence, KV head): every slot's mass to 0,
// then the attended list's blocks get max_g exp(block_lse - lse).
__global__ __launch_bounds__(256) void slot_mass_kernel(
    const float* __restrict__ block_lse, const float* __restrict__ lse,
    const int32_t* __restrict__ sel_count, const int32_t* __restrict__ sel_slots, int sel_stride,
    int Hq, int Hkv, int C, float* __restrict__ slot_mass) {
  const int j = blockIdx.x, b = blockIdx.y;
  const size_t u = (size_t)b * Hkv + j;
  const int G = Hq / Hkv;
  float* out = slot_mass + u * C;
  for (int c = threadIdx.x; c < C; c += 256) out[c] = 0.0f;
  __syncthreads();
  const int cnt = sel_count[u];
  for (int pos = threadIdx.x; pos < cnt; pos += 256) {
    float best = 0.0f;
    for (int g = 0; g < G; ++g) {
      const size_t row = (size_t)b * Hq + (size_t)j * G + g;
      best = fmaxf(best, expf(block_lse[row * sel_stride + pos] - lse[row]));
    }
    out[sel_slots[u * sel_stride + pos]] = best;
  }
}

hipError_t launch_cache_plan(const int32_t* sel, const int32_t* sel_count, int sel_stride, int B,
                             int Hkv, int maxN, int C, int32_t* slot_block, int32_t* block_slot,
                             const float* slot_mass, int32_t* sel_slots, int32_t* fetch_block,
                             int32_t* fetch_slot, int32_t* fetch_count, hipStream_t stream) {
  const dim3 grid(Hkv, B);
  const int ept = (C + kPlanThreads - 1) / kPlanThreads;
  const int ppt = (sel_stride + kPlanThreads - 1) / kPlanThreads;
  auto go = [&](auto e, auto p) {
    hipLaunchKernelGGL((cache_plan_kernel<decltype(e)::value, decltype(p)::value>), grid,
                       dim3(kPlanThreads), 0, stream, sel, sel_count, sel_stride, Hkv, maxN, C,
                       slot_block, block_slot, slot_mass, sel_slots, fetch_block, fetch_slot,
                       fetch_count);
    return hipGetLastError();
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  // sel_stride <= C, so ppt <= ept
  if (ept <= 1) return go(I1{}, I1{});
  if (ept <= 2) return ppt <= 1 ? go(I2{}, I1{}) : go(I2{}, I2{});
  if (ept <= 4) return ppt <= 1 ? go(I4{}, I1{}) : ppt <= 2 ? go(I4{}, I2{}) : go(I4{}, I4{});
  if (ept <= 8)
    return ppt <= 1 ? go(I8{}, I1{}) : ppt <= 2 ? go(I8{}, I2{}) : ppt <= 4 ? go(I8{}, I4{})
                                                                          : go(I8{}, I8{});
  return hipErrorInvalidValue;
}

hipError_t launch_cache_fetch(int tile_bytes, const void* k_pool, const void* v_pool,
                              const float* kv_scales, const int32_t* block_table,
                              const int32_t* fetch_block, const int32_t* fetch_slot,
                              const int32_t* fetch_count, int fetch_stride, int B, int Hkv,
                              int maxN, int C, void* cache_k, void* cache_v, float* cache_scales,
                              hipStream_t stream) {
  const dim3 grid(fetch_stride, Hkv, B);
  auto go = [&](auto tile) {
    hipLaunchKernelGGL((cache_fetch_kernel<decltype(tile)::value>), grid, dim3(kWave), 0, stream,
                       k_pool, v_pool, kv_scales, block_table, fetch_block, fetch_slot,
                       fetch_count, fetch_stride, Hkv, maxN, C, cache_k, cache_v, cache_scales);
    return hipGetLastError();
  };
  switch (tile_bytes) {
    case 512: return go(std::integral_constant<int, 512>{});
    case 1024: return go(std::integral_constant<int, 1024>{});
    case 2048: return go(std::integral_constant<int, 2048>{});
    case 4096: return go(std::integral_constant<int, 4096>{});
    case 8192: return go(std::integral_constant<int, 8192>{});
  }
  return hipErrorInvalidValue;
}

hipError_t launch_slot_mass(const float* block_lse, const float* lse, const int32_t* sel_count,
                            const int32_t* sel_slots, int sel_stride, int B, int Hq, int Hkv,
                            int C, float* slot_mass, hipStream_t stream) {
  hipLaunchKernelGGL(slot_mass_kernel, dim3(Hkv, B), dim3(256), 0, stream, block_lse, lse,
                     sel_count, sel_slots, sel_stride, Hq, Hkv, C, slot_mass);
  return hipGetLastError();
}

}  // namespace kvd

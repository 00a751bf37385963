// gfx950 kernel of the hot/cold tier policy (the tiered-offload blog, page
// replacement: pages whose heat has fallen move down a tier, and a cooldown
// after a demotion keeps a page from coming straight back; KVDrive §11: hot
// blocks stay at full precision, cold blocks are stored quantised).
//
//   tier_plan_kernel   one workgroup per sequence: a bitmap in LDS of the
//                      blocks any KV head selected in the step, then, in block
//                      order, each page's heat (an exponential average of its
//                      hits, fp32), its tier change, and a block scan that
//                      places the pages that changed in the demote and the
//                      promote list, block order kept.
//
// The heat update is written as one fused multiply-add for a hit and one
// product for a miss, so its fp32 result is a fixed function of the inputs.
#include <math.h>

#include "kvd_device.hpp"
#include "kvd_launch.hpp"

namespace kvd {

constexpr int kTierPlanThreads = 1024;
constexpr int kTierPlanWaves = kTierPlanThreads / kWave;
constexpr int kTierPlanEPT = 4;                    // consecutive blocks per thread and pass
constexpr int kTierPlanPass = kTierPlanThreads * kTierPlanEPT;
static_assert(kTierPlanPass < 65536, "the pass counts share one 32-bit scan word");

__global__ __launch_bounds__(kTierPlanThreads) void tier_plan_kernel(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int sel_stride,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int Hkv,
    int maxN, int num_pages, TierPolicy pol, int step, float* __restrict__ heat, uint8_t* __restrict__ tier,
    int32_t* __restrict__ stamp, int32_t* __restrict__ demote, int32_t* __restrict__ demote_count,
    int32_t* __restrict__ promote, int32_t* __restrict__ promote_count) {
  extern __shared__ uint32_t hitmap[];             // ceil(N / 32) words
  __shared__ uint32_t wsum[kTierPlanWaves];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const int L = seq_lens[b];
  const int N = min((L + kBlockSize - 1) / kBlockSize, maxN);
  for (int w = tid; w < (N + 31) / 32; w += kTierPlanThreads) hitmap[w] = 0u;
  __syncthreads();
  for (int j = 0; j < Hkv; ++j) {
    const size_t u = (size_t)b * Hkv + j;
    const int cnt = min(sel_count[u], sel_stride);
    const int32_t* list = sel + u * sel_stride;
    for (int pos = tid; pos < cnt; pos += kTierPlanThreads) {
      const int n = list[pos];
      if ((unsigned)n < (unsigned)N) atomicOr(&hitmap[n >> 5], 1u << (n & 31));
    }
  }
  __syncthreads();

  const int32_t* bt = block_table + (size_t)b * maxN;
  int32_t* dem = demote + (size_t)b * maxN;
  int32_t* pro = promote + (size_t)b * maxN;
  const int first_recent = L - pol.recent;         // tokens first_recent .. L - 1
  const float keep = 1.0f - pol.decay;
  uint32_t nd = 0, np = 0;                         // list entries before this pass (uniform)
  for (int c0 = 0; c0 < N; c0 += kTierPlanPass) {
    int pg[kTierPlanEPT];
    uint32_t down = 0u, up = 0u;
#pragma unroll
    for (int r = 0; r < kTierPlanEPT; ++r) {
      const int n = c0 + tid * kTierPlanEPT + r;
      pg[r] = -1;
      if (n < N) {
        const int p = bt[n];
        if ((unsigned)p >= (unsigned)num_pages) continue;   // not a page of the pools
        pg[r] = p;
        const bool hit = (hitmap[n >> 5] >> (n & 31)) & 1u;
        const bool recent = n * kBlockSize + kBlockSize - 1 >= first_recent;
        const float h0 = heat[p];
        const float h = hit ? fmaf(pol.decay, h0, keep) : pol.decay * h0;
        heat[p] = h;
        if (tier[p] == 0) {
          if (!recent && h < pol.cold_below) {
            tier[p] = 1;
            stamp[p] = step;
            down |= 1u << r;
          }
        } else if (recent ||
                   (h > pol.hot_above && (long)step - (long)stamp[p] >= (long)pol.cooldown)) {
          tier[p] = 0;
          up |= 1u << r;
        }
      }
    }
    // (demoted, promoted) counts of the thread in the high and low 16 bits
    const uint32_t packed = ((uint32_t)__popc(down) << 16) | (uint32_t)__popc(up);
    const uint32_t incl = wave_scan_add_u32(packed);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0u, total = 0u;
#pragma unroll
    for (int w = 0; w < kTierPlanWaves; ++w) {
      if (w < wave) before += wsum[w];
      total += wsum[w];
    }
    __syncthreads();                               // wsum is rewritten by the next pass
    const uint32_t ex = before + incl - packed;
    uint32_t d = nd + (ex >> 16), q = np + (ex & 0xFFFFu);
#pragma unroll
    for (int r = 0; r < kTierPlanEPT; ++r) {
      if ((down >> r) & 1u) dem[d++] = pg[r];
      if ((up >> r) & 1u) pro[q++] = pg[r];
    }
    nd += total >> 16;
    np += total & 0xFFFFu;
  }
  for (int n = (int)nd + tid; n < maxN; n += kTierPlanThreads) dem[n] = -1;
  for (int n = (int)np + tid; n < maxN; n += kTierPlanThreads) pro[n] = -1;
  if (tid == 0) {
    demote_count[b] = (int32_t)nd;
    promote_count[b] = (int32_t)np;
  }
}

hipError_t launch_tier_plan(const int32_t* sel, const int32_t* sel_count, int sel_stride,
                            const int32_t* block_table, const int32_t* seq_lens, int B, int Hkv,
                            int maxN, int num_pages, const TierPolicy& pol, int step, float* heat, uint8_t* tier,
                            int32_t* stamp, int32_t* demote, int32_t* demote_count,
                            int32_t* promote, int32_t* promote_count, hipStream_t stream) {
  if (maxN > kTierPlanMaxBlocks) return hipErrorInvalidValue;
  const size_t lds = (size_t)((maxN + 31) / 32) * sizeof(uint32_t);
  hipLaunchKernelGGL(tier_plan_kernel, dim3(B), dim3(kTierPlanThreads), lds, stream, sel,
                     sel_count, sel_stride, block_table, seq_lens, Hkv, maxN, num_pages, pol, step, heat,
                     tier, stamp, demote, demote_count, promote, promote_count);
  return hipGetLastError();
}

}  // namespace kvd

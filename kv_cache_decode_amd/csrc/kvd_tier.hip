// gfx950 kernels of the hot/cold tier policy (the tiered-offload blog, page
// replacement: pages whose heat has fallen move down a tier, and a cooldown
// after a demotion keeps a page from coming straight back; KVDrive §11: hot
// blocks stay at full precision, cold blocks are stored quantised).  Two
// launches:
//
//   tier_heat_kernel   one workgroup per (chunk of kTierHeatChunk blocks,
//                      sequence): a bitmap in LDS of the chunk's blocks that
//                      any KV head selected in the step, then per block its
//                      page's heat (an exponential average of its hits, fp32)
//                      and tier change, and the page id at the block's own
//                      position of the demote or the promote row (-1 where
//                      the page did not move).  The page state is reached
//                      through the block table, so its loads and stores are
//                      scattered: spreading them over many compute units is
//                      what sets this launch's time.
//   tier_list_kernel   one workgroup per sequence: compacts both rows in place
//                      with a block scan per pass of positions (each pass is
//                      read whole before any entry is written, and an entry
//                      never moves to a higher position), block order kept,
//                      then fills the rows with -1 after the last entry and
//                      writes the counts.
//
// The heat update is written as one fused multiply-add for a hit and one
// product for a miss, so its fp32 result is a fixed function of the inputs.
#include <math.h>

#include "kvd_device.hpp"
#include "kvd_launch.hpp"

namespace kvd {

constexpr int kTierHeatThreads = 256;
constexpr int kTierHeatEPT = 1;                    // blocks per thread (32 workgroups at 8192 blocks)
constexpr int kTierHeatChunk = kTierHeatThreads * kTierHeatEPT;
constexpr int kTierHeatSelR = 8;                   // selection entries per thread and round

constexpr int kTierListThreads = 1024;
constexpr int kTierListWaves = kTierListThreads / kWave;
constexpr int kTierListEPT = 4;                    // one 16-byte load per row and thread
constexpr int kTierListPass = kTierListThreads * kTierListEPT;
static_assert(kTierListPass < 65536, "the pass counts share one 32-bit scan word");

__global__ __launch_bounds__(kTierHeatThreads) void tier_heat_kernel(
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int sel_stride,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int Hkv,
    int maxN, int num_pages, TierPolicy pol, int step, float* __restrict__ heat,
    uint8_t* __restrict__ tier, int32_t* __restrict__ stamp, int32_t* __restrict__ demote,
    int32_t* __restrict__ promote) {
  constexpr int NT = kTierHeatThreads, EPT = kTierHeatEPT, SR = kTierHeatSelR;
  constexpr int CH = kTierHeatChunk;
  __shared__ uint32_t hitmap[CH / 32];
  const int b = blockIdx.y, tid = threadIdx.x;
  const int c0 = blockIdx.x * CH;
  const int32_t* bt = block_table + (size_t)b * maxN;
  // requested before the length arrives: the selection rows of all KV heads
  // (Hkv lists of sel_stride entries, one after the other in memory; read
  // whole, masked by their counts) and the chunk's block-table entries (the
  // row is readable up to maxN)
  const int rows = Hkv * sel_stride;
  const int32_t* selb = sel + (size_t)b * rows;
  const int32_t* cntb = sel_count + (size_t)b * Hkv;
  int sn[SR], sc[SR];
  auto load_sel = [&](int i0) {
#pragma unroll
    for (int r = 0; r < SR; ++r) {
      const int i = i0 + r * NT + tid;
      sn[r] = i < rows ? selb[i] : -1;
      sc[r] = i < rows ? cntb[i / sel_stride] : 0;
    }
  };
  int pg[EPT];
#pragma unroll
  for (int r = 0; r < EPT; ++r) {
    const int n = c0 + tid * EPT + r;
    pg[r] = n < maxN ? bt[n] : -1;
  }
  load_sel(0);
  const int L = seq_lens[b];
  const int N = min((L + kBlockSize - 1) / kBlockSize, maxN);
  if (c0 >= N) return;                             // workgroup-uniform
  // the pages' state, requested before the selection bitmap is built
  float h0[EPT];
  uint32_t t0[EPT];
  int32_t s0[EPT];
#pragma unroll
  for (int r = 0; r < EPT; ++r) {
    const int n = c0 + tid * EPT + r;
    if (n >= N || (unsigned)pg[r] >= (unsigned)num_pages) pg[r] = -1;   // not a page of the pools
    h0[r] = 0.0f;
    t0[r] = 0u;
    s0[r] = 0;
    if (pg[r] >= 0) {
      h0[r] = heat[pg[r]];
      t0[r] = tier[pg[r]];
      s0[r] = stamp[pg[r]];
    }
  }
  if (tid < CH / 32) hitmap[tid] = 0u;
  __syncthreads();
  for (int i0 = 0;;) {
#pragma unroll
    for (int r = 0; r < SR; ++r) {
      const int i = i0 + r * NT + tid;
      const int n = sn[r] - c0;                    // the block's bit in this chunk
      if (i < rows && i % sel_stride < sc[r] && sn[r] < N && (unsigned)n < (unsigned)CH)
        atomicOr(&hitmap[n >> 5], 1u << (n & 31));
    }
    i0 += SR * NT;
    if (i0 >= rows) break;
    load_sel(i0);
  }
  __syncthreads();

  const int first_recent = L - pol.recent;         // tokens first_recent .. L - 1
  const float keep = 1.0f - pol.decay;
#pragma unroll
  for (int r = 0; r < EPT; ++r) {
    const int n = c0 + tid * EPT + r;
    if (n >= N) continue;
    const int p = pg[r];
    int32_t down = -1, up = -1;
    if (p >= 0) {
      const bool hit = (hitmap[(n - c0) >> 5] >> ((n - c0) & 31)) & 1u;
      const bool recent = n * kBlockSize + kBlockSize - 1 >= first_recent;
      const float h = hit ? fmaf(pol.decay, h0[r], keep) : pol.decay * h0[r];
      heat[p] = h;
      if (t0[r] == 0u) {
        if (!recent && h < pol.cold_below) {
          tier[p] = 1;
          stamp[p] = step;
          down = p;
        }
      } else if (recent ||
                 (h > pol.hot_above && (long)step - (long)s0[r] >= (long)pol.cooldown)) {
        tier[p] = 0;
        up = p;
      }
    }
    demote[(size_t)b * maxN + n] = down;
    promote[(size_t)b * maxN + n] = up;
  }
}

__global__ __launch_bounds__(kTierListThreads) void tier_list_kernel(
    const int32_t* __restrict__ seq_lens, int maxN, int32_t* __restrict__ demote,
    int32_t* __restrict__ demote_count, int32_t* __restrict__ promote,
    int32_t* __restrict__ promote_count) {
  constexpr int NT = kTierListThreads, EPT = kTierListEPT;
  __shared__ uint32_t wsum[kTierListWaves];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid >> 6;
  const int L = seq_lens[b];
  const int N = min((L + kBlockSize - 1) / kBlockSize, maxN);
  int32_t* dem = demote + (size_t)b * maxN;
  int32_t* pro = promote + (size_t)b * maxN;
  // 16-byte loads where both rows start on a 16-byte boundary (a thread's EPT
  // positions are consecutive, so a lane-strided walk of single words would
  // touch every line EPT times)
  const bool aligned = ((reinterpret_cast<uintptr_t>(dem) | reinterpret_cast<uintptr_t>(pro)) & 15u) == 0;
  uint32_t nd = 0, np = 0;                         // list entries before this pass (uniform)
  for (int c0 = 0; c0 < N; c0 += kTierListPass) {
    int32_t dv[EPT], uv[EPT];
    const int n0 = c0 + tid * EPT;
    if (aligned && n0 + EPT <= N) {
      const int4 a = *reinterpret_cast<const int4*>(dem + n0);
      const int4 c = *reinterpret_cast<const int4*>(pro + n0);
      dv[0] = a.x; dv[1] = a.y; dv[2] = a.z; dv[3] = a.w;
      uv[0] = c.x; uv[1] = c.y; uv[2] = c.z; uv[3] = c.w;
    } else {
#pragma unroll
      for (int r = 0; r < EPT; ++r) {
        dv[r] = n0 + r < N ? dem[n0 + r] : -1;
        uv[r] = n0 + r < N ? pro[n0 + r] : -1;
      }
    }
    // (demoted, promoted) entries of the thread in the high and low 16 bits:
    // the scan needs every value the thread read, so the whole pass has been
    // read when the barrier below is passed, and only then is anything written
    uint32_t packed = 0u;
#pragma unroll
    for (int r = 0; r < EPT; ++r) packed += ((uint32_t)(dv[r] >= 0) << 16) | (uint32_t)(uv[r] >= 0);
    const uint32_t incl = wave_scan_add_u32(packed);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0u, total = 0u;
#pragma unroll
    for (int w = 0; w < kTierListWaves; ++w) {
      if (w < wave) before += wsum[w];
      total += wsum[w];
    }
    __syncthreads();                               // wsum is rewritten by the next pass
    const uint32_t ex = before + incl - packed;
    // an entry moves from position n to a position <= n, within this pass's
    // range or below it: no position a later pass reads is written
    uint32_t d = nd + (ex >> 16), q = np + (ex & 0xFFFFu);
#pragma unroll
    for (int r = 0; r < EPT; ++r) {
      if (dv[r] >= 0) dem[d++] = dv[r];
      if (uv[r] >= 0) pro[q++] = uv[r];
    }
    nd += total >> 16;
    np += total & 0xFFFFu;
  }
  for (int n = (int)nd + tid; n < maxN; n += NT) dem[n] = -1;
  for (int n = (int)np + tid; n < maxN; n += NT) pro[n] = -1;
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
  const dim3 grid((maxN + kTierHeatChunk - 1) / kTierHeatChunk, B);
  hipLaunchKernelGGL(tier_heat_kernel, grid, dim3(kTierHeatThreads), 0, stream, sel, sel_count,
                     sel_stride, block_table, seq_lens, Hkv, maxN, num_pages, pol, step, heat,
                     tier, stamp, demote, promote);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(tier_list_kernel, dim3(B), dim3(kTierListThreads), 0, stream, seq_lens, maxN,
                     demote, demote_count, promote, promote_count);
  return hipGetLastError();
}

}  // namespace kvd

// gfx950 kernel that turns K/V pages into quantised cold pages.
//
//   quantize_kernel<FP8>   per (page, KV head): amax of the valid slots, scale
//                          amax / 448, E4M3 codes round-to-nearest-even(x / scale)
//   quantize_kernel<INT4>  scale amax / 7, codes round-half-even(x / scale)
//                          clamped to [-7, 7], two per byte
//                          KVDrive §11 (cold blocks quantised, hot blocks kept in
//                          high precision); DirectKV review, assumption stress test
//                          (FP8/INT4 KV)
//
// The E4M3 format is the OCP 8-bit floating-point one (bias 7, no infinities,
// largest finite value 448).  Scale and quotient are correctly rounded fp32
// divisions, so the codes are a deterministic function of the stored values.
#include "kvd_device.hpp"
#include "kvd_dispatch.hpp"
#include "kvd_launch.hpp"

#ifndef KVD_QUANT_WGS_PER_CU
#define KVD_QUANT_WGS_PER_CU 16
#endif

namespace kvd {

// E codes of one lane chunk, packed little-endian into E/4 dwords.
template <int E>
struct CodeChunk {
  uint32_t w[E / 4];
};

template <int E>
__device__ inline void store_codes(uint8_t* dst, const CodeChunk<E>& cc) {
  if constexpr (E == 8) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(cc.w[0], cc.w[1]);
  } else {
    static_assert(E == 4, "4 or 8 channels per chunk");
    *reinterpret_cast<uint32_t*>(dst) = cc.w[0];
  }
}

// One wave per unit, a unit being one (page, KV head): lane (g, c) owns
// channel chunk c (E channels) of rows g, g + RG, g + 2 RG, ... (RG = 64 / LPR
// row groups, so one load instruction reads RG whole consecutive rows).  The
// K and V rows of the unit are requested together; each tensor's amax is
// reduced over the whole wave, and every lane then encodes and stores its own
// chunks.  Spreading a unit over all 64 lanes keeps a lane's share of the
// correctly rounded divisions at 16 / RG rows, which sets how long a wave
// takes when only a few pages are quantised (the demotions of one decode step).
constexpr int kFmtFp8 = 8, kFmtInt4 = 4;

template <typename DT, int D, int WAVES, int FMT>
__global__ __launch_bounds__(WAVES * kWave) void quantize_kernel(
    const void* __restrict__ k_cache, const void* __restrict__ v_cache,
    const int32_t* __restrict__ page_ids, const int32_t* __restrict__ valid_tokens, int n_ids,
    int Hkv, uint8_t* __restrict__ k8, uint8_t* __restrict__ v8, float* __restrict__ scales) {
  using G_ = RowGeom<DT, D>;
  using St = typename DT::storage;
  constexpr int E = G_::E, LPR = G_::LPR;
  constexpr int RG = kWave / LPR;                  // row groups: rows per load instruction
  constexpr int RPL = kBlockSize / RG;             // rows per lane
  static_assert(FMT == kFmtFp8 || E == 8, "INT4 pages hold 16-bit sources (8 channels per lane)");
  // code bytes per row and per lane chunk
  constexpr int RB = FMT == kFmtFp8 ? D : D / 2, CB = FMT == kFmtFp8 ? E : E / 2;
  const int lane = threadIdx.x & (kWave - 1);
  const int g = lane / LPR, c = lane % LPR;
  const long units = (long)n_ids * Hkv;
  const long nwaves = (long)gridDim.x * WAVES;
  // the wave's units are u0, u0 + nwaves, ...; lane l fetches the page id (and
  // valid count) of the l-th of the next 64 in one load, and a ballot lists
  // those with a page: skipped entries (negative ids) then cost no memory
  // round trip, however long the list
  for (long ub = (long)blockIdx.x * WAVES + (threadIdx.x >> 6); ub < units; ub += kWave * nwaves) {
    const long ul = ub + (long)lane * nwaves;
    const int il = ul < units ? (int)(ul / Hkv) : 0;
    const int pid_l = ul < units ? page_ids[il] : -1;
    const int nv_l = (ul < units && valid_tokens) ? valid_tokens[il] : kBlockSize;
    uint64_t todo = __ballot(pid_l >= 0);
    while (todo) {
      const int slot = __builtin_ctzll(todo);      // wave-uniform
      todo &= todo - 1;
      const long u = ub + (long)slot * nwaves;
      const int i = (int)(u / Hkv);
      const int j = (int)(u - (long)i * Hkv);
      const int pid = __builtin_amdgcn_readlane(pid_l, slot);
      const int nv = __builtin_amdgcn_readlane(nv_l, slot);
      const size_t tile = (size_t)pid * Hkv + j;
      uint4 w[2][RPL];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const St* src = static_cast<const St*>(t ? v_cache : k_cache) + tile * kBlockSize * D +
                        (size_t)c * E;
#pragma unroll
        for (int k = 0; k < RPL; ++k) w[t][k] = load16_stream(src + (size_t)(k * RG + g) * D);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint8_t* dst = (t ? v8 : k8) + tile * kBlockSize * RB + (size_t)c * CB;
        float amax = 0.0f;
#pragma unroll
        for (int k = 0; k < RPL; ++k) {
          if (k * RG + g < nv) {
            float f[E];
            DT::widen(w[t][k], f);
#pragma unroll
            for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(f[e]));
          }
        }
        amax = group_reduce<kWave, OpMax>(amax);
        const float sc = amax > 0.0f ? __fdiv_rn(amax, FMT == kFmtFp8 ? 448.0f : 7.0f) : 1.0f;
#pragma unroll
        for (int k = 0; k < RPL; ++k) {
          const int r = k * RG + g;
          if constexpr (FMT == kFmtFp8) {
            CodeChunk<E> cc;
#pragma unroll
            for (int q = 0; q < E / 4; ++q) cc.w[q] = 0u;
            if (r < nv) {
              float f[E];
              DT::widen(w[t][k], f);
#pragma unroll
              for (int e = 0; e < E; ++e)
                cc.w[e / 4] |= fp8_encode(__fdiv_rn(f[e], sc)) << (8 * (e % 4));
            }
            store_codes<E>(dst + (size_t)r * RB, cc);
          } else {
            uint32_t cw = 0u;                  // eight nibbles, channel e in bits 4e..4e+3
            if (r < nv) {
              float f[E];
              DT::widen(w[t][k], f);
#pragma unroll
              for (int e = 0; e < E; ++e) cw |= int4_encode(__fdiv_rn(f[e], sc)) << (4 * e);
            }
            *reinterpret_cast<uint32_t*>(dst + (size_t)r * RB) = cw;
          }
        }
        if (lane == 0) scales[tile * 2 + t] = sc;
      }
    }
  }
}

hipError_t launch_quantize(int fmt, int dtype, int D, const void* k_cache, const void* v_cache,
                           const int32_t* page_ids, const int32_t* valid_tokens, int n_ids,
                           int Hkv, uint8_t* k8, uint8_t* v8, float* scales, hipStream_t stream) {
  if (n_ids <= 0) return hipSuccess;
  return with_dtype(dtype, [&](auto dt) {
    return with_dim(D, [&](auto d) {
      using DT = decltype(dt);
      constexpr int DD = decltype(d)::value;
      constexpr int WAVES = 4;
      const long units = (long)n_ids * Hkv;          // one wave per unit up to the cap
      const long want = (units + WAVES - 1) / WAVES;
      const int grid = (int)std::min<long>(want, (long)cu_count() * KVD_QUANT_WGS_PER_CU);
      if (fmt == kFmtFp8) {
        hipLaunchKernelGGL((quantize_kernel<DT, DD, WAVES, kFmtFp8>), dim3(grid),
                           dim3(WAVES * kWave), 0, stream, k_cache, v_cache, page_ids,
                           valid_tokens, n_ids, Hkv, k8, v8, scales);
      } else if constexpr (DT::E == 8) {
        hipLaunchKernelGGL((quantize_kernel<DT, DD, WAVES, kFmtInt4>), dim3(grid),
                           dim3(WAVES * kWave), 0, stream, k_cache, v_cache, page_ids,
                           valid_tokens, n_ids, Hkv, k8, v8, scales);
      } else {
        return hipErrorInvalidValue;          // INT4 pages from 16-bit sources only
      }
      return hipGetLastError();
    });
  });
}

}  // namespace kvd

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

// Lane (us, c) owns channel chunk c (E channels) of unit us of a wave step, as
// in the index build: a unit is one (page, KV head); a wave step covers
// 64 / LPR consecutive units.  The lane keeps the unit's 16 rows of its chunk
// in registers, the LPR lanes of the unit reduce the amax, and every lane then
// encodes and stores its own chunk.  K and V are done one after the other.
constexpr int kFmtFp8 = 8, kFmtInt4 = 4;

template <typename DT, int D, int WAVES, int FMT>
__global__ __launch_bounds__(WAVES * kWave) void quantize_kernel(
    const void* __restrict__ k_cache, const void* __restrict__ v_cache,
    const int32_t* __restrict__ page_ids, const int32_t* __restrict__ valid_tokens, int n_ids,
    int Hkv, uint8_t* __restrict__ k8, uint8_t* __restrict__ v8, float* __restrict__ scales) {
  using G_ = RowGeom<DT, D>;
  using St = typename DT::storage;
  constexpr int E = G_::E, LPR = G_::LPR;
  static_assert(FMT == kFmtFp8 || E == 8, "INT4 pages hold 16-bit sources (8 channels per lane)");
  // code bytes per row and per lane chunk
  constexpr int RB = FMT == kFmtFp8 ? D : D / 2, CB = FMT == kFmtFp8 ? E : E / 2;
  constexpr int UPS = kWave / LPR;
  const int lane = threadIdx.x & (kWave - 1);
  const int us = lane / LPR, c = lane % LPR;
  const long units = (long)n_ids * Hkv;
  const long steps = (units + UPS - 1) / UPS;
  const long nwaves = (long)gridDim.x * WAVES;

  for (long step = (long)blockIdx.x * WAVES + (threadIdx.x >> 6); step < steps; step += nwaves) {
    const long u = step * UPS + us;
    if (u >= units) continue;                      // the whole unit's lanes skip together
    const int i = (int)(u / Hkv);
    const int j = (int)(u - (long)i * Hkv);
    const int pid = page_ids[i];
    if (pid < 0) continue;                         // a skipped list entry (unit-uniform)
    const size_t tile = (size_t)pid * Hkv + j;
    const int nv = valid_tokens ? valid_tokens[i] : kBlockSize;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const St* src = static_cast<const St*>(t ? v_cache : k_cache) + tile * kBlockSize * D +
                      (size_t)c * E;
      uint8_t* dst = (t ? v8 : k8) + tile * kBlockSize * RB + (size_t)c * CB;
      uint4 w[kBlockSize];
#pragma unroll
      for (int r = 0; r < kBlockSize; ++r) w[r] = load16_stream(src + (size_t)r * D);
      float amax = 0.0f;
#pragma unroll
      for (int r = 0; r < kBlockSize; ++r) {
        if (r < nv) {
          float f[E];
          DT::widen(w[r], f);
#pragma unroll
          for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(f[e]));
        }
      }
      amax = group_reduce<LPR, OpMax>(amax);
      const float sc = amax > 0.0f ? __fdiv_rn(amax, FMT == kFmtFp8 ? 448.0f : 7.0f) : 1.0f;
#pragma unroll
      for (int r = 0; r < kBlockSize; ++r) {
        if constexpr (FMT == kFmtFp8) {
          CodeChunk<E> cc;
#pragma unroll
          for (int k = 0; k < E / 4; ++k) cc.w[k] = 0u;
          if (r < nv) {
            float f[E];
            DT::widen(w[r], f);
#pragma unroll
            for (int e = 0; e < E; ++e)
              cc.w[e / 4] |= fp8_encode(__fdiv_rn(f[e], sc)) << (8 * (e % 4));
          }
          store_codes<E>(dst + (size_t)r * RB, cc);
        } else {
          uint32_t cw = 0u;                  // eight nibbles, channel e in bits 4e..4e+3
          if (r < nv) {
            float f[E];
            DT::widen(w[r], f);
#pragma unroll
            for (int e = 0; e < E; ++e) cw |= int4_encode(__fdiv_rn(f[e], sc)) << (4 * e);
          }
          *reinterpret_cast<uint32_t*>(dst + (size_t)r * RB) = cw;
        }
      }
      if (c == 0) scales[tile * 2 + t] = sc;
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
      constexpr int UPS = kWave / RowGeom<DT, DD>::LPR;
      const long steps = ((long)n_ids * Hkv + UPS - 1) / UPS;
      const long want = (steps + WAVES - 1) / WAVES;
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

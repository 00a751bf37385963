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
//
// bf16 sources take those quotients from a table.  A bf16 value is
// x = s 2^(E-127) 1.m with a 7-bit m (or a signed zero or subnormal for E = 0),
// and scaling by a power of two is exact, so RN(x / sc) = s 2^(E-127)
// RN(1.m / sc) wherever the right side is a normal fp32 number; where it is
// not, |x / sc| < 2^-126 and the code is a signed zero either way.  Per unit
// and tensor, the 128 correctly rounded RN(1.m / sc) go to LDS (two divisions
// per lane) and each quotient is one lookup and one product.  The E4M3 codes
// of those quotients come from v_cvt_pk_fp8_f32, which for every finite
// |y| < 464 gives the code of the rounding rule above (round to nearest even,
// subnormals kept; checked against it over all fp32 inputs); the quotients
// stay below 448 (1 + 2^-22).  INT4 quotients stay within 7 (1 + 2^-22), so
// their nearest integers need no clamp, and one fma with 1.5 * 2^23 rounds the
// (exact) product to the nearest integer, ties to even, in the low mantissa
// bits.  The unit maximum is taken over the bf16 magnitudes as 16-bit
// integers, whose order is that of the values, and a magnitude at or above
// 0x7f80 reveals an infinity or a NaN.  Units with a value that is not
// finite, or whose scale is outside [2^-125, 2^125] (so a table entry could
// overflow), take the maximum ignoring NaNs and divide.
#include <type_traits>

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

// Code stores are non-temporal: the pools are written once and read by later
// steps (over rotated full pools: FP8 150 -> 141 us, INT4 133 -> 121 us).
#ifndef KVD_QUANT_NT_STORE
#define KVD_QUANT_NT_STORE 1
#endif

typedef unsigned int u32x2_sv __attribute__((ext_vector_type(2)));

__device__ inline void store_code_word(uint8_t* dst, uint32_t w) {
  if constexpr (KVD_QUANT_NT_STORE)
    __builtin_nontemporal_store(w, reinterpret_cast<unsigned int*>(dst));
  else
    *reinterpret_cast<uint32_t*>(dst) = w;
}

template <int E>
__device__ inline void store_codes(uint8_t* dst, const CodeChunk<E>& cc) {
  if constexpr (E == 8) {
    if constexpr (KVD_QUANT_NT_STORE)
      __builtin_nontemporal_store(u32x2_sv{cc.w[0], cc.w[1]}, reinterpret_cast<u32x2_sv*>(dst));
    else
      *reinterpret_cast<uint2*>(dst) = make_uint2(cc.w[0], cc.w[1]);
  } else {
    static_assert(E == 4, "4 or 8 channels per chunk");
    store_code_word(dst, cc.w[0]);
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

typedef unsigned short u16x2_v __attribute__((ext_vector_type(2)));

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
  constexpr bool kTable = std::is_same<DT, BF16>::value;
  __shared__ float qtab[kTable ? WAVES : 1][2][128];   // RN(1.m / sc) of the wave's unit
  float* const tabw = qtab[kTable ? (threadIdx.x >> 6) : 0][0];
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
        auto amax_of = [&]() {                     // over the valid rows, NaNs ignored
          float a = 0.0f;
#pragma unroll
          for (int k = 0; k < RPL; ++k) {
            if (k * RG + g < nv) {
              float f[E];
              DT::widen(w[t][k], f);
#pragma unroll
              for (int e = 0; e < E; ++e) a = fmaxf(a, fabsf(f[e]));
            }
          }
          return a;
        };
        bool table = false;                        // wave-uniform
        float amax;
        if constexpr (kTable) {
          u16x2_v m2 = {0, 0};                     // largest magnitude bits of each half
#pragma unroll
          for (int k = 0; k < RPL; ++k) {
            if (k * RG + g < nv) {
              const uint32_t wv[4] = {w[t][k].x, w[t][k].y, w[t][k].z, w[t][k].w};
#pragma unroll
              for (int q = 0; q < 4; ++q)
                m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2_v, wv[q] & 0x7fff7fffu));
            }
          }
          const uint32_t mb = m2.x > m2.y ? m2.x : m2.y;
          table = __ballot(mb >= 0x7f80u) == 0ull;
          amax = table ? __uint_as_float(mb << 16) : amax_of();
        } else {
          amax = amax_of();
        }
        amax = group_reduce<kWave, OpMax>(amax);
        const float sc = amax > 0.0f ? __fdiv_rn(amax, FMT == kFmtFp8 ? 448.0f : 7.0f) : 1.0f;
        float* const tab = tabw + t * 128;
        if constexpr (kTable) {
          table = table && sc >= 0x1p-125f && sc <= 0x1p125f;
          if (table) {
            // the wave's earlier reads of this table were consumed before
            // these writes, and one wave's LDS operations run in order
            tab[lane] = __fdiv_rn(1.0f + (float)lane * 0x1p-7f, sc);
            tab[lane + 64] = __fdiv_rn(1.5f + (float)lane * 0x1p-7f, sc);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
          }
        }
        // quotient of bf16 word half (hi: bits 16..31) from the table
        auto tq = [&](uint32_t wd, bool hi) {
          const uint32_t m = hi ? (wd >> 16) & 0x7fu : wd & 0x7fu;
          const uint32_t p = (hi ? wd : wd << 16) & 0xff800000u;   // s 2^(E-127), or a signed zero
          return tab[m] * __uint_as_float(p);
        };
#pragma unroll
        for (int k = 0; k < RPL; ++k) {
          const int r = k * RG + g;
          const uint32_t wv[4] = {w[t][k].x, w[t][k].y, w[t][k].z, w[t][k].w};
          if constexpr (FMT == kFmtFp8) {
            CodeChunk<E> cc;
#pragma unroll
            for (int q = 0; q < E / 4; ++q) cc.w[q] = 0u;
            if (r < nv) {
              if (kTable && table) {
#pragma unroll
                for (int q = 0; q < E / 4; ++q) {
                  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(tq(wv[2 * q], false),
                                                                 tq(wv[2 * q], true), 0, false);
                  cc.w[q] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
                      tq(wv[2 * q + 1], false), tq(wv[2 * q + 1], true), lo, true);
                }
              } else {
                float f[E];
                DT::widen(w[t][k], f);
#pragma unroll
                for (int e = 0; e < E; ++e)
                  cc.w[e / 4] |= fp8_encode(__fdiv_rn(f[e], sc)) << (8 * (e % 4));
              }
            }
            store_codes<E>(dst + (size_t)r * RB, cc);
          } else {
            uint32_t cw = 0u;                  // eight nibbles, channel e in bits 4e..4e+3
            if (r < nv) {
              if (kTable && table) {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                  const uint32_t wd = wv[e / 2];
                  const bool hi = (e & 1) != 0;
                  const uint32_t m = hi ? (wd >> 16) & 0x7fu : wd & 0x7fu;
                  const uint32_t p = (hi ? wd : wd << 16) & 0xff800000u;
                  const float y = fmaf(tab[m], __uint_as_float(p), 0x1.8p23f);   // 1.5 * 2^23 + n
                  cw |= (__float_as_uint(y) & 15u) << (4 * e);
                }
              } else {
                float f[E];
                DT::widen(w[t][k], f);
#pragma unroll
                for (int e = 0; e < E; ++e) cw |= int4_encode(__fdiv_rn(f[e], sc)) << (4 * e);
              }
            }
            store_code_word(dst + (size_t)r * RB, cw);
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

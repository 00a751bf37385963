// Device helpers shared by the gfx950 kernels: storage-dtype traits (16-byte
// chunk loads and exact widening to fp32) and wave64 cross-lane reductions
// built from DPP row operations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvd {

constexpr int kWave = 64;
constexpr int kBlockSize = 16;  // tokens per KV page

// ---------------------------------------------------------------- dtypes
//
// Every kernel moves K/V/meta in 16-byte chunks (global_load_dwordx4), so a
// chunk holds E = 16 / sizeof(element) channels.

struct F32 {
  using storage = float;
  static constexpr int E = 4;
  __device__ static inline void widen(const uint4& w, float* f) {
    f[0] = __uint_as_float(w.x);
    f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z);
    f[3] = __uint_as_float(w.w);
  }
  __device__ static inline uint4 narrow_exact(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};

struct BF16 {
  using storage = uint16_t;
  static constexpr int E = 8;
  __device__ static inline void widen2(uint32_t w, float& lo, float& hi) {
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xffff0000u);
  }
  __device__ static inline void widen(const uint4& w, float* f) {
    widen2(w.x, f[0], f[1]);
    widen2(w.y, f[2], f[3]);
    widen2(w.z, f[4], f[5]);
    widen2(w.w, f[6], f[7]);
  }
  // Only for values that are exactly representable in bf16 (a min or max of
  // bf16 inputs): the low 16 bits of the fp32 pattern are zero.
  __device__ static inline uint32_t pack2(float lo, float hi) {
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
  }
  __device__ static inline uint4 narrow_exact(const float* f) {
    return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
  }
};

struct F16 {
  using storage = _Float16;
  static constexpr int E = 8;
  __device__ static inline void widen2(uint32_t w, float& lo, float& hi) {
    _Float16 a = __builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    _Float16 b = __builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    lo = (float)a;
    hi = (float)b;
  }
  __device__ static inline void widen(const uint4& w, float* f) {
    widen2(w.x, f[0], f[1]);
    widen2(w.y, f[2], f[3]);
    widen2(w.z, f[4], f[5]);
    widen2(w.w, f[6], f[7]);
  }
  __device__ static inline uint32_t pack2(float lo, float hi) {
    uint16_t a = __builtin_bit_cast(uint16_t, (_Float16)lo);
    uint16_t b = __builtin_bit_cast(uint16_t, (_Float16)hi);
    return (uint32_t)a | ((uint32_t)b << 16);
  }
  __device__ static inline uint4 narrow_exact(const float* f) {
    return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
  }
};

__device__ inline uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Loads of K/V (and key-pool) data that is read exactly once.  With
// KVD_NT_LOADS=1 (the default) they carry the non-temporal hint, so streamed
// bytes do not displace reusable lines in the caches; on the 128k GQA dense
// pass this took the kernel from 97.6 to 87.2 us.
#ifndef KVD_NT_LOADS
#define KVD_NT_LOADS 1
#endif
typedef unsigned int u32x4_v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_v __attribute__((ext_vector_type(2)));
__device__ inline uint4 load16_stream(const void* p) {
#if KVD_NT_LOADS
  const u32x4_v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_v*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}
__device__ inline uint2 load8_stream(const void* p) {
#if KVD_NT_LOADS
  const u32x2_v v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_v*>(p));
  return make_uint2(v.x, v.y);
#else
  return *reinterpret_cast<const uint2*>(p);
#endif
}
__device__ inline uint32_t load4_stream(const void* p) {
#if KVD_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<const unsigned int*>(p));
#else
  return *reinterpret_cast<const unsigned int*>(p);
#endif
}
__device__ inline uint32_t load2_stream(const void* p) {
#if KVD_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<const unsigned short*>(p));
#else
  return *reinterpret_cast<const unsigned short*>(p);
#endif
}
__device__ inline void store16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ inline void store8(void* p, const uint2& v) { *reinterpret_cast<uint2*>(p) = v; }
__device__ inline void store4(void* p, uint32_t v) { *reinterpret_cast<uint32_t*>(p) = v; }
__device__ inline void store2(void* p, uint32_t v) { *reinterpret_cast<uint16_t*>(p) = (uint16_t)v; }

// ---------------------------------------------------------------- FP8 E4M3 pages
//
// Cold K/V pages hold OCP FP8 E4M3 codes (1 byte per channel) with one fp32
// scale per (page, KV head) and tensor.  gfx950's v_cvt_pk_f32_fp8 decodes
// E4M3 exactly (every one of the 256 codes was checked on the GPU against the
// format's table); a decoded value has at most 4 significant bits and lies in
// [2^-9, 448], so it is also exact in bf16 and fp16.

typedef float f32x2_v __attribute__((ext_vector_type(2)));

__device__ inline void fp8x4_to_f32(uint32_t w, float* f) {
  const f32x2_v a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2_v b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = a.x;
  f[1] = a.y;
  f[2] = b.x;
  f[3] = b.y;
}

// Round an fp32 value to the nearest E4M3 code (ties to the even code);
// magnitudes of 464 and more saturate to 448.  Below 2^-6 the grid is the
// multiples of 2^-9; above, fp32's mantissa is cut to 3 bits with the usual
// round-half-even carry, and the exponent is rebiased from 127 to 7.
__device__ inline uint32_t fp8_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  uint32_t code;
  if (a > 0x7f800000u) code = 0x7fu;                          // NaN
  else if (a >= 0x43e80000u) code = 0x7eu;                    // >= 464
  else if (a < 0x3c800000u) code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  else code = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  return sign | code;
}

// ---------------------------------------------------------------- INT4 pages
//
// Cold K/V pages may hold symmetric INT4 codes n in [-7, 7] (two per byte,
// 4-bit two's complement, the even channel in the low nibble) with one fp32
// scale per (page, KV head) and tensor.  Small integers are exact in fp32,
// bf16 and fp16.

// Code e (0..7) of a dword of eight nibbles, sign-extended.
__device__ inline int int4_code(uint32_t w, int e) { return (int)(w << (28 - 4 * e)) >> 28; }

__device__ inline void int4x8_to_f32(uint32_t w, float* f) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (float)int4_code(w, e);
}

// Round an fp32 quotient x / scale to an INT4 code: nearest, ties to even,
// clamped to [-7, 7]; returned as its nibble.
__device__ inline uint32_t int4_encode(float y) {
  const float r = fminf(fmaxf(__builtin_rintf(y), -7.0f), 7.0f);
  return (uint32_t)(int)r & 15u;
}

// ---------------------------------------------------------------- matrix cores
//
// v_mfma_f32_16x16x32_{bf16,f16}: D (16 x 16, fp32) = A (16 x 32) B (32 x 16) + C.
// Lane l holds A[l % 16][8 (l / 16) .. + 8], B[8 (l / 16) .. + 8][l % 16] (eight
// 16-bit values, 16 bytes) and D[4 (l / 16) + i][l % 16] for i = 0..3.

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

template <typename DT>
__device__ inline f32x4_v mfma_16x16x32(const uint4& a, const uint4& b, f32x4_v c);
template <>
__device__ inline f32x4_v mfma_16x16x32<BF16>(const uint4& a, const uint4& b, f32x4_v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a),
                                                 __builtin_bit_cast(bf16x8_v, b), c, 0, 0, 0);
}
template <>
__device__ inline f32x4_v mfma_16x16x32<F16>(const uint4& a, const uint4& b, f32x4_v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_v, a),
                                                __builtin_bit_cast(f16x8_v, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- lane shuffles
//
// DPP controls (gfx9 encoding): quad_perm, row_mirror (lane i <-> 15-i in a
// 16-lane row), row_half_mirror (i <-> 7-i in each 8-lane half row).

enum : int {
  kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
  kDppHalfMirror = 0x141,
  kDppMirror = 0x140,
};

template <int CTRL>
__device__ inline float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ inline float xor16(float v) {
  // ds_swizzle bit mode inside each 32-lane half: and 0x1F, or 0, xor 0x10.
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}
__device__ inline float xor32(float v) { return __shfl_xor(v, 32, kWave); }

// Max over lanes l, l ^ 16, l ^ 32 and l ^ 48 (one lane of each 16-lane row)
// with gfx950's row-swap permutes, which stay in the VALU (no LDS round trip):
// permlane16_swap of a register with itself returns, per lane, its own value
// and that of lane l ^ 16 (in one order or the other); permlane32_swap the same
// for l ^ 32.  Every lane of the wave must be active.
__device__ inline float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

struct OpSum {
  __device__ static inline float apply(float a, float b) { return a + b; }
};
struct OpMax {
  __device__ static inline float apply(float a, float b) { return fmaxf(a, b); }
};
struct OpMin {
  __device__ static inline float apply(float a, float b) { return fminf(a, b); }
};

// All-reduce over aligned groups of N lanes (N = 1..64, a power of two); every
// lane of a group ends with the group's result.  Each step pairs a lane with a
// lane of the other half of its current group, which is enough for sum, min
// and max once the lower levels are uniform.
template <int N, typename Op>
__device__ inline float group_reduce(float v) {
  if constexpr (N >= 2) v = Op::apply(v, dpp<kDppXor1>(v));
  if constexpr (N >= 4) v = Op::apply(v, dpp<kDppXor2>(v));
  if constexpr (N >= 8) v = Op::apply(v, dpp<kDppHalfMirror>(v));
  if constexpr (N >= 16) v = Op::apply(v, dpp<kDppMirror>(v));
  if constexpr (N >= 32) v = Op::apply(v, xor16(v));
  if constexpr (N >= 64) v = Op::apply(v, xor32(v));
  return v;
}

// Reduce across the row groups of a wave: lanes l and l ^ k for k = N .. 32,
// i.e. over all lanes with the same position inside their N-lane group.  The
// pairing is a true xor so values that differ inside a group stay apart.
template <int N, typename Op>
__device__ inline float cross_group_reduce(float v) {
  static_assert(N >= 8 && N <= 64, "row groups are 8..64 lanes wide");
  if constexpr (N <= 8) v = Op::apply(v, __shfl_xor(v, 8, kWave));
  if constexpr (N <= 16) v = Op::apply(v, xor16(v));
  if constexpr (N <= 32) v = Op::apply(v, xor32(v));
  return v;
}

// ---------------------------------------------------------------- integer wave ops
//
// Without LDS round trips: DPP row_shr:n (each 16-lane row shifted up by n
// lanes; lanes with no source read 0), row_bcast:15 / row_bcast:31 (lane 15 /
// lane 31 fed to the rows enabled by the row mask), and readlane.  Every lane
// of the wave must be active.

enum : int {
  kDppRowShr1 = 0x111,
  kDppRowShr2 = 0x112,
  kDppRowShr4 = 0x114,
  kDppRowShr8 = 0x118,
  kDppRowBcast15 = 0x142,
  kDppRowBcast31 = 0x143,
};

template <int CTRL, int ROW_MASK = 0xF>
__device__ inline uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}

// inclusive prefix sum over the wave's 64 lanes
__device__ inline uint32_t wave_scan_add_u32(uint32_t v) {
  v += dpp_u32<kDppRowShr1>(v);
  v += dpp_u32<kDppRowShr2>(v);
  v += dpp_u32<kDppRowShr4>(v);
  v += dpp_u32<kDppRowShr8>(v);
  v += dpp_u32<kDppRowBcast15, 0xA>(v);   // row 0's total into row 1, row 2's into row 3
  v += dpp_u32<kDppRowBcast31, 0xC>(v);   // rows 0-1's total into rows 2 and 3
  return v;
}

struct MinU32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return min(a, b); }
};
struct MaxU32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return max(a, b); }
};
struct AddU32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};

// all-reduce over the wave: inside each 16-lane row with DPP, then the four
// row results read as scalars (the result is wave-uniform)
template <typename Op>
__device__ inline uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, dpp_u32<kDppXor1>(v));
  v = op(v, dpp_u32<kDppXor2>(v));
  v = op(v, dpp_u32<kDppHalfMirror>(v));
  v = op(v, dpp_u32<kDppMirror>(v));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return op(op(r0, r1), op(r2, r3));
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline int lane_id() { return __lane_id(); }

__device__ inline int readlane(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }

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

}  // namespace kvd

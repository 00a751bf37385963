// Read-ceiling probes that the benchmark reports the kernels against: they
// move the same kind of bytes as the path but compute nothing (an XOR of
// what they load, one word written per workgroup or wave so no load is dead).
//
//   stream_read_kernel  one buffer read with 16-byte non-temporal loads, one
//                       contiguous range per workgroup (also over mapped host
//                       memory: the kernel-side host-read rate)
//   gather_read_kernel  the dense decode attention's own loads: per (split,
//                       KV head, sequence) wave the K and V tiles of its pages
//                       in block-table order, in the matrix-core kernel's lane
//                       layout, one page ahead
//
// And one probe of an instruction the quantizer relies on:
//
//   fp8_convert_kernel  every fp32 bit pattern through v_cvt_pk_fp8_f32 (as
//                       the first operand, and XOR 0x80012345 as the second)
//                       against fp8_encode, the E4M3 rounding rule the codes
//                       are defined by; mismatches counted per magnitude class
#include "kvd_device.hpp"
#include "kvd_dispatch.hpp"
#include "kvd_launch.hpp"

namespace kvd {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(
    const uint8_t* __restrict__ buf, size_t chunks, uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[kProbeThreads / kWave];
  // one contiguous range of 16-byte chunks per workgroup, four loads in flight
  // per lane (a grid-stride walk over the same buffer was measured slower)
  constexpr int U = 4;
  const size_t per = (chunks + gridDim.x - 1) / gridDim.x;
  const size_t c0 = min((size_t)blockIdx.x * per, chunks), c1 = min(c0 + per, chunks);
  uint4 acc = make_uint4(0, 0, 0, 0);
  size_t i = c0 + threadIdx.x;
  for (; i + (U - 1) * kProbeThreads < c1; i += U * kProbeThreads) {
    uint4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = load16_stream(buf + (i + (size_t)u * kProbeThreads) * 16);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc.x ^= r[u].x; acc.y ^= r[u].y; acc.z ^= r[u].z; acc.w ^= r[u].w;
    }
  }
  for (; i < c1; i += kProbeThreads) {
    const uint4 a = load16_stream(buf + i * 16);
    acc.x ^= a.x; acc.y ^= a.y; acc.z ^= a.z; acc.w ^= a.w;
  }
  uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v ^= (uint32_t)__shfl_xor((int)v, off, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / kWave; ++w) t ^= red[w];
    sink[blockIdx.x] = t;
  }
}

template <typename DT, int D, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) void gather_read_kernel(
    const void* __restrict__ k_cache, const void* __restrict__ v_cache,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int Hkv,
    int maxN, int S, uint32_t* __restrict__ sink) {
  using St = typename DT::storage;
  constexpr int KS = D / 32, NDW = D / 32;
  const int lane = threadIdx.x & (kWave - 1);
  const int s = blockIdx.x * WAVES + (threadIdx.x >> 6);
  if (s >= S) return;
  const int j = blockIdx.y, b = blockIdx.z;
  const int col = lane & 15, grp = lane >> 4;
  const int nb = (seq_lens[b] + kBlockSize - 1) / kBlockSize;
  const int chunk = (nb + S - 1) / S;
  const int p0 = min(s * chunk, nb), p1 = min(p0 + chunk, nb);
  const size_t page_stride = (size_t)Hkv * kBlockSize * D;
  const St* kb = static_cast<const St*>(k_cache) + (size_t)j * kBlockSize * D + (size_t)col * D + 8 * grp;
  const St* vb = static_cast<const St*>(v_cache) + (size_t)j * kBlockSize * D +
                 (size_t)(4 * grp) * D + 2 * NDW * col;
  const int32_t* bt_row = block_table + (size_t)b * maxN;
  struct Regs {
    uint4 k[KS];
    uint4 v[4];
  };
  auto load = [&](Regs& r, int page) {
    const size_t off = (size_t)page * page_stride;
#pragma unroll
    for (int st = 0; st < KS; ++st) r.k[st] = load16_stream(kb + off + 32 * st);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (NDW == 4) {
        r.v[i] = load16_stream(vb + off + (size_t)i * D);
      } else {
        const uint2 t = load8_stream(vb + off + (size_t)i * D);
        r.v[i] = make_uint4(t.x, t.y, 0, 0);
      }
    }
  };
  uint32_t acc = 0;
  auto fold = [&](const Regs& r) {
#pragma unroll
    for (int st = 0; st < KS; ++st) acc ^= r.k[st].x ^ r.k[st].y ^ r.k[st].z ^ r.k[st].w;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc ^= r.v[i].x ^ r.v[i].y ^ r.v[i].z ^ r.v[i].w;
  };
  // page ids 64 at a time, one per lane, broadcast with readlane (as the
  // attention does: no scalar load on the path from one page to the next)
  for (int base = p0; base < p1; base += kWave) {
    const int cnt = min(kWave, p1 - base);
    const int my_page = lane < cnt ? bt_row[base + lane] : 0;
    Regs cur, nxt;
    load(cur, readlane(my_page, 0));
    for (int it = 0; it + 1 < cnt; ++it) {
      load(nxt, readlane(my_page, it + 1));
      fold(cur);
      cur = nxt;
    }
    fold(cur);
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, kWave);
  if (lane == 0) sink[((size_t)b * Hkv + j) * S + s] = acc;
}

// magnitude classes of an fp32 input: finite below 464 (where the quantizer
// uses the instruction), finite from 464 up, infinity, NaN
__device__ inline int fp8_probe_class(uint32_t u) {
  const uint32_t a = u & 0x7fffffffu;
  return a < 0x43e80000u ? 0 : a < 0x7f800000u ? 1 : a == 0x7f800000u ? 2 : 3;
}

__global__ void fp8_convert_init_kernel(unsigned long long* counts, uint32_t* first) {
  const int i = threadIdx.x;
  if (i < kProbeFp8Classes) {
    counts[i] = 0ull;
    first[i] = 0xffffffffu;
  }
}

__global__ __launch_bounds__(kProbeThreads) void fp8_convert_kernel(unsigned long long* counts,
                                                                   uint32_t* first) {
  unsigned long long c[kProbeFp8Classes];
  uint32_t f[kProbeFp8Classes];
#pragma unroll
  for (int k = 0; k < kProbeFp8Classes; ++k) {
    c[k] = 0ull;
    f[k] = 0xffffffffu;
  }
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 32); i += stride) {
    const uint32_t u0 = (uint32_t)i, u1 = u0 ^ 0x80012345u;
    const uint32_t hw = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(u0),
                                                                   __uint_as_float(u1), 0, false);
    const uint32_t v[2] = {u0, u1};
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      if (((hw >> (8 * o)) & 0xffu) != fp8_encode(__uint_as_float(v[o]))) {
        const int k = fp8_probe_class(v[o]);
#pragma unroll
        for (int q = 0; q < kProbeFp8Classes; ++q) {   // registers stay statically indexed
          if (q == k) {
            c[q] += 1ull;
            f[q] = min(f[q], v[o]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kProbeFp8Classes; ++k) {
    if (c[k]) {
      atomicAdd(&counts[k], c[k]);
      atomicMin(&first[k], f[k]);
    }
  }
}

hipError_t launch_fp8_convert(unsigned long long* counts, uint32_t* first, hipStream_t stream) {
  hipLaunchKernelGGL(fp8_convert_init_kernel, dim3(1), dim3(kWave), 0, stream, counts, first);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fp8_convert_kernel, dim3(cu_count() * 8), dim3(kProbeThreads), 0, stream,
                     counts, first);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int sink_words,
                              hipStream_t stream) {
  const size_t chunks = bytes / 16;
  const int grid = std::min<int>(sink_words, cu_count() * 8);
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(kProbeThreads), 0, stream,
                     static_cast<const uint8_t*>(buf), chunks, sink);
  return hipGetLastError();
}

hipError_t launch_gather_read(int dtype, int D, const void* k_cache, const void* v_cache,
                              const int32_t* block_table, const int32_t* seq_lens, int B, int Hkv,
                              int maxN, int S, uint32_t* sink, hipStream_t stream) {
  if (dtype == 0) return hipErrorInvalidValue;          // the 16-bit lane layout only
  return with_dtype(dtype, [&](auto dt) {
    return with_dim(D, [&](auto d) {
      constexpr int WAVES = 2;
      hipLaunchKernelGGL((gather_read_kernel<decltype(dt), decltype(d)::value, WAVES>),
                         dim3((S + WAVES - 1) / WAVES, Hkv, B), dim3(WAVES * kWave), 0, stream,
                         k_cache, v_cache, block_table, seq_lens, Hkv, maxN, S, sink);
      return hipGetLastError();
    });
  });
}

}  // namespace kvd

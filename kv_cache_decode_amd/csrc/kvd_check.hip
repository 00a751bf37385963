// gfx950 kernel that checks the device-side tables a decode call trusts.
//
//   check_tables_kernel  one workgroup per sequence b: L_b against [1, maxN*bs],
//                        the page ids of its live blocks against [0, P), and
//                        (when a selection is given) every (b, KV head) list:
//                        its count against [0, min(sel_stride, N_b)] and its
//                        entries strictly ascending inside [0, N_b)
//
// The kernel only reads the tables (every index it forms is bounded by maxN,
// Hkv and sel_stride, not by the data) and writes one result word per sequence.
#include "kvd_device.hpp"
#include "kvd_launch.hpp"

namespace kvd {

constexpr int kCheckThreads = 256;

__global__ __launch_bounds__(kCheckThreads) void check_tables_kernel(
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int sel_stride,
    int Hkv, int maxN, int num_pages, uint32_t* __restrict__ result) {
  __shared__ uint32_t bits_s;
  const int b = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) bits_s = 0u;
  __syncthreads();
  uint32_t bits = 0u;
  const long L = seq_lens[b];
  int nb = 0;
  if (L < 1 || L > (long)maxN * kBlockSize) {
    bits |= kCheckBadSeqLen;                    // the tables past this are not checked
  } else {
    nb = (int)((L + kBlockSize - 1) / kBlockSize);
    const int32_t* bt = block_table + (size_t)b * maxN;
    for (int n = tid; n < nb; n += kCheckThreads) {
      const int32_t p = bt[n];
      if (p < 0 || p >= num_pages) bits |= kCheckBadPageId;
    }
    if (sel) {
      for (int j = 0; j < Hkv; ++j) {
        const int32_t cnt = sel_count[(size_t)b * Hkv + j];
        if (cnt < 0 || cnt > sel_stride || cnt > nb) {
          if (tid == 0) bits |= kCheckBadSelCount;
          continue;
        }
        const int32_t* row = sel + ((size_t)b * Hkv + j) * sel_stride;
        for (int i = tid; i < cnt; i += kCheckThreads) {
          const int32_t n = row[i];
          if (n < 0 || n >= nb || (i > 0 && row[i - 1] >= n)) bits |= kCheckBadSelBlock;
        }
      }
    }
  }
  if (bits) atomicOr(&bits_s, bits);             // workgroup-local (LDS)
  __syncthreads();
  if (tid == 0) result[b] = bits_s;
}

hipError_t launch_check_tables(const int32_t* block_table, const int32_t* seq_lens,
                               const int32_t* sel, const int32_t* sel_count, int sel_stride,
                               int B, int Hkv, int maxN, int num_pages, uint32_t* result,
                               hipStream_t stream) {
  hipLaunchKernelGGL(check_tables_kernel, dim3(B), dim3(kCheckThreads), 0, stream, block_table,
                     seq_lens, sel, sel_count, sel_stride, Hkv, maxN, num_pages, result);
  return hipGetLastError();
}

}  // namespace kvd

// Host-side dispatch from runtime (dtype, head_dim, group size) to the
// compile-time kernel instances; included by the kernel sources only.
#pragma once

#include <type_traits>

#include "kvd_device.hpp"

namespace kvd {

// Map a runtime (dtype, head_dim, group size) to the compile-time instance;
// dtype codes follow kv_dtype (0 fp32, 1 fp16, 2 bf16).  Unknown values return
// hipErrorInvalidValue (the C ABI rejects them before this point).

template <typename F>
inline hipError_t with_dtype(int dtype, F&& f) {
  switch (dtype) {
    case 0: return f(F32{});
    case 1: return f(F16{});
    case 2: return f(BF16{});
  }
  return hipErrorInvalidValue;
}

template <typename F>
inline hipError_t with_dim(int D, F&& f) {
  switch (D) {
    case 64: return f(std::integral_constant<int, 64>{});
    case 128: return f(std::integral_constant<int, 128>{});
  }
  return hipErrorInvalidValue;
}

template <typename F>
inline hipError_t with_group(int G, F&& f) {
  switch (G) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 8: return f(std::integral_constant<int, 8>{});
  }
  return hipErrorInvalidValue;
}

}  // namespace kvd

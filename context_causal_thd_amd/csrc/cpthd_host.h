// Host-side helpers shared by the C-ABI entry points.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "../../include/cpthd.h"
#include "../../include/cpthd_timing.h"

namespace cpthd {

// A launch a call leaves out: its (start, stop) event pair, when the caller
// supplied one, is recorded back to back, so it times zero work.
inline int skip_launch(hipEvent_t* events, int n_events, int slot, hipStream_t stream) {
  if (!events || n_events < 2 * (slot + 1)) return CPTHD_OK;
  if (hipEventRecord(events[2 * slot], stream) != hipSuccess ||
      hipEventRecord(events[2 * slot + 1], stream) != hipSuccess)
    return CPTHD_ERR_LAUNCH;
  return CPTHD_OK;
}

// Launch `kernel` on `stream`; when the caller supplied a (start, stop) event
// pair for launch number `slot`, record it around the kernel.
template <typename... Params, typename... Args>
inline int launch(void (*kernel)(Params...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                  hipEvent_t* events, int n_events, int slot, Args... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "argument count");
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return skip_launch(events, n_events, slot, stream);
  auto tup = std::make_tuple(static_cast<Params>(args)...);
  void* ptrs[sizeof...(Params) + 1];
  std::apply([&](auto&... a) {
    int i = 0;
    ((ptrs[i++] = (void*)&a), ...);
  }, tup);
  hipError_t err;
  if (events && n_events >= 2 * (slot + 1)) {
    err = hipExtLaunchKernel((const void*)kernel, grid, block, ptrs, shmem, stream, events[2 * slot],
                             events[2 * slot + 1], 0);
  } else {
    err = hipLaunchKernel((const void*)kernel, grid, block, ptrs, shmem, stream);
  }
  return err == hipSuccess ? CPTHD_OK : CPTHD_ERR_LAUNCH;
}

inline int check_strategy(int32_t strategy) {
  return (strategy == CPTHD_DUAL_CHUNK_SWAP || strategy == CPTHD_NO_LOAD_BALANCE ||
          strategy == CPTHD_PACKED_SUPER_SEQUENCE)
             ? CPTHD_OK
             : CPTHD_ERR_STRATEGY;
}

// The whole-buffer mirrored strategy cuts T into 2*cp_size equal chunks.
inline int check_strategy_tokens(int32_t strategy, int64_t T, int32_t cp) {
  return (strategy == CPTHD_PACKED_SUPER_SEQUENCE && T % (2 * (int64_t)cp)) ? CPTHD_ERR_TOKENS : CPTHD_OK;
}

inline int check_tokens(int64_t T, int64_t capacity, int32_t cp, int32_t num_docs) {
  if (T <= 0 || num_docs < 1) return CPTHD_ERR_TOKENS;
  if (capacity < T) return CPTHD_ERR_TOKENS;
  if (T % cp) return CPTHD_ERR_TOKENS;
  if (capacity > INT32_MAX) return CPTHD_ERR_TOKENS;
  return CPTHD_OK;
}

// Kernels reading the rank-major all-gathered K/V address all T rows through
// one 32-bit buffer descriptor.
inline int check_allgathered_bytes(int64_t T, int32_t Hkv, int32_t D) {
  return T * Hkv * D * 2 < ((int64_t)1 << 31) ? CPTHD_OK : CPTHD_ERR_TOKENS;
}

inline int check_heads(int32_t Hq, int32_t Hkv, int32_t D) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv) return CPTHD_ERR_HEADS;
  if (Hq / Hkv > 64) return CPTHD_ERR_HEADS;
  if (D != 16 && D != 32 && D != 64 && D != 128) return CPTHD_ERR_HEADS;
  return CPTHD_OK;
}

}  // namespace cpthd

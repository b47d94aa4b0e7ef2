// HBM read-bandwidth probe (include/w12_probe.h): streams a buffer once with
// the 16-byte non-temporal loads the GEMM kernels use for records, so the
// GEMM's achieved bandwidth can be set beside what a plain read reaches on
// the same device, with the same occupancy choices.
#include <string.h>

#include "w12_internal.h"
#include "w12_probe.h"

namespace w12 {

// HW_REG_XCC_ID (hardware register 20), bits 3..0: the XCD running the wave.
constexpr int kHwRegXccId = 20 | (0 << 6) | (3 << 11);

template <int LD>
__device__ __forceinline__ void read_range(const uint8_t* buf, uint64_t lo, uint64_t hi, uint64_t first,
                                           uint64_t step, uint32_t& acc) {
  // words [lo, hi), this thread's first word `first`, LD loads `step` apart in
  // flight (an index past hi - 1 re-reads hi - 1; its value is folded too)
  for (uint64_t i = first; i < hi; i += step * LD) {
    uint4 v[LD];
#pragma unroll
    for (int j = 0; j < LD; ++j) {
      const uint64_t q = i + (uint64_t)j * step;
      v[j] = load_stream16(buf + 16 * (q < hi ? q : hi - 1));
    }
#pragma unroll
    for (int j = 0; j < LD; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  (void)lo;
}

template <int LD>
__global__ __launch_bounds__(1024) void k_probe_read(const uint8_t* __restrict__ buf, uint64_t n16, int mode,
                                                     uint64_t piece16, uint32_t* ctr, uint64_t* stamps, int never,
                                                     uint32_t* sink) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t B = blockDim.x;
  uint32_t acc = 0;
  if (mode == W12_PROBE_STATIC) {
    const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const uint64_t lo = min((uint64_t)blockIdx.x * per, n16), hi = min(lo + per, n16);
    read_range<LD>(buf, lo, hi, lo + threadIdx.x, B, acc);
  } else if (mode == W12_PROBE_STRIDE) {
    const uint64_t T = (uint64_t)gridDim.x * B;
    read_range<LD>(buf, 0, n16, (uint64_t)blockIdx.x * B + threadIdx.x, T, acc);
  } else if (mode == W12_PROBE_PIECES) {
    for (uint64_t lo = (uint64_t)blockIdx.x * piece16; lo < n16; lo += (uint64_t)gridDim.x * piece16)
      read_range<LD>(buf, lo, min(lo + piece16, n16), lo + threadIdx.x, B, acc);
  } else {
    // chunks of 4 passes of the workgroup's loads, taken in order from ctr[0];
    // the next chunk's number is fetched while the current one streams
    __shared__ uint32_t next;
    const uint64_t cw = B * LD * 4;
    const uint32_t nch = (uint32_t)((n16 + cw - 1) / cw);
    if (threadIdx.x == 0) next = atomicAdd(&ctr[0], 1u);
    __syncthreads();
    uint32_t c = next;
    while (c < nch) {
      __syncthreads();  // every thread has read `next`
      if (threadIdx.x == 0) next = atomicAdd(&ctr[0], 1u);
      const uint64_t lo = (uint64_t)c * cw, hi = min(lo + cw, n16);
      read_range<LD>(buf, lo, hi, lo + threadIdx.x, B, acc);
      __syncthreads();  // `next` is visible
      c = next;
    }
    // every workgroup has taken its last number once ctr[1] counts all of
    // them: the last one clears both counters for the next call
    if (threadIdx.x == 0) {
      const uint32_t done = __hip_atomic_fetch_add(&ctr[1], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (done == gridDim.x - 1) {
        __hip_atomic_store(&ctr[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctr[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if ((int)threadIdx.x == never) sink[blockIdx.x] = acc;  // never true: keeps the loads
  if (stamps) {
    __syncthreads();  // every wave's loads have returned (their data was folded)
    if (threadIdx.x == 0) {
      stamps[3 * (uint64_t)blockIdx.x] = t0;
      stamps[3 * (uint64_t)blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
      stamps[3 * (uint64_t)blockIdx.x + 2] = (uint64_t)__builtin_amdgcn_s_getreg(kHwRegXccId) & 15u;
    }
  }
}

}  // namespace w12

extern "C" int w12_probe_read(const void* buf, size_t bytes, int grid, int block, int loads, int mode,
                              size_t piece, int lds_bytes, uint64_t* stamps, void* ws, size_t ws_bytes,
                              void* stream) {
  using namespace w12;
  if (!buf || (reinterpret_cast<uintptr_t>(buf) & 15u) || bytes == 0 || bytes % 16 != 0 ||
      bytes > ((size_t)1 << 40))
    return W12_E_INVALID_ARG;
  if (grid < 1 || grid > (1 << 20) || block < 64 || block > 1024 || block % 64 != 0) return W12_E_INVALID_ARG;
  if (mode < W12_PROBE_STATIC || mode > W12_PROBE_PIECES) return W12_E_INVALID_ARG;
  if (mode == W12_PROBE_PIECES && (piece == 0 || piece % 16 != 0 || piece > bytes)) return W12_E_INVALID_ARG;
  if (lds_bytes < 0 || lds_bytes > 160 * 1024 - 64) return W12_E_INVALID_ARG;
  if (!ws || ws_bytes < W12_PROBE_WS_BYTES) return W12_E_WORKSPACE;
  uint32_t* ctr = reinterpret_cast<uint32_t*>(ws);
  uint32_t* sink = ctr + 32;
  const uint8_t* b = reinterpret_cast<const uint8_t*>(buf);
  const uint64_t n16 = bytes / 16;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 g(grid), t(block);
  switch (loads) {
    case 1: hipLaunchKernelGGL(k_probe_read<1>, g, t, lds_bytes, s, b, n16, mode, piece / 16, ctr, stamps, -1, sink); break;
    case 2: hipLaunchKernelGGL(k_probe_read<2>, g, t, lds_bytes, s, b, n16, mode, piece / 16, ctr, stamps, -1, sink); break;
    case 4: hipLaunchKernelGGL(k_probe_read<4>, g, t, lds_bytes, s, b, n16, mode, piece / 16, ctr, stamps, -1, sink); break;
    case 8: hipLaunchKernelGGL(k_probe_read<8>, g, t, lds_bytes, s, b, n16, mode, piece / 16, ctr, stamps, -1, sink); break;
    default: return W12_E_INVALID_ARG;
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? W12_OK : W12_E_HIP;
}

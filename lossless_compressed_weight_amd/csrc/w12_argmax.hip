// Per-row argmax over fp32 logits already in memory (the second pass of the
// LM-head argmax above 16 activation rows; SpecPilot Appendix E, the W12 LM
// head): y[m][0 .. N) -> the lowest n attaining the maximum, and that maximum.
//
// Workgroup (chunk, m) folds kArgChunk columns of row m into one 64-bit key
// (argmax_key: a larger value wins, the lower index wins equal values) and
// takes the atomic maximum into keys[m]. The last of a row's workgroups to
// arrive (a counter per row) writes idx[m] and max_logit[m] and clears the
// row's key and counter for the next call.
#include "w12_internal.h"

namespace w12 {

namespace {

constexpr int kArgThreads = 256;
constexpr int kArgChunk = 16384;  // columns per workgroup: 64 values per thread in 16-byte pieces
constexpr int kKeyStride = 32;    // keys and counters 256 bytes apart (separate lines and channels)

__global__ __launch_bounds__(kArgThreads) void k_rows_argmax(const float* __restrict__ y, int64_t ldy, int n, int M,
                                                            unsigned long long* keys, uint32_t* ctr, int32_t* idx,
                                                            float* maxv, const uint32_t* gate) {
  __shared__ unsigned long long wk[kArgThreads / 64];
  if (gated_off(gate)) return;
  const int m = blockIdx.y, c0 = blockIdx.x * kArgChunk;
  const float* yr = y + (int64_t)m * ldy;
  unsigned long long best = 0ull;
  // sixteen 16-byte loads per thread, all in flight together: N is a multiple
  // of 16, so a piece is wholly inside or wholly past the row, and a piece
  // past the row loads the row's last piece instead (no branch, so no wait
  // between the loads) and is skipped below
  constexpr int kPieces = kArgChunk / (4 * kArgThreads);
  float4 v[kPieces];
#pragma unroll
  for (int j = 0; j < kPieces; ++j) {
    const int c = c0 + 4 * (j * kArgThreads + (int)threadIdx.x);
    v[j] = *reinterpret_cast<const float4*>(yr + min(c, n - 4));
  }
#pragma unroll
  for (int j = 0; j < kPieces; ++j) {
    const int c = c0 + 4 * (j * kArgThreads + (int)threadIdx.x);
    if (c < n) {
      const float e[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned long long key = argmax_key(e[i], (uint32_t)(c + i));
        best = key > best ? key : best;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long t = __shfl_xor(best, o, 64);
    best = t > best ? t : best;
  }
  if ((threadIdx.x & 63) == 0) wk[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kArgThreads / 64; ++w) best = wk[w] > best ? wk[w] : best;
    // The maximum is an agent-scope atomic, performed at the device's
    // coherence point; waiting for it to complete before counting this
    // workgroup in means the last one to arrive reads every maximum there.
    // (Release/acquire fences at agent scope would also write back and
    // invalidate the XCD's whole L2 in every workgroup: 12 us more per call.)
    unsigned long long* key_m = keys + (int64_t)m * kKeyStride;
    uint32_t* ctr_m = ctr + (int64_t)m * 2 * kKeyStride;
    __hip_atomic_fetch_max(key_m, best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    // one counter per activation row, so the rows' workgroups do not queue
    // on a single address
    const bool last =
        __hip_atomic_fetch_add(ctr_m, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1u;
    if (last) {
      const unsigned long long key = __hip_atomic_load(key_m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      idx[m] = (int32_t)(0xFFFFFFFFu - (uint32_t)key);
      if (maxv) maxv[m] = key_value(key);
      __hip_atomic_store(key_m, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctr_m, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

hipError_t launch_rows_argmax(const float* y, int64_t ldy, int n, int M, unsigned long long* keys, uint32_t* ctr,
                              int32_t* idx, float* maxv, const uint32_t* gate, hipStream_t s) {
  if (M < 1 || M > kArgThreads || n < 1 || n % 16 != 0 || ldy % 4 != 0 ||
      (reinterpret_cast<uintptr_t>(y) & 15u) != 0)
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((n + kArgChunk - 1) / kArgChunk), (unsigned)M);
  hipLaunchKernelGGL(k_rows_argmax, grid, dim3(kArgThreads), 0, s, y, ldy, n, M, keys, ctr, idx, maxv, gate);
  return hipGetLastError();
}

}  // namespace w12

// W12 skinny GEMM kernels for gfx950: y[M, N] = x[M, K] W^T over W12 records.
//
// SpecPilot (arXiv 2611.02501) section 4.1 and Figure 5b: the kernel decodes
// records in registers so that the weight stream hides the decode, and splits
// the reduction loop over workgroups in a fixed order (stream-K), so results
// are deterministic. Section 4.3: the Q pass reads only the 8-bit view.
// Appendix E: the LM head in W12, here fused with a per-row argmax.
//
// Work decomposition (both kernels): the matrix is a sequence of row tiles
// (64 rows for the GEMV kernel, 16 for the MFMA kernel), each a sequence of
// units of 256 columns along K (one pipeline stage for each of a workgroup's
// four waves, so trip counts are exact). Workgroup p owns the contiguous unit
// range [p U / P, (p+1) U / P).
//
// A segment (the units of one tile that a workgroup owns) yields, per output
// row and activation row, A = sum of x * w' over its columns, where w' is the
// weight decoded with a fixed exponent bias (w = w' 2^(E_n - 127)), plus the
// escape corrections of its columns: CN = sum of x * placeholder and CP = sum
// of x * exact escape value. The segment's value is (A 2^(E_n-127) - CN) + CP.
// The scales and corrections are gathered by a helper wave while the
// streaming waves run, so finishing a segment needs no global loads.
//
// A tile covered by one workgroup is finished there. A tile split between
// workgroups: each stores its segment value in a fixed slot (2p for a
// workgroup's first tile, 2p+1 for its last) and counts itself in the tile's
// counter; the last to arrive adds the slots in workgroup order (so the result
// does not depend on arrival order) and writes the tile. Counters wrap back to
// zero, so every call leaves them zeroed for the next one.
#include "w12_internal.h"

namespace w12 {

constexpr int kUnitCols = 256;

// -------------------------------------------------------------- stream-K map
__device__ __forceinline__ int64_t unit_start(int64_t p, int64_t units, int P) { return p * units / P; }

// Workgroup owning unit u.
__device__ __forceinline__ int unit_owner(int64_t u, int64_t units, int P) {
  return (int)(((u + 1) * P + units - 1) / units) - 1;
}

__device__ __forceinline__ bool wg_empty(int q, const GemmParams& a) {
  return unit_start(q, a.units, a.P) == unit_start(q + 1, a.units, a.P);
}

// Slot of workgroup q's segment of tile t.
__device__ __forceinline__ int tile_slot(int q, int64_t t, const GemmParams& a) {
  return (unit_start(q, a.units, a.P) / a.ku == t) ? 2 * q : 2 * q + 1;
}

// -------------------------------------------------------------- outputs
__device__ __forceinline__ void emit(const GemmParams& a, int n, int m, float v, unsigned long long* kbest) {
  if (n >= a.n) return;
  if (a.mode == kModeStore) {
    if (a.y_f32) reinterpret_cast<float*>(a.y)[(int64_t)m * a.ldy + n] = v;
    else reinterpret_cast<uint16_t*>(a.y)[(int64_t)m * a.ldy + n] = f32_to_bf16_rne(v);
  } else {
    atomicMax(&kbest[m], argmax_key(v, (uint32_t)n));
  }
}

// Cross-workgroup exchange without an L2 writeback: segment values and keys
// are written and read with agent-scope atomic stores and loads (coherent
// across the XCDs' separate L2 caches); each thread waits until its own
// stores are acknowledged, then one thread counts the workgroup in.
__device__ __forceinline__ void store_shared(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_shared(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_shared(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long load_shared(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Count this workgroup into counter c (n arrivals in all; the counter wraps to
// 0 on the last). Returns, to every thread, whether this workgroup was last.
__device__ __forceinline__ bool arrive(uint32_t* c, uint32_t n, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);  // this thread's coherent stores are acknowledged
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __builtin_amdgcn_atomic_inc32(c, n - 1, __ATOMIC_RELAXED, "agent");
    *flag = old == n - 1;
  }
  __syncthreads();
  return *flag;
}

// Finish segment values value(m, row) of tile t (tile_rows rows from output
// row row0): written directly for a whole tile, through the slots and the
// tile counter for a split one.
template <class ValFn>
__device__ __forceinline__ void finish_segment(const GemmParams& a, int64_t t, int tile_rows, int row0, bool whole,
                                               int p, ValFn value, unsigned long long* kbest, int* flag) {
  const int nval = a.m * tile_rows;
  if (whole) {
    for (int i = threadIdx.x; i < nval; i += blockDim.x) {
      const int m = i / tile_rows, row = i % tile_rows;
      emit(a, row0 + row, m, value(m, row), kbest);
    }
    return;
  }
  float* dst = a.part + (int64_t)tile_slot(p, t, a) * a.m * tile_rows;
  for (int i = threadIdx.x; i < nval; i += blockDim.x) {
    const int m = i / tile_rows, row = i % tile_rows;
    store_shared(&dst[m * tile_rows + row], value(m, row));
  }
  const int64_t u_first = t * a.ku, u_last = min(a.units, (t + 1) * a.ku) - 1;
  const int pa = unit_owner(u_first, a.units, a.P), pb = unit_owner(u_last, a.units, a.P);
  uint32_t c = 0;
  for (int q = pa; q <= pb; ++q) c += !wg_empty(q, a);
  // a workgroup owns the first unit of at most one split tile, so the owner's
  // index names the tile's counter
  if (arrive(&a.ctr[pa], c, flag)) {
    for (int i = threadIdx.x; i < nval; i += blockDim.x) {
      const int m = i / tile_rows, row = i % tile_rows;
      float v = 0.f;
      for (int q = pa; q <= pb; ++q) {
        if (wg_empty(q, a)) continue;
        v += load_shared(&a.part[((int64_t)tile_slot(q, t, a) * a.m + m) * tile_rows + row]);
      }
      emit(a, row0 + row, m, v, kbest);
    }
  }
  __syncthreads();
}

// Argmax mode: publish this workgroup's best key per activation row; the last
// workgroup to finish reduces all of them into idx / max.
__device__ __forceinline__ void finish_argmax(const GemmParams& a, int p, unsigned long long* kbest, int* flag) {
  __syncthreads();
  if (threadIdx.x < a.m) store_shared(&a.keys[(int64_t)p * a.m + threadIdx.x], kbest[threadIdx.x]);
  if (arrive(&a.ctr[kMaxGrid], (uint32_t)a.P, flag)) {
    if (threadIdx.x < a.m) {
      unsigned long long best = 0ull;
      for (int q = 0; q < a.P; ++q) {
        const unsigned long long k = load_shared(&a.keys[(int64_t)q * a.m + threadIdx.x]);
        best = k > best ? k : best;
      }
      a.idx[threadIdx.x] = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
      if (a.maxv) a.maxv[threadIdx.x] = key_value(best);
    }
  }
}

// -------------------------------------------------------------- escapes
// First escape of row n with column >= c0 (binary search in the row's
// column-sorted list), and the end of the row's list.
__device__ __forceinline__ uint32_t esc_lower_bound(const GemmParams& a, int n, uint32_t c0, uint32_t* end) {
  uint32_t lo = a.row_ptr[n], hi = a.row_ptr[n + 1];
  *end = hi;
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (a.esc[mid].x < c0) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// The weight the main loop used for an escape: its placeholder, seen through
// the Q view (low nibble 1000) in the Q pass.
__device__ __forceinline__ float esc_placeholder(const GemmParams& a, uint32_t packed) {
  uint32_t ph = packed >> 16;
  if (a.q) ph = (ph & 0xFFF0u) | 0x8u;
  return bf16_to_f32(ph);
}

__device__ __forceinline__ float dot2_bf16(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, x), acc,
                                         false);
}

// Software pipeline over the units [u, ue) of one segment with two register
// stages: the loads of unit u+1 are in flight while unit u is computed. All
// loads are unconditional (a prefetch past the last unit re-reads it and is
// unused) and nothing with a data-dependent number of loads runs between
// them, so the compiler's vmcnt waits stay exact and the prefetch overlaps.
template <class Stage, class Load, class Compute>
__device__ __forceinline__ void pipeline(int u, int ue, Load&& load, Compute&& compute) {
  // Loop invariant: at the top, only stage a's loads (unit u + i) are in flight.
  Stage sa, sb;
  load(sa, u);
  const int n = ue - u;
  int i = 0;
  for (; i + 2 <= n; i += 2) {
    load(sb, u + i + 1);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the math
    compute(sa);
    load(sa, min(u + i + 2, ue - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(sb);
  }
  if (i < n) compute(sa);
}

// ============================================================== GEMV (M < 16)
// A wave covers 64 rows (lane = row, four 16-row blocks) and one 16-column
// group per step: each lane loads the 16 view bytes and 8 B-plane bytes of its
// own row, rebuilds 16 weights and accumulates M dot products. The activations
// of a step are the same for every lane, so they come through scalar loads and
// feed v_dot2c_f32_bf16 as its SGPR operand; no cross-lane reduction is
// needed. In a unit (16 groups) streaming wave w takes groups w, w+4, w+8,
// w+12; the four waves' sums are added through LDS in wave order.
//
// Both kernels run a fifth, helper wave beside the four streaming ones: it
// reads the per-row scales and gathers the escape corrections of the
// segment's columns (irregular, latency-bound work with its own wait
// counters), so the streaming waves never stall on it.
constexpr int kGemvTileRows = 64;
constexpr int kGemvSteps = 4;  // column groups per wave per unit
constexpr int kStreamWaves = 4;
constexpr int kThreads = (kStreamWaves + 1) * 64;

template <int M, bool Q>
struct GemvStage {
  uint4 v[kGemvSteps];
  uint2 b[kGemvSteps];
  int g;
};

template <int M>
struct GemvShared {
  float acc[kStreamWaves][M][kGemvTileRows];
  float cn[M][kGemvTileRows];
  float cp[M][kGemvTileRows];
  float scale[kGemvTileRows];
};

template <int M, bool Q>
__global__ __launch_bounds__(kThreads) void k_gemv(GemmParams a, const uint16_t* __restrict__ x) {
  __shared__ GemvShared<M> sh;
  __shared__ unsigned long long kbest[M];
  __shared__ int flag;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = blockIdx.x;
  const int64_t u0 = unit_start(p, a.units, a.P), u1 = unit_start(p + 1, a.units, a.P);
  const uint32_t c3800 = opaque_vgpr(0x38003800u);
  const int64_t ldx = a.ldx;
  if (threadIdx.x < M) kbest[threadIdx.x] = 0ull;
  for (int64_t u = u0; u < u1;) {
    const int tile = (int)(u / a.ku);
    const int k0 = (int)(u - (int64_t)tile * a.ku);
    const int k1 = (int)min((int64_t)a.ku, u1 - (int64_t)tile * a.ku);
    // lane -> row tile*64 + lane; rows past N read block 0 of the tile
    const int row = tile * kGemvTileRows + lane;
    const bool ok = row < a.n;
    if (wave < kStreamWaves) {
      const uint8_t* tile_rec = a.rec + (int64_t)tile * 4 * a.kb * kRecBytes;
      const uint32_t soff = ok ? (uint32_t)(lane >> 4) * (uint32_t)(a.kb * kRecBytes) : 0u;
      const uint32_t voff = soff + (lane & 15) * 16, boff = soff + kViewBytes + (lane & 15) * 8;
      float acc[M];
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = 0.f;
      auto load = [&](GemvStage<M, Q>& st, int kk) {
        st.g = kk * 16 + wave;
#pragma unroll
        for (int j = 0; j < kGemvSteps; ++j) {
          const int gj = st.g + 4 * j;
          const uint32_t sb = (uint32_t)(gj >> 5) * kRecBytes;
          st.v[j] = *reinterpret_cast<const uint4*>(tile_rec + (sb + (gj & 31) * 256 + voff));
          if (!Q) st.b[j] = *reinterpret_cast<const uint2*>(tile_rec + (sb + (gj & 31) * 128 + boff));
        }
      };
      auto compute = [&](const GemvStage<M, Q>& st) {
#pragma unroll
        for (int j = 0; j < kGemvSteps; ++j) {
          const int gj = st.g + 4 * j;
          uint32_t d[8];
          decode16_scaled<Q>(st.v[j], Q ? make_uint2(0, 0) : st.b[j], d, c3800);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const uint32_t* xp = reinterpret_cast<const uint32_t*>(x + (int64_t)m * ldx + gj * 16);
#pragma unroll
            for (int t = 0; t < 8; ++t) acc[m] = dot2_bf16(d[t], xp[t], acc[m]);
          }
        }
      };
      pipeline<GemvStage<M, Q>>(k0, k1, load, compute);
#pragma unroll
      for (int m = 0; m < M; ++m) sh.acc[wave][m][lane] = acc[m];
    } else {
      // helper: scale and escape corrections of this lane's row over the
      // segment's columns, in column order
      float cn[M], cp[M];
#pragma unroll
      for (int m = 0; m < M; ++m) cn[m] = cp[m] = 0.f;
      if (a.fix && ok) {
        uint32_t end;
        const uint32_t c0 = (uint32_t)k0 * kUnitCols, c1 = (uint32_t)k1 * kUnitCols;
        for (uint32_t i = esc_lower_bound(a, row, c0, &end); i < end; ++i) {
          const uint2 e = a.esc[i];
          if (e.x >= c1) break;
          const float ph = esc_placeholder(a, e.y), ex = bf16_to_f32(e.y & 0xFFFFu);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const float xv = bf16_to_f32(x[(int64_t)m * ldx + e.x]);
            cn[m] = fmaf(xv, ph, cn[m]);
            cp[m] = fmaf(xv, ex, cp[m]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        sh.cn[m][lane] = cn[m];
        sh.cp[m][lane] = cp[m];
      }
      sh.scale[lane] = pow2_scale(a.e_top[ok ? row : 0]);
    }
    __syncthreads();
    auto value = [&](int m, int r) {
      float A = sh.acc[0][m][r];
#pragma unroll
      for (int w = 1; w < kStreamWaves; ++w) A += sh.acc[w][m][r];
      return (A * sh.scale[r] - sh.cn[m][r]) + sh.cp[m][r];
    };
    const bool whole = (k0 == 0 && k1 == a.ku);
    finish_segment(a, tile, kGemvTileRows, tile * kGemvTileRows, whole, p, value, kbest, &flag);
    __syncthreads();
    u = (int64_t)tile * a.ku + k1;
  }
  if (a.mode == kModeArgmax) finish_argmax(a, p, kbest, &flag);
}

// ============================================================== MFMA (M >= 16)
// v_mfma_f32_16x16x32_bf16 with A = 16 weight rows x 32 columns decoded in
// registers and B = 32 columns x 16 activation rows loaded straight from
// global memory. A wave's 1 KB view load of one 64-column chunk of a 16-row
// block gives lane l row l%16 and columns 16 (l/16) .. +15: exactly the A
// operands of two MFMAs; the B operands use the same lane -> column map.
// A unit is 4 chunks (256 columns); streaming wave w takes chunk w. Whole
// 16-row blocks are processed R at a time so one activation load serves R
// blocks. The four waves' sums are added through LDS in wave order; the
// helper wave gathers scales and escape corrections meanwhile.
constexpr int kMfmaTileRows = 16;

// Blocks per group: 4 up to two m-tiles; 2 beyond, which keeps the kernel's
// registers within the architectural VGPRs (with four blocks and four m-tiles
// the compiler's register assignment produced wrong results).
template <int MT>
constexpr int kMfmaR = MT <= 2 ? 4 : 2;

template <int MT, int RG, bool Q>
struct MfmaStage {
  uint4 x[MT][2];
  uint4 v[RG];
  uint2 b[RG];
};

template <int MT>
struct MfmaShared {
  float red[kStreamWaves][kMfmaR<MT>][MT][4][64];  // per wave: C of each block and m-tile
  float cn[kMfmaR<MT> * 16][MT * 16];              // escape corrections per (row, m)
  float cp[kMfmaR<MT> * 16][MT * 16];
  float scale[kMfmaR<MT> * 16];
};

// One group: RG consecutive 16-row blocks starting at block s, units [k0, k1).
template <int MT, int RG, bool Q>
__device__ __forceinline__ void mfma_group(const GemmParams& a, int s, int k0, int k1, int wave, int lane,
                                           MfmaShared<MT>& sh) {
  if (wave == kStreamWaves) {
    // helper: lane = row of the group; escape corrections for every m, in
    // column order, sixteen activation rows at a time
    const int rows = RG * 16;
    if (lane < rows) {
      const int n = s * 16 + lane;
      sh.scale[lane] = pow2_scale(a.e_top[n]);
      const uint32_t c0 = (uint32_t)k0 * kUnitCols, c1 = (uint32_t)k1 * kUnitCols;
      uint32_t end = 0, first = 0;
      if (a.fix) first = esc_lower_bound(a, n, c0, &end);
      for (int m0 = 0; m0 < a.m; m0 += 16) {
        float cn[16], cp[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) cn[j] = cp[j] = 0.f;
        for (uint32_t i = first; i < end; ++i) {
          const uint2 e = a.esc[i];
          if (e.x >= c1) break;
          const float ph = esc_placeholder(a, e.y), ex = bf16_to_f32(e.y & 0xFFFFu);
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int m = min(m0 + j, a.m - 1);
            const float xv = bf16_to_f32(a.x[(int64_t)m * a.ldx + e.x]);
            cn[j] = fmaf(xv, ph, cn[j]);
            cp[j] = fmaf(xv, ex, cp[j]);
          }
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          sh.cn[lane][m0 + j] = cn[j];
          sh.cp[lane][m0 + j] = cp[j];
        }
      }
    }
    return;
  }
  f32x4_t acc[RG][MT];
#pragma unroll
  for (int j = 0; j < RG; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[j][mt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const uint32_t c3800 = opaque_vgpr(0x38003800u);
  // activation row mt*16 + lane%16, columns 16 (lane/16) + 0..15 of the chunk:
  // per-lane byte offsets from the chunk. Past M the lane reads row 0: those
  // B columns only feed output columns m >= M, which are never stored, so the
  // loads need no predicate.
  uint32_t xoff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = mt * 16 + (lane & 15);
    xoff[mt] = (uint32_t)((row < a.m ? row : 0) * a.ldx + (lane >> 4) * 16) * 2u;
  }
  const uint8_t* blk = a.rec + (int64_t)s * a.kb * kRecBytes;
  const uint32_t blk_stride = (uint32_t)(a.kb * kRecBytes);
  auto load = [&](MfmaStage<MT, RG, Q>& st, int kk) {
    const int c = kk * 4 + wave;
    const char* xc = reinterpret_cast<const char*>(a.x + c * 64);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint4* xp = reinterpret_cast<const uint4*>(xc + xoff[mt]);
      st.x[mt][0] = xp[0];
      st.x[mt][1] = xp[1];
    }
    const uint32_t rec_off = (uint32_t)(c >> 3) * kRecBytes;
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      const uint32_t o = j * blk_stride + rec_off;
      st.v[j] = *reinterpret_cast<const uint4*>(blk + (o + (c & 7) * 1024 + lane * 16));
      if (!Q) st.b[j] = *reinterpret_cast<const uint2*>(blk + (o + kViewBytes + (c & 7) * 512 + lane * 8));
    }
  };
  auto compute = [&](const MfmaStage<MT, RG, Q>& st) {
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      uint32_t d[8];
      decode16_scaled<Q>(st.v[j], Q ? make_uint2(0, 0) : st.b[j], d, c3800);
      const uint4 a0 = make_uint4(d[0], d[1], d[2], d[3]);
      const uint4 a1 = make_uint4(d[4], d[5], d[6], d[7]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0),
                                                             __builtin_bit_cast(bf16x8_t, st.x[mt][0]),
                                                             acc[j][mt], 0, 0, 0);
        acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1),
                                                             __builtin_bit_cast(bf16x8_t, st.x[mt][1]),
                                                             acc[j][mt], 0, 0, 0);
      }
    }
  };
  pipeline<MfmaStage<MT, RG, Q>>(k0, k1, load, compute);
  // C layout of a 16x16 MFMA: lane l holds rows 4 (l/16) + i, column l % 16.
#pragma unroll
  for (int j = 0; j < RG; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sh.red[wave][j][mt][i][lane] = acc[j][mt][i];
}

template <int MT, bool Q>
__global__ __launch_bounds__(kThreads) void k_mfma(GemmParams a) {
  __shared__ MfmaShared<MT> sh;
  __shared__ unsigned long long kbest[MT * 16];
  __shared__ int flag;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = blockIdx.x;
  const int64_t u0 = unit_start(p, a.units, a.P), u1 = unit_start(p + 1, a.units, a.P);
  if (threadIdx.x < MT * 16) kbest[threadIdx.x] = 0ull;
  for (int64_t u = u0; u < u1;) {
    const int s = (int)(u / a.ku);
    const int k0 = (int)(u - (int64_t)s * a.ku);
    int rg, k1;
    if (k0 == 0 && (int64_t)(s + 1) * a.ku <= u1) {
      rg = (int)min((int64_t)kMfmaR<MT>, (u1 - u) / a.ku);
      k1 = a.ku;
    } else {
      rg = 1;
      k1 = (int)min((int64_t)a.ku, u1 - (int64_t)s * a.ku);
    }
    if constexpr (kMfmaR<MT> == 4) {
      switch (rg) {
        case 1: mfma_group<MT, 1, Q>(a, s, k0, k1, wave, lane, sh); break;
        case 2: mfma_group<MT, 2, Q>(a, s, k0, k1, wave, lane, sh); break;
        case 3: mfma_group<MT, 3, Q>(a, s, k0, k1, wave, lane, sh); break;
        default: mfma_group<MT, 4, Q>(a, s, k0, k1, wave, lane, sh); break;
      }
    } else {
      if (rg == 1) mfma_group<MT, 1, Q>(a, s, k0, k1, wave, lane, sh);
      else mfma_group<MT, 2, Q>(a, s, k0, k1, wave, lane, sh);
    }
    __syncthreads();
    const bool whole = (k0 == 0 && k1 == a.ku);
    // C of block j at (row, m): lane (row/4)*16 + m%16, element row%4, m-tile m/16
    auto value = [&](int m, int rr) {
      const int j = rr >> 4, row = rr & 15;
      const int mt = m >> 4, l = (row >> 2) * 16 + (m & 15), i = row & 3;
      float A = sh.red[0][j][mt][i][l];
#pragma unroll
      for (int w = 1; w < kStreamWaves; ++w) A += sh.red[w][j][mt][i][l];
      return (A * sh.scale[rr] - sh.cn[rr][m]) + sh.cp[rr][m];
    };
    finish_segment(a, s, rg * kMfmaTileRows, s * kMfmaTileRows, whole, p, value, kbest, &flag);
    __syncthreads();
    u = (int64_t)(s + rg - 1) * a.ku + k1;
  }
  if (a.mode == kModeArgmax) finish_argmax(a, p, kbest, &flag);
}

// ============================================================== planning
GemmPlan plan_gemm(int64_t n, int64_t k, int64_t m, int op, int path, int64_t grid_override) {
  GemmPlan pl{};
  pl.mfma = (path == 2) || (path == 0 && m >= 16);
  if (pl.mfma) {
    pl.tile_rows = kMfmaTileRows;
    pl.ku = (int)(k / kUnitCols);
    pl.tiles = (int)(n / 16);
  } else {
    pl.tile_rows = kGemvTileRows;
    pl.ku = (int)(k / kUnitCols);
    pl.tiles = (int)((n + kGemvTileRows - 1) / kGemvTileRows);
  }
  pl.units = (int64_t)pl.tiles * pl.ku;
  // One resident round of workgroups (occupancy set by the kernels' register
  // and LDS use); at least a few units per workgroup.
  const int64_t mt = (m + 15) / 16;
  const int64_t per_cu = pl.mfma ? (mt == 1 ? 4 : 2) : 4;
  int64_t P = kNumCU * per_cu;
  const int64_t min_units = 2;
  if (pl.units / min_units < P) P = pl.units / min_units;
  if (grid_override > 0) P = grid_override;
  if (P > kMaxGrid) P = kMaxGrid;
  if (P > pl.units) P = pl.units;
  if (P < 1) P = 1;
  pl.P = (int)P;
  const int64_t mm = pl.mfma ? ((m + 15) / 16) * 16 : m;
  pl.ctr_bytes = kCounterBytes;
  pl.part_bytes = (size_t)(2 * P) * (size_t)mm * pl.tile_rows * sizeof(float);
  pl.key_bytes = (op == W12_OP_LMHEAD_ARGMAX) ? (size_t)P * (size_t)m * 8 : 0;
  return pl;
}

template <bool Q>
static hipError_t launch_gemv_m(const GemmPlan& pl, const GemmParams& p, hipStream_t s) {
  const dim3 grid(pl.P), block(kThreads);
  switch (p.m) {
#define W12_GEMV_CASE(MM) \
  case MM: hipLaunchKernelGGL((k_gemv<MM, Q>), grid, block, 0, s, p, p.x); break;
    W12_GEMV_CASE(1) W12_GEMV_CASE(2) W12_GEMV_CASE(3) W12_GEMV_CASE(4) W12_GEMV_CASE(5) W12_GEMV_CASE(6)
    W12_GEMV_CASE(7) W12_GEMV_CASE(8) W12_GEMV_CASE(9) W12_GEMV_CASE(10) W12_GEMV_CASE(11) W12_GEMV_CASE(12)
    W12_GEMV_CASE(13) W12_GEMV_CASE(14) W12_GEMV_CASE(15) W12_GEMV_CASE(16)
#undef W12_GEMV_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool Q>
static hipError_t launch_mfma_m(const GemmPlan& pl, const GemmParams& p, hipStream_t s) {
  const dim3 grid(pl.P), block(kThreads);
  switch ((p.m + 15) / 16) {
    case 1: hipLaunchKernelGGL((k_mfma<1, Q>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((k_mfma<2, Q>), grid, block, 0, s, p); break;
    case 3: hipLaunchKernelGGL((k_mfma<3, Q>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((k_mfma<4, Q>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmPlan& pl, GemmParams p, hipStream_t s, int* unsupported) {
  *unsupported = 0;
  p.units = pl.units;
  p.ku = pl.ku;
  p.tiles = pl.tiles;
  p.P = pl.P;
  if (!pl.mfma && p.m > 16) {
    *unsupported = 1;
    return hipSuccess;
  }
  return pl.mfma ? (p.q ? launch_mfma_m<true>(pl, p, s) : launch_mfma_m<false>(pl, p, s))
                 : (p.q ? launch_gemv_m<true>(pl, p, s) : launch_gemv_m<false>(pl, p, s));
}

}  // namespace w12

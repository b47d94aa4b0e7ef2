// W12 skinny GEMM kernels for gfx950: y[M, N] = x[M, K] W^T over W12 records.
//
// SpecPilot (arXiv 2611.02501) section 4.1 and Figure 5b: the kernel decodes
// records in registers so that the weight stream hides the decode, and splits
// the reduction loop over workgroups in a fixed order (stream-K), so results
// are deterministic. Section 4.3: the Q pass reads only the 8-bit view.
// Appendix E: the LM head in W12, here fused with a per-row argmax.
//
// Work decomposition (both kernels): the matrix is a sequence of tiles of rows
// (64 rows for the GEMV kernel, 16 for the MFMA kernel), each a sequence of
// units along K (128 columns for GEMV, 256 for MFMA: one pipeline stage of
// every wave of a workgroup, so trip counts are exact). Workgroup p owns the
// contiguous unit range [p U / P, (p+1) U / P). A tile covered by one
// workgroup is finished there (per-row scale, escape fix-up, output); a tile
// split between workgroups leaves fp32 partial sums in fixed slots (2p for a
// workgroup's first tile, 2p+1 for its last), which k_reduce adds in workgroup
// order.
#include "w12_internal.h"

namespace w12 {

// -------------------------------------------------------------- shared pieces
__device__ __forceinline__ int64_t unit_start(int64_t p, int64_t units, int P) { return p * units / P; }

// Workgroup owning unit u.
__device__ __forceinline__ int unit_owner(int64_t u, int64_t units, int P) {
  return (int)(((u + 1) * P + units - 1) / units) - 1;
}

// Scale, escape fix-up, then either store y[m, n] or fold the value into the
// workgroup's argmax key for row m.
__device__ __forceinline__ void finish_value(const GemmParams& a, int n, int m, float s,
                                             unsigned long long* kbest) {
  if (n >= a.n) return;
  float v = s * pow2_scale(a.e_top[n]);
  if (a.fix) {
    const uint16_t* xr = a.x + (int64_t)m * a.ldx;
    const uint32_t e0 = a.row_ptr[n], e1 = a.row_ptr[n + 1];
    for (uint32_t i = e0; i < e1; ++i) {
      const uint2 e = a.esc[i];
      const float xv = bf16_to_f32(xr[e.x]);
      uint32_t ph = e.y >> 16;
      if (a.q) ph = (ph & 0xFFF0u) | 0x8u;
      v = fmaf(-xv, bf16_to_f32(ph), v);
      v = fmaf(xv, bf16_to_f32(e.y & 0xFFFFu), v);
    }
  }
  if (a.mode == kModeStore) {
    if (a.y_f32) reinterpret_cast<float*>(a.y)[(int64_t)m * a.ldy + n] = v;
    else reinterpret_cast<uint16_t*>(a.y)[(int64_t)m * a.ldy + n] = f32_to_bf16_rne(v);
  } else {
    atomicMax(&kbest[m], argmax_key(v, (uint32_t)n));
  }
}

__device__ __forceinline__ float dot2_bf16(uint32_t w, uint32_t x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, x), acc,
                                         false);
}

// Software pipeline over the units [u, ue) of one segment with two register
// stages: the loads of the next unit are in flight while the current one is
// computed. All loads are unconditional (the prefetch past the last unit
// re-reads the last unit and is never used), so the compiler can count them
// with vmcnt across the loop.
template <class Stage, class Load, class Compute>
__device__ __forceinline__ void pipeline(int u, int ue, Load&& load, Compute&& compute) {
  if (u >= ue) return;
  Stage sa, sb;
  load(sa, u);
  for (;;) {
    load(sb, min(u + 1, ue - 1));
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the math
    compute(sa);
    if (++u == ue) break;
    load(sa, min(u + 1, ue - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(sb);
    if (++u == ue) break;
  }
}

// ============================================================== GEMV (M < 16)
// A wave covers 64 rows (lane = row, four 16-row blocks) and one 16-column
// group per step: each lane loads 16 view bytes and 8 B-plane bytes of its own
// row, rebuilds 16 weights and accumulates M dot products. The activations of
// a step are the same for all lanes, so they come through scalar loads and
// feed v_dot2c_f32_bf16 as its SGPR operand; no cross-lane reduction is needed.
// A unit is 8 column groups (128 columns); wave w takes groups w and w + 4.
// The four waves' sums are added through LDS in wave order.
constexpr int kGemvTileRows = 64;
constexpr int kGemvUnitCols = 128;

// Activations are prefetched into SGPRs with the weights when they fit
// (M <= 4); otherwise they are read right before use.
template <int M>
constexpr bool kGemvPrefetchX = M <= 4;

template <int M, bool Q>
struct GemvStage {
  uint4 v[2];
  uint2 b[2];
  int g;
  uint32_t x[kGemvPrefetchX<M> ? 2 : 1][kGemvPrefetchX<M> ? M : 1][8];
};

template <int M, bool Q>
__global__ __launch_bounds__(256) void k_gemv(GemmParams a, const uint16_t* __restrict__ x) {
  __shared__ float red[4 * M * kGemvTileRows];
  __shared__ unsigned long long kbest[M];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = blockIdx.x;
  const int64_t u0 = unit_start(p, a.units, a.P), u1 = unit_start(p + 1, a.units, a.P);
  const uint32_t c3800 = 0x38003800u;
  const int64_t ldx = a.ldx;
  if (threadIdx.x < M) kbest[threadIdx.x] = 0ull;
  const int first_tile = (int)(u0 / a.ku);
  for (int64_t u = u0; u < u1;) {
    const int tile = (int)(u / a.ku);
    const int k0 = (int)(u - (int64_t)tile * a.ku);
    const int k1 = (int)min((int64_t)a.ku, u1 - (int64_t)tile * a.ku);
    // lane -> row: block tile*4 + lane/16, row lane%16; rows past N read block 0
    const bool ok = (tile * 4 + (lane >> 4)) * kRecRows < a.n;
    const uint8_t* tile_rec = a.rec + (int64_t)tile * 4 * a.kb * kRecBytes;
    const uint32_t soff = ok ? (uint32_t)(lane >> 4) * (uint32_t)(a.kb * kRecBytes) : 0u;
    const uint32_t voff = soff + (lane & 15) * 16, boff = soff + kViewBytes + (lane & 15) * 8;
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;
    auto load = [&](GemvStage<M, Q>& st, int kk) {
      st.g = kk * 8 + wave;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int gj = st.g + 4 * j;
        const uint32_t sb = (uint32_t)(gj >> 5) * kRecBytes;
        st.v[j] = *reinterpret_cast<const uint4*>(tile_rec + (sb + (gj & 31) * 256 + voff));
        if (!Q) st.b[j] = *reinterpret_cast<const uint2*>(tile_rec + (sb + (gj & 31) * 128 + boff));
        if constexpr (kGemvPrefetchX<M>) {
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const uint32_t* xp = reinterpret_cast<const uint32_t*>(x + (int64_t)m * ldx + gj * 16);
#pragma unroll
            for (int t = 0; t < 8; ++t) st.x[j][m][t] = xp[t];
          }
        }
      }
    };
    auto compute = [&](const GemvStage<M, Q>& st) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int gj = st.g + 4 * j;
        uint32_t d[8];
        decode16_scaled<Q>(st.v[j], Q ? make_uint2(0, 0) : st.b[j], d, c3800);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const uint32_t* xp = reinterpret_cast<const uint32_t*>(x + (int64_t)m * ldx + gj * 16);
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const uint32_t xv = kGemvPrefetchX<M> ? st.x[kGemvPrefetchX<M> ? j : 0][kGemvPrefetchX<M> ? m : 0][t]
                                                  : xp[t];
            acc[m] = dot2_bf16(d[t], xv, acc[m]);
          }
        }
      }
    };
    pipeline<GemvStage<M, Q>>(k0, k1, load, compute);
#pragma unroll
    for (int m = 0; m < M; ++m) red[(wave * M + m) * kGemvTileRows + lane] = acc[m];
    __syncthreads();
    const bool whole = (k0 == 0 && k1 == a.ku);
    const int slot = (tile == first_tile) ? 2 * p : 2 * p + 1;
    for (int i = threadIdx.x; i < M * kGemvTileRows; i += 256) {
      const int m = i / kGemvTileRows, row = i % kGemvTileRows;
      float s = red[(0 * M + m) * kGemvTileRows + row];
      s += red[(1 * M + m) * kGemvTileRows + row];
      s += red[(2 * M + m) * kGemvTileRows + row];
      s += red[(3 * M + m) * kGemvTileRows + row];
      if (whole) finish_value(a, tile * kGemvTileRows + row, m, s, kbest);
      else a.part[((int64_t)slot * M + m) * kGemvTileRows + row] = s;
    }
    __syncthreads();
    u = (int64_t)tile * a.ku + k1;
  }
  if (a.mode == kModeArgmax) {
    __syncthreads();
    if (threadIdx.x < M) a.keys[(int64_t)p * M + threadIdx.x] = kbest[threadIdx.x];
  }
}

// ============================================================== MFMA (M >= 16)
// v_mfma_f32_16x16x32_bf16 with A = 16 weight rows x 32 columns decoded in
// registers and B = 32 columns x 16 activation rows loaded straight from
// global memory. A wave's 1 KB view load of one 64-column chunk of a 16-row
// block gives lane l row l%16 and columns 16 (l/16) .. +15: exactly the A
// operands of two MFMAs; the B operands use the same lane -> column map.
// A unit is 4 chunks (256 columns); wave w takes chunk w. Whole 16-row blocks
// are processed R at a time so one activation load serves R blocks. The four
// waves' sums are added through LDS in wave order.
constexpr int kMfmaR = 4;
constexpr int kMfmaTileRows = 16;
constexpr int kMfmaUnitCols = 256;

template <int MT, int RG, bool Q>
struct MfmaStage {
  uint4 x[MT][2];
  uint4 v[RG];
  uint2 b[RG];
};

// One group: RG consecutive 16-row blocks starting at block s, units [k0, k1).
template <int MT, int RG, bool Q>
__device__ __forceinline__ void mfma_group(const GemmParams& a, int s, int k0, int k1, int wave, int lane,
                                           float* red) {
  f32x4_t acc[RG][MT];
#pragma unroll
  for (int j = 0; j < RG; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[j][mt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const uint32_t c3800 = 0x38003800u;
  // activation row mt*16 + lane%16 (row 0 and a zero operand past M), columns
  // 16 (lane/16) + 0..15 of the chunk: per-lane byte offsets from the chunk
  uint32_t ok_mask = 0;
  uint32_t xoff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = mt * 16 + (lane & 15);
    const bool ok = row < a.m;
    ok_mask |= ok ? (1u << mt) : 0u;
    xoff[mt] = (uint32_t)((ok ? row : 0) * a.ldx + (lane >> 4) * 16) * 2u;
  }
  const uint8_t* blk = a.rec + (int64_t)s * a.kb * kRecBytes;
  const uint32_t blk_stride = (uint32_t)(a.kb * kRecBytes);
  auto load = [&](MfmaStage<MT, RG, Q>& st, int kk) {
    const int c = kk * 4 + wave;
    const char* xc = reinterpret_cast<const char*>(a.x + c * 64);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint4* xp = reinterpret_cast<const uint4*>(xc + xoff[mt]);
      const uint4 x0 = xp[0], x1 = xp[1];
      const bool ok = (ok_mask >> mt) & 1u;
      st.x[mt][0] = ok ? x0 : make_uint4(0, 0, 0, 0);
      st.x[mt][1] = ok ? x1 : make_uint4(0, 0, 0, 0);
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
      for (int i = 0; i < 4; ++i) red[(((wave * kMfmaR + j) * MT + mt) * 4 + i) * 64 + lane] = acc[j][mt][i];
}

template <int MT, bool Q>
__global__ __launch_bounds__(256) void k_mfma(GemmParams a) {
  __shared__ float red[4 * kMfmaR * MT * 4 * 64];
  __shared__ unsigned long long kbest[MT * 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = blockIdx.x;
  const int64_t u0 = unit_start(p, a.units, a.P), u1 = unit_start(p + 1, a.units, a.P);
  if (threadIdx.x < MT * 16) kbest[threadIdx.x] = 0ull;
  const int first_tile = (int)(u0 / a.ku);
  for (int64_t u = u0; u < u1;) {
    const int s = (int)(u / a.ku);
    const int k0 = (int)(u - (int64_t)s * a.ku);
    int rg, k1;
    if (k0 == 0 && (int64_t)(s + 1) * a.ku <= u1) {
      rg = (int)min((int64_t)kMfmaR, (u1 - u) / a.ku);
      k1 = a.ku;
    } else {
      rg = 1;
      k1 = (int)min((int64_t)a.ku, u1 - (int64_t)s * a.ku);
    }
    switch (rg) {
      case 1: mfma_group<MT, 1, Q>(a, s, k0, k1, wave, lane, red); break;
      case 2: mfma_group<MT, 2, Q>(a, s, k0, k1, wave, lane, red); break;
      case 3: mfma_group<MT, 3, Q>(a, s, k0, k1, wave, lane, red); break;
      default: mfma_group<MT, 4, Q>(a, s, k0, k1, wave, lane, red); break;
    }
    __syncthreads();
    const bool whole = (k0 == 0 && k1 == a.ku);
    const int slot = (s == first_tile) ? 2 * p : 2 * p + 1;
    const int rows = rg * 16;
    for (int q = threadIdx.x; q < rows * a.m; q += 256) {
      const int m = q / rows, rr = q % rows;
      const int j = rr >> 4, row = rr & 15;
      const int mt = m >> 4, l = (row >> 2) * 16 + (m & 15), i = row & 3;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) v += red[(((w * kMfmaR + j) * MT + mt) * 4 + i) * 64 + l];
      if (whole) finish_value(a, (s + j) * 16 + row, m, v, kbest);
      else a.part[((int64_t)slot * a.m + m) * kMfmaTileRows + row] = v;
    }
    __syncthreads();
    u = (int64_t)(s + rg - 1) * a.ku + k1;
  }
  if (a.mode == kModeArgmax) {
    __syncthreads();
    if (threadIdx.x < a.m) a.keys[(int64_t)p * a.m + threadIdx.x] = kbest[threadIdx.x];
  }
}

// ============================================================== reduce / finalize
// Block b (boundary between workgroups b-1 and b, b = 1..P-1): if that boundary
// falls inside a tile and is the first boundary in it, sum the tile's partial
// slots in workgroup order and finish it.
__global__ __launch_bounds__(256) void k_reduce(GemmParams a, int tile_rows) {
  __shared__ unsigned long long kbest[W12_MAX_M];
  const int b = blockIdx.x + 1;
  if (threadIdx.x < a.m) kbest[threadIdx.x] = 0ull;
  __syncthreads();
  const int64_t ub = unit_start(b, a.units, a.P);
  const int64_t t = ub / a.ku;
  const bool mine = b < a.P && ub < a.units && (ub % a.ku) != 0 &&
                    unit_start(b - 1, a.units, a.P) <= t * a.ku;
  if (mine) {
    const int pa = unit_owner(t * a.ku, a.units, a.P);
    const int pb = unit_owner(min(a.units, (t + 1) * a.ku) - 1, a.units, a.P);
    for (int q = threadIdx.x; q < tile_rows * a.m; q += blockDim.x) {
      const int m = q / tile_rows, row = q % tile_rows;
      float v = 0.f;
      for (int pp = pa; pp <= pb; ++pp) {
        const int64_t sp = unit_start(pp, a.units, a.P);
        if (sp == unit_start(pp + 1, a.units, a.P)) continue;
        const int slot = (sp / a.ku == t) ? 2 * pp : 2 * pp + 1;
        v += a.part[((int64_t)slot * a.m + m) * tile_rows + row];
      }
      finish_value(a, (int)(t * tile_rows) + row, m, v, kbest);
    }
  }
  if (a.mode == kModeArgmax) {
    __syncthreads();
    if (threadIdx.x < a.m) a.keys[((int64_t)a.P + blockIdx.x) * a.m + threadIdx.x] = kbest[threadIdx.x];
  }
}

__global__ __launch_bounds__(64) void k_argmax_final(const unsigned long long* __restrict__ keys, int nslots,
                                                     int m, int32_t* __restrict__ idx,
                                                     float* __restrict__ maxv) {
  const int i = threadIdx.x;
  if (i >= m) return;
  unsigned long long best = 0ull;
  for (int s = 0; s < nslots; ++s) {
    const unsigned long long k = keys[(int64_t)s * m + i];
    best = k > best ? k : best;
  }
  idx[i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
  if (maxv) maxv[i] = key_value(best);
}

// ============================================================== planning
GemmPlan plan_gemm(int64_t n, int64_t k, int64_t m, int op, int path, int64_t grid_override) {
  GemmPlan pl{};
  pl.mfma = (path == 2) || (path == 0 && m >= 16);
  if (pl.mfma) {
    pl.tile_rows = kMfmaTileRows;
    pl.ku = (int)(k / kMfmaUnitCols);
    pl.tiles = (int)(n / 16);
  } else {
    pl.tile_rows = kGemvTileRows;
    pl.ku = (int)(k / kGemvUnitCols);
    pl.tiles = (int)((n + kGemvTileRows - 1) / kGemvTileRows);
  }
  pl.units = (int64_t)pl.tiles * pl.ku;
  // One resident round of workgroups (occupancy set by the kernels' register
  // and LDS use); at least a few units per workgroup.
  const int64_t mt = (m + 15) / 16;
  const int64_t per_cu = pl.mfma ? (mt == 1 ? 4 : (mt == 2 ? 2 : 1)) : 4;
  int64_t P = kNumCU * per_cu;
  const int64_t min_units = pl.mfma ? 4 : 8;
  if (pl.units / min_units < P) P = pl.units / min_units;
  if (grid_override > 0) P = grid_override;
  if (P > pl.units) P = pl.units;
  if (P < 1) P = 1;
  pl.P = (int)P;
  const int64_t mm = pl.mfma ? ((m + 15) / 16) * 16 : m;
  pl.part_bytes = (size_t)(2 * P) * (size_t)mm * pl.tile_rows * sizeof(float);
  pl.key_bytes = (op == W12_OP_LMHEAD_ARGMAX) ? (size_t)(2 * P) * (size_t)m * 8 : 0;
  return pl;
}

template <bool Q>
static hipError_t launch_gemv_m(const GemmPlan& pl, const GemmParams& p, hipStream_t s) {
  const dim3 grid(pl.P), block(256);
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
  const dim3 grid(pl.P), block(256);
  switch ((p.m + 15) / 16) {
    case 1: hipLaunchKernelGGL((k_mfma<1, Q>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((k_mfma<2, Q>), grid, block, 0, s, p); break;
    case 3: hipLaunchKernelGGL((k_mfma<3, Q>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((k_mfma<4, Q>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// True if some boundary between workgroups falls inside a tile.
static bool has_split_tiles(const GemmPlan& pl) {
  for (int64_t b = 1; b < pl.P; ++b) {
    const int64_t ub = b * pl.units / pl.P;
    if (ub % pl.ku != 0) return true;
  }
  return false;
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
  hipError_t e = pl.mfma ? (p.q ? launch_mfma_m<true>(pl, p, s) : launch_mfma_m<false>(pl, p, s))
                         : (p.q ? launch_gemv_m<true>(pl, p, s) : launch_gemv_m<false>(pl, p, s));
  if (e != hipSuccess) return e;
  if (p.mode == kModeArgmax || has_split_tiles(pl)) {
    if (pl.P > 1) {
      hipLaunchKernelGGL(k_reduce, dim3(pl.P - 1), dim3(256), 0, s, p, pl.tile_rows);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (p.mode == kModeArgmax) {
    const int nslots = pl.P + (pl.P - 1);
    hipLaunchKernelGGL(k_argmax_final, dim3(1), dim3(64), 0, s, p.keys, nslots, p.m, p.idx, p.maxv);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace w12

// Escape fix-up for matrices with dense escape lists (SpecPilot, arXiv
// 2611.02501, section 4.1: the sparse per-channel list restores the exact
// weights). The GEMM kernel runs without escape work and leaves the fp32 sums
// A of every output (the escapes' placeholders multiplied in place of their
// values) in the workspace; this kernel then applies, per output row n and
// activation row m,
//     y = (A - CN) + CP,  CN = sum x * placeholder,  CP = sum x * exact value,
// both sums over the row's escapes, one fused multiply-add per escape in
// column order within each of S slices of the row's list and the slices then
// added in order, and rounds once to the output type. In the Q pass the
// placeholder term is the placeholder's 8-bit view (low nibble at its
// midpoint), which is what the Q pass multiplied.
//
// A workgroup takes R consecutive output rows; their escape lists are one
// contiguous range of the list, which the workgroup copies into LDS with
// coalesced loads (in pieces of kFixEntCap entries). Walk: MP = M rounded up
// to a power of two; a lane holds V = min(MP, 8) activation rows, so O = MP / V
// lanes cover all of them and the workgroup's 256 threads are G = 256 / O
// groups of O lanes, S per output row (R = G / S): group s of a row walks the
// s-th of S equal slices of the row's list in column order, reading each entry
// from LDS and, for its column, its V activations from the transposed copy
// xT[K][mm] as one piece of up to 16 bytes. Epilogue: the slices' sums meet in
// LDS and are added in slice order by threads laid over consecutive rows, so
// that the loads of A and the stores of y are contiguous runs of each
// activation row. S (host side) follows the matrix's average escapes per row,
// about one batch of kFixBatch per slice, and is capped so that the grid's
// lanes stay within about one pass of the device; the order, like the split
// of K in the GEMM, therefore depends only on the matrix, N, K and M.
#include "w12_internal.h"

namespace w12 {

namespace {

constexpr int kFixThreads = 256;
constexpr int kFixBatch = 8;              // escapes whose activation loads a lane issues together
constexpr int kFixEntCap = 2048;          // escape entries per LDS piece
// Lanes of one pass of the device with LDS and registers allowing four
// workgroups per CU (256 CUs x 1024 threads), plus a quarter.
constexpr int64_t kFixLanes = 327680;
constexpr int kFixEntPerThread = kFixEntCap / kFixThreads;

// V consecutive bf16 activations as packed 32-bit words (the low half only for V = 1)
template <int V>
struct XPiece {
  uint32_t w[(V + 1) / 2];
};
template <int V>
__device__ __forceinline__ XPiece<V> load_piece(const uint16_t* p) {
  XPiece<V> r;
  if constexpr (V == 1) {
    r.w[0] = *p;
  } else if constexpr (V == 2) {
    r.w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (V == 4) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    r.w[0] = t.x;
    r.w[1] = t.y;
  } else {
    const uint4 t = *reinterpret_cast<const uint4*>(p);
    r.w[0] = t.x;
    r.w[1] = t.y;
    r.w[2] = t.z;
    r.w[3] = t.w;
  }
  return r;
}
template <int V>
__device__ __forceinline__ float piece_at(const XPiece<V>& x, int v) {
  const uint32_t w = x.w[v >> 1];
  return __uint_as_float((v & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

// Workgroup i runs on XCD i % 8: consecutive row blocks are dealt to one XCD,
// so the blocks that share cache lines of A and y share its L2.
__device__ __forceinline__ int xcd_block(int i, int nb) {
  const int x = i % 8, j = i / 8, q = nb / 8, r = nb % 8;
  return x * q + min(x, r) + j;
}

template <int MP>
__global__ __launch_bounds__(kFixThreads) void k_fix_dense(FixParams p) {
  constexpr int V = MP < 8 ? MP : 8;  // activation rows per lane
  constexpr int O = MP / V;           // lanes per group
  constexpr int G = kFixThreads / O;  // groups per workgroup
  __shared__ float part[2][G][MP + 1];
  __shared__ uint32_t rp[G + 1];
  __shared__ uint2 ents[kFixEntCap];
  const int S = p.slices;             // groups per output row (a power of two <= G)
  const int R = G / S;                // rows per workgroup, a power of two
  const int lr = __ffs(R) - 1;
  const int t = threadIdx.x;
  const int n0 = xcd_block(blockIdx.x, gridDim.x) * R;
  const int nr = min(R, p.n - n0);    // rows of this workgroup, >= 1
  for (int i = t; i <= nr; i += kFixThreads) rp[i] = p.row_ptr[n0 + i];  // nr + 1 offsets, up to 257
  // epilogue items t + 256 j = (activation row m, output row n0 + r), their
  // sums A requested now so that they arrive during the walk
  float av[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = t + kFixThreads * j, r = i & (R - 1), m = i >> lr;
    av[j] = (m < p.m && r < nr) ? p.a[(int64_t)m * p.n + n0 + r] : 0.f;
  }
  __syncthreads();
  const int g = t / O, o = t % O;
  const int m0 = o * V;               // this lane's first activation row
  const int s = g % S, rr = g / S;
  // lanes whose rows all lie past M load nothing (xT has mm >= M columns, a
  // multiple of 16, so a piece that starts below M is wholly inside its row)
  const bool active = rr < nr && m0 < p.m;
  uint32_t e = 0, end = 0;
  if (active) {
    const uint32_t a0 = rp[rr], c = rp[rr + 1] - a0;
    e = a0 + (uint32_t)(((uint64_t)c * (uint32_t)s) / (uint32_t)S);
    end = a0 + (uint32_t)(((uint64_t)c * (uint32_t)(s + 1)) / (uint32_t)S);
  }
  float cn[V], cp[V];
#pragma unroll
  for (int v = 0; v < V; ++v) cn[v] = cp[v] = 0.f;
  // byte offsets within xT fit 32 bits (K <= 2^23 rows of at most 64 activations: under 2^30 bytes)
  const char* xtb = reinterpret_cast<const char*>(p.xt + m0);
  const uint32_t xrow = 2u * (uint32_t)p.mm;
  const uint32_t E0 = rp[0], E1 = rp[nr];
  for (uint32_t c0 = E0; c0 < E1; c0 += kFixEntCap) {  // the same pieces in every thread
    const uint32_t c1 = min(c0 + (uint32_t)kFixEntCap, E1);
    uint2 tmp[kFixEntPerThread];
#pragma unroll
    for (int j = 0; j < kFixEntPerThread; ++j) {
      const uint32_t q = c0 + (uint32_t)(t + kFixThreads * j);
      tmp[j] = q < c1 ? p.esc[q] : make_uint2(0u, 0u);
    }
    __syncthreads();  // the previous piece's readers are done
#pragma unroll
    for (int j = 0; j < kFixEntPerThread; ++j) {
      const uint32_t q = c0 + (uint32_t)(t + kFixThreads * j);
      if (q < c1) ents[q - c0] = tmp[j];
    }
    __syncthreads();
    uint32_t lo = max(e, c0);
    const uint32_t hi = min(end, c1);
    while (__any(lo < hi)) {
      const uint32_t left = lo < hi ? hi - lo : 0u;  // entries this lane still has in the piece
      uint2 ent[kFixBatch];
#pragma unroll
      for (int j = 0; j < kFixBatch; ++j) ent[j] = (uint32_t)j < left ? ents[lo - c0 + j] : make_uint2(0u, 0u);
      XPiece<V> xv[kFixBatch];
#pragma unroll
      for (int j = 0; j < kFixBatch; ++j) {
        if constexpr (V == 1) {
          // one activation row: the compiler would wait on each conditional
          // 2-byte load before the next, so every lane loads (an entry past
          // its slice reads column 0, in bounds) and the FMAs skip it below
          xv[j] = load_piece<V>(reinterpret_cast<const uint16_t*>(xtb + ((uint32_t)j < left ? ent[j].x : 0u) * xrow));
        } else if ((uint32_t)j < left) {
          xv[j] = load_piece<V>(reinterpret_cast<const uint16_t*>(xtb + ent[j].x * xrow));
        } else {
#pragma unroll
          for (int i = 0; i < (V + 1) / 2; ++i) xv[j].w[i] = 0u;
        }
      }
#pragma unroll
      for (int j = 0; j < kFixBatch; ++j) {
        if ((uint32_t)j < left) {
          const uint32_t ph = ent[j].y >> 16;
          const float pv = bf16_to_f32(p.q ? ((ph & 0xFFF0u) | 0x8u) : ph);
          const float ev = bf16_to_f32(ent[j].y & 0xFFFFu);
#pragma unroll
          for (int v = 0; v < V; ++v) {
            const float xf = piece_at<V>(xv[j], v);
            cn[v] = fmaf(xf, pv, cn[v]);
            cp[v] = fmaf(xf, ev, cp[v]);
          }
        }
      }
      lo += left < (uint32_t)kFixBatch ? left : (uint32_t)kFixBatch;
    }
  }
#pragma unroll
  for (int v = 0; v < V; ++v) {
    part[0][g][m0 + v] = cn[v];
    part[1][g][m0 + v] = cp[v];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = t + kFixThreads * j, r = i & (R - 1), m = i >> lr;
    if (m < p.m && r < nr) {
      const int g0 = r * S;
      float tn = part[0][g0][m], tp = part[1][g0][m];
      for (int u = 1; u < S; ++u) {  // slices in order
        tn += part[0][g0 + u][m];
        tp += part[1][g0 + u][m];
      }
      const float v = (av[j] - tn) + tp;
      const int64_t at = (int64_t)m * p.ldy + n0 + r;
      if (p.y_f32)
        reinterpret_cast<float*>(p.y)[at] = v;
      else
        reinterpret_cast<uint16_t*>(p.y)[at] = f32_to_bf16_rne(v);
    }
  }
}

int lanes_per_group(int m) {
  int mp = 1;
  while (mp < m) mp <<= 1;
  return mp < 8 ? 1 : mp / 8;
}

}  // namespace

int fix_slices(int64_t n, int64_t n_esc, int m) {
  const int o = lanes_per_group(m), groups = kFixThreads / o;
  const int64_t per_row = n > 0 ? (n_esc + n - 1) / n : 0;
  int s = 1;
  // about one batch per slice, while the lanes stay within about one pass of the device
  while (s < groups && (int64_t)s * kFixBatch < per_row && n * o * 2 * s <= kFixLanes) s <<= 1;
  return s;
}

hipError_t launch_fix_dense(const FixParams& p, hipStream_t s) {
  int mp = 1;
  while (mp < p.m) mp <<= 1;
  const int groups = kFixThreads / lanes_per_group(p.m);
  if (mp > 64 || p.n < 1 || p.mm < p.m || p.mm % 16 != 0 || p.slices < 1 || p.slices > groups ||
      (p.slices & (p.slices - 1)) != 0 || (reinterpret_cast<uintptr_t>(p.xt) & 15u) != 0)
    return hipErrorInvalidValue;
  const int rows_per_wg = groups / p.slices;
  const dim3 grid((unsigned)(((int64_t)p.n + rows_per_wg - 1) / rows_per_wg)), block(kFixThreads);
  switch (mp) {
    case 1: hipLaunchKernelGGL(k_fix_dense<1>, grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL(k_fix_dense<2>, grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL(k_fix_dense<4>, grid, block, 0, s, p); break;
    case 8: hipLaunchKernelGGL(k_fix_dense<8>, grid, block, 0, s, p); break;
    case 16: hipLaunchKernelGGL(k_fix_dense<16>, grid, block, 0, s, p); break;
    case 32: hipLaunchKernelGGL(k_fix_dense<32>, grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL(k_fix_dense<64>, grid, block, 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace w12

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
// Lanes: a workgroup of 256 threads is G = 256 / MP groups of MP lanes (MP =
// M rounded up to a power of two, lane m of a group = activation row m). The
// groups take G / S output rows, S groups per row: group s of a row walks the
// s-th of S equal slices of the row's escape list in column order, reading
// each escape entry once per group (one request) and the activations of its
// column for all m from the transposed copy xT[K][MM] (one contiguous piece).
// The slices' sums are then added in slice order through LDS. S follows the
// matrix's average escapes per row (host side), so the order, like the split
// of K in the GEMM, depends only on the matrix, N, K and M.
#include "w12_internal.h"

namespace w12 {

namespace {

constexpr int kFixThreads = 256;
constexpr int kFixBatch = 16;  // escapes whose loads a lane issues together

template <int MP>
__global__ __launch_bounds__(kFixThreads) void k_fix_dense(FixParams p) {
  constexpr int G = kFixThreads / MP;  // groups per workgroup
  __shared__ float part[2][G][MP];
  const int S = p.slices;               // groups per output row (a power of two <= G)
  const int g = threadIdx.x / MP, m = threadIdx.x % MP;
  const int s = g % S;
  const int row = blockIdx.x * (G / S) + g / S;
  const bool active = row < p.n && m < p.m;  // lanes past M load nothing (xT has mm <= MP columns)
  uint32_t e = 0, end = 0;
  if (active) {
    const uint32_t a0 = p.row_ptr[row], a1 = p.row_ptr[row + 1];
    const uint32_t c = a1 - a0;
    e = a0 + (uint32_t)(((uint64_t)c * (uint32_t)s) / (uint32_t)S);
    end = a0 + (uint32_t)(((uint64_t)c * (uint32_t)(s + 1)) / (uint32_t)S);
  }
  // the output's sum A, requested now so that it arrives during the walk
  const float a = (active && s == 0) ? p.a[(int64_t)m * p.n + row] : 0.f;
  float cn = 0.f, cp = 0.f;
  while (__any(e < end)) {
    const uint32_t left = e < end ? end - e : 0u;  // entries this lane still has
    uint2 ent[kFixBatch];
#pragma unroll
    for (int j = 0; j < kFixBatch; ++j) ent[j] = (uint32_t)j < left ? p.esc[e + j] : make_uint2(0u, 0u);
    float xv[kFixBatch];
#pragma unroll
    for (int j = 0; j < kFixBatch; ++j)
      xv[j] = (uint32_t)j < left ? bf16_to_f32(p.xt[(int64_t)ent[j].x * p.mm + m]) : 0.f;
#pragma unroll
    for (int j = 0; j < kFixBatch; ++j) {
      if ((uint32_t)j < left) {
        const uint32_t ph = ent[j].y >> 16;
        const float pv = bf16_to_f32(p.q ? ((ph & 0xFFF0u) | 0x8u) : ph);
        cn = fmaf(xv[j], pv, cn);
        cp = fmaf(xv[j], bf16_to_f32(ent[j].y & 0xFFFFu), cp);
      }
    }
    e += left < (uint32_t)kFixBatch ? left : (uint32_t)kFixBatch;
  }
  part[0][g][m] = cn;
  part[1][g][m] = cp;
  __syncthreads();
  if (!active || s != 0) return;
  float tn = part[0][g][m], tp = part[1][g][m];
  for (int t = 1; t < S; ++t) {  // slices in order
    tn += part[0][g + t][m];
    tp += part[1][g + t][m];
  }
  const float v = (a - tn) + tp;
  if (p.y_f32)
    reinterpret_cast<float*>(p.y)[(int64_t)m * p.ldy + row] = v;
  else
    reinterpret_cast<uint16_t*>(p.y)[(int64_t)m * p.ldy + row] = f32_to_bf16_rne(v);
}

}  // namespace

int fix_slices(int64_t n, int64_t n_esc, int m) {
  int mp = 1;
  while (mp < m) mp <<= 1;
  const int groups = kFixThreads / mp;
  const int64_t per_row = n > 0 ? (n_esc + n - 1) / n : 0;
  int s = 1;
  while (s < groups && (int64_t)s * kFixBatch < per_row) s <<= 1;  // about one batch per slice
  return s;
}

hipError_t launch_fix_dense(const FixParams& p, hipStream_t s) {
  int mp = 1;
  while (mp < p.m) mp <<= 1;
  const int groups = kFixThreads / mp;
  if (mp > 64 || p.slices < 1 || p.slices > groups || (p.slices & (p.slices - 1)) != 0) return hipErrorInvalidValue;
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

// W12 encode, decode and descriptor validation kernels for gfx950.
//
// SpecPilot (arXiv 2611.02501) section 4.1: per output channel, choose the
// 16-binade window holding the most weights, store in-window weights in 12
// bits, send the rest to an exact per-channel escape list; at load time check
// every decoded tensor bit for bit. Bit and byte positions: include/w12.h.
#include "w12_internal.h"

namespace w12 {

// ---------------------------------------------------------------- window choice
// One wave per row: 256-bin histogram of the normal exponents in LDS, then
// each lane scores up to four candidate window tops. The packed key
// count << 8 | E makes a single max pick the largest count and, among equal
// counts, the largest top E (the tie rule of format v1).
__global__ __launch_bounds__(256) void k_plan(const uint16_t* __restrict__ w, int n, int k,
                                              uint8_t* __restrict__ e_top, uint32_t* __restrict__ cnt) {
  __shared__ uint32_t hist[4][256];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wave;
  for (int i = lane; i < 256; i += 64) hist[wave][i] = 0;
  __syncthreads();
  int emax = 0;
  if (row < n) {
    const uint4* wr = reinterpret_cast<const uint4*>(w + (int64_t)row * k);
    for (int i = lane; i < k / 8; i += 64) {
      const uint4 q = wr[i];
      const uint32_t h[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t e = (h[j >> 1] >> ((j & 1) * 16 + 7)) & 0xFFu;
        if (e >= 1 && e <= 254) {
          atomicAdd(&hist[wave][e], 1u);
          emax = e > (uint32_t)emax ? (int)e : emax;
        }
      }
    }
  }
  __syncthreads();
  if (row >= n) return;
  for (int off = 32; off > 0; off >>= 1) emax = max(emax, __shfl_xor(emax, off));
  const int cap = emax > 16 ? emax : 16;
  uint32_t best = 0;
  for (int top = 16 + lane; top <= cap; top += 64) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) c += hist[wave][top - 15 + j];
    const uint32_t key = (c << 8) | (uint32_t)top;
    best = key > best ? key : best;
  }
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(best, off);
    best = o > best ? o : best;
  }
  if (lane == 0) {
    e_top[row] = (uint8_t)(best & 0xFFu);
    cnt[row] = (uint32_t)k - (best >> 8);
  }
}

// Exclusive prefix sum of the per-row escape counts -> CSR row pointers.
// One workgroup; each thread sums a contiguous slice, then a block scan.
__global__ __launch_bounds__(1024) void k_scan(const uint32_t* __restrict__ cnt, int n,
                                               uint32_t* __restrict__ row_ptr) {
  __shared__ uint32_t sums[1024];
  const int t = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int a = min(n, t * per), b = min(n, a + per);
  uint32_t local = 0;
  for (int i = a; i < b; ++i) local += cnt[i];
  sums[t] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const uint32_t v = t >= off ? sums[t - off] : 0u;
    __syncthreads();
    sums[t] += v;
    __syncthreads();
  }
  uint32_t run = sums[t] - local;  // exclusive
  for (int i = a; i < b; ++i) {
    row_ptr[i] = run;
    run += cnt[i];
  }
  if (t == 1023) row_ptr[n] = sums[1023];
}

// ---------------------------------------------------------------- pack
// One workgroup per 16-row block, one wave per row. Per record, lane L takes
// the 8 columns 8L..8L+7 of the row: G = L/2, t = 8 (L%2) .. +7. It writes 8
// view bytes and one B dword, and its escapes at the row's CSR offset plus the
// number of escapes in lower columns (wave prefix sum in lane order).
__global__ __launch_bounds__(1024) void k_pack(const uint16_t* __restrict__ w, int n, int k,
                                               const uint8_t* __restrict__ e_top,
                                               const uint32_t* __restrict__ row_ptr,
                                               uint8_t* __restrict__ rec, w12_escape* __restrict__ esc,
                                               uint32_t esc_cap) {
  const int lane = threadIdx.x & 63;
  const int r = threadIdx.x >> 6;
  const int rb = blockIdx.x;
  const int row = rb * kRecRows + r;
  const int kb_count = k / kRecCols;
  const int E = e_top[row];
  const int lo = E - 15;
  const uint4* wr = reinterpret_cast<const uint4*>(w + (int64_t)row * k);
  uint32_t out_pos = row_ptr[row];
  const int G = lane >> 1, t8 = lane & 1;
  for (int kb = 0; kb < kb_count; ++kb) {
    const uint4 q = wr[kb * 64 + lane];
    const uint32_t h[4] = {q.x, q.y, q.z, q.w};
    uint32_t view[2] = {0, 0};
    uint32_t ml[8];
    uint32_t ph[8];
    uint32_t mask = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t bits = (h[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
      const int s = bits >> 15, e = (bits >> 7) & 0xFF, m = bits & 0x7F;
      const bool normal = e >= 1 && e <= 254;
      const bool inwin = normal && e >= lo && e <= E;
      const bool above = (e == 255) || (normal && e > E);
      const int off = inwin ? e - lo : (above ? 15 : 0);
      const int mh = inwin ? (m >> 4) : (above ? 7 : 0);
      const int l4 = inwin ? (m & 15) : (above ? 15 : 0);
      view[j >> 2] |= (uint32_t)((s << 7) | (off << 3) | mh) << ((j & 3) * 8);
      ml[j] = (uint32_t)l4;
      ph[j] = ((uint32_t)s << 15) | ((uint32_t)(off + lo) << 7) | ((uint32_t)mh << 4) | (uint32_t)l4;
      mask |= inwin ? 0u : (1u << j);
    }
    uint32_t bdw = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) bdw |= ((ml[j] << 4) | ml[j + 4]) << (8 * j);
    uint8_t* rp = rec + ((int64_t)rb * kb_count + kb) * kRecBytes;
    *reinterpret_cast<uint2*>(rp + (G * 16 + r) * 16 + 8 * t8) = make_uint2(view[0], view[1]);
    *reinterpret_cast<uint32_t*>(rp + kViewBytes + (G * 16 + r) * 8 + 4 * t8) = bdw;
    // escapes, in column order
    const uint32_t pc = __popc(mask);
    uint32_t incl = pc;
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    const uint32_t total = __shfl(incl, 63);
    uint32_t pos = out_pos + incl - pc;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (mask & (1u << j)) {
        const uint32_t bits = (h[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
        w12_escape ev;
        ev.col = (uint32_t)(kb * kRecCols + lane * 8 + j);
        ev.bits = (uint16_t)bits;
        ev.ph = (uint16_t)ph[j];
        if (pos < esc_cap) esc[pos] = ev;  // never past the caller's buffer
        ++pos;
      }
    }
    out_pos += total;
  }
}

// ---------------------------------------------------------------- decode
// One thread per 16-column group of one row (512 per record): rebuild the 16
// BF16 weights with their true exponents, then overwrite the escapes of that
// group (found by binary search in the row's sorted escape list), then one
// 32-byte store.
__global__ __launch_bounds__(256) void k_decode(const uint8_t* __restrict__ rec, const uint8_t* __restrict__ e_top,
                                                const uint32_t* __restrict__ row_ptr,
                                                const uint2* __restrict__ esc, int n, int k,
                                                uint16_t* __restrict__ out) {
  const int kb_count = k / kRecCols;
  const int64_t rid = blockIdx.x >> 1;  // record
  const int q = (blockIdx.x & 1) * 256 + threadIdx.x;  // G*16 + r
  const int G = q >> 4, r = q & 15;
  const int rb = (int)(rid / kb_count), kb = (int)(rid % kb_count);
  const int row = rb * kRecRows + r;
  const uint8_t* rp = rec + rid * kRecBytes;
  const uint4 v = *reinterpret_cast<const uint4*>(rp + q * 16);
  const uint2 b = *reinterpret_cast<const uint2*>(rp + kViewBytes + q * 8);
  const uint32_t bias = (uint32_t)(e_top[row] - 15) << 7;
  uint32_t d[8];
  decode16_exact(v, b, d, bias | (bias << 16));
  const uint32_t c_lo = (uint32_t)(kb * kRecCols + G * 16);
  uint32_t a = row_ptr[row], z = row_ptr[row + 1];
  while (a < z) {  // first escape with col >= c_lo
    const uint32_t mid = (a + z) >> 1;
    if (esc[mid].x < c_lo) a = mid + 1; else z = mid;
  }
  const uint32_t end = row_ptr[row + 1];
  for (uint32_t i = a; i < end; ++i) {
    const uint2 e = esc[i];
    const uint32_t t = e.x - c_lo;
    if (t >= 16) break;
    const uint32_t bits = e.y & 0xFFFFu;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (t == (uint32_t)j) {
        d[j >> 1] = (j & 1) ? ((d[j >> 1] & 0x0000FFFFu) | (bits << 16)) : ((d[j >> 1] & 0xFFFF0000u) | bits);
      }
    }
  }
  uint4* op = reinterpret_cast<uint4*>(out + (int64_t)row * k + c_lo);
  op[0] = make_uint4(d[0], d[1], d[2], d[3]);
  op[1] = make_uint4(d[4], d[5], d[6], d[7]);
}

// ---------------------------------------------------------------- validate
__global__ __launch_bounds__(256) void k_validate(const uint8_t* __restrict__ e_top,
                                                  const uint32_t* __restrict__ row_ptr,
                                                  const uint2* __restrict__ esc, int n, int k, int64_t n_esc,
                                                  uint32_t* __restrict__ flag) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= n) return;
  bool bad = false;
  const int E = e_top[row];
  bad |= E < 16 || E > 254;
  const uint32_t a = row_ptr[row], z = row_ptr[row + 1];
  if (row == 0) bad |= a != 0;
  if (row == n - 1) bad |= (int64_t)z != n_esc;
  bad |= z < a || (int64_t)z > n_esc;
  if (!bad) {
    uint32_t prev = 0;
    for (uint32_t i = a; i < z; ++i) {
      const uint32_t c = esc[i].x;
      bad |= c >= (uint32_t)k || (i > a && c <= prev);
      prev = c;
    }
  }
  if (bad) atomicOr(flag, 1u);
}

__global__ void k_zero_u32(uint32_t* p) { *p = 0u; }

// ---------------------------------------------------------------- launchers
hipError_t launch_plan(const uint16_t* w, int n, int k, uint8_t* e_top, uint32_t* cnt, hipStream_t s) {
  hipLaunchKernelGGL(k_plan, dim3((n + 3) / 4), dim3(256), 0, s, w, n, k, e_top, cnt);
  return hipGetLastError();
}

hipError_t launch_scan(const uint32_t* cnt, int n, uint32_t* row_ptr, hipStream_t s) {
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, cnt, n, row_ptr);
  return hipGetLastError();
}

hipError_t launch_pack(const uint16_t* w, int n, int k, const uint8_t* e_top, const uint32_t* row_ptr,
                       uint8_t* rec, w12_escape* esc, uint32_t esc_cap, hipStream_t s) {
  hipLaunchKernelGGL(k_pack, dim3(n / kRecRows), dim3(1024), 0, s, w, n, k, e_top, row_ptr, rec, esc, esc_cap);
  return hipGetLastError();
}

hipError_t launch_decode(const w12_matrix* m, uint16_t* out, hipStream_t s) {
  const int n = (int)m->n, k = (int)m->k;
  const int64_t records = (int64_t)(n / kRecRows) * (k / kRecCols);
  hipLaunchKernelGGL(k_decode, dim3((unsigned)(records * 2)), dim3(256), 0, s, m->records, m->e_top,
                     m->esc_row_ptr, reinterpret_cast<const uint2*>(m->esc), n, k, out);
  return hipGetLastError();
}

hipError_t launch_validate(const w12_matrix* m, uint32_t* flag, hipStream_t s) {
  const int n = (int)m->n;
  hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(1), 0, s, flag);
  hipLaunchKernelGGL(k_validate, dim3((n + 255) / 256), dim3(256), 0, s, m->e_top, m->esc_row_ptr,
                     reinterpret_cast<const uint2*>(m->esc), n, (int)m->k, m->n_esc, flag);
  return hipGetLastError();
}

}  // namespace w12

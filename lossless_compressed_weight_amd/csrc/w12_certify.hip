// Certified argmax LM head (SpecPilot, arXiv 2611.02501, section 4.1, the
// certified LM head paragraph; section 4.3, zero-copy Q pass): logits from a Q
// copy of the head plus a per-row Cauchy-Schwarz bound on that copy's error
// rule out every vocabulary row that cannot hold the argmax; the rows left are
// rescored with their exact weights, and the full head runs instead when any
// activation row keeps more than W12_CERT_MAX_SURVIVORS rows.
//
// The Q copy is the 8-bit view of the W12 records with the escapes applied
// (the Q pass of w12_gemm_q8 with W12_Q8_APPLY_ESCAPES), so no second copy of
// the head is stored. For row n with exact weights w_n, view weights v_n
// (placeholders at escapes) and Q weights q_n (v_n with escapes exact):
//   r_n = ||w_n - q_n||_2,  a_n = ||w_n||_2 + ||v_n||_2.
// For activation row x the true logit l_n = x.w_n and the fp32 Q logit lq_n
// satisfy |l_n - lq_n| <= ||x|| (r_n + c a_n), c = 4 K u / (1 - K u),
// u = 2^-24: Cauchy-Schwarz for the view's dropped bits, and a bound on the
// rounding of any fp32 summation order of the Q pass (its escape terms
// included). Row n is ruled out when lq_n + ||x|| (r_n + c a_n) is below
// max_j (lq_j - ||x|| (r_j + c a_j)).
//
// Kernels, in stream order after the Q pass:
//   k_cert_lower   per (chunk of rows, activation row): ||x||, the chunk's
//                  largest lower and upper bounds (kept per chunk)
//   k_cert_select  the best lower bound of the activation row (a maximum over
//                  its chunks); chunks whose largest upper bound reaches it
//                  list their surviving rows
//   k_cert_rescore one wave per (activation row, survivor): exact dot product
//                  from the record bytes and the escape list, 64-bit argmax
//                  key; the row's last pair writes its index and maximum. A row
//                  past the cap raises the gate instead.
// The full fused head then runs gated on the flag.
#include "w12_internal.h"

namespace w12 {

namespace {

constexpr int kCertChunk = 2048;   // rows per chunk (8 per thread of 256)
constexpr int kCertThreads = 256;
static_assert(kCertChunk % kCertThreads == 0, "whole rows per thread");

// Wave sums in a fixed order (butterfly over the 64 lanes).
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Order-preserving 32-bit key of a float (larger value, larger key; any NaN
// sorts above +inf, -0 as +0); 0 is below every key and means "none yet".
__device__ __forceinline__ uint32_t ord32(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord32(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Rounded-up float of a non-negative double, with a relative margin that
// covers the double sums' own rounding.
__device__ __forceinline__ float up_f32(double v) {
  return __double2float_ru(v * (1.0 + 0x1p-40));
}

// ---------------------------------------------------------------- bounds
// One wave per row: the lanes cover two records per step (lane l: record
// kb + l / 32, 16-column group l % 32), decode view and B exactly and with the
// midpoint nibble, and sum in float64; escapes then swap their placeholder
// terms for their exact values.
__global__ __launch_bounds__(kCertThreads) void k_cert_bounds(const uint8_t* __restrict__ rec,
                                                              const uint8_t* __restrict__ e_top,
                                                              const uint32_t* __restrict__ row_ptr,
                                                              const uint2* __restrict__ esc, int n, int k,
                                                              float* __restrict__ bounds) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kCertThreads / 64) + (threadIdx.x >> 6);
  if (row >= n) return;  // whole waves leave together: row is uniform per wave
  const int kb_count = k / kRecCols;
  const int r = row & 15;
  const uint8_t* blk = rec + (int64_t)(row >> 4) * kb_count * kRecBytes;
  const uint32_t bias = (uint32_t)(e_top[row] - 15) << 7;
  const uint32_t bias2 = bias | (bias << 16);
  const int G = lane & 31;
  double sd = 0.0, sw = 0.0, sv = 0.0;
  for (int kb = lane >> 5; kb < kb_count; kb += 2) {
    const uint8_t* rp = blk + (int64_t)kb * kRecBytes;
    const uint4 v = *reinterpret_cast<const uint4*>(rp + (G * 16 + r) * 16);
    const uint2 b = *reinterpret_cast<const uint2*>(rp + kViewBytes + (G * 16 + r) * 8);
    uint32_t dw[8], dv[8];
    decode16_exact(v, b, dw, bias2);
    // the view alone: every dropped nibble at its midpoint (no shift needed,
    // both nibbles of 0x80 bytes are the same after the shift's effect)
    dv[0] = pair_exact(v.x, 0x80808080u, kSelPair01, bias2);
    dv[1] = pair_exact(v.x, 0x80808080u, kSelPair23, bias2);
    dv[2] = pair_exact(v.y, 0x80808080u, kSelPair01, bias2);
    dv[3] = pair_exact(v.y, 0x80808080u, kSelPair23, bias2);
    dv[4] = pair_exact(v.z, 0x80808080u, kSelPair01, bias2);
    dv[5] = pair_exact(v.z, 0x80808080u, kSelPair23, bias2);
    dv[6] = pair_exact(v.w, 0x80808080u, kSelPair01, bias2);
    dv[7] = pair_exact(v.w, 0x80808080u, kSelPair23, bias2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const double w = (double)bf16_to_f32(h ? dw[j] >> 16 : dw[j] & 0xFFFFu);
        const double q = (double)bf16_to_f32(h ? dv[j] >> 16 : dv[j] & 0xFFFFu);
        sd += (w - q) * (w - q);
        sw += w * w;
        sv += q * q;
      }
    }
  }
  // escapes: the decode gave the placeholder ph there; the view holds ph with
  // its low nibble at the midpoint. Exact weight = bits; Q weight = bits too.
  bool bad = false;
  const uint32_t e0 = row_ptr[row], e1 = row_ptr[row + 1];
  for (uint32_t i = e0 + lane; i < e1; i += 64) {
    const uint2 e = esc[i];
    const uint32_t bits = e.y & 0xFFFFu, ph = e.y >> 16;
    const double we = (double)bf16_to_f32(bits);
    const double wp = (double)bf16_to_f32(ph);
    const double vp = (double)bf16_to_f32((ph & 0xFFF0u) | 0x8u);
    if (!isfinite(we)) bad = true;
    sd -= (wp - vp) * (wp - vp);
    sw += (isfinite(we) ? we * we : 0.0) - wp * wp;
  }
  sd = wave_sum_f64(sd);
  sw = wave_sum_f64(sw);
  sv = wave_sum_f64(sv);
  bad = __any(bad);
  if (lane == 0) {
    const float inf = __builtin_inff();
    bounds[2 * (int64_t)row] = bad ? inf : up_f32(sqrt(fmax(sd, 0.0)));
    bounds[2 * (int64_t)row + 1] = bad ? inf : up_f32(sqrt(fmax(sw, 0.0)) + sqrt(fmax(sv, 0.0)));
  }
}

// ---------------------------------------------------------------- per call
struct CertArgs {
  const uint16_t* x;
  int64_t ldx;
  const float* lq;       // Q-copy logits [M][N], fp32
  const float* bounds;   // [N][2]: r_n, a_n
  CertZero* z;
  CertCall* cc;
  float* ub_chunk;       // [M][chunks]: each chunk's largest upper bound
  float* lb_chunk;       // [M][chunks]: each chunk's largest lower bound
  uint32_t* list;        // [M][cap]
  int n, k, m, chunks, cap;
  double slack;
};

// Thread t sums x[t]^2, x[t + 256]^2, ... in order; the loads of 24 terms go
// out together, all of a row up to K = 6144 (past K they are zero, which
// leaves the sum as it is).
__device__ double row_norm(const uint16_t* x, int k, double* red) {
  constexpr int kBatch = 24;
  double s = 0.0;
  for (int i0 = threadIdx.x; i0 < k; i0 += kBatch * kCertThreads) {
    float v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = i0 + j * kCertThreads;
      const float xi = bf16_to_f32(x[min(i, k - 1)]);  // clamped in bounds, so the loads carry no branches
      v[j] = i < k ? xi : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const double d = (double)v[j];
      s += d * d;
    }
  }
  s = wave_sum_f64(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kCertThreads / 64; ++w) t += red[w];
  return sqrt(t);
}

// Per (chunk of rows, activation row m): ||x_m||, the chunk's largest lower
// and upper bounds. (One atomic maximum per activation row instead, from
// every chunk, queued the chunks' workgroups on one cache line: 24 us at
// M = 16 for the 151936-row head.)
__global__ __launch_bounds__(kCertThreads) void k_cert_lower(CertArgs a) {
  __shared__ double red[kCertThreads / 64];
  __shared__ float lo_w[kCertThreads / 64], hi_w[kCertThreads / 64];
  const int chunk = blockIdx.x, m = blockIdx.y;
  const int r0 = chunk * kCertChunk;
  // the thread's rows of the chunk: their loads go out first, with those of
  // x's norm, then the bounds
  constexpr int kRows = kCertChunk / kCertThreads;
  float lqv[kRows];
  float2 bd[kRows];
#pragma unroll
  for (int j = 0; j < kRows; ++j) {
    // rows past N load row N - 1 (in bounds, no branch) and are skipped below
    const int row = min(r0 + j * kCertThreads + (int)threadIdx.x, a.n - 1);
    lqv[j] = a.lq[(int64_t)m * a.n + row];
    bd[j] = make_float2(a.bounds[2 * row], a.bounds[2 * row + 1]);
  }
  const double xn = row_norm(a.x + (int64_t)m * a.ldx, a.k, red);
  if (chunk == 0 && threadIdx.x == 0) {
    a.cc->xnorm[m] = xn;
    a.cc->count[m] = 0u;  // the survivors are counted by k_cert_select
  }
  float lo = -__builtin_inff(), hi = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < kRows; ++j) {
    if (r0 + j * kCertThreads + (int)threadIdx.x >= a.n) break;
    const double lq = (double)lqv[j];
    const double width = xn * ((double)bd[j].x + a.slack * (double)bd[j].y);
    const double lower = isfinite(width) ? lq - width : -__builtin_inf();
    const double upper = lq + width;
    lo = fmaxf(lo, __double2float_rd(lower));                 // NaN ignored
    hi = fmaxf(hi, isnan(upper) ? __builtin_inff() : __double2float_ru(upper));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = fmaxf(lo, __shfl_xor(lo, o, 64));
    hi = fmaxf(hi, __shfl_xor(hi, o, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    lo_w[threadIdx.x >> 6] = lo;
    hi_w[threadIdx.x >> 6] = hi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kCertThreads / 64; ++w) {
      lo = fmaxf(lo, lo_w[w]);
      hi = fmaxf(hi, hi_w[w]);
    }
    a.lb_chunk[(int64_t)m * a.chunks + chunk] = lo;
    a.ub_chunk[(int64_t)m * a.chunks + chunk] = hi;
  }
}

// Chunks whose largest upper bound reaches the best lower bound list their
// surviving rows (the count may pass the cap; entries past it are dropped).
__global__ __launch_bounds__(kCertThreads) void k_cert_select(CertArgs a) {
  __shared__ uint32_t lo_w[kCertThreads / 64];
  const int chunk = blockIdx.x, m = blockIdx.y;
  // the activation row's best lower bound: the largest of its chunks' (as
  // order-preserving keys, so the maximum does not depend on the order)
  uint32_t key = 0u;
  for (int c = threadIdx.x; c < a.chunks; c += kCertThreads) {
    const uint32_t kc = ord32(a.lb_chunk[(int64_t)m * a.chunks + c]);
    key = kc > key ? kc : key;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t t = __shfl_xor(key, o, 64);
    key = t > key ? t : key;
  }
  if ((threadIdx.x & 63) == 0) lo_w[threadIdx.x >> 6] = key;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kCertThreads / 64; ++w) key = lo_w[w] > key ? lo_w[w] : key;
  const float best_lower = unord32(key);
  if (a.ub_chunk[(int64_t)m * a.chunks + chunk] < best_lower) return;  // nothing here can win
  const double xn = a.cc->xnorm[m];
  const int lane = threadIdx.x & 63;
  const int r0 = chunk * kCertChunk;
  // the thread's rows: all loads first (rows past N load row N - 1, in bounds,
  // and are not kept), then the survivors are listed
  constexpr int kRows = kCertChunk / kCertThreads;
  float lqv[kRows];
  float2 bd[kRows];
#pragma unroll
  for (int j = 0; j < kRows; ++j) {
    const int row = min(r0 + j * kCertThreads + (int)threadIdx.x, a.n - 1);
    lqv[j] = a.lq[(int64_t)m * a.n + row];
    bd[j] = make_float2(a.bounds[2 * row], a.bounds[2 * row + 1]);
  }
#pragma unroll
  for (int j = 0; j < kRows; ++j) {
    const int row = r0 + j * kCertThreads + (int)threadIdx.x;
    const double width = xn * ((double)bd[j].x + a.slack * (double)bd[j].y);
    const bool keep = row < a.n && !((double)lqv[j] + width < (double)best_lower);
    const uint64_t ballot = __ballot(keep);
    if (ballot == 0) continue;
    uint32_t pos0 = 0;
    if (lane == 0)
      pos0 = __hip_atomic_fetch_add(&a.cc->count[m], (uint32_t)__popcll(ballot), __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    pos0 = __shfl(pos0, 0, 64);
    if (keep) {
      const uint32_t pos = pos0 + (uint32_t)__popcll(ballot & ((1ull << lane) - 1ull));
      if (pos < (uint32_t)a.cap) a.list[(int64_t)m * a.cap + pos] = (uint32_t)row;
    }
  }
}

struct RescoreArgs {
  const uint8_t* rec;
  const uint8_t* e_top;
  const uint32_t* row_ptr;
  const uint2* esc;
  const uint16_t* x;
  int64_t ldx;
  CertZero* z;
  CertCall* cc;
  const uint32_t* list;
  int32_t* idx;
  float* maxv;
  int32_t* survivors;
  int n, k, m, cap;
};

__device__ __forceinline__ int32_t sat_i32(uint32_t c) { return c > 0x7FFFFFFFu ? 0x7FFFFFFF : (int32_t)c; }

// One wave per (activation row, surviving row), waves striding over the
// flattened lists. The dot product runs over the exact decode (placeholders at
// escapes), then each escape adds x * (exact - placeholder); both in fp32 in a
// fixed order, so a pair's logit does not depend on the schedule. The last of
// row m's pairs to finish writes idx[m] and max_logit[m]. When any row kept
// more than the cap, nothing is rescored: the full head's gate goes up.
__global__ __launch_bounds__(kCertThreads) void k_cert_rescore(RescoreArgs a) {
  const int lane = threadIdx.x & 63;
  // per-activation-row counts and their inclusive prefix (lane = row)
  uint32_t c = 0;
  if (lane < a.m) c = a.cc->count[lane];
  const bool fallback = __ballot(c > (uint32_t)a.cap) != 0ull;
  if (blockIdx.x == 0 && threadIdx.x < 64) {
    if (threadIdx.x == 0)
      __hip_atomic_store(&a.cc->flag, fallback ? 1u : 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lane < a.m && (fallback || c == 0u)) {
      // the full head answers (or, with no survivor at all, which the bounds
      // rule out, index 0): only the counts are reported here
      if (a.survivors) a.survivors[lane] = sat_i32(c);
      if (!fallback) {
        a.idx[lane] = 0;
        if (a.maxv) a.maxv[lane] = -__builtin_inff();
      }
    }
  }
  if (fallback) return;
  uint32_t incl = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  const uint32_t total = __shfl(incl, 63, 64);
  const int waves = gridDim.x * (kCertThreads / 64);
  const int kb_count = a.k / kRecCols;
  const int G = lane & 31;
  for (uint32_t t = blockIdx.x * (kCertThreads / 64) + (threadIdx.x >> 6); t < total; t += (uint32_t)waves) {
    const uint64_t past = __ballot(incl > t);           // rows whose prefix passes t
    const int m = __builtin_ctzll(past);
    const uint32_t cm = __shfl(c, m, 64);
    const uint32_t excl = __shfl(incl - c, m, 64);
    const uint32_t row = a.list[(int64_t)m * a.cap + (t - excl)];
    const int r = row & 15;
    const uint8_t* blk = a.rec + (int64_t)(row >> 4) * kb_count * kRecBytes;
    const uint32_t bias = (uint32_t)(a.e_top[row] - 15) << 7;
    const uint32_t bias2 = bias | (bias << 16);
    const uint16_t* xr = a.x + (int64_t)m * a.ldx;
    float acc = 0.f;
    // records kb = lane / 32 + 2 i, four at a time with every load issued first
    constexpr int kRB = 4;
    for (int kb0 = lane >> 5; kb0 < kb_count; kb0 += 2 * kRB) {
      uint4 v[kRB], x0[kRB], x1[kRB];
      uint2 b[kRB];
#pragma unroll
      for (int i = 0; i < kRB; ++i) {
        const int kb = kb0 + 2 * i;
        if (kb < kb_count) {
          const uint8_t* rp = blk + (int64_t)kb * kRecBytes;
          v[i] = *reinterpret_cast<const uint4*>(rp + (G * 16 + r) * 16);
          b[i] = *reinterpret_cast<const uint2*>(rp + kViewBytes + (G * 16 + r) * 8);
          const uint4* xp = reinterpret_cast<const uint4*>(xr + kb * kRecCols + G * 16);
          x0[i] = xp[0];
          x1[i] = xp[1];
        }
      }
#pragma unroll
      for (int i = 0; i < kRB; ++i) {
        if (kb0 + 2 * i < kb_count) {
          const uint32_t xw[8] = {x0[i].x, x0[i].y, x0[i].z, x0[i].w, x1[i].x, x1[i].y, x1[i].z, x1[i].w};
          uint32_t d[8];
          decode16_exact(v[i], b[i], d, bias2);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            acc = fmaf(bf16_to_f32(d[j] & 0xFFFFu), bf16_to_f32(xw[j] & 0xFFFFu), acc);
            acc = fmaf(bf16_to_f32(d[j] >> 16), bf16_to_f32(xw[j] >> 16), acc);
          }
        }
      }
    }
    float corr = 0.f;
    const uint32_t e0 = a.row_ptr[row], e1 = a.row_ptr[row + 1];
    for (uint32_t i = e0 + lane; i < e1; i += 64) {
      const uint2 e = a.esc[i];
      const float xv = bf16_to_f32(xr[e.x]);
      corr = fmaf(xv, bf16_to_f32(e.y & 0xFFFFu), corr);
      corr = fmaf(-xv, bf16_to_f32(e.y >> 16), corr);
    }
    const float logit = wave_sum_f32(acc) + wave_sum_f32(corr);
    if (lane == 0) {
      // the key and the count are atomics at the coherence point; the count
      // goes in only once the key has, so the row's last pair reads them all
      __hip_atomic_fetch_max(&a.z->best[m], argmax_key(logit, row), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      const uint32_t d = __hip_atomic_fetch_add(&a.z->done[m], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (d == cm - 1u) {
        const unsigned long long key = __hip_atomic_load(&a.z->best[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        a.idx[m] = (int32_t)(0xFFFFFFFFu - (uint32_t)key);
        if (a.maxv) a.maxv[m] = key_value(key);
        if (a.survivors) a.survivors[m] = sat_i32(cm);
        __hip_atomic_store(&a.z->best[m], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.z->done[m], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

}  // namespace

hipError_t launch_cert_bounds(const w12_matrix* m, float* bounds, hipStream_t s) {
  const int n = (int)m->n;
  const int per = kCertThreads / 64;
  hipLaunchKernelGGL(k_cert_bounds, dim3((n + per - 1) / per), dim3(kCertThreads), 0, s, m->records, m->e_top,
                     m->esc_row_ptr, reinterpret_cast<const uint2*>(m->esc), n, (int)m->k, bounds);
  return hipGetLastError();
}

int cert_chunks(int64_t n) { return (int)((n + kCertChunk - 1) / kCertChunk); }

hipError_t launch_cert(const w12_matrix* mat, const uint16_t* x, int64_t ldx, int M, const float* lq,
                       const float* bounds, CertZero* z, CertCall* cc, float* ub_chunk, float* lb_chunk,
                       uint32_t* list, int32_t* idx,
                       float* maxv, int32_t* survivors, hipStream_t s) {
  CertArgs a{};
  a.x = x;
  a.ldx = ldx;
  a.lq = lq;
  a.bounds = bounds;
  a.z = z;
  a.cc = cc;
  a.ub_chunk = ub_chunk;
  a.lb_chunk = lb_chunk;
  a.list = list;
  a.n = (int)mat->n;
  a.k = (int)mat->k;
  a.m = M;
  a.chunks = cert_chunks(mat->n);
  a.cap = W12_CERT_MAX_SURVIVORS;
  const double ku = (double)mat->k * 0x1p-24;
  a.slack = 4.0 * ku / (1.0 - ku);
  hipLaunchKernelGGL(k_cert_lower, dim3(a.chunks, M), dim3(kCertThreads), 0, s, a);
  hipLaunchKernelGGL(k_cert_select, dim3(a.chunks, M), dim3(kCertThreads), 0, s, a);
  RescoreArgs r{};
  r.rec = mat->records;
  r.e_top = mat->e_top;
  r.row_ptr = mat->esc_row_ptr;
  r.esc = reinterpret_cast<const uint2*>(mat->esc);
  r.x = x;
  r.ldx = ldx;
  r.z = z;
  r.cc = cc;
  r.list = list;
  r.idx = idx;
  r.maxv = maxv;
  r.survivors = survivors;
  r.n = a.n;
  r.k = a.k;
  r.m = M;
  r.cap = a.cap;
  hipLaunchKernelGGL(k_cert_rescore, dim3(kNumCU), dim3(kCertThreads), 0, s, r);
  return hipGetLastError();
}

}  // namespace w12

// W12 GEMM, MFMA stream kernel for gfx950: y[M, N] = x[M, K] W^T for 3 to 64
// activation rows, in store mode (exact GEMM and Q pass).
//
// SpecPilot (arXiv 2611.02501) section 4.1 and Figure 5b: records are decoded
// in registers so that the weight stream hides the decode, the escape list
// restores every weight exactly, and the reduction over K is split over
// workgroups in a fixed order (stream-K), so results are deterministic.
// Section 4.3: the Q pass reads only the 8-bit view.
//
// Layout of the work. A workgroup has eight waves and every wave streams. A
// unit is 512 columns of a tile (one record per 16-row block); wave w takes
// its 64-column chunk w, so one record load per block serves all eight waves
// and one activation load serves every block of the tile. A whole tile is
// four 16-row blocks (two beyond 32 activation rows, for registers). With P
// workgroups and T whole tiles, workgroup p owns tiles [p D, (p+1) D),
// D = T / P; the rows left over are cut into split tiles whose units are
// shared evenly by all workgroups (stream-K), streamed first.
//
// Decode. Weights are rebuilt with their true exponent (off + E_n - 15), so
// an escape's exact BF16 bits are a valid operand: the wave substitutes them
// for the placeholder in its decoded registers before the MFMA, and the
// matrix cores multiply the exact weight (they keep subnormal inputs and
// results). There is no separate fix-up pass and no activation gather. Each
// wave takes its escapes for a segment from an LDS list that it builds at the
// segment's start from the CSR escape list, while the segment's first two
// units load. Entries beyond the list's capacity are corrected after the
// segment's stream: the partial sums get x * (-placeholder) then x * exact,
// two fused multiply-adds per activation row (exact when x is one-hot).
//
// Activations. The B operand of v_mfma_f32_16x16x32_bf16 comes from
// row-major x with no pre-pass: lane l needs activation row l % 16 of its
// m-tile at the 16 columns of the view load that give its A operands. Read
// that way, one load instruction would touch 16 rows' lines, half of each;
// instead each wave loads its 64-column chunk as whole 128-byte lines (eight
// rows per instruction) and turns it into operand order through a small
// per-wave LDS area.
//
// End of a segment. Each wave leaves its MFMA accumulators in LDS; after a
// barrier all 512 threads add the eight waves' sums in wave order and either
// write the tile's outputs or, for a split tile, publish the values in the
// workgroup's slot: every thread stores its values with agent-scope atomic
// stores and waits until they have completed, then wave 0 counts the
// workgroup into the tile's counter. The last workgroup to arrive adds all
// slots (agent-scope atomic loads) in workgroup order after its own work is
// streamed and writes the tile; counters wrap back to zero.
#include "w12_internal.h"

namespace w12 {
namespace mx {

constexpr int kWaves = 8;                  // streaming waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kUnitCols = 64 * kWaves;     // a unit: one 64-column chunk per wave
constexpr int kWgPerCU = 8 / kWaves;       // workgroups per compute unit (eight waves per CU)
constexpr int kCap = 256;  // escape substitutions one wave holds per segment
constexpr int kRedRow = 65;  // floats per row of the reduction area (64 lanes + 1 of padding)
constexpr int kXsRow = 144;  // bytes per activation row of a wave's staging area (128 + 16 of padding)

template <int MT>
constexpr int kRG = MT <= 2 ? 4 : 2;  // 16-row blocks of a whole tile

// -------------------------------------------------------------- schedule
// floor(x / y) for x < 2^40, 0 < y < 2^31: the double quotient is within one
// of the exact one, and one integer step corrects it.
__device__ __forceinline__ uint32_t div_floor(uint64_t x, uint32_t y) {
  uint32_t q = (uint32_t)((double)x / (double)y);
  const uint64_t qy = (uint64_t)q * y;
  if (qy > x) --q;
  else if (qy + y <= x) ++q;
  return q;
}

// First split unit of workgroup q (q in [0, P]); unit u is column unit u % ku
// of split tile u / ku.
__device__ __forceinline__ uint32_t sk_start(const MxParams& a, int q) {
  return div_floor((uint64_t)q * (uint64_t)a.sk_units, (uint32_t)a.P);
}

// Workgroup owning split unit u.
__device__ __forceinline__ int sk_owner(const MxParams& a, uint32_t u) {
  return (int)div_floor(((uint64_t)u + 1) * (uint64_t)a.P + (uint64_t)a.sk_units - 1, (uint32_t)a.sk_units) - 1;
}

// Workgroup q's slot for split tile t: 2q if t is its first split tile, 2q+1
// if its second; -1 if q owns no unit of t.
__device__ __forceinline__ int part_slot(const MxParams& a, int q, int t) {
  const uint32_t s = sk_start(a, q), e = sk_start(a, q + 1);
  const uint32_t t0 = (uint32_t)t * (uint32_t)a.ku, t1 = t0 + (uint32_t)a.ku;
  if (s >= e || e <= t0 || s >= t1) return -1;
  return 2 * q + ((s >= t0) ? 0 : 1);
}

struct Seg {
  int row0;    // first row
  int rg;      // 16-row blocks (fewer than the tile's only at the end of the matrix)
  int k0, k1;  // units [k0, k1)
  int tile;    // split tile index (whole tile: -1)
  int part;    // which of this workgroup's split tiles, 0 or 1 (whole tile: -1)
};

struct SegList {
  int n, nsk;
  Seg sk0, sk1;
  int dp0;
};

template <int TB>
__device__ __forceinline__ Seg split_seg(const MxParams& a, int t, int k0, int k1, int part) {
  const int r0 = a.sk_row0 + t * TB * 16;
  return Seg{r0, min(TB, (a.n - r0) >> 4), k0, k1, t, part};
}

// The segments of workgroup p: its split ones (the shorter first), then its
// whole tiles.
template <int TB>
__device__ __forceinline__ SegList seg_list(const MxParams& a, int p) {
  SegList L;
  L.dp0 = p * a.dp;
  L.nsk = 0;
  L.sk0 = L.sk1 = Seg{0, 0, 0, 0, -1, -1};
  const uint32_t s0 = sk_start(a, p), s1 = sk_start(a, p + 1);
  if (s1 > s0) {
    const int ta = (int)div_floor(s0, (uint32_t)a.ku), tz = (int)div_floor(s1 - 1, (uint32_t)a.ku);
    const uint32_t ua = (uint32_t)ta * (uint32_t)a.ku, uz = (uint32_t)tz * (uint32_t)a.ku;
    const Seg A = split_seg<TB>(a, ta, (int)(s0 - ua), ta == tz ? (int)(s1 - ua) : a.ku, 0);
    if (ta == tz) {
      L.nsk = 1;
      L.sk0 = A;
    } else {
      const Seg B = split_seg<TB>(a, tz, 0, (int)(s1 - uz), 1);
      L.nsk = 2;
      const bool b_first = (B.k1 - B.k0) < (A.k1 - A.k0);
      L.sk0 = b_first ? B : A;
      L.sk1 = b_first ? A : B;
    }
  }
  L.n = L.nsk + a.dp;
  return L;
}

template <int GB>
__device__ __forceinline__ Seg seg_at(const MxParams& a, const SegList& L, int i) {
  if (i < L.nsk) return i == 0 ? L.sk0 : L.sk1;
  const int r0 = (L.dp0 + i - L.nsk) * GB * 16;
  return Seg{r0, min(GB, (a.n - r0) >> 4), 0, a.ku, -1, -1};
}

// -------------------------------------------------------------- LDS
template <int MT>
struct Lds {
  // each wave's MFMA accumulators of the current segment: [block][m-tile][element][lane],
  // rows padded to 65 floats so that the reduction's reads (64 output rows of
  // one activation row) spread over the banks
  float red[kWaves][kRG<MT>][MT][4][kRedRow];
  // per wave: the segment's escape substitutions {packed target and bits,
  // unit}, their count, and the row pointers of the segment's rows
  uint2 list[kWaves][kCap];
  uint32_t rp[kWaves][65];
  int last[2];  // split tiles this workgroup finishes last: tile + 1, or 0
  // per wave: its 64-column chunk of x for the current unit, rows padded to
  // 144 bytes so that the operand-order reads spread over the banks
  alignas(16) uint8_t xs[kWaves][16 * MT][kXsRow];
};

// -------------------------------------------------------------- decode
// 16 weights with their true exponent; in Q mode the four dropped mantissa
// bits are 1000 (the midpoint) and plane B is not read.
template <bool Q>
__device__ __forceinline__ void decode16(uint4 v, uint2 b, uint32_t* d, uint32_t bias2) {
  const uint32_t b0 = Q ? 0x80808080u : b.x, b1 = Q ? 0x80808080u : b.y;
  const uint32_t b0s = Q ? b0 : (b0 << 4), b1s = Q ? b1 : (b1 << 4);
  d[0] = pair_exact(v.x, b0, kSelPair01, bias2);
  d[1] = pair_exact(v.x, b0, kSelPair23, bias2);
  d[2] = pair_exact(v.y, b0s, kSelPair01, bias2);
  d[3] = pair_exact(v.y, b0s, kSelPair23, bias2);
  d[4] = pair_exact(v.z, b1, kSelPair01, bias2);
  d[5] = pair_exact(v.z, b1, kSelPair23, bias2);
  d[6] = pair_exact(v.w, b1s, kSelPair01, bias2);
  d[7] = pair_exact(v.w, b1s, kSelPair23, bias2);
}

// Packed substitution: bits 15..0 the exact BF16, bit 16 the half of the
// register (odd column), bits 19..17 the register (column % 16 / 2), bits
// 21..20 the 16-row block, bits 27..22 the lane (16 (column % 64 / 16) + row % 16).
__device__ __forceinline__ uint32_t pack_sub(uint32_t col, int r, uint32_t bits) {
  const uint32_t tl = ((col >> 4) & 3u) * 16u + ((uint32_t)r & 15u);
  return (bits & 0xFFFFu) | (col & 1u) << 16 | ((col >> 1) & 7u) << 17 | ((uint32_t)r >> 4) << 20 | tl << 22;
}

// Replace one decoded weight (register jr = 8 block + register, chosen by the
// uniform `info`) in lane info >> 22.
template <int RG>
__device__ __forceinline__ void substitute(uint32_t (&d)[RG][8], uint32_t info, int lane) {
  const uint32_t jr = (info >> 17) & 31u;
  const bool mine = (uint32_t)lane == (info >> 22);
  const bool hi = (info >> 16) & 1u;
  const uint32_t keep = hi ? 0x0000FFFFu : 0xFFFF0000u;
  const uint32_t nv = hi ? (info << 16) : (info & 0xFFFFu);
#pragma unroll
  for (int q = 0; q < RG * 8; ++q)
    if ((uint32_t)q == jr) d[q >> 3][q & 7] = mine ? ((d[q >> 3][q & 7] & keep) | nv) : d[q >> 3][q & 7];
}

// Row r (0 .. R-1) of escape entry `idx`: the largest r with rp[r] <= idx.
__device__ __forceinline__ int entry_row(const uint32_t* rp, int R, uint32_t idx) {
  int lo = 0, hi = R;  // rp[lo] <= idx < rp[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (rp[mid] <= idx) lo = mid; else hi = mid;
  }
  return lo;
}

constexpr int kEscBatch = 8;  // entry loads per lane in flight while building a list (512 entries)

// The wave's escapes of segment s (rows row0 .. row0 + R - 1, units [k0, k1),
// 64-column chunk `wave` of each unit), in CSR order: the first kCap go to the
// LDS list; returns how many there are.
// The first batch of a segment's escape entries, [e0, e0 + 64 kEscBatch).
__device__ __forceinline__ void load_entries(const MxParams& a, uint32_t b, uint32_t e1, int lane,
                                             uint2 (&ev)[kEscBatch]) {
#pragma unroll
  for (int k = 0; k < kEscBatch; ++k) {
    const uint32_t idx = b + 64 * k + lane;
    ev[k] = idx < e1 ? a.esc[idx] : make_uint2(0xFFFFFFFFu, 0u);
  }
}

// r_lane and e1 are the row pointers of row row0 + lane and of row row0 + R,
// ev the first batch of entries; the caller loads both ahead of the
// segment's first weight loads (the entries after the row pointers arrive),
// so neither round trip queues behind the weight stream.
template <int MT>
__device__ __forceinline__ int build_list(const MxParams& a, Lds<MT>& sh, const Seg& s, int wave, int lane,
                                          uint32_t r_lane, uint32_t e1, const uint2 (&ev0)[kEscBatch]) {
  const int R = s.rg * 16;
  uint32_t* rp = sh.rp[wave];
  if (lane < R) rp[lane] = r_lane;
  if (lane == 0) rp[R] = e1;
  __builtin_amdgcn_wave_barrier();
  const uint32_t e0 = __builtin_amdgcn_readfirstlane(r_lane);
  int cnt = 0;
  for (uint32_t b = e0; b < e1; b += 64 * kEscBatch) {
    uint2 ev[kEscBatch];
    if (b == e0) {
#pragma unroll
      for (int k = 0; k < kEscBatch; ++k) ev[k] = ev0[k];
    } else {
      load_entries(a, b, e1, lane, ev);
    }
#pragma unroll
    for (int k = 0; k < kEscBatch; ++k) {
      const uint32_t idx = b + 64 * k + lane;
      const uint32_t col = ev[k].x, u = col / kUnitCols;
      const bool keep = idx < e1 && u >= (uint32_t)s.k0 && u < (uint32_t)s.k1 && (col >> 6) % kWaves == (uint32_t)wave;
      const uint64_t bal = __ballot(keep);
      if (keep) {
        const int pos = cnt + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        if (pos < kCap) sh.list[wave][pos] = make_uint2(pack_sub(col, entry_row(rp, R, idx), ev[k].y), u);
      }
      cnt += __popcll(bal);
    }
  }
  __builtin_amdgcn_wave_barrier();  // the list is written before the stream reads it
  return cnt;
}

// Entries of the wave's escape list beyond kCap, after the stream, on the
// wave's accumulators in LDS: the MFMA multiplied the placeholder (seen
// through the Q view in the Q pass), so each entry's row gets x * (-placeholder)
// and then x * exact value for every activation row, entry by entry in CSR
// order. The accumulator of (row r, activation row m) is element r % 4 of
// lane 16 (r % 16 / 4) + m % 16 in block r / 16, m-tile m / 16.
template <int MT, bool Q>
__device__ __forceinline__ void overflow_fix(const MxParams& a, Lds<MT>& sh, const Seg& s, int wave, int lane) {
  const int R = s.rg * 16;
  const uint32_t* rp = sh.rp[wave];
  const uint32_t e0 = rp[0], e1 = rp[R];
  int cnt = 0;
  for (uint32_t b = e0; b < e1; b += 64) {
    const uint32_t idx = b + lane;
    const uint2 ev = idx < e1 ? a.esc[idx] : make_uint2(0xFFFFFFFFu, 0u);
    const uint32_t col = ev.x, u = col / kUnitCols;
    const bool keep = idx < e1 && u >= (uint32_t)s.k0 && u < (uint32_t)s.k1 && (col >> 6) % kWaves == (uint32_t)wave;
    uint64_t bal = __ballot(keep);
    const int nk = __popcll(bal);
    // the first kCap kept entries were substituted in the stream
    const int skip = cnt >= kCap ? 0 : min(kCap - cnt, nk);
    for (int i = 0; i < skip; ++i) bal &= bal - 1;
    cnt += nk;
    const int r_lane = entry_row(rp, R, idx);
    while (bal) {
      const int src = __builtin_ctzll(bal);
      bal &= bal - 1;
      const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)col, src);
      const uint32_t bits = (uint32_t)__builtin_amdgcn_readlane((int)ev.y, src);
      const int r = __builtin_amdgcn_readlane(r_lane, src);
      uint32_t ph = bits >> 16;
      if (Q) ph = (ph & 0xFFF0u) | 0x8u;
      const float nph = -bf16_to_f32(ph), ex = bf16_to_f32(bits & 0xFFFFu);
      if ((lane >> 4) == ((r & 15) >> 2)) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = mt * 16 + (lane & 15);
          if (m < a.m) {
            const float xv = bf16_to_f32(a.x[(int64_t)m * a.ldx + c]);
            float& acc = sh.red[wave][r >> 4][mt][r & 3][lane];
            acc = fmaf(xv, ex, fmaf(xv, nph, acc));
          }
        }
      }
    }
  }
}

// -------------------------------------------------------------- stream
template <int MT, int RG, bool Q>
struct Stage {
  uint4 x[MT][2];
  uint4 v[RG];
  uint2 b[RG];
};

// One wave's part of segment s: stream its chunk of every unit, substitute
// escapes, and leave its accumulators in sh.red[wave]. Returns the wave's
// escape count of the segment (those beyond kCap still need overflow_fix).
template <int MT, int RG, bool Q>
__device__ __forceinline__ int seg_stream(const MxParams& a, Lds<MT>& sh, const Seg& s, int wave, int lane) {
  // exponent bias per block for this lane's row (l % 16 of the block)
  uint32_t bias[RG];
#pragma unroll
  for (int j = 0; j < RG; ++j) {
    const int n = min(s.row0 + 16 * j + (lane & 15), a.n - 1);
    const uint32_t e = ((uint32_t)a.e_top[n] - 15u) << 7;
    bias[j] = e | e << 16;
  }
  const uint8_t* blk = a.rec + (int64_t)(s.row0 >> 4) * a.kb * kRecBytes;
  const uint32_t blk_stride = (uint32_t)a.kb * kRecBytes;
  const uint32_t voff = (uint32_t)lane * 16u, boff = kViewBytes + (uint32_t)lane * 8u;
  // Activations: load i of a unit takes rows 8 i .. 8 i + 7 of the wave's
  // 64-column chunk, lane l row 8 i + l / 8 and bytes 16 (l % 8) of its
  // 128, so each load is eight whole lines (rows past M read row M - 1;
  // they only feed outputs that are not stored).
  const uint16_t* xr[2 * MT];
#pragma unroll
  for (int i = 0; i < 2 * MT; ++i)
    xr[i] = a.x + (int64_t)min(8 * i + (lane >> 3), a.m - 1) * a.ldx + wave * 64 + (lane & 7) * 8;
  uint8_t* xs = &sh.xs[wave][0][0];
  const uint32_t xs_w = (uint32_t)(lane >> 3) * kXsRow + (uint32_t)(lane & 7) * 16u;
  const uint32_t xs_r = (uint32_t)(lane & 15) * kXsRow + (uint32_t)(lane >> 4) * 32u;
  auto load = [&](Stage<MT, RG, Q>& st, int u) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        st.x[mt][h] = *reinterpret_cast<const uint4*>(xr[2 * mt + h] + (int64_t)u * kUnitCols);
    // this wave's 64-column chunk c of the row: record c / 8, chunk c % 8 in it
    const uint32_t c = (uint32_t)u * kWaves + (uint32_t)wave;
    const uint32_t rec_off = (c >> 3) * kRecBytes;
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      const uint32_t o = (uint32_t)j * blk_stride + rec_off;
      st.v[j] = load_stream16(blk + (o + (c & 7) * 1024u + voff));
      if (!Q) st.b[j] = load_stream8(blk + (o + (c & 7) * 512u + boff));
    }
  };
  f32x4_t acc[RG][MT];
#pragma unroll
  for (int j = 0; j < RG; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[j][mt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  int ne = 0;  // escape substitutions in the list
  auto compute = [&](const Stage<MT, RG, Q>& st, int u) {
    // through LDS into operand order: lane l gets activation row l % 16 of
    // each m-tile, bytes 32 (l / 16) .. +31 of the chunk (the columns of its
    // A operands). One wave's LDS accesses complete in order, so the next
    // unit's writes cannot overtake these reads.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *reinterpret_cast<u32x4_t*>(xs + xs_w + (2 * mt + h) * 8 * kXsRow) = __builtin_bit_cast(u32x4_t, st.x[mt][h]);
    __builtin_amdgcn_wave_barrier();
    uint4 xb[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      xb[mt][0] = __builtin_bit_cast(uint4, *reinterpret_cast<const u32x4_t*>(xs + xs_r + mt * 16 * kXsRow));
      xb[mt][1] = __builtin_bit_cast(uint4, *reinterpret_cast<const u32x4_t*>(xs + xs_r + mt * 16 * kXsRow + 16));
    }
    __builtin_amdgcn_wave_barrier();
    uint32_t d[RG][8];
#pragma unroll
    for (int j = 0; j < RG; ++j) decode16<Q>(st.v[j], Q ? make_uint2(0, 0) : st.b[j], d[j], bias[j]);
    for (int b0 = 0; b0 < ne; b0 += 64) {
      const uint2 e = b0 + lane < ne ? sh.list[wave][b0 + lane] : make_uint2(0u, 0xFFFFFFFFu);
      uint64_t bal = __ballot(e.y == (uint32_t)u);
      while (bal) {
        const int src = __builtin_ctzll(bal);
        bal &= bal - 1;
        substitute<RG>(d, (uint32_t)__builtin_amdgcn_readlane((int)e.x, src), lane);
      }
    }
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      const uint4 a0 = make_uint4(d[j][0], d[j][1], d[j][2], d[j][3]);
      const uint4 a1 = make_uint4(d[j][4], d[j][5], d[j][6], d[j][7]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0),
                                                             __builtin_bit_cast(bf16x8_t, xb[mt][0]), acc[j][mt], 0,
                                                             0, 0);
        acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1),
                                                             __builtin_bit_cast(bf16x8_t, xb[mt][1]), acc[j][mt], 0,
                                                             0, 0);
      }
    }
  };
  // Two register stages. The loads of the first two units go out before the
  // escape list is built (its dependent round trips overlap them); in the
  // loop, unit i + 2 loads while unit i + 1's data arrive and unit i computes.
  const int u0 = s.k0, n = s.k1 - s.k0;
  int cnt = 0;
  // The escape list's round trips (row pointers, then the first batch of
  // entries) go out ahead of the segment's weight loads, so they do not queue
  // behind them; the list is built while the first two units load.
  uint32_t r_lane = 0u, e1 = 0u;
  uint2 ev0[kEscBatch];
  if (a.fix) {
    r_lane = a.row_ptr[s.row0 + min(lane, s.rg * 16)];
    e1 = a.row_ptr[s.row0 + s.rg * 16];
    load_entries(a, __builtin_amdgcn_readfirstlane(r_lane), e1, lane, ev0);
  }
  Stage<MT, RG, Q> sa, sb;
  load(sa, u0);
  if (n > 1) load(sb, u0 + 1);
  if (a.fix) {
    cnt = build_list<MT>(a, sh, s, wave, lane, r_lane, e1, ev0);
    ne = min(cnt, kCap);
  }
  if (n == 1) {
    compute(sa, u0);
  } else {
    int i = 0;
    for (; i + 3 < n; i += 2) {
      compute(sa, u0 + i);
      load(sa, u0 + i + 2);
      compute(sb, u0 + i + 1);
      load(sb, u0 + i + 3);
    }
    compute(sa, u0 + i);
    if (n - i == 3) {
      load(sa, u0 + i + 2);
      compute(sb, u0 + i + 1);
      compute(sa, u0 + i + 2);
    } else {
      compute(sb, u0 + i + 1);
    }
  }
  // C layout of a 16x16 MFMA: lane l holds rows 4 (l / 16) + e, activation row l % 16
#pragma unroll
  for (int j = 0; j < RG; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) sh.red[wave][j][mt][e][lane] = acc[j][mt][e];
  return cnt;
}

// -------------------------------------------------------------- outputs
template <int J, int MS>
__device__ __forceinline__ void store_y(const MxParams& a, int n, int m0, const float (&v)[J]) {
  if (a.y_f32) {
    float* y = reinterpret_cast<float*>(a.y) + n;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (m0 + MS * j < a.m) y[(int64_t)(m0 + MS * j) * a.ldy] = v[j];
  } else {
    uint16_t* y = reinterpret_cast<uint16_t*>(a.y) + n;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (m0 + MS * j < a.m) y[(int64_t)(m0 + MS * j) * a.ldy] = f32_to_bf16_rne(v[j]);
  }
}

// Sum of the eight waves' accumulators (in wave order) for row r of the tile
// and activation rows m0 + MS j.
template <int MT, int RG, int J, int MS>
__device__ __forceinline__ void wave_sums(const Lds<MT>& sh, int r, int m0, float (&v)[J]) {
  const int j = r >> 4, e = r & 3, lq = ((r & 15) >> 2) * 16;
#pragma unroll
  for (int q = 0; q < J; ++q) {
    const int m = min(m0 + MS * q, 16 * MT - 1);
    const int mt = m >> 4, ln = lq + (m & 15);
    float s = sh.red[0][j][mt][e][ln];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += sh.red[w][j][mt][e][ln];
    v[q] = s;
  }
}

// Workgroups that hold units of split tile t, and how many of them there are
// (wave-uniform; every lane of the calling wave active).
__device__ __forceinline__ int tile_sharers(const MxParams& a, int t, int& pa, int& pb, int lane) {
  const uint32_t u_first = (uint32_t)t * (uint32_t)a.ku;
  pa = sk_owner(a, u_first);
  pb = sk_owner(a, u_first + (uint32_t)a.ku - 1);
  int cnt = 0;
  for (int q0 = pa; q0 <= pb; q0 += 64) {
    const int q = q0 + lane;
    cnt += __popcll(__ballot(q <= pb && part_slot(a, q, t) >= 0));
  }
  return cnt;
}

// ============================================================== kernel
template <int MT, bool Q, int TB>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_mx(MxParams a) {
  constexpr int RG = kRG<MT>;
  constexpr int MM = 16 * MT;
  constexpr int ROWS = RG * 16;       // rows of a whole tile
  constexpr int TS = TB * 16;         // rows of a split tile
  constexpr int MS = kThreads / ROWS; // activation-row step of a thread's outputs
  constexpr int J = (MM + MS - 1) / MS;
  __shared__ Lds<MT> sh;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int p = blockIdx.x;
  const SegList L = seg_list<TB>(a, p);
  // split tiles this workgroup counted itself into: tile, sharers [pa, pb]
  // and their count (wave 0), the counter's old value (thread 0)
  int np = 0;
  int t0 = 0, pa0 = 0, pb0 = 0, c0 = 0, t1 = 0, pa1 = 0, pb1 = 0, c1 = 0;
  uint32_t old0 = 0u, old1 = 0u;
  const int r = t % ROWS, m0 = t / ROWS;
  for (int i = 0; i < L.n; ++i) {
    const Seg s = seg_at<RG>(a, L, i);
    int cnt;
    if constexpr (RG == 4) {
      switch (s.rg) {
        case 1: cnt = seg_stream<MT, 1, Q>(a, sh, s, wave, lane); break;
        case 2: cnt = seg_stream<MT, 2, Q>(a, sh, s, wave, lane); break;
        case 3: cnt = seg_stream<MT, 3, Q>(a, sh, s, wave, lane); break;
        default: cnt = seg_stream<MT, 4, Q>(a, sh, s, wave, lane); break;
      }
    } else {
      if (s.rg == 1) cnt = seg_stream<MT, 1, Q>(a, sh, s, wave, lane);
      else cnt = seg_stream<MT, RG, Q>(a, sh, s, wave, lane);
    }
    if (cnt > kCap) overflow_fix<MT, Q>(a, sh, s, wave, lane);
    __syncthreads();
    float v[J];
    wave_sums<MT, RG, J, MS>(sh, r, m0, v);
    if (s.tile < 0) {
      if (r < s.rg * 16) store_y<J, MS>(a, s.row0 + r, m0, v);
      __syncthreads();  // sh.red is free for the next segment
      continue;
    }
    // split tile: every thread stores its values in the workgroup's slot with
    // agent-scope atomic stores, which complete at the device's coherence
    // point; each wave waits for its stores, and once all have (barrier),
    // wave 0 counts the workgroup in. (Release and acquire fences at agent
    // scope would write back and invalidate the whole L2 of the XCD, which
    // under the weight stream took 10-30 us.)
    {
      float* slot = a.part + (int64_t)(2 * p + s.part) * MM * TS;
      if (r < TS) {
#pragma unroll
        for (int q = 0; q < J; ++q) {
          const int m = m0 + MS * q;
          if (m < a.m) __hip_atomic_store(&slot[m * TS + r], v[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
    }
    __syncthreads();
    if (wave == 0) {
      int pa, pb;
      const int cnt = tile_sharers(a, s.tile, pa, pb, lane);
      // The owner of a split tile's first unit owns no other tile's first
      // unit (a workgroup's split units span at most one tile's length), so
      // its index names the tile's counter.
      uint32_t old = 0u;
      if (lane == 0) old = __builtin_amdgcn_atomic_inc32(&a.ctr[pa], (uint32_t)cnt - 1u, __ATOMIC_RELAXED, "agent");
      if (np == 0) t0 = s.tile, pa0 = pa, pb0 = pb, c0 = cnt, old0 = old;
      else t1 = s.tile, pa1 = pa, pb1 = pb, c1 = cnt, old1 = old;
    }
    ++np;
  }
  if (np == 0) return;
  // Split tiles this workgroup was last on: add every sharer's slot in
  // workgroup order and write the tile.
  if (t == 0) {
    sh.last[0] = (np > 0 && old0 == (uint32_t)c0 - 1u) ? 1 : 0;
    sh.last[1] = (np > 1 && old1 == (uint32_t)c1 - 1u) ? 1 : 0;
    // tiles and sharers travel through LDS (only wave 0 knows them)
    sh.rp[0][0] = (uint32_t)t0, sh.rp[0][1] = (uint32_t)pa0, sh.rp[0][2] = (uint32_t)pb0;
    sh.rp[0][3] = (uint32_t)t1, sh.rp[0][4] = (uint32_t)pa1, sh.rp[0][5] = (uint32_t)pb1;
  }
  __syncthreads();
  for (int c = 0; c < np; ++c) {
    if (!sh.last[c]) continue;
    const int tile = (int)sh.rp[0][3 * c], pa = (int)sh.rp[0][3 * c + 1], pb = (int)sh.rp[0][3 * c + 2];
    const int n0 = a.sk_row0 + tile * TS;
    // thread t: row t % TS, activation rows t / TS + (512 / TS) q
    constexpr int MS2 = kThreads / TS, J2 = (MM + MS2 - 1) / MS2;
    const int r2 = t % TS, mb = t / TS;
    float acc[J2];
#pragma unroll
    for (int q = 0; q < J2; ++q) acc[q] = 0.f;
    bool started = false;  // the sum starts from the first slot (keeps the sign of a zero sum)
    for (int qg = pa; qg <= pb; ++qg) {
      const int sl = part_slot(a, qg, tile);
      if (sl < 0) continue;
      const float* slot = a.part + (int64_t)sl * MM * TS;
#pragma unroll
      for (int q = 0; q < J2; ++q) {
        const int m = mb + MS2 * q;
        const float x = m < a.m ? __hip_atomic_load(&slot[m * TS + r2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                : 0.f;
        acc[q] = started ? acc[q] + x : x;
      }
      started = true;
    }
    if (n0 + r2 < a.n) store_y<J2, MS2>(a, n0 + r2, mb, acc);
  }
}

}  // namespace mx

// ============================================================== planning
MxPlan plan_mx(int64_t n, int64_t k, int64_t m, int64_t grid_override) {
  MxPlan pl{};
  const int64_t mt = (m + 15) / 16;
  pl.gb = mt <= 2 ? 4 : 2;
  const int64_t kb = k / mx::kUnitCols;  // units per row
  const int64_t nb = n / 16;
  const int64_t tiles = (nb + pl.gb - 1) / pl.gb;
  // Eight streaming waves per compute unit (kWgPerCU workgroups); with fewer
  // tiles than workgroup slots, c equal sharers per tile (c * T workgroups),
  // or whole tiles on T workgroups when the idle slots cost little.
  const int64_t slots = (int64_t)kNumCU * mx::kWgPerCU;
  int64_t P = slots;
  if (grid_override > 0) {
    P = grid_override;
  } else if (tiles < slots) {
    const int64_t c = slots / tiles;
    if (c >= 2) {
      P = c * tiles;
    } else {
      const int64_t tile_bytes = pl.gb * 16 * k * 3 / 2;
      if (tile_bytes * (slots - tiles) <= kWholeTileSlack * slots) P = tiles;
    }
  }
  if (P > kMaxGrid) P = kMaxGrid;
  if (P > tiles * kb) P = tiles * kb;
  if (P < 1) P = 1;
  pl.P = (int)P;
  pl.dp = (int)(tiles / P);
  // blocks left for split tiles (none when the whole tiles reach past N)
  const int64_t rem = nb - P * pl.dp * pl.gb > 0 ? nb - P * pl.dp * pl.gb : 0;
  // Split tiles are whole-tile sized when many rows are left, single blocks
  // when few are (fewer sharers, so fewer slots for the last one to add).
  pl.tb = rem >= (P / 4) * pl.gb ? pl.gb : 1;
  pl.sk_row0 = (int)(P * pl.dp * pl.gb * 16);
  pl.sk_tiles = (int)((rem + pl.tb - 1) / pl.tb);
  pl.sk_units = (int64_t)pl.sk_tiles * kb;
  pl.part_bytes = (size_t)(2 * P) * (size_t)(mt * 16) * (size_t)(pl.tb * 16) * sizeof(float);
  pl.threads = mx::kThreads;
  pl.unit_cols = mx::kUnitCols;
  return pl;
}

template <bool Q>
static hipError_t launch_mx_q(const MxPlan& pl, const MxParams& p, hipStream_t s) {
  const dim3 grid(pl.P), block(mx::kThreads);
  const bool single = pl.tb == 1;
  switch ((p.m + 15) / 16) {
#define W12_MX_CASE(MT)                                                                             \
  case MT:                                                                                          \
    if (single) hipLaunchKernelGGL((mx::k_mx<MT, Q, 1>), grid, block, 0, s, p);                    \
    else hipLaunchKernelGGL((mx::k_mx<MT, Q, mx::kRG<MT>>), grid, block, 0, s, p);                  \
    break;
    W12_MX_CASE(1) W12_MX_CASE(2) W12_MX_CASE(3) W12_MX_CASE(4)
#undef W12_MX_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mx(const MxPlan& pl, MxParams p, hipStream_t s) {
  p.ku = p.k / mx::kUnitCols;
  p.P = pl.P;
  p.dp = pl.dp;
  p.sk_row0 = pl.sk_row0;
  p.sk_units = pl.sk_units;
  return p.q ? launch_mx_q<true>(pl, p, s) : launch_mx_q<false>(pl, p, s);
}

}  // namespace w12

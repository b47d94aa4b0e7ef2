// W12 skinny GEMM kernels for gfx950: y[M, N] = x[M, K] W^T over W12 records.
//
// SpecPilot (arXiv 2611.02501) section 4.1 and Figure 5b: the kernel decodes
// records in registers so that the weight stream hides the decode, and splits
// the reduction over workgroups in a fixed order (stream-K), so results are
// deterministic. Section 4.3: the Q pass reads only the 8-bit view.
// Appendix E: the LM head in W12, here fused with a per-row argmax.
//
// Work: the matrix is a sequence of row tiles (64 rows for the GEMV kernel,
// 16 for the MFMA kernel), each a sequence of units of 256 columns. With P
// workgroups (one per compute unit) and T tiles, workgroup p owns the whole
// tiles [p D, (p+1) D), D = T / P, and an even share of the units of the
// remaining T - P D tiles (stream-K). A segment is the units of one tile (or
// of a group of whole tiles) that a workgroup processes in one pass.
//
// Each workgroup runs four streaming waves and one helper wave. The streaming
// waves only stream records and activations: per segment they leave their
// partial sums in LDS (double-buffered) and raise a counter; they never wait
// for the helper's memory round trips. The helper does everything with
// dependent round trips: it adds the partial sums, gathers the per-row scales
// and escape corrections, and finishes segments - whole tiles by storing
// them, split tiles by the exchange below. A workgroup streams its (short)
// split segments first, so their exchange overlaps its whole tiles.
//
// Segment value, per output row and activation row: A = sum of x * w' over the
// segment's columns, where w' is the weight decoded with a fixed exponent
// bias (w = w' 2^(E_n - 127)); CN = sum of x * placeholder and CP = sum of x *
// exact value over the segment's escapes. The value is (A 2^(E_n-127) - CN) + CP.
//
// Split tiles: each workgroup stores its segment value in a fixed slot (2p for
// its first split tile, 2p+1 for its second) and counts itself in the tile's
// counter; the last to arrive adds the slots in workgroup order (so the result
// does not depend on arrival order) and writes the tile. Counters wrap back to
// zero, so every call leaves them zeroed for the next one.
#include "w12_internal.h"

namespace w12 {

constexpr int kUnitCols = 256;
constexpr int kStreamWaves = 4;
constexpr int kThreads = (kStreamWaves + 1) * 64;
constexpr int kSlots = 3;       // segments the helper holds at once

// -------------------------------------------------------------- schedule
// floor(x / y) for x < 2^40, 0 < y < 2^31: the double quotient is within one
// of the exact one, and one integer step corrects it. (Inline 64-bit integer
// division would cost far more code.)
__device__ __forceinline__ uint32_t div_floor(uint64_t x, uint32_t y) {
  uint32_t q = (uint32_t)((double)x / (double)y);
  const uint64_t qy = (uint64_t)q * y;
  if (qy > x) --q;
  else if (qy + y <= x) ++q;
  return q;
}

// First split unit of workgroup q (q in [0, P]).
__device__ __forceinline__ uint32_t sk_start(const GemmParams& a, int q) {
  return (uint32_t)a.sk_base + div_floor((uint64_t)q * (uint64_t)a.sk_units, (uint32_t)a.P);
}

// Workgroup owning split unit u.
__device__ __forceinline__ int sk_owner(const GemmParams& a, uint32_t u) {
  const uint64_t v = u - (uint32_t)a.sk_base;
  return (int)div_floor((v + 1) * (uint64_t)a.P + (uint64_t)a.sk_units - 1, (uint32_t)a.sk_units) - 1;
}

// Workgroup q's slot for split tile t: 2q if t is its first split tile, 2q+1
// if its second; -1 if q owns no split unit.
__device__ __forceinline__ int part_slot(const GemmParams& a, int q, int t) {
  const uint32_t s = sk_start(a, q), e = sk_start(a, q + 1);
  if (s == e) return -1;
  const uint32_t t0 = (uint32_t)t * (uint32_t)a.ku;
  return 2 * q + ((s >= t0 && s < t0 + (uint32_t)a.ku) ? 0 : 1);
}

struct Seg {
  int tile;    // first tile
  int rg;      // tiles (whole-tile groups of the MFMA kernel; 1 otherwise)
  int k0, k1;  // units [k0, k1) of each tile
  int part;    // split tile: 0 or 1 (which of this workgroup's split tiles); -1: whole
};

// The segments of workgroup p: nsk split ones (shorter first), then whole
// tiles in groups of at most rmax.
struct SegList {
  int n, nsk;
  Seg sk0, sk1;
  int dp0, D, rmax;
};

__device__ __forceinline__ SegList seg_list(const GemmParams& a, int p, int rmax) {
  SegList L;
  L.rmax = rmax;
  L.D = a.dp;
  L.dp0 = p * a.dp;
  L.nsk = 0;
  L.sk0 = L.sk1 = Seg{0, 1, 0, 0, 0};
  const uint32_t s0 = sk_start(a, p), s1 = sk_start(a, p + 1);
  if (s1 > s0) {
    const int ta = (int)div_floor(s0, (uint32_t)a.ku), tb = (int)div_floor(s1 - 1, (uint32_t)a.ku);
    const uint32_t ua = (uint32_t)ta * (uint32_t)a.ku, ub = (uint32_t)tb * (uint32_t)a.ku;
    const Seg A{ta, 1, (int)(s0 - ua), ta == tb ? (int)(s1 - ua) : a.ku, 0};
    if (ta == tb) {
      L.nsk = 1;
      L.sk0 = A;
    } else {
      const Seg B{tb, 1, 0, (int)(s1 - ub), 1};
      L.nsk = 2;
      const bool b_first = (B.k1 - B.k0) < (A.k1 - A.k0);
      L.sk0 = b_first ? B : A;
      L.sk1 = b_first ? A : B;
    }
  }
  L.n = L.nsk + (a.dp + rmax - 1) / rmax;
  return L;
}

__device__ __forceinline__ Seg seg_at(const GemmParams& a, const SegList& L, int i) {
  if (i < L.nsk) return i == 0 ? L.sk0 : L.sk1;
  const int j = i - L.nsk;
  return Seg{L.dp0 + j * L.rmax, min(L.rmax, L.D - j * L.rmax), 0, a.ku, -1};
}

// -------------------------------------------------------------- outputs
// Cross-workgroup exchange without an L2 writeback: slot values and keys are
// written and read with agent-scope atomic stores and loads (coherent across
// the XCDs' separate L2 caches); the helper waits until its stores are
// acknowledged before it counts the workgroup in.
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

__device__ __forceinline__ void emit(const GemmParams& a, int n, int m, float v, unsigned long long* kbest) {
  if (a.mode == kModeStore) {
    if (a.y_f32) reinterpret_cast<float*>(a.y)[(int64_t)m * a.ldy + n] = v;
    else reinterpret_cast<uint16_t*>(a.y)[(int64_t)m * a.ldy + n] = f32_to_bf16_rne(v);
  } else {
    atomicMax(&kbest[m], argmax_key(v, (uint32_t)n));
  }
}

// -------------------------------------------------------------- escapes
// The helper gathers a segment's escape corrections in three memory round
// trips whatever the rows' escape counts (up to a few hundred entries): the
// row pointers of the segment's rows; all their entries at once (lane = entry),
// filtered to the segment's columns and appended to a list in LDS; then, with
// lane = activation row, the activations of 32 or 64 listed entries at a time,
// summed per row in column order.
constexpr int kEscLoad = 8;    // entries per lane per load round trip
constexpr int kEscList = 64 * kEscLoad;

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

// ============================================================== helper wave
// Per-segment state the helper keeps in LDS, in slot (segment index % 3):
// the segment's values [m][row] (first the plain sums A, then the finished
// values), its corrections CN and CP, and its rows' scales; plus the work
// list of the corrections.
template <int MM, int ROWS>
struct HelperLds {
  float cv[kSlots][MM][ROWS];
  float cn[kSlots][MM][ROWS];
  float cp[kSlots][MM][ROWS];
  float scale[kSlots][ROWS];
  unsigned long long kbest[MM];
  uint32_t rp[3][ROWS + 1];                   // row pointers of each target's rows
  alignas(16) uint32_t ecol[kEscList];        // listed entries: column,
  uint32_t ebits[kEscList];                   // original BF16 | placeholder << 16,
  uint32_t erow[kEscList];                    // target * 256 + row
  alignas(16) float xs[64][20];  // gathered activations [entry][activation row], rows padded
  float eph[64], eex[64];    // placeholder and exact value of a pass's entries
  int poff[64];              // exchange: slots of a chunk of participants
  uint32_t ready[2];  // streaming waves done with the partial buffer (cumulative)
  uint32_t consumed;  // segments whose partial sums the helper has taken
};

// Handshakes between the streaming waves and the helper through LDS counters
// (no barrier, so neither side waits for the other's memory round trips).
// Every wait ends: the helper waits only for counters the streaming waves
// raise after each segment, and a streaming wave only for the helper to take
// the segment two back, which needs nothing from that wave.
__device__ __forceinline__ void lds_wait_geq(const uint32_t* c, uint32_t v) {
  while (__hip_atomic_load(c, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < v) __builtin_amdgcn_s_sleep(1);
}
__device__ __forceinline__ void lds_add(uint32_t* c) {
  __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_set(uint32_t* c, uint32_t v) {
  __hip_atomic_store(c, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Upper bound of j in the nondecreasing rp[0 .. rows]: the row holding entry j.
__device__ __forceinline__ int rp_row(const uint32_t* rp, int rows, uint32_t j) {
  int lo = 0, hi = rows;  // rp[lo] <= j < rp[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (rp[mid] <= j) lo = mid; else hi = mid;
  }
  return lo;
}

// Add the listed entries [0, n) to the corrections, 64 at a time with
// lane = entry. Entries come sorted by (target, row, column), so each row's
// entries of a pass are a run of lanes: the activations of all entries are
// gathered at once (16 activation rows per round trip) and parked in LDS,
// then the first lane of each run sums the run in column order and adds it
// to the row's LDS sums (a run split across passes adds its parts in order).
template <int MM, int ROWS, bool XT>
__device__ __forceinline__ void esc_list_apply(const GemmParams& a, HelperLds<MM, ROWS>& h, int n, int slot0,
                                               int slot1, int slot2, int lane) {
  // target t's slot is bits 4t .. 4t+3 (arithmetic, not a select, so the
  // slot stays an index into the LDS arrays)
  const uint32_t slots = (uint32_t)slot0 | (uint32_t)slot1 << 4 | (uint32_t)slot2 << 8;
  for (int e0 = 0; e0 < n; e0 += 64) {
    const int ne = min(64, n - e0);
    const bool live = lane < ne;
    const int e = e0 + (live ? lane : 0);
    const uint32_t col = live ? h.ecol[e] : 0u, bits = live ? h.ebits[e] : 0u;
    const uint32_t tr = live ? h.erow[e] : 0xFFFFFFFFu;
    const bool head = live && (lane == 0 || h.erow[e - 1] != tr);
    int len = 0;
    if (head) {
      len = 1;
      while (lane + len < ne && h.erow[e + len] == tr) ++len;
    }
    h.eph[lane] = esc_placeholder(a, bits);
    h.eex[lane] = bf16_to_f32(bits & 0xFFFFu);
    const uint32_t sl = (slots >> (4 * ((tr >> 8) & 3u))) & 15u, r = tr & 255u;
    // XT: the entry's activations for all rows, one line of the transposed copy
    constexpr int XW = XT ? MM / 2 : 1;
    uint32_t xw[XW];
    if constexpr (XT) {
      const uint4* xp = reinterpret_cast<const uint4*>(a.xt + (size_t)col * MM);
#pragma unroll
      for (int i = 0; i < MM / 8; ++i) {
        const uint4 v = xp[i];
        xw[4 * i] = v.x, xw[4 * i + 1] = v.y, xw[4 * i + 2] = v.z, xw[4 * i + 3] = v.w;
      }
    }
#pragma unroll
    for (int m0 = 0; m0 < (XT ? MM : 64); m0 += 16) {
      if (m0 >= a.m) break;
      float xv[16];
      if constexpr (XT) {
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          const uint32_t w = xw[(m0 + j) / 2];
          xv[j] = bf16_to_f32(w & 0xFFFFu);
          xv[j + 1] = bf16_to_f32(w >> 16);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int m = (m0 + j < a.m) ? m0 + j : 0;
          xv[j] = bf16_to_f32(a.x[(int64_t)m * a.ldx + col]);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(&h.xs[lane][4 * q]) =
            make_float4(xv[4 * q], xv[4 * q + 1], xv[4 * q + 2], xv[4 * q + 3]);
      if (head) {
        float sn[16], sp[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) sn[j] = sp[j] = 0.f;
        for (int k = 0; k < len; ++k) {
          const float ph = h.eph[lane + k], ex = h.eex[lane + k];
          float xk[16];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 v = *reinterpret_cast<const float4*>(&h.xs[lane + k][4 * q]);
            xk[4 * q] = v.x, xk[4 * q + 1] = v.y, xk[4 * q + 2] = v.z, xk[4 * q + 3] = v.w;
          }
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            sn[j] = fmaf(xk[j], ph, sn[j]);
            sp[j] = fmaf(xk[j], ex, sp[j]);
          }
        }
        // all reads before any write (the compiler cannot tell the LDS
        // addresses apart and would otherwise wait on each access)
        float on[16], op[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int m = m0 + j < MM ? m0 + j : MM - 1;
          on[j] = h.cn[sl][m][r];
          op[j] = h.cp[sl][m][r];
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (m0 + j < a.m && m0 + j < MM) {
            h.cn[sl][m0 + j][r] = on[j] + sn[j];
            h.cp[sl][m0 + j][r] = op[j] + sp[j];
          }
        }
      }
    }
  }
}

// A correction target: slot, rows row0 + r for r < rows, columns [c0, c1).
struct Tgt {
  int slot, row0, rows;
  uint32_t c0, c1;
};

template <class T>
__device__ __forceinline__ T pick3(int t, T a, T b, T c) { return t == 0 ? a : t == 1 ? b : c; }

// Scales and escape corrections of up to three segments (targets) at once,
// in two steps: corr_rows (row pointers and scales; sums cleared), then
// corr_list (entries, activations, sums).
template <int MM, int ROWS>
__device__ __forceinline__ void corr_rows(const GemmParams& a, HelperLds<MM, ROWS>& h, int nt, Tgt g0t, Tgt g1t,
                                          Tgt g2t, int lane) {
  // row pointers and scales: every load first (clamped indices), one round trip
  uint32_t etv[3], rpv[3], rpe[3];
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const Tgt T = t == 0 ? g0t : t == 1 ? g1t : g2t;
    const int n = T.row0 + lane;
    etv[t] = a.e_top[min(n, a.n - 1)];
    rpv[t] = a.row_ptr[min(n, a.n)];
    rpe[t] = a.row_ptr[min(T.row0 + T.rows, a.n)];
  }
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    const Tgt T = t == 0 ? g0t : t == 1 ? g1t : g2t;
    if (t < nt) {
      if (lane < T.rows && lane < ROWS) {
        h.scale[T.slot][lane] = pow2_scale(etv[t]);
#pragma unroll
        for (int m = 0; m < MM; ++m) h.cn[T.slot][m][lane] = h.cp[T.slot][m][lane] = 0.f;
        h.rp[t][lane] = rpv[t];
      }
      if (lane == 0) h.rp[t][T.rows] = rpe[t];
    }
  }
}

template <int MM, int ROWS, bool XT>
__device__ __forceinline__ void corr_list(const GemmParams& a, HelperLds<MM, ROWS>& h, int t_first, int nt, Tgt g0t,
                                          Tgt g1t, Tgt g2t, int lane) {
  if (!a.fix) return;
  // the targets' entries as one index space [0, J): target t holds
  // [pre_t, pre_t + size_t), its entries [E0_t, E0_t + size_t)
  // (targets before t_first count as empty)
  const uint32_t E00 = __builtin_amdgcn_readfirstlane(h.rp[0][0]);
  const uint32_t E10 = t_first > 0 ? E00 : __builtin_amdgcn_readfirstlane(h.rp[0][g0t.rows]);
  const uint32_t E01 = nt > 1 ? __builtin_amdgcn_readfirstlane(h.rp[1][0]) : 0u;
  const uint32_t E11 = nt > 1 && t_first <= 1 ? __builtin_amdgcn_readfirstlane(h.rp[1][g1t.rows]) : E01;
  const uint32_t E02 = nt > 2 ? __builtin_amdgcn_readfirstlane(h.rp[2][0]) : 0u;
  const uint32_t E12 = nt > 2 ? __builtin_amdgcn_readfirstlane(h.rp[2][g2t.rows]) : E02;
  const uint32_t pre1 = E10 - E00, pre2 = pre1 + (E11 - E01), J = pre2 + (E12 - E02);
  for (uint32_t b0 = 0; b0 < J; b0 += kEscList) {
    uint2 e[kEscLoad];
    uint32_t gj[kEscLoad];
    int tt[kEscLoad];
#pragma unroll
    for (int k = 0; k < kEscLoad; ++k) {
      const uint32_t g = b0 + 64 * k + lane;
      tt[k] = g < pre1 ? 0 : g < pre2 ? 1 : 2;
      gj[k] = g - pick3(tt[k], 0u, pre1, pre2) + pick3(tt[k], E00, E01, E02);
      e[k] = g < J ? a.esc[gj[k]] : make_uint2(0xFFFFFFFFu, 0u);
    }
    int n = 0;
#pragma unroll
    for (int k = 0; k < kEscLoad; ++k) {
      const int t = tt[k];
      const bool in = b0 + 64 * k + lane < J && e[k].x >= pick3(t, g0t.c0, g1t.c0, g2t.c0) &&
                      e[k].x < pick3(t, g0t.c1, g1t.c1, g2t.c1);
      const uint64_t bal = __ballot(in);
      if (in) {
        const int pos = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        const int r = rp_row(h.rp[t], pick3(t, g0t.rows, g1t.rows, g2t.rows), gj[k]);
        h.ecol[pos] = e[k].x;
        h.ebits[pos] = e[k].y;
        h.erow[pos] = (uint32_t)(t * 256 + r);
      }
      n += __popcll(bal);
    }
    esc_list_apply<MM, ROWS, XT>(a, h, n, g0t.slot, g1t.slot, g2t.slot, lane);
  }
}

template <int MM, int ROWS, bool XT>
__device__ __forceinline__ void corrections(const GemmParams& a, HelperLds<MM, ROWS>& h, int nt, Tgt g0t, Tgt g1t,
                                            Tgt g2t, int lane) {
  corr_rows(a, h, nt, g0t, g1t, g2t, lane);
  corr_list<MM, ROWS, XT>(a, h, 0, nt, g0t, g1t, g2t, lane);
}

// Rows of a segment.
__device__ __forceinline__ int seg_rows(const Seg& s, int tile_rows) { return s.rg * tile_rows; }

// value = (A * scale - CN) + CP for every (row, m) of slot sl.
// (Each chunk of 8 is read before it is written: the compiler cannot tell
// the LDS addresses apart and would otherwise wait on every access.)
template <int MM, int ROWS>
__device__ __forceinline__ void apply(const GemmParams& a, HelperLds<MM, ROWS>& h, int sl, int rows, int lane) {
  if (lane < rows && lane < ROWS) {
    const float s = h.scale[sl][lane];
#pragma unroll
    for (int m0 = 0; m0 < MM; m0 += 8) {
      float c[8], cn[8], cp[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int m = m0 + j < MM ? m0 + j : MM - 1;
        c[j] = h.cv[sl][m][lane], cn[j] = h.cn[sl][m][lane], cp[j] = h.cp[sl][m][lane];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (m0 + j < MM && m0 + j < a.m) h.cv[sl][m0 + j][lane] = (c[j] * s - cn[j]) + cp[j];
    }
  }
}

// Whole-tile segment si (slot si % 3): its finished values are written out.
template <int MM, int ROWS, int TR>
__device__ __forceinline__ void emit_whole(const GemmParams& a, HelperLds<MM, ROWS>& h, const SegList& L, int si,
                                           int lane) {
  const Seg s = seg_at(a, L, si);
  const int sl = si % kSlots, rows = seg_rows(s, TR), n0 = s.tile * TR;
  if (lane < rows && lane < ROWS && n0 + lane < a.n) {
#pragma unroll
    for (int m = 0; m < MM; ++m)
      if (m < a.m) emit(a, n0 + lane, m, h.cv[sl][m][lane], h.kbest);
  }
}

// The exchange of one or two of a workgroup's split segments [b0, b1).
// Begin: store this workgroup's segment values in its fixed slots, then count
// it into each tile. End: for the tiles it was last on, add all slots in
// workgroup order and write the tile. In the exchange a lane serves row
// lane % TR and activation rows lane / TR + (64 / TR) j.
struct Xch {
  int n;              // split segments
  int t0, t1;         // their tiles
  int pa0, pa1, pb0, pb1;  // participants of each tile
  uint64_t last;      // bit c: this workgroup finishes tile c
};

template <int MM, int ROWS, int TR>
__device__ __forceinline__ Xch xch_begin(const GemmParams& a, HelperLds<MM, ROWS>& h, const SegList& L, int p,
                                         int b0, int b1, int lane) {
  constexpr int LPR = 64 / TR;
  constexpr int MJ = (MM + LPR - 1) / LPR;
  const int r = lane % TR, mq = lane / TR;
  Xch X{b1 - b0, 0, 0, 0, 0, 0, 0, 0ull};
  uint32_t cnt0 = 0, cnt1 = 0;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c < X.n) {
      const int si = b0 + c, sl = si % kSlots;
      const Seg s = seg_at(a, L, si);
      float* dst = a.part + (int64_t)(2 * p + s.part) * MM * TR;
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        const int m = mq + LPR * j;
        if (m < a.m) store_shared(&dst[m * TR + r], h.cv[sl][m][r]);
      }
      // participants and how many own split units (64 workgroups at a time)
      const uint32_t u_first = (uint32_t)s.tile * (uint32_t)a.ku;
      const int pa = sk_owner(a, u_first), pb = sk_owner(a, u_first + (uint32_t)a.ku - 1);
      uint32_t cnt = 0;
      for (int q0 = pa; q0 <= pb; q0 += 64) {
        const int q = q0 + lane;
        cnt += __popcll(__ballot(q <= pb && part_slot(a, q, s.tile) >= 0));
      }
      if (c == 0) X.t0 = s.tile, X.pa0 = pa, X.pb0 = pb, cnt0 = cnt;
      else X.t1 = s.tile, X.pa1 = pa, X.pb1 = pb, cnt1 = cnt;
    }
  }
  if (X.n == 0) return X;
  __builtin_amdgcn_s_waitcnt(0);  // the slot stores are acknowledged
  // lane c counts this workgroup into split tile c; a workgroup owns the first
  // unit of at most one split tile, so the owner's index names the counter
  bool last = false;
  if (lane < X.n) {
    const uint32_t c = lane == 0 ? cnt0 : cnt1;
    const int pa = lane == 0 ? X.pa0 : X.pa1;
    last = __builtin_amdgcn_atomic_inc32(&a.ctr[pa], c - 1, __ATOMIC_RELAXED, "agent") == c - 1;
  }
  X.last = __ballot(last);
  return X;
}

template <int MM, int ROWS, int TR>
__device__ __forceinline__ void xch_end(const GemmParams& a, HelperLds<MM, ROWS>& h, const Xch& X, int lane) {
  constexpr int LPR = 64 / TR;
  constexpr int MJ = (MM + LPR - 1) / LPR;
  constexpr int QC = MJ <= 4 ? 16 : MJ <= 8 ? 8 : 4;  // slots loaded per round trip
  const int r = lane % TR, mq = lane / TR;
  for (int c = 0; c < X.n; ++c) {
    if (!((X.last >> c) & 1)) continue;
    const int t = c == 0 ? X.t0 : X.t1;
    const int pa = c == 0 ? X.pa0 : X.pa1, pb = c == 0 ? X.pb0 : X.pb1;
    const int n0 = t * TR;
    float v[MJ];
#pragma unroll
    for (int j = 0; j < MJ; ++j) v[j] = 0.f;
    bool started = false;  // adds start from the first slot (keeps the sign of a zero sum)
    for (int q0 = pa; q0 <= pb; q0 += 64) {
      const int nq = min(64, pb - q0 + 1);
      h.poff[lane] = lane < nq ? part_slot(a, q0 + lane, t) : -1;
      for (int i0 = 0; i0 < nq; i0 += QC) {
        float tv[QC][MJ];
        int sl[QC];
#pragma unroll
        for (int u = 0; u < QC; ++u) {
          sl[u] = i0 + u < nq ? h.poff[i0 + u] : -1;
          const int64_t base = (int64_t)max(sl[u], 0) * MM * TR;
#pragma unroll
          for (int j = 0; j < MJ; ++j) {
            const int m = mq + LPR * j;
            tv[u][j] = (sl[u] >= 0 && m < a.m) ? load_shared(&a.part[base + m * TR + r]) : 0.f;
          }
        }
#pragma unroll
        for (int u = 0; u < QC; ++u) {
          if (sl[u] < 0) continue;
#pragma unroll
          for (int j = 0; j < MJ; ++j) v[j] = started ? v[j] + tv[u][j] : tv[u][j];
          started = true;
        }
      }
    }
    if (n0 + r < a.n) {
#pragma unroll
      for (int j = 0; j < MJ; ++j) {
        const int m = mq + LPR * j;
        if (m < a.m) emit(a, n0 + r, m, v[j], h.kbest);
      }
    }
  }
}

// Argmax mode: publish this workgroup's best key per activation row; the last
// workgroup to finish reduces all of them into idx / max.
template <int MM, int ROWS>
__device__ __forceinline__ void finish_argmax(const GemmParams& a, HelperLds<MM, ROWS>& h, int p, int lane) {
  if (lane < a.m) store_shared(&a.keys[(int64_t)p * a.m + lane], h.kbest[lane]);
  __builtin_amdgcn_s_waitcnt(0);
  bool last = false;
  if (lane == 0)
    last = __builtin_amdgcn_atomic_inc32(&a.ctr[kMaxGrid], (uint32_t)a.P - 1, __ATOMIC_RELAXED, "agent") ==
           (uint32_t)a.P - 1;
  if (__ballot(last) == 0) return;
  if (lane < a.m) {
    unsigned long long best = 0ull;
    for (int q = 0; q < a.P; ++q) {
      const unsigned long long k = load_shared(&a.keys[(int64_t)q * a.m + lane]);
      best = k > best ? k : best;
    }
    a.idx[lane] = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
    if (a.maxv) a.maxv[lane] = key_value(best);
  }
}

// Correction target for segment j: its rows and columns.
__device__ __forceinline__ Tgt seg_target(const GemmParams& a, const SegList& L, int j, int tile_rows) {
  const Seg s = seg_at(a, L, j);
  return Tgt{j % kSlots, s.tile * tile_rows, seg_rows(s, tile_rows), (uint32_t)s.k0 * kUnitCols,
             (uint32_t)s.k1 * kUnitCols};
}

// The helper wave. It finishes the segments in stream order (two split
// segments together when the second is short): corrections of the segment,
// take its partial sums as the streaming waves leave them, apply
// (A 2^(E_n-127) - CN) + CP, then write a whole tile or start the exchange of
// a split one; while the exchange's stores and count are in flight it gathers
// the corrections of the next segments (whose slots are free by then).
constexpr int kMergeUnits = 8;  // a split segment this short joins the previous one's exchange

template <int MM, int ROWS, int TR, class Compact>
__device__ __forceinline__ void helper(const GemmParams& a, HelperLds<MM, ROWS>& h, const SegList& L, int p,
                                       int lane, Compact&& compact) {
  constexpr bool XT = TR == 16;  // the MFMA kernel reads the transposed activations
  if (lane < MM) h.kbest[lane] = 0ull;
  const int n = L.n;
  const Tgt z{0, 0, 0, 0, 0};
  int corr_end = 0;  // segments [0, corr_end) have their corrections
  // corrections of segments [corr_end, j1), three at a time
  auto corr_upto = [&](int j1) {
    while (corr_end < j1) {
      const int nt = min(3, j1 - corr_end);
      corrections<MM, ROWS, XT>(a, h, nt, seg_target(a, L, corr_end, TR),
                                nt > 1 ? seg_target(a, L, corr_end + 1, TR) : z,
                                nt > 2 ? seg_target(a, L, corr_end + 2, TR) : z, lane);
      corr_end += nt;
    }
  };
  // the segments finished together from b0: two split ones when the second is short
  auto group_end = [&](int b0) {
    if (b0 + 1 < L.nsk) {
      const Seg s1 = seg_at(a, L, b0 + 1);
      if (s1.k1 - s1.k0 <= kMergeUnits) return b0 + 2;
    }
    return b0 + 1;
  };
  corr_upto(group_end(0));
  for (int b0 = 0; b0 < n;) {
    const bool split = b0 < L.nsk;
    const int b1 = group_end(b0);  // (its corrections were gathered ahead)
    for (int i = b0; i < b1; ++i) {
      lds_wait_geq(&h.ready[i & 1], (uint32_t)kStreamWaves * (uint32_t)(i / 2 + 1));
      compact(i & 1, i % kSlots, seg_at(a, L, i));
      lds_set(&h.consumed, (uint32_t)(i + 1));
      apply(a, h, i % kSlots, seg_rows(seg_at(a, L, i), TR), lane);
    }
    Xch X{0, 0, 0, 0, 0, 0, 0, 0ull};
    if (split) X = xch_begin<MM, ROWS, TR>(a, h, L, p, b0, b1, lane);
    else emit_whole<MM, ROWS, TR>(a, h, L, b0, lane);
    // segments before b1 are done with their slots: those of b1 .. b1 + 2 are
    // free (this also covers the next group)
    corr_upto(min(n, b1 + kSlots));
    if (split) xch_end<MM, ROWS, TR>(a, h, X, lane);
    b0 = b1;
  }
  if (a.mode == kModeArgmax) finish_argmax(a, h, p, lane);
}

// ============================================================== GEMV (M < 16)
// A streaming wave covers 64 rows (lane = row, four 16-row blocks) and one
// 16-column group per step: each lane loads the 16 view bytes and 8 B-plane
// bytes of its own row, rebuilds 16 weights and accumulates M dot products.
// The activations of a step are the same for every lane, so they come
// through scalar loads and feed v_dot2c_f32_bf16 as its SGPR operand; no
// cross-lane reduction is needed. In a unit (16 groups) streaming wave w
// takes groups w, w+4, w+8, w+12.
constexpr int kGemvTileRows = 64;
constexpr int kGemvSteps = 4;  // column groups per wave per unit

template <int M, bool Q>
struct GemvStage {
  uint4 v[kGemvSteps];
  uint2 b[kGemvSteps];
  int g;
};

template <int M>
struct GemvLds {
  float part[2][kStreamWaves][M][kGemvTileRows];  // streaming waves' sums, double-buffered
  HelperLds<M, kGemvTileRows> h;
};

template <int M, bool Q>
__global__ __launch_bounds__(kThreads) void k_gemv(GemmParams a, const uint16_t* __restrict__ x) {
  __shared__ GemvLds<M> sh;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = blockIdx.x;
  const SegList L = seg_list(a, p, 1);
  if (threadIdx.x == 0) sh.h.ready[0] = sh.h.ready[1] = sh.h.consumed = 0;
  __syncthreads();
  if (wave == kStreamWaves) {
    auto compact = [&](int buf, int sl, const Seg&) {
      // all reads before any write (the compiler would wait on each access)
      float t[kStreamWaves][M];
#pragma unroll
      for (int w = 0; w < kStreamWaves; ++w)
#pragma unroll
        for (int m = 0; m < M; ++m) t[w][m] = sh.part[buf][w][m][lane];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float v = t[0][m];
#pragma unroll
        for (int w = 1; w < kStreamWaves; ++w) v += t[w][m];
        sh.h.cv[sl][m][lane] = v;
      }
    };
    helper<M, kGemvTileRows, kGemvTileRows>(a, sh.h, L, p, lane, compact);
    return;
  }
  const uint32_t c3800 = opaque_vgpr(0x38003800u);
  const int64_t ldx = a.ldx;
  for (int i = 0; i < L.n; ++i) {
    const Seg s = seg_at(a, L, i);
    // lane -> row s.tile * 64 + lane; rows past N read block 0 of the tile
    const int row = s.tile * kGemvTileRows + lane;
    const uint8_t* tile_rec = a.rec + (int64_t)s.tile * 4 * a.kb * kRecBytes;
    const uint32_t soff = row < a.n ? (uint32_t)(lane >> 4) * (uint32_t)(a.kb * kRecBytes) : 0u;
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
    pipeline<GemvStage<M, Q>>(s.k0, s.k1, load, compute);
    if (i >= 2) lds_wait_geq(&sh.h.consumed, (uint32_t)(i - 1));
#pragma unroll
    for (int m = 0; m < M; ++m) sh.part[i & 1][wave][m][lane] = acc[m];
    if (lane == 0) lds_add(&sh.h.ready[i & 1]);
  }
}

// ============================================================== MFMA (M >= 16)
// v_mfma_f32_16x16x32_bf16 with A = 16 weight rows x 32 columns decoded in
// registers and B = 32 columns x 16 activation rows loaded straight from
// global memory. A wave's 1 KB view load of one 64-column chunk of a 16-row
// block gives lane l row l%16 and columns 16 (l/16) .. +15: exactly the A
// operands of two MFMAs; the B operands use the same lane -> column map.
// A unit is 4 chunks (256 columns); streaming wave w takes chunk w. Whole
// 16-row tiles are processed RG at a time so one activation load serves RG
// tiles.
constexpr int kMfmaTileRows = 16;

// Tiles per group: 4 up to two m-tiles, 2 beyond (registers and LDS).
template <int MT>
constexpr int kMfmaR = MT <= 2 ? 4 : 2;

template <int MT, int RG, bool Q>
struct MfmaStage {
  uint4 x[MT][2];
  uint4 v[RG];
  uint2 b[RG];
};

template <int MT>
struct MfmaLds {
  alignas(16) float part[2][kStreamWaves][kMfmaR<MT>][MT][4][64];  // C of each tile and m-tile, double-buffered
  HelperLds<MT * 16, kMfmaR<MT> * 16> h;
};

// One segment: RG consecutive 16-row tiles starting at tile s, units [k0, k1).
template <int MT, int RG, bool Q>
__device__ __forceinline__ void mfma_group(const GemmParams& a, int s, int k0, int k1, int wave, int lane,
                                           float (*part)[kMfmaR<MT>][MT][4][64], int seg, const uint32_t* consumed) {
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
  if (seg >= 2) lds_wait_geq(consumed, (uint32_t)(seg - 1));
  // C layout of a 16x16 MFMA: lane l holds rows 4 (l/16) + i, column l % 16.
#pragma unroll
  for (int j = 0; j < RG; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[wave][j][mt][i][lane] = acc[j][mt][i];
}

template <int MT, bool Q>
__global__ __launch_bounds__(kThreads) void k_mfma(GemmParams a) {
  __shared__ MfmaLds<MT> sh;
  constexpr int R = kMfmaR<MT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = blockIdx.x;
  const SegList L = seg_list(a, p, R);
  if (threadIdx.x == 0) sh.h.ready[0] = sh.h.ready[1] = sh.h.consumed = 0;
  __syncthreads();
  if (wave == kStreamWaves) {
    // C of tile j at (row, m): lane (row/4)*16 + m%16, element row%4, m-tile m/16
    auto compact = [&](int buf, int sl, const Seg& s) {
      const int rr = lane;
      if (rr < s.rg * 16) {
        const int j = rr >> 4, row = rr & 15, i = row & 3, lb = (row >> 2) * 16;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          // the four waves' 16 values of this m-tile, all read before any write
          float t[kStreamWaves][16];
#pragma unroll
          for (int w = 0; w < kStreamWaves; ++w)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 v = *reinterpret_cast<const float4*>(&sh.part[buf][w][j][mt][i][lb + 4 * q]);
              t[w][4 * q] = v.x, t[w][4 * q + 1] = v.y, t[w][4 * q + 2] = v.z, t[w][4 * q + 3] = v.w;
            }
#pragma unroll
          for (int mm = 0; mm < 16; ++mm) {
            float v = t[0][mm];
#pragma unroll
            for (int w = 1; w < kStreamWaves; ++w) v += t[w][mm];
            sh.h.cv[sl][mt * 16 + mm][rr] = v;
          }
        }
      }
    };
    helper<MT * 16, R * 16, kMfmaTileRows>(a, sh.h, L, p, lane, compact);
    return;
  }
  for (int i = 0; i < L.n; ++i) {
    const Seg s = seg_at(a, L, i);
    if constexpr (R == 4) {
      switch (s.rg) {
        case 1: mfma_group<MT, 1, Q>(a, s.tile, s.k0, s.k1, wave, lane, sh.part[i & 1], i, &sh.h.consumed); break;
        case 2: mfma_group<MT, 2, Q>(a, s.tile, s.k0, s.k1, wave, lane, sh.part[i & 1], i, &sh.h.consumed); break;
        case 3: mfma_group<MT, 3, Q>(a, s.tile, s.k0, s.k1, wave, lane, sh.part[i & 1], i, &sh.h.consumed); break;
        default: mfma_group<MT, 4, Q>(a, s.tile, s.k0, s.k1, wave, lane, sh.part[i & 1], i, &sh.h.consumed); break;
      }
    } else {
      if (s.rg == 1) mfma_group<MT, 1, Q>(a, s.tile, s.k0, s.k1, wave, lane, sh.part[i & 1], i, &sh.h.consumed);
      else mfma_group<MT, 2, Q>(a, s.tile, s.k0, s.k1, wave, lane, sh.part[i & 1], i, &sh.h.consumed);
    }
    if (lane == 0) lds_add(&sh.h.ready[i & 1]);
  }
}

// ============================================================== activation transpose
// x [M, K] -> xt [K, MM]: 32 columns per workgroup through LDS, read in
// 16-byte pieces along rows of x and written in 16-byte pieces along rows of xt.
__global__ __launch_bounds__(256) void k_xpose(const uint16_t* __restrict__ x, int64_t ldx, int M, int MM,
                                               uint16_t* __restrict__ xt) {
  __shared__ uint16_t t[64][32 + 8];  // [m][column], rows padded to keep 16-byte alignment
  const int c0 = blockIdx.x * 32;
  // MM rows x 4 pieces of 8 columns
  for (int i = threadIdx.x; i < MM * 4; i += 256) {
    const int m = i >> 2, q = i & 3;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (m < M) v = *reinterpret_cast<const uint4*>(x + (int64_t)m * ldx + c0 + 8 * q);
    *reinterpret_cast<uint4*>(&t[m][8 * q]) = v;
  }
  __syncthreads();
  // 32 columns x MM / 8 pieces of 8 activation rows
  const int pr = MM / 8;
  for (int i = threadIdx.x; i < 32 * pr; i += 256) {
    const int c = i / pr, q = i - c * pr;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)t[8 * q + 2 * j][c] | (uint32_t)t[8 * q + 2 * j + 1][c] << 16;
    *reinterpret_cast<uint4*>(xt + (int64_t)(c0 + c) * MM + 8 * q) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t launch_xpose(const uint16_t* x, int64_t ldx, int M, int mm, int K, uint16_t* xt, hipStream_t s) {
  if (mm > 64 || mm % 16 != 0 || M > mm || K % 32 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_xpose, dim3(K / 32), dim3(256), 0, s, x, ldx, M, mm, xt);
  return hipGetLastError();
}

// ============================================================== planning
GemmPlan plan_gemm(int64_t n, int64_t k, int64_t m, int op, int path, int64_t grid_override) {
  GemmPlan pl{};
  pl.mfma = (path == 2) || (path == 0 && m >= 16);
  pl.ku = (int)(k / kUnitCols);
  if (pl.mfma) {
    pl.tile_rows = kMfmaTileRows;
    pl.tiles = (int)(n / kMfmaTileRows);
  } else {
    pl.tile_rows = kGemvTileRows;
    pl.tiles = (int)((n + kGemvTileRows - 1) / kGemvTileRows);
  }
  pl.units = (int64_t)pl.tiles * pl.ku;
  // One workgroup per compute unit: its four streaming waves keep enough
  // loads in flight, and the whole tiles go round-robin over the CUs.
  int64_t P = kNumCU;
  if (grid_override > 0) P = grid_override;
  if (P > kMaxGrid) P = kMaxGrid;
  if (P > pl.units) P = pl.units;
  if (P < 1) P = 1;
  pl.P = (int)P;
  pl.dp = (int)(pl.tiles / P);
  pl.sk_base = (int64_t)P * pl.dp * pl.ku;
  pl.sk_units = pl.units - pl.sk_base;
  const int64_t mm = pl.mfma ? ((m + 15) / 16) * 16 : m;
  pl.ctr_bytes = kCounterBytes;
  pl.part_bytes = (size_t)(2 * P) * (size_t)mm * pl.tile_rows * sizeof(float);
  pl.key_bytes = (op == W12_OP_LMHEAD_ARGMAX) ? (size_t)P * (size_t)m * 8 : 0;
  pl.xt_bytes = pl.mfma ? (size_t)k * (size_t)mm * sizeof(uint16_t) : 0;
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
  p.dp = pl.dp;
  p.sk_base = pl.sk_base;
  p.sk_units = pl.sk_units;
  if (!pl.mfma && p.m > 16) {
    *unsupported = 1;
    return hipSuccess;
  }
  return pl.mfma ? (p.q ? launch_mfma_m<true>(pl, p, s) : launch_mfma_m<false>(pl, p, s))
                 : (p.q ? launch_gemv_m<true>(pl, p, s) : launch_gemv_m<false>(pl, p, s));
}

}  // namespace w12

// W12 skinny GEMM kernels for gfx950: y[M, N] = x[M, K] W^T over W12 records.
//
// SpecPilot (arXiv 2611.02501) section 4.1 and Figure 5b: the kernel decodes
// records in registers so that the weight stream hides the decode, and splits
// the reduction over workgroups in a fixed order (stream-K), so results are
// deterministic. Section 4.3: the Q pass reads only the 8-bit view.
// Appendix E: the LM head in W12, here fused with a per-row argmax.
//
// Work: rows come in 16-row blocks and columns in units of 256. A whole tile
// is GB blocks (64 rows; 32 for the MFMA kernel beyond 32 activation rows).
// With P workgroups (one per compute unit) and T whole tiles, workgroup p owns
// the tiles [p D, (p+1) D), D = T / P. The rows left after the P D tiles are
// cut into split tiles of TB blocks (GB, or a single block when few rows are
// left, so that each split tile has few sharers) and their units are shared
// evenly by all workgroups (stream-K). A segment is the units of one tile that
// a workgroup processes in one pass.
//
// Each workgroup runs four streaming waves and one helper wave. The streaming
// waves only stream records and activations: per segment they leave their
// partial sums in LDS (double-buffered) and raise a counter; they never wait
// for the helper's memory round trips. The helper does everything with
// dependent round trips: it adds the partial sums, gathers the per-row scales
// and escape corrections, and finishes segments - whole tiles by storing
// them, split tiles by the exchange below. A workgroup streams its (short)
// split segments first, so their exchange overlaps its whole tiles. The last
// piece of its work, after the stream, is shared by all five waves.
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

// Split units are numbered from the first split tile: unit u is column unit
// u % ku of split tile u / ku.
// First split unit of workgroup q (q in [0, P]).
__device__ __forceinline__ uint32_t sk_start(const GemmParams& a, int q) {
  return div_floor((uint64_t)q * (uint64_t)a.sk_units, (uint32_t)a.P);
}

// Workgroup owning split unit u.
__device__ __forceinline__ int sk_owner(const GemmParams& a, uint32_t u) {
  return (int)div_floor(((uint64_t)u + 1) * (uint64_t)a.P + (uint64_t)a.sk_units - 1, (uint32_t)a.sk_units) - 1;
}

// Workgroup q's slot for split tile t: 2q if t is its first split tile, 2q+1
// if its second; -1 if q owns no split unit.
__device__ __forceinline__ int part_slot(const GemmParams& a, int q, int t) {
  const uint32_t s = sk_start(a, q), e = sk_start(a, q + 1);
  if (s == e) return -1;
  const uint32_t t0 = (uint32_t)t * (uint32_t)a.ku;
  return 2 * q + ((s >= t0 && s < t0 + (uint32_t)a.ku) ? 0 : 1);
}

// First row of split tile t.
template <int TB>
__device__ __forceinline__ int split_row0(const GemmParams& a, int t) {
  return a.sk_row0 + t * TB * 16;
}

struct Seg {
  int row0;    // first row
  int rg;      // 16-row blocks (fewer than the tile's only at the end of the matrix)
  int k0, k1;  // units [k0, k1)
  int tile;    // split tile index (whole tile: -1)
  int part;    // which of this workgroup's split tiles, 0 or 1 (whole tile: -1)
};

// The segments of workgroup p: nsk split ones (shorter first), then its D
// whole tiles.
struct SegList {
  int n, nsk;
  Seg sk0, sk1;
  int dp0;
};

template <int TB>
__device__ __forceinline__ Seg split_seg(const GemmParams& a, int t, int k0, int k1, int part) {
  const int r0 = split_row0<TB>(a, t);
  return Seg{r0, min(TB, (a.n - r0) >> 4), k0, k1, t, part};
}

template <int TB>
__device__ __forceinline__ SegList seg_list(const GemmParams& a, int p) {
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
__device__ __forceinline__ Seg seg_at(const GemmParams& a, const SegList& L, int i) {
  if (i < L.nsk) return i == 0 ? L.sk0 : L.sk1;
  const int r0 = (L.dp0 + i - L.nsk) * GB * 16;
  return Seg{r0, min(GB, (a.n - r0) >> 4), 0, a.ku, -1, -1};
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

// One lane's outputs: v[j] is activation row m0 + MS j at output column n.
// The bound, address and stride live in vector registers (the helper is short
// of scalar ones; kept there, each store would first reload them), and the
// dtype branch sits outside the per-value loop.
template <int J, int MS>
__device__ __forceinline__ void store_values(const GemmParams& a, int n, int m0, const float (&v)[J]) {
  const int mend = (int)opaque_vgpr((uint32_t)a.m);
  const uint32_t ld = opaque_vgpr((uint32_t)a.ldy);  // ldy < 2^31 (checked by the API)
  const uint64_t step = (uint64_t)ld * (uint64_t)MS;
  const uint64_t off = (uint64_t)ld * (uint64_t)(uint32_t)m0 + (uint64_t)(uint32_t)n;
  if (a.y_f32) {
    float* y = reinterpret_cast<float*>(a.y) + off;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (m0 + MS * j < mend) y[step * j] = v[j];
  } else {
    uint16_t* y = reinterpret_cast<uint16_t*>(a.y) + off;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (m0 + MS * j < mend) y[step * j] = f32_to_bf16_rne(v[j]);
  }
}

__device__ __forceinline__ unsigned long long max_u64(unsigned long long x, unsigned long long y) {
  return x > y ? x : y;
}

// Lane i takes the key of lane (i - CTRL + 0x120) mod 16 of its 16-lane row (row rotate).
template <int CTRL>
__device__ __forceinline__ unsigned long long row_ror_u64(unsigned long long k) {
  const int lo = (int)(uint32_t)k, hi = (int)(uint32_t)(k >> 32);
  const uint32_t l = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, 0xF, 0xF, false);
  const uint32_t h = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, 0xF, 0xF, false);
  return (unsigned long long)h << 32 | l;
}

__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long k, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), l);
  return (unsigned long long)hi << 32 | lo;
}

// Argmax: lane m of the helper keeps kb, the largest key of activation row m
// seen so far. argmax_absorb folds in one key per lane (0: none); each group
// of G lanes (G = 64, 32 or 16) holds keys of one activation row, m0 + g for
// group g. Rotations by 1, 2, 4 and 8 leave every lane of a 16-lane row with
// the row's largest key. All lanes must be active.
template <int G>
__device__ __forceinline__ void argmax_absorb(unsigned long long& kb, unsigned long long key, int m0, int lane) {
  key = max_u64(key, row_ror_u64<0x121>(key));
  key = max_u64(key, row_ror_u64<0x122>(key));
  key = max_u64(key, row_ror_u64<0x124>(key));
  key = max_u64(key, row_ror_u64<0x128>(key));
  const unsigned long long g0 = readlane_u64(key, 0), g1 = readlane_u64(key, 16), g2 = readlane_u64(key, 32),
                           g3 = readlane_u64(key, 48);
  if constexpr (G == 64) {
    if (lane == m0) kb = max_u64(kb, max_u64(max_u64(g0, g1), max_u64(g2, g3)));
  } else if constexpr (G == 32) {
    const int d = lane - m0;
    const unsigned long long g = d == 0 ? max_u64(g0, g1) : max_u64(g2, g3);
    if (d >= 0 && d < 2) kb = max_u64(kb, g);
  } else {
    const int d = lane - m0;
    const unsigned long long g = d == 0 ? g0 : d == 1 ? g1 : d == 2 ? g2 : g3;
    if (d >= 0 && d < 4) kb = max_u64(kb, g);
  }
}

// Each lane: the largest value of its 16-lane row (DPP row rotations). All lanes active.
__device__ __forceinline__ uint32_t row_ror_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x121, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x122, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x124, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x128, 0xF, 0xF, false));
  return v;
}

// -------------------------------------------------------------- escapes
// The helper gathers the escape corrections of up to three segments in three
// memory round trips for up to a few hundred entries: the row pointers of the
// segments' rows; all their entries at once (lane = entry), filtered to the
// segments' columns and appended to a list in LDS; then the activations of the
// listed entries (lane = entry again), whose products are added to the rows'
// sums in column order.
// Entries per lane per load round trip (fewer where registers are scarce,
// beyond 32 activation rows), and the list capacity they fill.
template <int MM>
constexpr int kEscLoad = MM > 32 ? 8 : 16;
constexpr int kEscList = 64 * 16;

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
// Argmax of whole tiles: for up to 16 activation rows each lane
// keeps the largest value of its own rows (the high half of the argmax key, in
// a register) and the row that gave it (in LDS, lbi), updated only on a
// strictly larger value, so among equal values the first row in stream order
// (the lowest) stays; the pairs are folded into kb once at the end. Beyond 16
// activation rows the registers run out (the kernels for 17..32 rows sit at
// the 256-register limit) and each tile is folded at once.
template <int MM>
constexpr int kLaneBest = MM <= 16 ? MM : 0;
template <int MM>
constexpr int kLaneBestN = kLaneBest<MM> > 0 ? kLaneBest<MM> : 1;  // array extent
// Row length (elements) of the escape activation staging area: rows of a
// multiple of 8 activations get 16 bytes of padding, so that 16-byte accesses
// of eight consecutive lanes (one row each) fall in different LDS banks.
template <int MM>
constexpr int kStageRow = MM % 8 == 0 ? MM + 8 : MM;

// Per-segment state the helper keeps in LDS, in slot (segment index % 3):
// the segment's plain sums A [m][row], its corrections CN and CP, and its
// rows' scales; plus the work list of the corrections.
template <int MM, int ROWS>
struct HelperLds {
  float cv[kSlots][MM][ROWS];
  float cn[kSlots][MM][ROWS];
  float cp[kSlots][MM][ROWS];
  float scale[kSlots][ROWS];
  uint32_t rp[3][ROWS + 1];                   // row pointers of each target's rows
  alignas(16) uint32_t ecol[kEscList];        // listed entries: column,
  uint32_t ebits[kEscList];                   // original BF16 | placeholder << 16,
  uint32_t erow[kEscList];                    // target * 256 + row
  int poff[64];              // exchange: slots of a chunk of participants
  uint32_t ready[2];  // streaming waves done with the partial buffer (cumulative)
  uint32_t consumed;  // segments whose partial sums the helper has taken
  // The workgroup's final work, which all five waves share: published (fin = 1)
  // by the helper once it knows it: the outputs of whole segment fin_si (if
  // not -1), and the sums of the fin_n split tiles this workgroup is last on.
  uint32_t fin;
  int fin_si, fin_n, fin_t[2], fin_pa[2], fin_pb[2];
  uint32_t lbi[kLaneBestN<MM>][64];  // argmax: row of each lane's best value per activation row
  // escapes, up to 32 activation rows: a pass's activations [entry][activation row],
  // its run starts and then its entry count
  alignas(16) uint16_t xs[MM <= 32 ? 64 : 1][kStageRow<MM>];
  int rs[MM <= 32 ? 65 : 1];
};

// Handshakes between the streaming waves and the helper through LDS counters
// (no barrier, so neither side waits for the other's memory round trips).
// Every wait ends: the helper waits only for counters the streaming waves
// raise after each segment; a streaming wave waits only for the helper to take
// the segment two back, which needs nothing from that wave, and at the end for
// the helper's notice of the final work, which every path of the helper posts.
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

// Add the listed entries [0, n) to the corrections, 64 at a time. Entries
// come sorted by (target, row, column), so each row's entries of a pass are a
// run of lanes, and every row's sums must grow in column order, one fused
// multiply-add per entry (a run split across passes continues in the next
// pass). Two ways give the same sums bit for bit; each pass takes the cheaper:
// - rounds: lane = entry; in round k the k-th entry of every run adds its
//   products to its row's sums in LDS. L rounds (L: the longest run), each a
//   dependent LDS read-modify-write of 2 MM sums: good for many short runs;
// - runs: the pass's activations are staged in LDS; each run gets G lanes, one
//   per activation row, that walk its entries in order with the sums in
//   registers. ceil(R / (64 / G)) groups of runs (R: the runs), each about
//   L / 8 LDS round trips: good for few long runs (dense escape rows).
// The activations of PB passes' entries are gathered in one round trip and
// stay in registers: from the transposed copy when there is one (XT, one line
// per entry), else from x (one load per activation row).
template <int MM>
constexpr int kRunLanes = MM <= 1 ? 1 : MM <= 2 ? 2 : MM <= 4 ? 4 : MM <= 8 ? 8 : MM <= 16 ? 16 : MM <= 32 ? 32 : 64;

template <int MM, int ROWS, bool XT>
__device__ __forceinline__ void esc_passes(const GemmParams& a, HelperLds<MM, ROWS>& h, int n, int slot0,
                                           int slot1, int slot2, int lane) {
  // target t's slot is bits 4t .. 4t+3 (arithmetic, not a select, so the
  // slot stays an index into the LDS arrays)
  const uint32_t slots = (uint32_t)slot0 | (uint32_t)slot1 << 4 | (uint32_t)slot2 << 8;
  // activation loads per lane and pass; the loads of PB passes go out together
  // (within a register budget of LB loads)
  constexpr int LP = XT ? MM / 8 : MM;
  constexpr int LB = XT ? (MM > 32 ? 8 : 16) : (MM > 32 ? 64 : 2 * MM > 16 ? 2 * MM : 16);
  constexpr int PB = LP >= LB ? 1 : (LB / LP > kEscLoad<MM> ? kEscLoad<MM> : LB / LP);
  constexpr int C = MM < 16 ? MM : 16;  // activation rows per batch of LDS reads
  constexpr int G = kRunLanes<MM>, RPG = 64 / G;
  for (int e00 = 0; e00 < n; e00 += 64 * PB) {
    // XT: the entry's activations for all rows, one line of the transposed
    // copy (rows past M are zero there); otherwise one load per row (rows
    // past M repeat row 0; their sums are never used)
    uint4 xq[PB][XT ? MM / 8 : 1];
    uint16_t xg[PB][XT ? 1 : MM];
#pragma unroll
    for (int pp = 0; pp < PB; ++pp) {
      const int e = e00 + 64 * pp + lane;
      const uint32_t col = e < n ? h.ecol[e] : 0u;
      if constexpr (XT) {
        const uint4* xp = reinterpret_cast<const uint4*>(a.xt + (size_t)col * MM);
#pragma unroll
        for (int i = 0; i < MM / 8; ++i) xq[pp][i] = xp[i];
      } else {
#pragma unroll
        for (int m = 0; m < MM; ++m) xg[pp][m] = a.x[(int64_t)(m < a.m ? m : 0) * a.ldx + col];
      }
    }
#pragma unroll
    for (int pp = 0; pp < PB; ++pp) {
      const int e0 = e00 + 64 * pp;
      if (e0 < n) {
        const int ne = min(64, n - e0);
        const bool live = lane < ne;
        const int e = e0 + (live ? lane : 0);
        const uint32_t tr = live ? h.erow[e] : 0xFFFFFFFFu;
        const uint32_t tp = lane > 0 ? h.erow[max(e - 1, 0)] : 0xFFFFFFFEu;
        const bool head = live && (lane == 0 || tp != tr);
        const uint64_t H = __ballot(head);
        // position in the run: lanes since the closest head at or below this lane
        const uint64_t below = H & (lane == 63 ? ~0ull : (2ull << lane) - 1ull);
        const int pos = below ? lane - (63 - __clzll(below)) : 0;
        // the runs and the longest one (uniform)
        const int R = __popcll(H);
        const uint32_t lmax = row_ror_max_u32(live ? (uint32_t)pos + 1u : 0u);
        const int L = (int)max(max((uint32_t)__builtin_amdgcn_readlane((int)lmax, 0),
                                   (uint32_t)__builtin_amdgcn_readlane((int)lmax, 16)),
                               max((uint32_t)__builtin_amdgcn_readlane((int)lmax, 32),
                                   (uint32_t)__builtin_amdgcn_readlane((int)lmax, 48)));
        // estimated cycles of each way (an LDS round trip ~150 cycles); the
        // runs must win by 4x, as the estimate flatters them on short runs
        // (measured: 1 us per call on a normal matrix at M = 32 with 1x)
        const int cost_rounds = L * (150 + 6 * MM);
        const int cost_runs = ((R + RPG - 1) / RPG) * (((L + 7) >> 3) * 150 + 8 * L) + 4 * MM;
        // (beyond 32 activation rows only the rounds: the kernels have no registers to spare)
        if constexpr (MM <= 32) {
          if (4 * cost_runs < cost_rounds) {
            // runs: stage the activations [entry][activation row] and the run
            // starts, then each run's lanes walk its entries
#pragma unroll
            for (int m0 = 0; m0 < MM; m0 += 8) {
              if constexpr (XT) {
                *reinterpret_cast<uint4*>(&h.xs[lane][m0]) = xq[pp][m0 / 8];
              } else {
#pragma unroll
                for (int m = m0; m < m0 + 8 && m < MM; ++m) h.xs[lane][m] = xg[pp][m];
              }
            }
            if (head) h.rs[__builtin_amdgcn_mbcnt_hi((uint32_t)(H >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)H, 0u))] = lane;
            if (lane == 0) h.rs[R] = ne;
            __builtin_amdgcn_wave_barrier();
            for (int g0 = 0; g0 < R; g0 += RPG) {
              const int j = g0 + lane / G, m = lane % G;
              if (j < R && m < MM) {
                const int q0 = h.rs[j], q1 = h.rs[j + 1];
                const uint32_t row = h.erow[e0 + q0];
                const uint32_t sl = (slots >> (4 * ((row >> 8) & 3u))) & 15u, r = row & 255u;
                float cn = h.cn[sl][m][r], cp = h.cp[sl][m][r];
                for (int q = q0; q < q1; q += 8) {
                  // eight entries' loads first, then their products in order
                  uint32_t bb[8];
                  uint16_t xx[8];
#pragma unroll
                  for (int i = 0; i < 8; ++i) {
                    const int qi = min(q + i, q1 - 1);
                    bb[i] = h.ebits[e0 + qi];
                    xx[i] = h.xs[qi][m];
                  }
#pragma unroll
                  for (int i = 0; i < 8; ++i) {
                    if (q + i < q1) {
                      const float x = bf16_to_f32(xx[i]);
                      cn = fmaf(x, esc_placeholder(a, bb[i]), cn);
                      cp = fmaf(x, bf16_to_f32(bb[i] & 0xFFFFu), cp);
                    }
                  }
                }
                h.cn[sl][m][r] = cn;
                h.cp[sl][m][r] = cp;
              }
            }
            __builtin_amdgcn_wave_barrier();
            continue;
          }
        }
        const uint32_t bits = h.ebits[e];
        const float ph = esc_placeholder(a, bits), ex = bf16_to_f32(bits & 0xFFFFu);
        const uint32_t sl = (slots >> (4 * ((tr >> 8) & 3u))) & 15u, r = live ? tr & 255u : 0u;
        float xv[MM];
#pragma unroll
        for (int m = 0; m < MM; m += 2) {
          if constexpr (XT) {
            const uint4 q = xq[pp][m / 8];
            const int w = (m % 8) / 2;
            const uint32_t u = w == 0 ? q.x : w == 1 ? q.y : w == 2 ? q.z : q.w;
            xv[m] = bf16_to_f32(u & 0xFFFFu);
            xv[m + 1] = bf16_to_f32(u >> 16);
          } else {
            xv[m] = bf16_to_f32(xg[pp][m]);
            if (m + 1 < MM) xv[m + 1] = bf16_to_f32(xg[pp][m + 1 < MM ? m + 1 : m]);
          }
        }
        for (int k = 0; k < L; ++k) {
          if (live && pos == k) {
#pragma unroll
            for (int m0 = 0; m0 < MM; m0 += C) {
              // all reads before any write (the compiler cannot tell the LDS
              // addresses apart and would otherwise wait on each access)
              float on[C], op[C];
#pragma unroll
              for (int j = 0; j < C; ++j) on[j] = h.cn[sl][m0 + j][r], op[j] = h.cp[sl][m0 + j][r];
#pragma unroll
              for (int j = 0; j < C; ++j) {
                h.cn[sl][m0 + j][r] = fmaf(xv[m0 + j], ph, on[j]);
                h.cp[sl][m0 + j][r] = fmaf(xv[m0 + j], ex, op[j]);
              }
            }
          }
        }
      }
    }
  }
}

template <int MM, int ROWS, bool XT>
__device__ __forceinline__ void esc_list_apply(const GemmParams& a, HelperLds<MM, ROWS>& h, int n, int slot0,
                                               int slot1, int slot2, int lane) {
  if (XT && a.xt) esc_passes<MM, ROWS, XT>(a, h, n, slot0, slot1, slot2, lane);
  else esc_passes<MM, ROWS, false>(a, h, n, slot0, slot1, slot2, lane);
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
  constexpr int EL = kEscLoad<MM>;
  for (uint32_t b0 = 0; b0 < J; b0 += 64 * EL) {
    uint2 e[EL];
    uint32_t gj[EL];
    int tt[EL];
#pragma unroll
    for (int k = 0; k < EL; ++k) {
      const uint32_t g = b0 + 64 * k + lane;
      tt[k] = g < pre1 ? 0 : g < pre2 ? 1 : 2;
      gj[k] = g - pick3(tt[k], 0u, pre1, pre2) + pick3(tt[k], E00, E01, E02);
      e[k] = g < J ? a.esc[gj[k]] : make_uint2(0xFFFFFFFFu, 0u);
    }
    int n = 0;
#pragma unroll
    for (int k = 0; k < EL; ++k) {
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

// Finished values (A * scale - CN) + CP of row r, activation rows m0 + MS j,
// from slot sl. All LDS reads come first (the compiler cannot tell the LDS
// addresses apart and would otherwise wait on every access).
template <int J, int MS, int MM, int ROWS>
__device__ __forceinline__ void seg_values(const HelperLds<MM, ROWS>& h, int sl, int r, int m0, float (&v)[J]) {
  const float s = h.scale[sl][r];
  float c[J], cn[J], cp[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int m = m0 + MS * j < MM ? m0 + MS * j : MM - 1;
    c[j] = h.cv[sl][m][r], cn[j] = h.cn[sl][m][r], cp[j] = h.cp[sl][m][r];
  }
#pragma unroll
  for (int j = 0; j < J; ++j) v[j] = (c[j] * s - cn[j]) + cp[j];
}

// The largest key over all 64 lanes (every lane must be active).
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long key) {
  key = max_u64(key, row_ror_u64<0x121>(key));
  key = max_u64(key, row_ror_u64<0x122>(key));
  key = max_u64(key, row_ror_u64<0x124>(key));
  key = max_u64(key, row_ror_u64<0x128>(key));
  return max_u64(max_u64(readlane_u64(key, 0), readlane_u64(key, 16)),
                 max_u64(readlane_u64(key, 32), readlane_u64(key, 48)));
}

// One activation row m of a 64-row tile (lane = row n0 + lane): fold the
// tile's best key into lane m's kb. The value half of the keys is reduced
// first (DPP row maxima, then the four rows); the lowest valid lane holding
// it gives the index half, so ties go to the lowest row. All lanes active.
__device__ __forceinline__ void argmax_tile64(unsigned long long& kb, float v, bool valid, int n0, int m, int lane) {
  const uint32_t hi = valid ? (uint32_t)(argmax_key(v, 0u) >> 32) : 0u;
  const uint32_t rm = row_ror_max_u32(hi);
  const uint32_t mx = max(max((uint32_t)__builtin_amdgcn_readlane((int)rm, 0), (uint32_t)__builtin_amdgcn_readlane((int)rm, 16)),
                          max((uint32_t)__builtin_amdgcn_readlane((int)rm, 32), (uint32_t)__builtin_amdgcn_readlane((int)rm, 48)));
  const uint64_t cand = __ballot(valid && hi == mx);
  if (cand != 0 && lane == m) {
    const uint32_t n = (uint32_t)(n0 + __builtin_ctzll(cand));
    kb = max_u64(kb, (unsigned long long)mx << 32 | (0xFFFFFFFFu - n));
  }
}


// Whole-tile segment si (slot si % 3), lane = row: its outputs or argmax keys.
template <int MM, int ROWS>
__device__ __forceinline__ void emit_whole(const GemmParams& a, HelperLds<MM, ROWS>& h, const SegList& L, int si,
                                           int lane, unsigned long long& kb,
                                           uint32_t (&lbv)[kLaneBestN<MM>]) {
  const Seg s = seg_at<ROWS / 16>(a, L, si);
  const int sl = si % kSlots, n0 = s.row0;
  const bool valid = lane < s.rg * 16 && lane < ROWS;
  const int r = lane < ROWS ? lane : ROWS - 1;
  constexpr int C = MM < 16 ? MM : 16;
  constexpr int LB = kLaneBest<MM>;
  if constexpr (LB > 0) {
    if (a.mode == kModeArgmax) {
      constexpr int CL = LB < C ? LB : C;
#pragma unroll
      for (int m0 = 0; m0 < LB; m0 += CL) {
        float v[CL];
        seg_values<CL, 1>(h, sl, r, m0, v);
#pragma unroll
        for (int j = 0; j < CL; ++j) {
          const uint32_t hv = valid ? (uint32_t)(argmax_key(v[j], 0u) >> 32) : 0u;
          if (hv > lbv[m0 + j]) {
            lbv[m0 + j] = hv;
            h.lbi[m0 + j][lane] = (uint32_t)(n0 + lane);
          }
        }
      }
      if constexpr (LB < MM) {
#pragma unroll 1
        for (int m0 = LB; m0 < MM; m0 += C) {
          if (m0 < a.m) {
            float v[C];
            seg_values<C, 1>(h, sl, r, m0, v);
#pragma unroll
            for (int j = 0; j < C; ++j)
              if (m0 + j < a.m) argmax_tile64(kb, v[j], valid, n0, m0 + j, lane);
          }
        }
      }
      return;
    }
  }
#pragma unroll 1
  for (int m0 = 0; m0 < MM; m0 += C) {
    if (m0 < a.m) {
      float v[C];
      seg_values<C, 1>(h, sl, r, m0, v);
      if (a.mode == kModeStore) {
        if (valid) store_values<C, 1>(a, n0 + lane, m0, v);
      } else {
#pragma unroll
        for (int j = 0; j < C; ++j)
          if (m0 + j < a.m) argmax_tile64(kb, v[j], valid, n0, m0 + j, lane);
      }
    }
  }
}

// The exchange of one or two of a workgroup's split segments [b0, b1).
// Begin: store this workgroup's segment values in its fixed slots, then count
// it into each tile. End: for the tiles it was last on, add all slots in
// workgroup order and write the tile. In the exchange a lane serves row
// lane % TS and activation rows lane / TS + (64 / TS) j (TS: rows of a split
// tile).
struct Xch {
  int n;              // split segments
  int t0, t1;         // their tiles
  int pa0, pa1, pb0, pb1;  // participants of each tile
  uint64_t last;      // bit c: this workgroup finishes tile c
};

template <int MM, int ROWS, int TS>
__device__ __forceinline__ Xch xch_begin(const GemmParams& a, HelperLds<MM, ROWS>& h, const SegList& L, int p,
                                         int b0, int b1, int lane) {
  constexpr int LPR = 64 / TS;
  constexpr int MJ = (MM + LPR - 1) / LPR;
  const int r = lane % TS, mq = lane / TS;
  Xch X{b1 - b0, 0, 0, 0, 0, 0, 0, 0ull};
  uint32_t cnt0 = 0, cnt1 = 0;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c < X.n) {
      const int si = b0 + c, sl = si % kSlots;
      const Seg s = seg_at<ROWS / 16>(a, L, si);
      float* dst = a.part + (int64_t)(2 * p + s.part) * MM * TS;
      constexpr int JC = MJ < 8 ? MJ : 8;  // values per batch of LDS reads
#pragma unroll
      for (int j0 = 0; j0 < MJ; j0 += JC) {
        float v[JC];
        seg_values<JC, LPR>(h, sl, r, mq + LPR * j0, v);
#pragma unroll
        for (int j = 0; j < JC; ++j) {
          const int m = mq + LPR * (j0 + j);
          if (m < a.m) store_shared(&dst[m * TS + r], v[j]);
        }
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

// Finished values of one lane (row n0 + r, activation rows m0 + LPR j): its
// outputs, or its argmax keys.
template <int J, int LPR, int TS>
__device__ __forceinline__ void xch_out(const GemmParams& a, int n0, int r, int m0, const float (&v)[J], int lane,
                                        unsigned long long& kb) {
  if (a.mode == kModeStore) {
    if (n0 + r < a.n) store_values<J, LPR>(a, n0 + r, m0, v);
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const bool ok = n0 + r < a.n && m0 + LPR * j < a.m;
      argmax_absorb<TS>(kb, ok ? argmax_key(v[j], (uint32_t)(n0 + r)) : 0ull, m0 - lane / TS + LPR * j, lane);
    }
  }
}

template <int MM, int ROWS, int TS>
__device__ __forceinline__ void xch_end(const GemmParams& a, HelperLds<MM, ROWS>& h, const Xch& X, int lane,
                                        unsigned long long& kb) {
  constexpr int LPR = 64 / TS;
  constexpr int MJ = (MM + LPR - 1) / LPR;
  constexpr int JC = MJ < 8 ? MJ : 8;       // values per lane per pass
  constexpr int QC = JC <= 4 ? 16 : 8;      // slots loaded per round trip
  constexpr int JP = MJ < 4 ? MJ : 4;       // pipelined passes: values per lane
  constexpr int QP = MM > 32 ? 4 : 8;       // and slots (at most QP sharers)
  const int r = lane % TS, mq = lane / TS;
  for (int c = 0; c < X.n; ++c) {
    if (!((X.last >> c) & 1)) continue;
    const int t = c == 0 ? X.t0 : X.t1;
    const int pa = c == 0 ? X.pa0 : X.pa1, pb = c == 0 ? X.pb0 : X.pb1;
    const int n0 = split_row0<TS / 16>(a, t);
    const int np = pb - pa + 1;  // workgroups that may hold units of the tile
    if (MJ > JP && MM <= 32 && np <= QP) {
      // Few sharers: their slots once, then passes over the activation rows
      // with the next pass's loads in flight while this one is added up.
      h.poff[lane] = lane < np ? part_slot(a, pa + lane, t) : -1;
      int64_t base[QP];
      bool has[QP];  // the workgroup holds units of the tile (the first one always does)
#pragma unroll
      for (int u = 0; u < QP; ++u) {
        const int sl = u < np ? h.poff[u] : -1;
        base[u] = (int64_t)max(sl, 0) * MM * TS;
        has[u] = sl >= 0;
      }
      auto load = [&](float (&tv)[QP][JP], int j0) {
#pragma unroll
        for (int u = 0; u < QP; ++u)
#pragma unroll
          for (int j = 0; j < JP; ++j) {
            const int m = mq + LPR * (j0 + j);
            tv[u][j] = (has[u] && m < a.m) ? load_shared(&a.part[base[u] + m * TS + r]) : 0.f;
          }
      };
      auto finish = [&](const float (&tv)[QP][JP], int j0) {
        float v[JP];
#pragma unroll
        for (int j = 0; j < JP; ++j) v[j] = tv[0][j];
#pragma unroll
        for (int u = 1; u < QP; ++u)
#pragma unroll
          for (int j = 0; j < JP; ++j)
            if (has[u]) v[j] += tv[u][j];
        xch_out<JP, LPR, TS>(a, n0, r, mq + LPR * j0, v, lane, kb);
      };
      const int jend = min(MJ, (a.m + LPR - 1) / LPR);  // passes past M hold nothing
      float ta[QP][JP], tb[QP][JP];
      load(ta, 0);
      for (int j0 = 0; j0 < jend; j0 += 2 * JP) {
        if (j0 + JP < jend) load(tb, j0 + JP);
        finish(ta, j0);
        if (j0 + JP < jend) {
          if (j0 + 2 * JP < jend) load(ta, j0 + 2 * JP);
          finish(tb, j0 + JP);
        }
      }
      continue;
    }
#pragma unroll 1
    for (int j0 = 0; j0 < MJ && LPR * j0 < a.m; j0 += JC) {
      float v[JC];
#pragma unroll
      for (int j = 0; j < JC; ++j) v[j] = 0.f;
      bool started = false;  // adds start from the first slot (keeps the sign of a zero sum)
      for (int q0 = pa; q0 <= pb; q0 += 64) {
        const int nq = min(64, pb - q0 + 1);
        h.poff[lane] = lane < nq ? part_slot(a, q0 + lane, t) : -1;
        for (int i0 = 0; i0 < nq; i0 += QC) {
          float tv[QC][JC];
          int sl[QC];
#pragma unroll
          for (int u = 0; u < QC; ++u) {
            sl[u] = i0 + u < nq ? h.poff[i0 + u] : -1;
            const int64_t base = (int64_t)max(sl[u], 0) * MM * TS;
#pragma unroll
            for (int j = 0; j < JC; ++j) {
              const int m = mq + LPR * (j0 + j);
              tv[u][j] = (sl[u] >= 0 && m < a.m) ? load_shared(&a.part[base + m * TS + r]) : 0.f;
            }
          }
#pragma unroll
          for (int u = 0; u < QC; ++u) {
            if (sl[u] < 0) continue;
#pragma unroll
            for (int j = 0; j < JC; ++j) v[j] = started ? v[j] + tv[u][j] : tv[u][j];
            started = true;
          }
        }
      }
      xch_out<JC, LPR, TS>(a, n0, r, mq + LPR * j0, v, lane, kb);
    }
  }
}

// Argmax mode: publish this workgroup's best key per activation row; the last
// workgroup to finish reduces all of them into idx / max, lane = workgroup
// (64 at a time) and 8 activation rows per round trip.
__device__ __forceinline__ void finish_argmax(const GemmParams& a, int p, int lane, unsigned long long kb) {
  if (lane < a.m) store_shared(&a.keys[(int64_t)p * a.m + lane], kb);
  __builtin_amdgcn_s_waitcnt(0);
  bool last = false;
  if (lane == 0)
    last = __builtin_amdgcn_atomic_inc32(&a.ctr[kMaxGrid], (uint32_t)a.P - 1, __ATOMIC_RELAXED, "agent") ==
           (uint32_t)a.P - 1;
  if (__ballot(last) == 0) return;
  constexpr int MC = 8, QB = 4;
  for (int m0 = 0; m0 < a.m; m0 += MC) {
    unsigned long long best[MC];
#pragma unroll
    for (int j = 0; j < MC; ++j) best[j] = 0ull;
    for (int q0 = 0; q0 < a.P; q0 += 64 * QB) {
      unsigned long long k[MC][QB];
#pragma unroll
      for (int j = 0; j < MC; ++j)
#pragma unroll
        for (int i = 0; i < QB; ++i) {
          const int q = q0 + 64 * i + lane, m = m0 + j;
          k[j][i] = (q < a.P && m < a.m) ? load_shared(&a.keys[(int64_t)q * a.m + m]) : 0ull;
        }
#pragma unroll
      for (int j = 0; j < MC; ++j)
#pragma unroll
        for (int i = 0; i < QB; ++i) best[j] = max_u64(best[j], k[j][i]);
    }
#pragma unroll
    for (int j = 0; j < MC; ++j) {
      const unsigned long long b = wave_max_u64(best[j]);
      if (lane == 0 && m0 + j < a.m) {
        a.idx[m0 + j] = (int32_t)(0xFFFFFFFFu - (uint32_t)(b & 0xFFFFFFFFull));
        if (a.maxv) a.maxv[m0 + j] = key_value(b);
      }
    }
  }
}

// ------------------------------------------------------------ final work
// The last piece of a workgroup's work comes after its stream, when the
// streaming waves are idle: so all five waves share it, worker w taking
// every fifth activation row (store mode; the argmax keys stay with the
// helper, which holds them).
constexpr int kWorkers = kStreamWaves + 1;

// Split tile t, which this workgroup is last on: worker w's share of the sums
// of all sharers' slots, added in workgroup order (the same order as the
// helper alone would use).
template <int MM, int TS>
__device__ __forceinline__ void xch_sum_share(const GemmParams& a, int t, int pa, int pb, int lane, int w) {
  constexpr int LPR = 64 / TS;
  constexpr int MJ = (MM + LPR - 1) / LPR;
  constexpr int J = (MJ + kWorkers - 1) / kWorkers;
  constexpr int QX = 8;  // slots loaded per round trip
  const int r = lane % TS, mq = lane / TS;
  const int n0 = split_row0<TS / 16>(a, t);
  float v[J];
#pragma unroll
  for (int i = 0; i < J; ++i) v[i] = 0.f;
  bool started = false;  // adds start from the first slot (keeps the sign of a zero sum)
  for (int q0 = pa; q0 <= pb; q0 += QX) {
    const int nq = min(QX, pb - q0 + 1);
    const int mine = lane < nq ? part_slot(a, q0 + lane, t) : -1;
    float tv[QX][J];
    bool has[QX];
#pragma unroll
    for (int u = 0; u < QX; ++u) {
      const int sl = u < nq ? __builtin_amdgcn_readlane(mine, u) : -1;
      has[u] = sl >= 0;
      const int64_t base = (int64_t)max(sl, 0) * MM * TS;
#pragma unroll
      for (int i = 0; i < J; ++i) {
        const int m = mq + LPR * (w + kWorkers * i);
        tv[u][i] = (has[u] && m < a.m) ? load_shared(&a.part[base + m * TS + r]) : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < QX; ++u) {
      if (!has[u]) continue;
#pragma unroll
      for (int i = 0; i < J; ++i) v[i] = started ? v[i] + tv[u][i] : tv[u][i];
      started = true;
    }
  }
  if (n0 + r < a.n) store_values<J, LPR * kWorkers>(a, n0 + r, mq + LPR * w, v);
}

// Worker w's share of the final work the helper published.
template <int MM, int ROWS, int TS>
__device__ __forceinline__ void final_share(const GemmParams& a, const HelperLds<MM, ROWS>& h, const SegList& L,
                                            int lane, int w) {
  const int si = __builtin_amdgcn_readfirstlane(h.fin_si);
  if (si >= 0) {
    const Seg s = seg_at<ROWS / 16>(a, L, si);
    constexpr int J = (MM + kWorkers - 1) / kWorkers;
    const int r = lane < ROWS ? lane : ROWS - 1;
    float v[J];
    seg_values<J, kWorkers>(h, si % kSlots, r, w, v);
    if (lane < s.rg * 16 && lane < ROWS) store_values<J, kWorkers>(a, s.row0 + lane, w, v);
  }
  const int nn = __builtin_amdgcn_readfirstlane(h.fin_n);
  for (int c = 0; c < nn; ++c)
    xch_sum_share<MM, TS>(a, __builtin_amdgcn_readfirstlane(h.fin_t[c]), __builtin_amdgcn_readfirstlane(h.fin_pa[c]),
                          __builtin_amdgcn_readfirstlane(h.fin_pb[c]), lane, w);
}

// Correction target for segment j: its rows and columns.
template <int GB>
__device__ __forceinline__ Tgt seg_target(const GemmParams& a, const SegList& L, int j) {
  const Seg s = seg_at<GB>(a, L, j);
  return Tgt{j % kSlots, s.row0, s.rg * 16, (uint32_t)s.k0 * kUnitCols,
             (uint32_t)s.k1 * kUnitCols};
}

// The helper wave. It finishes the segments in stream order (two split
// segments together when the second is short): corrections of the segment,
// take its partial sums as the streaming waves leave them, then write a whole
// tile's values (A 2^(E_n-127) - CN) + CP or start the exchange of a split
// one; while the exchange's stores and count are in flight it gathers the
// corrections of the next segments (whose slots are free by then).
constexpr int kMergeUnits = 8;  // a split segment this short joins the previous one's exchange

template <int MM, int ROWS, int TS, bool XT, class Compact>
__device__ __forceinline__ void helper(const GemmParams& a, HelperLds<MM, ROWS>& h, const SegList& L, int p,
                                       int lane, Compact&& compact) {
  // Instruction issue priority over the streaming waves: the helper's work is
  // a chain of short dependent steps, the streaming waves' is not.
  __builtin_amdgcn_s_setprio(3);
  constexpr int GB = ROWS / 16;  // 16-row blocks of a whole tile
  unsigned long long kb = 0ull;  // argmax: lane m's best key of activation row m
  uint32_t lbv[kLaneBestN<MM>];  // argmax: this lane's best value per activation row (0: none)
#pragma unroll
  for (int m = 0; m < kLaneBestN<MM>; ++m) lbv[m] = 0u;
  const int n = L.n;
  const Tgt z{0, 0, 0, 0, 0};
  int corr_end = 0;  // segments [0, corr_end) have their corrections
  // corrections of segments [corr_end, j1), three at a time
  auto corr_upto = [&](int j1) {
    while (corr_end < j1) {
      const int nt = min(3, j1 - corr_end);
      corrections<MM, ROWS, XT>(a, h, nt, seg_target<GB>(a, L, corr_end),
                                nt > 1 ? seg_target<GB>(a, L, corr_end + 1) : z,
                                nt > 2 ? seg_target<GB>(a, L, corr_end + 2) : z, lane);
      corr_end += nt;
    }
  };
  // the segments finished together from b0: two split ones when the second is short
  auto group_end = [&](int b0) {
    if (b0 + 1 < L.nsk) {
      const Seg s1 = seg_at<GB>(a, L, b0 + 1);
      if (s1.k1 - s1.k0 <= kMergeUnits) return b0 + 2;
    }
    return b0 + 1;
  };
  // the first three segments' corrections in one pass (the round trips cost
  // the same for one target as for three)
  corr_upto(min(n, kSlots));
  // Store mode, when a split tile's sum is a long job (more than 8 values per
  // lane): the sums of the split tiles this workgroup is last on wait for the
  // shared final work (a workgroup has at most two split tiles). Short sums
  // are done at once, hidden behind the stream.
  const bool store = a.mode == kModeStore;
  constexpr bool kDefer = (MM + 64 / TS - 1) / (64 / TS) > 8;
  const bool defer = store && kDefer;
  int npend = 0, pt0 = 0, pa0 = 0, pb0 = 0, pt1 = 0, pa1 = 0, pb1 = 0;
  auto publish = [&](int si) {
    if (lane == 0) {
      h.fin_si = si;
      h.fin_n = npend;
      h.fin_t[0] = pt0, h.fin_pa[0] = pa0, h.fin_pb[0] = pb0;
      h.fin_t[1] = pt1, h.fin_pa[1] = pa1, h.fin_pb[1] = pb1;
    }
    lds_set(&h.fin, 1u);
  };
  for (int b0 = 0; b0 < n;) {
    const bool split = b0 < L.nsk;
    const int b1 = group_end(b0);  // (their corrections were gathered ahead)
    for (int i = b0; i < b1; ++i) {
      lds_wait_geq(&h.ready[i & 1], (uint32_t)kStreamWaves * (uint32_t)(i / 2 + 1));
      compact(i & 1, i % kSlots, seg_at<GB>(a, L, i));
      lds_set(&h.consumed, (uint32_t)(i + 1));
    }
    // the last group of a store-mode call is part of the shared final work
    const bool shared = b1 == n && store;
    Xch X{0, 0, 0, 0, 0, 0, 0, 0ull};
    if (split) X = xch_begin<MM, ROWS, TS>(a, h, L, p, b0, b1, lane);
    else if (!shared) emit_whole<MM, ROWS>(a, h, L, b0, lane, kb, lbv);
    if ((defer || shared) && split) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (c < X.n && ((X.last >> c) & 1)) {
          const int t = c == 0 ? X.t0 : X.t1, qa = c == 0 ? X.pa0 : X.pa1, qb = c == 0 ? X.pb0 : X.pb1;
          if (npend == 0) pt0 = t, pa0 = qa, pb0 = qb;
          else pt1 = t, pa1 = qa, pb1 = qb;
          ++npend;
        }
      }
    }
    if (shared) {
      publish(split ? -1 : b0);
      final_share<MM, ROWS, TS>(a, h, L, lane, kStreamWaves);
      return;
    }
    // segments before b1 are done with their slots: those of b1 .. b1 + 2 are
    // free (this also covers the next group)
    corr_upto(min(n, b1 + kSlots));
    if (split && !defer) xch_end<MM, ROWS, TS>(a, h, X, lane, kb);
    b0 = b1;
  }
  if (a.mode == kModeArgmax) {
    if constexpr (kLaneBest<MM> > 0) {
#pragma unroll
      for (int m = 0; m < kLaneBest<MM>; ++m)
        if (m < a.m) {
          const unsigned long long key =
              lbv[m] ? ((unsigned long long)lbv[m] << 32 | (0xFFFFFFFFu - h.lbi[m][lane])) : 0ull;
          argmax_absorb<64>(kb, key, m, lane);
        }
    }
    finish_argmax(a, p, lane, kb);
  }
  // no segments, or argmax mode: nothing (else) to share
  publish(-1);
}

// ============================================================== GEMV (lane per row; chosen for M <= 2)
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
  if (gated_off(a.gate)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = blockIdx.x;
  const SegList L = seg_list<kGemvTileRows / 16>(a, p);
  if (threadIdx.x == 0) sh.h.ready[0] = sh.h.ready[1] = sh.h.consumed = sh.h.fin = 0;
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
    helper<M, kGemvTileRows, kGemvTileRows, false>(a, sh.h, L, p, lane, compact);
    return;
  }
  const uint32_t c3800 = opaque_vgpr(0x38003800u);
  const int64_t ldx = a.ldx;
  for (int i = 0; i < L.n; ++i) {
    const Seg s = seg_at<kGemvTileRows / 16>(a, L, i);
    // lane -> row s.row0 + lane; rows past N read block 0 of the tile
    const int row = s.row0 + lane;
    const uint8_t* tile_rec = a.rec + (int64_t)(s.row0 >> 4) * a.kb * kRecBytes;
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
        st.v[j] = load_stream16(tile_rec + (sb + (gj & 31) * 256 + voff));
        if (!Q) st.b[j] = load_stream8(tile_rec + (sb + (gj & 31) * 128 + boff));
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
  // the workgroup's final work, shared with the helper
  lds_wait_geq(&sh.h.fin, 1u);
  final_share<M, kGemvTileRows, kGemvTileRows>(a, sh.h, L, lane, wave);
}

// ============================================================== MFMA with helper waves (chosen from M = 3)
// v_mfma_f32_16x16x32_bf16 with A = 16 weight rows x 32 columns decoded in
// registers and B = 32 columns x 16 activation rows loaded straight from
// global memory. A wave's 1 KB view load of one 64-column chunk of a 16-row
// block gives lane l row l%16 and columns 16 (l/16) .. +15: exactly the A
// operands of two MFMAs; the B operands use the same lane -> column map.
// A unit is 4 chunks (256 columns); streaming wave w takes chunk w. A tile is
// up to four 16-row blocks, so one activation load serves all of them.
// 16-row blocks per tile: 4 up to two m-tiles, 2 beyond (registers and LDS).
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
  // up to 16 activation rows: each streaming wave's 64-column chunk of x on
  // its way into operand order, 16-byte slots swizzled by row (see mfma_group)
  alignas(16) uint8_t xs[MT == 1 ? kStreamWaves : 1][MT == 1 ? 16 : 1][MT == 1 ? 128 : 16];
  HelperLds<MT * 16, kMfmaR<MT> * 16> h;
};

// One segment: the RG 16-row blocks starting at block s, units [k0, k1).
template <int MT, int RG, bool Q>
__device__ __forceinline__ void mfma_group(const GemmParams& a, int s, int k0, int k1, int wave, int lane,
                                           float (*part)[kMfmaR<MT>][MT][4][64], int seg, const uint32_t* consumed,
                                           uint8_t* xs) {
  f32x4_t acc[RG][MT];
#pragma unroll
  for (int j = 0; j < RG; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[j][mt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  const uint32_t c3800 = opaque_vgpr(0x38003800u);
  // B operands: for chunk c, MFMA half h and m-tile mt, lane l needs the 8
  // activations of row mt*16 + l%16 at columns 16 (l/16) + 8h + 0..7 of the
  // chunk. From 17 rows on they come from the copy of x in operand order (one
  // contiguous kilobyte per load). Up to 16 rows the wave loads its chunk of
  // row-major x as whole 128-byte lines instead, rows 8h .. 8h + 7 in load h
  // (lane l: row 8h + l/8, bytes 16 (l%8); rows past M read row M - 1, which
  // only feeds outputs that are not stored), and turns it into operand order
  // through its LDS area, where 16-byte slot j of row r sits at slot
  // j ^ ((r / 2) % 8) so that the rows an operand read takes hit different
  // banks. (Beyond one m-tile the kernel's LDS has no room for this, and the
  // round trip in every unit cost more than the copy.)
  const uint8_t* xk = reinterpret_cast<const uint8_t*>(a.xk) + lane * 16;
  uint32_t xo[2] = {0u, 0u}, xs_w[2] = {0u, 0u}, xs_r[2] = {0u, 0u};
  if constexpr (MT == 1) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t rw = 8u * h + (uint32_t)(lane >> 3), rr = (uint32_t)(lane & 15);
      xo[h] = 2u * ((uint32_t)min((int)rw, a.m - 1) * (uint32_t)a.ldx + (uint32_t)((lane & 7) * 8));
      xs_w[h] = rw * 128u + ((((uint32_t)lane & 7u) ^ ((rw >> 1) & 7u)) << 4);
      xs_r[h] = rr * 128u + ((((uint32_t)(lane >> 4) * 2u + h) ^ ((rr >> 1) & 7u)) << 4);
    }
  }
  const char* xrow = reinterpret_cast<const char*>(a.x);
  const uint8_t* blk = a.rec + (int64_t)s * a.kb * kRecBytes;
  const uint32_t blk_stride = (uint32_t)(a.kb * kRecBytes);
  // The wave's chunks: chunk w of every unit, except that wave 0 (which
  // shares its SIMD with the helper wave and streams ~6-8% slower) leaves
  // its chunk of the segment's last d units to waves 1, 2, 3 in turn. Each
  // wave's sums cover whatever columns it takes, and the helper adds the four
  // in a fixed order, so the result stays deterministic.
  const int nu = k1 - k0;
  const int d = (nu + 8) >> 4;
  const int items = wave == 0 ? nu - d : nu + (d > wave - 1 ? (d - wave + 3) / 3 : 0);
  auto chunk_of = [&](int i) {
    return wave == 0 ? 4 * (k0 + i) : (i < nu ? 4 * (k0 + i) + wave : 4 * (k1 - d + (wave - 1) + 3 * (i - nu)));
  };
  auto load = [&](MfmaStage<MT, RG, Q>& st, int i) {
    const int c = chunk_of(i);
    if constexpr (MT == 1) {
#pragma unroll
      for (int h = 0; h < 2; ++h) st.x[0][h] = *reinterpret_cast<const uint4*>(xrow + (xo[h] + (uint32_t)c * 128u));
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        st.x[mt][0] = *reinterpret_cast<const uint4*>(xk + ((size_t)(2 * c) * MT + mt) * 1024);
        st.x[mt][1] = *reinterpret_cast<const uint4*>(xk + ((size_t)(2 * c + 1) * MT + mt) * 1024);
      }
    }
    const uint32_t rec_off = (uint32_t)(c >> 3) * kRecBytes;
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      const uint32_t o = j * blk_stride + rec_off;
      st.v[j] = load_stream16(blk + (o + (c & 7) * 1024 + lane * 16));
      if (!Q) st.b[j] = load_stream8(blk + (o + kViewBytes + (c & 7) * 512 + lane * 8));
    }
  };
  auto compute = [&](const MfmaStage<MT, RG, Q>& st) {
    uint4 xb[MT][2];
    if constexpr (MT == 1) {
      // one wave's LDS accesses complete in order, so the next unit's writes
      // cannot overtake these reads
#pragma unroll
      for (int h = 0; h < 2; ++h) *reinterpret_cast<u32x4_t*>(xs + xs_w[h]) = __builtin_bit_cast(u32x4_t, st.x[0][h]);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int h = 0; h < 2; ++h) xb[0][h] = __builtin_bit_cast(uint4, *reinterpret_cast<const u32x4_t*>(xs + xs_r[h]));
      __builtin_amdgcn_wave_barrier();
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) xb[mt][0] = st.x[mt][0], xb[mt][1] = st.x[mt][1];
    }
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      uint32_t d[8];
      decode16_scaled<Q>(st.v[j], Q ? make_uint2(0, 0) : st.b[j], d, c3800);
      const uint4 a0 = make_uint4(d[0], d[1], d[2], d[3]);
      const uint4 a1 = make_uint4(d[4], d[5], d[6], d[7]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0),
                                                             __builtin_bit_cast(bf16x8_t, xb[mt][0]),
                                                             acc[j][mt], 0, 0, 0);
        acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1),
                                                             __builtin_bit_cast(bf16x8_t, xb[mt][1]),
                                                             acc[j][mt], 0, 0, 0);
      }
    }
  };
  pipeline<MfmaStage<MT, RG, Q>>(0, items, load, compute);
  if (seg >= 2) lds_wait_geq(consumed, (uint32_t)(seg - 1));
  // C layout of a 16x16 MFMA: lane l holds rows 4 (l/16) + i, column l % 16.
#pragma unroll
  for (int j = 0; j < RG; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[wave][j][mt][i][lane] = acc[j][mt][i];
}

// TB: 16-row blocks of a split tile (1 or R).
template <int MT, bool Q, int TB>
__global__ __launch_bounds__(kThreads) void k_mfma(GemmParams a) {
  __shared__ MfmaLds<MT> sh;
  if (gated_off(a.gate)) return;
  constexpr int R = kMfmaR<MT>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = blockIdx.x;
  const SegList L = seg_list<TB>(a, p);
  if (threadIdx.x == 0) sh.h.ready[0] = sh.h.ready[1] = sh.h.consumed = sh.h.fin = 0;
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
    helper<MT * 16, R * 16, TB * 16, true>(a, sh.h, L, p, lane, compact);
    return;
  }
  for (int i = 0; i < L.n; ++i) {
    const Seg s = seg_at<R>(a, L, i);
    const int b = s.row0 >> 4;  // first 16-row block
    if constexpr (R == 4) {
      switch (s.rg) {
        case 1: mfma_group<MT, 1, Q>(a, b, s.k0, s.k1, wave, lane, sh.part[i & 1], i, &sh.h.consumed, &sh.xs[MT == 1 ? wave : 0][0][0]); break;
        case 2: mfma_group<MT, 2, Q>(a, b, s.k0, s.k1, wave, lane, sh.part[i & 1], i, &sh.h.consumed, &sh.xs[MT == 1 ? wave : 0][0][0]); break;
        case 3: mfma_group<MT, 3, Q>(a, b, s.k0, s.k1, wave, lane, sh.part[i & 1], i, &sh.h.consumed, &sh.xs[MT == 1 ? wave : 0][0][0]); break;
        default: mfma_group<MT, 4, Q>(a, b, s.k0, s.k1, wave, lane, sh.part[i & 1], i, &sh.h.consumed, &sh.xs[MT == 1 ? wave : 0][0][0]); break;
      }
    } else {
      if (s.rg == 1) mfma_group<MT, 1, Q>(a, b, s.k0, s.k1, wave, lane, sh.part[i & 1], i, &sh.h.consumed, &sh.xs[MT == 1 ? wave : 0][0][0]);
      else mfma_group<MT, 2, Q>(a, b, s.k0, s.k1, wave, lane, sh.part[i & 1], i, &sh.h.consumed, &sh.xs[MT == 1 ? wave : 0][0][0]);
    }
    if (lane == 0) lds_add(&sh.h.ready[i & 1]);
  }
  // the workgroup's final work, shared with the helper
  lds_wait_geq(&sh.h.fin, 1u);
  final_share<MT * 16, R * 16, TB * 16>(a, sh.h, L, lane, wave);
}

// ============================================================== activation transpose
// x [M, K] -> xt [K, MM] and xk (the MFMA kernel's B operand order): 32
// columns per workgroup through LDS, read in 16-byte pieces along rows of x and
// written in 16-byte pieces.
__global__ __launch_bounds__(256) void k_xpose(const uint16_t* __restrict__ x, int64_t ldx, int M, int MM,
                                               uint16_t* __restrict__ xt, uint16_t* __restrict__ xk,
                                               const uint32_t* __restrict__ gate) {
  __shared__ uint16_t t[64][32 + 8];  // [m][column], rows padded to keep 16-byte alignment
  if (gated_off(gate)) return;
  const int c0 = blockIdx.x * 32;
  // MM rows x 4 pieces of 8 columns
  for (int i = threadIdx.x; i < MM * 4; i += 256) {
    const int m = i >> 2, q = i & 3;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (m < M) v = *reinterpret_cast<const uint4*>(x + (int64_t)m * ldx + c0 + 8 * q);
    *reinterpret_cast<uint4*>(&t[m][8 * q]) = v;
  }
  __syncthreads();
  // xt: 32 columns x MM / 8 pieces of 8 activation rows
  const int pr = MM / 8;
  if (xt) {
    for (int i = threadIdx.x; i < 32 * pr; i += 256) {
      const int c = i / pr, q = i - c * pr;
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)t[8 * q + 2 * j][c] | (uint32_t)t[8 * q + 2 * j + 1][c] << 16;
      *reinterpret_cast<uint4*>(xt + (int64_t)(c0 + c) * MM + 8 * q) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  // xk: MM rows x 4 pieces of 8 columns, each to its operand slot
  if (xk) {
    const int MT = MM / 16;
    for (int i = threadIdx.x; i < MM * 4; i += 256) {
      const int m = i >> 2, col = c0 + 8 * (i & 3);
      const int ch = col >> 6, w = col & 63, q = w >> 4, h = (w >> 3) & 1;
      const int64_t o = ((((int64_t)(2 * ch + h) * MT + (m >> 4)) * 4 + q) * 16 + (m & 15)) * 8;
      *reinterpret_cast<uint4*>(xk + o) = *reinterpret_cast<const uint4*>(&t[m][8 * (i & 3)]);
    }
  }
}

hipError_t launch_xpose(const uint16_t* x, int64_t ldx, int M, int mm, int K, uint16_t* xt, uint16_t* xk,
                        const uint32_t* gate, hipStream_t s) {
  if (mm > 64 || mm % 16 != 0 || M > mm || K % 64 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_xpose, dim3(K / 32), dim3(256), 0, s, x, ldx, M, mm, xt, xk, gate);
  return hipGetLastError();
}

// ============================================================== planning
GemmPlan plan_gemm(int64_t n, int64_t k, int64_t m, int op, int path, int64_t grid_override) {
  GemmPlan pl{};
  // The GEMV kernel takes its activations as scalar operands; past two rows
  // they no longer stay in the scalar cache, and the MFMA kernel (M padded to
  // 16) is faster from M = 3 up (measured over M = 1 .. 16).
  pl.mfma = (path == 2) || (path == 0 && m >= 3);
  pl.ku = (int)(k / kUnitCols);
  const int64_t mt = (m + 15) / 16;
  pl.gb = pl.mfma ? (mt <= 2 ? kMfmaR<1> : kMfmaR<3>) : kGemvTileRows / 16;
  const int64_t nb = n / 16;
  const int64_t tiles = (nb + pl.gb - 1) / pl.gb;
  // One workgroup per compute unit: its four streaming waves keep enough
  // loads in flight, and the whole tiles go round-robin over the CUs.
  int64_t P = kNumCU;
  if (grid_override > 0) {
    P = grid_override;
  } else if (tiles < kNumCU) {
    // Fewer tiles than CUs: every tile is split. Splitting each tile into the
    // same number c of parts (c * tiles workgroups) beats spreading the units
    // over all CUs, where tiles have unequal parts and workgroups two of them
    // (measured on 6144 x 5120, 5120 x 6144 and 5120 x 17408 at M = 1 .. 64).
    const int64_t c = kNumCU / tiles;
    if (c >= 2) {
      P = c * tiles;
    } else {
      // One part per tile (whole tiles, no exchange) leaves kNumCU - tiles
      // CUs idle: worth it while the extra bytes per workgroup stay small
      // against what the exchange of split tiles costs.
      const int64_t tile_bytes = pl.gb * 16 * k * 3 / 2;
      if (tile_bytes * (kNumCU - tiles) <= kWholeTileSlack * kNumCU) P = tiles;
    }
  }
  if (P > kMaxGrid) P = kMaxGrid;
  if (P > tiles * pl.ku) P = tiles * pl.ku;
  if (P < 1) P = 1;
  pl.P = (int)P;
  pl.dp = (int)(tiles / P);
  // Blocks left for the split tiles. When P * dp covers every tile and the
  // last tile is partial (N not a multiple of the tile height), the whole
  // tiles already reach past N: nothing is left (seg_at clips the last tile).
  const int64_t rem = nb - P * pl.dp * pl.gb > 0 ? nb - P * pl.dp * pl.gb : 0;
  // Split tiles are whole-tile sized when many rows are left (a few sharers
  // each) and single blocks when few are: a tile shared by many workgroups
  // would leave its last workgroup many partial sums to read. (The GEMV
  // kernel's lanes are the 64 rows of a tile, so its tiles are always whole.)
  pl.tb = (!pl.mfma || rem >= (P / 4) * pl.gb) ? pl.gb : 1;
  pl.sk_row0 = (int)(P * pl.dp * pl.gb * 16);
  pl.sk_tiles = (int)((rem + pl.tb - 1) / pl.tb);
  pl.sk_units = (int64_t)pl.sk_tiles * pl.ku;
  pl.tile_rows = pl.tb * 16;
  const int64_t mm = pl.mfma ? mt * 16 : m;
  pl.ctr_bytes = kCounterBytes;
  pl.part_bytes = (size_t)(2 * P) * (size_t)mm * pl.tile_rows * sizeof(float);
  pl.key_bytes = (op == W12_OP_LMHEAD_ARGMAX) ? (size_t)P * (size_t)m * 8 : 0;
  pl.xt_bytes = pl.mfma ? (size_t)k * (size_t)mm * sizeof(uint16_t) : 0;
  pl.xk_bytes = pl.xt_bytes;
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
  const bool single = pl.tb == 1;
  switch ((p.m + 15) / 16) {
#define W12_MFMA_CASE(MT)                                                                          \
  case MT:                                                                                         \
    if (single) hipLaunchKernelGGL((k_mfma<MT, Q, 1>), grid, block, 0, s, p);                      \
    else hipLaunchKernelGGL((k_mfma<MT, Q, kMfmaR<MT>>), grid, block, 0, s, p);                     \
    break;
    W12_MFMA_CASE(1) W12_MFMA_CASE(2) W12_MFMA_CASE(3) W12_MFMA_CASE(4)
#undef W12_MFMA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmPlan& pl, GemmParams p, hipStream_t s, int* unsupported) {
  *unsupported = 0;
  p.ku = pl.ku;
  p.P = pl.P;
  p.dp = pl.dp;
  p.sk_row0 = pl.sk_row0;
  p.sk_units = pl.sk_units;
  if (!pl.mfma && p.m > 16) {
    *unsupported = 1;
    return hipSuccess;
  }
  return pl.mfma ? (p.q ? launch_mfma_m<true>(pl, p, s) : launch_mfma_m<false>(pl, p, s))
                 : (p.q ? launch_gemv_m<true>(pl, p, s) : launch_gemv_m<false>(pl, p, s));
}

}  // namespace w12

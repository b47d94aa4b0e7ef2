// Internal definitions shared by the libw12 translation units: format
// constants, the in-register decode of W12 records, and kernel launchers.
//
// Format (SpecPilot, arXiv 2611.02501, section 4.1 and Figure 5; bit and byte
// positions as fixed in include/w12.h): a lane that loads the 16 view bytes of
// one row and 16 consecutive columns (a uint4) and the matching 8 B-plane
// bytes (a uint2) rebuilds all 16 BF16 weights with three VALU operations per
// pair of weights.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "w12.h"

namespace w12 {

constexpr int kRecRows = W12_REC_ROWS;        // 16
constexpr int kRecCols = W12_REC_COLS;        // 512
constexpr int kRecBytes = W12_REC_BYTES;      // 12288
constexpr int kViewBytes = W12_REC_VIEW_BYTES;  // 8192
constexpr int kNumCU = 256;                   // MI355X compute units (sizes the stream-K grid)
constexpr int kMaxGrid = 4096;                // most workgroups a GEMM launch uses
constexpr int64_t kWholeTileSlack = 192 << 10;  // extra bytes per workgroup whole tiles may cost (see plan_gemm)
// Counter words at the start of every GEMM workspace: one per workgroup (the
// split tile whose first unit it owns) plus the argmax completion counter.
// Same size and place for every op and shape, and zero between calls.
constexpr size_t kCounterBytes = W12_WS_COUNTER_BYTES;
// Escape lines per matrix row (escapes x padded activation rows / N) above
// which the MFMA kernel reads escape activations from a transposed copy of x.
constexpr int64_t kXtEscRowLines = 16;
// Layout of the counter region: the GEMM kernels' counters, then the state of
// the two-pass argmax (a line of keys and a line of counters per activation
// row), then the certified head's accumulators. All of it is zero between
// calls, at the same place for every op and M, so one workspace serves any mix.
constexpr size_t kKernelCounterBytes = 16640;
constexpr size_t kArgmaxStateOffset = kKernelCounterBytes;
constexpr size_t kArgmaxStateBytes = 256;  // per activation row, keys and counters each
constexpr size_t kCertZeroOffset = kArgmaxStateOffset + 2 * W12_MAX_M * kArgmaxStateBytes;
static_assert(kKernelCounterBytes >= (kMaxGrid + 1) * sizeof(uint32_t), "counter region too small");

typedef short short2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Record loads: read once per GEMM, so marked non-temporal (streamed through
// the caches with low retention; the activations, read by every workgroup,
// stay cached instead).
__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_stream8(const uint8_t* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}

// v_perm_b32 selectors over {S0 = view dword, S1 = B dword}: the result holds
// two 16-bit halves [B byte | view byte] for weights (t, t+1) of the dword.
constexpr uint32_t kSelPair01 = 0x05010400u;  // bytes B0, V0, B1, V1
constexpr uint32_t kSelPair23 = 0x07030602u;  // bytes B2, V2, B3, V3

// Arithmetic shift right by 4 of both 16-bit halves (v_pk_ashrrev_i16).
// A half [v | b] (view byte v high, B byte b low) becomes
//   bit 15..11 = s, bits 10..7 = off, bits 6..4 = mh, bits 3..0 = high nibble of b.
__device__ __forceinline__ uint32_t pk_ashr4(uint32_t p) {
  short2_t s = __builtin_bit_cast(short2_t, p);
  s = s >> (short2_t){4, 4};
  return __builtin_bit_cast(uint32_t, s);
}

// (mask & a) | (~mask & b): the compiler selects v_bfi_b32. Written in C, not
// inline asm, so the compiler sees a VALU write and keeps the wait states an
// MFMA reading the result needs.
__device__ __forceinline__ uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) {
  return (mask & a) | (~mask & b);
}

// A value held in a VGPR that the compiler may not constant-fold (the empty asm
// emits no instruction). Keeps 0x38003800 out of folding so that bfi below
// stays one v_bfi_b32 (SGPR mask, VGPR constant) instead of an AND and an OR
// with two literals.
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t v) {
  asm("" : "+v"(v));
  return v;
}

// Two weights in the GEMM's scaled domain: the exponent field becomes
// 112 + off (bits 14..11 forced to 0111), so the pair holds w * 2^(127 - E_n)
// exactly; the per-row factor 2^(E_n - 127) is applied to the fp32 sum.
__device__ __forceinline__ uint32_t pair_scaled(uint32_t v, uint32_t b, uint32_t sel, uint32_t c3800) {
  return bfi(0x78007800u, c3800, pk_ashr4(__builtin_amdgcn_perm(v, b, sel)));
}

// Two weights with their true exponent off + E_n - 15 (exact decode).
__device__ __forceinline__ uint32_t pair_exact(uint32_t v, uint32_t b, uint32_t sel, uint32_t bias2) {
  return (pk_ashr4(__builtin_amdgcn_perm(v, b, sel)) & 0x87FF87FFu) + bias2;
}

// B dword layout: byte j holds ml(t=j) in its high nibble and ml(t=j+4) in its
// low nibble, for the 8 weights t = 0..7 the dword covers. Shifting the dword
// left by 4 moves the low nibbles into the high-nibble positions.
// In Q mode b0 = b1 = 0x80808080 and no shift is applied: every ml is 1000.
template <bool kQ>
__device__ __forceinline__ void decode16_scaled(uint4 v, uint2 b, uint32_t* d, uint32_t c3800) {
  const uint32_t b0 = kQ ? 0x80808080u : b.x, b1 = kQ ? 0x80808080u : b.y;
  const uint32_t b0s = kQ ? b0 : (b0 << 4), b1s = kQ ? b1 : (b1 << 4);
  d[0] = pair_scaled(v.x, b0, kSelPair01, c3800);
  d[1] = pair_scaled(v.x, b0, kSelPair23, c3800);
  d[2] = pair_scaled(v.y, b0s, kSelPair01, c3800);
  d[3] = pair_scaled(v.y, b0s, kSelPair23, c3800);
  d[4] = pair_scaled(v.z, b1, kSelPair01, c3800);
  d[5] = pair_scaled(v.z, b1, kSelPair23, c3800);
  d[6] = pair_scaled(v.w, b1s, kSelPair01, c3800);
  d[7] = pair_scaled(v.w, b1s, kSelPair23, c3800);
}

__device__ __forceinline__ void decode16_exact(uint4 v, uint2 b, uint32_t* d, uint32_t bias2) {
  const uint32_t b0s = b.x << 4, b1s = b.y << 4;
  d[0] = pair_exact(v.x, b.x, kSelPair01, bias2);
  d[1] = pair_exact(v.x, b.x, kSelPair23, bias2);
  d[2] = pair_exact(v.y, b0s, kSelPair01, bias2);
  d[3] = pair_exact(v.y, b0s, kSelPair23, bias2);
  d[4] = pair_exact(v.z, b.y, kSelPair01, bias2);
  d[5] = pair_exact(v.z, b.y, kSelPair23, bias2);
  d[6] = pair_exact(v.w, b1s, kSelPair01, bias2);
  d[7] = pair_exact(v.w, b1s, kSelPair23, bias2);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// 2^(E - 127) for E in [1, 254]: an fp32 with exponent field E.
__device__ __forceinline__ float pow2_scale(uint32_t e_top) { return __uint_as_float(e_top << 23); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Order-preserving 64-bit argmax key: a larger value gives a larger key, and
// among equal values the lowest index gives the larger key. -0 counts as +0.
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t n) {
  uint32_t u = __float_as_uint(v + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned long long)(0xFFFFFFFFu - n);
}

__device__ __forceinline__ float key_value(unsigned long long key) {
  uint32_t u = (uint32_t)(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

// Parameters of the GEMM kernels (passed by value).
struct GemmParams {
  const uint8_t* rec;
  const uint8_t* e_top;
  const uint32_t* row_ptr;
  const uint2* esc;          // w12_escape as {col, bits | ph << 16}
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* xt;        // x transposed, [K][16 * ceil(M / 16)], rows past M zero (or null)
  const uint16_t* xk;        // x in MFMA operand order (MFMA kernel), rows past M zero:
                             // [K / 64][2][MT][4][16][8], one kilobyte per chunk, half and m-tile
  void* y;
  int64_t ldy;
  uint32_t* ctr;             // split-tile counters [tiles], then the argmax counter; zero between calls
  float* part;               // partial-sum slots [2P][M][tile_rows]
  unsigned long long* keys;  // per-workgroup argmax keys [P][M]
  int32_t* idx;              // argmax outputs [M]
  float* maxv;               // argmax values [M] (may be null)
  int64_t sk_units;          // units (split tile x 256 columns) of the split (stream-K) tiles
  int sk_row0;               // first row of the split tiles
  int n, k;
  int kb;                    // records per 16-row block (K / 512)
  int ku;                    // units per row of tiles (K / 256)
  int P;                     // workgroups
  int dp;                    // whole tiles per workgroup
  int m;                     // activation rows
  int y_f32;
  int mode;                  // 0 = store Y, 1 = argmax keys
  int fix;                   // apply the escape fix-up
  int q;                     // Q pass (fix-up subtracts the Q view of the placeholder)
  const uint32_t* gate;      // null, or a device word: the kernel does nothing when it reads 0
};

enum { kModeStore = 0, kModeArgmax = 1 };

// A launch-time switch written by an earlier kernel on the same stream: every
// workgroup reads it first and returns at once when it is zero (all of a
// workgroup's threads read the same word, so they leave together, before any
// barrier). Read with an agent-scope load so no stale cached copy is seen.
__device__ __forceinline__ bool gated_off(const uint32_t* gate) {
  return gate != nullptr && __hip_atomic_load(gate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u;
}

// launchers (return a hipError_t)
hipError_t launch_plan(const uint16_t* w, int n, int k, uint8_t* e_top, uint32_t* cnt, hipStream_t s);
hipError_t launch_scan(const uint32_t* cnt, int n, uint32_t* row_ptr, hipStream_t s);
hipError_t launch_pack(const uint16_t* w, int n, int k, const uint8_t* e_top, const uint32_t* row_ptr,
                       uint8_t* rec, w12_escape* esc, uint32_t esc_cap, hipStream_t s);
hipError_t launch_decode(const w12_matrix* m, uint16_t* out, hipStream_t s);
hipError_t launch_validate(const w12_matrix* m, uint32_t* flag, hipStream_t s);

struct GemmPlan {
  bool mfma;
  int P;
  int gb;         // 16-row blocks of a whole tile
  int tb;         // 16-row blocks of a split tile
  int tile_rows;  // rows of a split tile (16 tb)
  int ku;
  int dp;
  int sk_row0;
  int sk_tiles;
  int64_t sk_units;
  size_t ctr_bytes;
  size_t part_bytes;
  size_t key_bytes;
  size_t xt_bytes;
  size_t xk_bytes;
};
GemmPlan plan_gemm(int64_t n, int64_t k, int64_t m, int op, int path, int64_t grid_override);
hipError_t launch_gemm(const GemmPlan& plan, GemmParams p, hipStream_t s, int* unsupported);

// ------------------------------------------------------------------ dense escapes
// The escape fix-up as a kernel of its own after a GEMM run without escape
// work (w12_fixup.hip): y = (a - CN) + CP per output.
struct FixParams {
  const float* a;            // fp32 sums with the placeholders in place [M][N] (row stride N)
  const uint32_t* row_ptr;
  const uint2* esc;
  const uint16_t* xt;        // activations transposed [K][mm], rows past M zero
  void* y;
  int64_t ldy;
  int n, m, mm;
  int y_f32;
  int q;                     // Q pass: the placeholder term uses the placeholder's view
  int slices;                // groups per output row (fix_slices)
};
int fix_slices(int64_t n, int64_t n_esc, int m);
hipError_t launch_fix_dense(const FixParams& p, hipStream_t s);

// ------------------------------------------------------------------ argmax of stored logits
// The LM-head argmax above 16 activation rows: the GEMM stores fp32 logits,
// then this kernel folds each row (w12_argmax.hip). keys and ctr hold one
// 256-byte line per activation row (kArgmaxStateBytes), zero before the call;
// the last workgroup of each row clears its line again.
constexpr int kFusedArgmaxMaxM = 16;  // the fused argmax keeps its per-lane fold up to here
hipError_t launch_rows_argmax(const float* y, int64_t ldy, int n, int M, unsigned long long* keys, uint32_t* ctr,
                              int32_t* idx, float* maxv, const uint32_t* gate, hipStream_t s);

// ------------------------------------------------------------------ certified LM head
// State of the certified head (w12_certify.hip). CertZero accumulates, so it
// lives in the counter region (kCertZeroOffset): zero before a workspace's
// first use and left zero by every call (a row's last rescored pair clears
// its key and done count). CertCall is written by every call before it is
// read.
constexpr int kCertMaxM = 64;
struct CertZero {
  unsigned long long best[kCertMaxM];  // argmax keys of the rescored rows
  uint32_t done[kCertMaxM];            // survivors rescored
};
struct CertCall {
  double xnorm[kCertMaxM];             // ||x_m||_2
  uint32_t count[kCertMaxM];           // surviving rows
  uint32_t flag;                       // any row over the cap: the full head's gate
};
static_assert(kCertZeroOffset + sizeof(CertZero) <= kCounterBytes, "counter region too small");
int cert_chunks(int64_t n);
hipError_t launch_cert_bounds(const w12_matrix* m, float* bounds, hipStream_t s);
hipError_t launch_cert(const w12_matrix* mat, const uint16_t* x, int64_t ldx, int M, const float* lq,
                       const float* bounds, CertZero* z, CertCall* cc, float* ub_chunk, float* lb_chunk,
                       uint32_t* list, int32_t* idx, float* maxv, int32_t* survivors, hipStream_t s);

// ------------------------------------------------------------------ stream kernel
// The MFMA stream kernel (w12_gemm_mx.hip): eight streaming waves per
// workgroup, activations read straight from x, escapes substituted into the
// decoded weights in registers (exact decode), no helper wave and no
// activation pre-pass.
struct MxParams {
  const uint8_t* rec;
  const uint8_t* e_top;
  const uint32_t* row_ptr;
  const uint2* esc;          // w12_escape as {col, bits | ph << 16}
  const uint16_t* x;
  int64_t ldx;
  void* y;
  int64_t ldy;
  uint32_t* ctr;             // split-tile counters [sk_tiles]; zero between calls
  float* part;               // split slots [2P][MM][tile_rows]
  int64_t sk_units;          // units of the split tiles
  int sk_row0;               // first row of the split tiles
  int n, k;
  int kb;                    // records per 16-row block: K / 512
  int ku;                    // stream-K units per 16-row block: K / unit width
  int P;                     // workgroups
  int dp;                    // whole tiles per workgroup
  int m;                     // activation rows
  int y_f32;
  int fix;                   // substitute the exact escape values
  int q;                     // Q pass: dropped mantissa bits at their midpoint
};

struct MxPlan {
  int P;
  int gb;         // 16-row blocks of a whole tile
  int tb;         // 16-row blocks of a split tile
  int dp;
  int sk_row0;
  int sk_tiles;
  int64_t sk_units;
  size_t part_bytes;
  int threads;    // threads per workgroup
  int unit_cols;  // columns of a stream-K unit
};
// Largest K the stream kernel takes (its per-segment unit count fits the
// escape bucket arithmetic); larger K runs the helper-wave kernel.
constexpr int64_t kMxMaxK = (int64_t)1 << 20;
MxPlan plan_mx(int64_t n, int64_t k, int64_t m, int64_t grid_override);
hipError_t launch_mx(const MxPlan& plan, MxParams p, hipStream_t s);
// x [M, K] (row stride ldx) -> xt [K, mm] (mm = 16 * ceil(M / 16)) and xk (MFMA operand order), rows
// past M zero; either output may be null.
hipError_t launch_xpose(const uint16_t* x, int64_t ldx, int M, int mm, int K, uint16_t* xt, uint16_t* xk,
                        const uint32_t* gate,
                        hipStream_t s);

}  // namespace w12

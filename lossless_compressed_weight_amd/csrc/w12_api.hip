// C ABI of libw12 (declared in include/w12.h): argument checks, workspace
// sizing and dispatch to the gfx950 kernels. Every check runs before any HIP
// call, so invalid arguments never launch anything.
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "w12_internal.h"

using namespace w12;

// The workspace of w12_gemm_noalloc: counter words and partial sums in a
// file-scope device array instead of caller memory. Every device the library
// runs on holds its own copy until the process ends. In host code the array's
// name is no device address: host code uses only the address
// hipGetSymbolAddress returns for the current device, kept per device.
static __device__ __align__(256) uint8_t scratch[W12_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;
// Test hooks (w12_set_tuning): per thread, so that a test forcing a kernel
// or a grid never changes what another thread's calls compute.
thread_local int g_tune_path = 0;
thread_local int64_t g_tune_grid = 0;

// The stream kernel takes matrices whose escapes are sparse enough for its
// per-wave substitution lists: at most this many escapes per row on average
// (the synthetic workloads have about 1.4; the escape-stress workload 56).
constexpr int64_t kMxMaxEscPerRow = 8;

int hip_fail(hipError_t e, const char* where) {
  g_last_error = std::string(where) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
  return W12_E_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// N % 16, K % 512, sizes that fit the kernels' 32-bit indices.
int check_shape(int64_t n, int64_t k) {
  if (n <= 0 || k <= 0 || n % W12_REC_ROWS != 0 || k % W12_REC_COLS != 0) return W12_E_UNSUPPORTED_SHAPE;
  if (n > (int64_t)1 << 28 || k > (int64_t)1 << 23 || n * k > (int64_t)0xFFFFFFFFll) return W12_E_UNSUPPORTED_SHAPE;
  return W12_OK;
}

int check_matrix(const w12_matrix* m) {
  if (!m) return W12_E_INVALID_ARG;
  if (m->format_version != W12_FORMAT_VERSION) return W12_E_VERSION;
  const int s = check_shape(m->n, m->k);
  if (s != W12_OK) return s;
  if (!m->records || !m->e_top || !m->esc_row_ptr || m->n_esc < 0) return W12_E_INVALID_ARG;
  if (m->n_esc > 0 && !m->esc) return W12_E_INVALID_ARG;
  if (m->n_esc > m->n * m->k) return W12_E_INVALID_ARG;
  if (!aligned16(m->records)) return W12_E_INVALID_ARG;
  return W12_OK;
}

int check_gemm_args(const w12_matrix* m, const void* x, int64_t M, int64_t ldx, const void* y, int64_t ldy,
                    int y_dtype) {
  int s = check_matrix(m);
  if (s != W12_OK) return s;
  if (M < 1 || M > W12_MAX_M) return W12_E_M_RANGE;
  if (!x || !y) return W12_E_INVALID_ARG;
  if (ldx < m->k || ldx % 8 != 0 || ldx > ((int64_t)1 << 25) || !aligned16(x)) return W12_E_INVALID_ARG;
  if (ldy < m->n || ldy > INT32_MAX) return W12_E_INVALID_ARG;
  if (y_dtype != W12_BF16 && y_dtype != W12_F32) return W12_E_INVALID_ARG;
  return W12_OK;
}

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// workspace of the helper-wave kernels: [counters | partial slots | argmax
// keys | transposed x | x in MFMA operand order], each 256-byte aligned
size_t gemm_ws_bytes(const GemmPlan& pl) {
  return round256(pl.ctr_bytes) + round256(pl.part_bytes) + round256(pl.key_bytes) + round256(pl.xt_bytes) +
         round256(pl.xk_bytes);
}

// workspace of the stream kernel: [counters | partial slots]
size_t mx_ws_bytes(const MxPlan& pl) { return round256(kCounterBytes) + round256(pl.part_bytes); }

GemmPlan make_plan(int64_t n, int64_t k, int64_t M, int op) {
  return plan_gemm(n, k, M, op, g_tune_path == 3 ? 2 : (g_tune_path == 4 ? 0 : g_tune_path), g_tune_grid);
}

// Matrices with more escapes than this per row on average (the escape-stress
// workload has about 55, the normal ones about 1.4) take the dense path: the
// GEMM without escape work, then the fix-up kernel (w12_fixup.hip) with every
// lane busy, instead of the per-segment fix-up on one helper wave per CU.
constexpr int64_t kDenseEscPerRow = 8;

bool dense_path(const w12_matrix* m, int op, bool fix) {
  if (!fix || op == W12_OP_LMHEAD_ARGMAX || m->n_esc == 0) return false;
  if (g_tune_path == 4) return true;
  return g_tune_path == 0 && m->n_esc > kDenseEscPerRow * m->n;
}

// The kernel a call runs: the lane-per-row GEMV for M <= 2; from M = 3 an
// MFMA kernel. The stream kernel takes matrices with fewer 64-row tiles than
// compute units (every tile shared by several workgroups) up to 32 activation
// rows, where its direct escape substitution and absent pre-pass pay; the
// helper-wave kernel takes the rest (whole tiles per workgroup, whose escape
// work and exchanges its helper wave overlaps with the stream), the fused
// argmax, dense escapes and very long rows. Measured per call on MI355X at
// M = 32: 6144 x 5120 19.6 vs 24.2 us, 5120 x 6144 19.2 vs 23.6,
// 5120 x 17408 35.6 vs 37.7, 17408 x 5120 35.8 vs 32.4 (stream vs helper);
// the same order at M = 24, 48 and 64.
// The copies of x that one activation transpose kernel writes before the
// helper-wave MFMA kernel: beyond 16 activation rows its B operands in operand
// order (xk; up to 16 rows the kernel stages x through LDS itself), and, with
// many escapes per row, the activations of each escape column (xT: one cache
// line per escape instead of one per activation row). Up to 16 rows the
// escapes' activations are gathered from x unless a workgroup has more than
// kGatherEscPerWg of them (measured at M = 16: the 151936-row LM head, ~830
// per workgroup, 6% slower gathering; 17408x5120, ~93, 2% faster with no
// pre-pass at all, 8% at M = 3..8).
constexpr int64_t kGatherEscPerWg = 256;
struct XCopies {
  bool xt, xk;
};
XCopies x_copies(const w12_matrix* m, const GemmPlan& pl, int64_t M, bool fix) {
  XCopies c{false, false};
  if (!pl.mfma) return c;
  const int64_t mm = ((M + 15) / 16) * 16;
  c.xk = M > 16;
  const bool many = fix && m->n_esc > 0 && m->n_esc * mm > kXtEscRowLines * m->n;
  c.xt = many && (c.xk || m->n_esc > kGatherEscPerWg * (int64_t)pl.P);
  return c;
}

int choose_kernel(int64_t n, int64_t k, int64_t n_esc, int64_t M, int op, bool fix, const GemmPlan& old) {
  const bool mx_ok = op != W12_OP_LMHEAD_ARGMAX && k <= kMxMaxK;
  if (g_tune_path == 4) fix = false;  // the dense path runs its GEMM without escape work
  if (g_tune_path == 1) return W12_KERNEL_GEMV;
  if (g_tune_path == 2) return W12_KERNEL_MFMA_HELPER;
  if (g_tune_path == 3) return mx_ok ? W12_KERNEL_MFMA_STREAM : W12_KERNEL_MFMA_HELPER;
  if (!old.mfma) return W12_KERNEL_GEMV;
  const int64_t tiles = (n / 16 + 3) / 4;  // 64-row tiles
  // Up to 16 activation rows the helper-wave kernel runs without a pre-pass
  // and is the faster one on long rows and on matrices of few tiles
  // (measured at M = 8: 5120x17408 29.1 against 31.4 us, 1024x5120 12.8
  // against 14.3; 6144x5120, 5120x6144 and 8192x5120 within 1 us either way).
  const bool stream_rows = M > 16 || (tiles >= 32 && k <= 8192);
  if (mx_ok && tiles < kNumCU && stream_rows && (!fix || n_esc <= kMxMaxEscPerRow * n)) return W12_KERNEL_MFMA_STREAM;
  return W12_KERNEL_MFMA_HELPER;
}

size_t ws_bytes_any(int64_t n, int64_t k, int64_t M, int op);

// Workspace of the certified head: [GEMM region shared by the Q pass and the
// gated full head | CertCall | Q logits [M][N] | chunk upper and lower bounds [2][M][chunks] | lists];
// CertZero sits in the counter region at the start of the GEMM region.
struct CertLayout {
  size_t gemm, state, logits, ub, list, total;
};
CertLayout cert_layout(int64_t n, int64_t k, int64_t M) {
  CertLayout c{};
  const size_t g = std::max(ws_bytes_any(n, k, M, W12_OP_GEMM_Q8), ws_bytes_any(n, k, M, W12_OP_LMHEAD_ARGMAX));
  c.gemm = round256(g);
  c.state = c.gemm;
  c.logits = c.state + round256(sizeof(CertCall));
  c.ub = c.logits + round256((size_t)M * (size_t)n * sizeof(float));
  c.list = c.ub + round256(2 * (size_t)M * (size_t)cert_chunks(n) * sizeof(float));
  c.total = c.list + round256((size_t)M * W12_CERT_MAX_SURVIVORS * sizeof(uint32_t));
  return c;
}

// Every GEMM kernel plan for this shape fits in this much workspace.
size_t ws_bytes_kernels(int64_t n, int64_t k, int64_t M, int op) {
  size_t b = gemm_ws_bytes(make_plan(n, k, M, op));
  if (op != W12_OP_LMHEAD_ARGMAX && k <= kMxMaxK) {
    const size_t bx = mx_ws_bytes(plan_mx(n, k, M, g_tune_grid));
    if (bx > b) b = bx;
  }
  return b;
}

// The dense path's workspace: [kernel plans | fp32 sums [M][N] | xT [K][mm]].
struct DenseLayout {
  size_t main, a, xt, total;
};
DenseLayout dense_layout(int64_t n, int64_t k, int64_t M, int op) {
  DenseLayout d{};
  d.main = round256(ws_bytes_kernels(n, k, M, op));
  d.a = d.main;
  d.xt = d.a + round256((size_t)M * (size_t)n * sizeof(float));
  d.total = d.xt + round256((size_t)k * (size_t)(((M + 15) / 16) * 16) * sizeof(uint16_t));
  return d;
}

// The two-pass argmax's workspace: [kernel plans of both ops | fp32 logits [M][N]]; its keys and
// counters are in the counter region (kArgmaxStateOffset).
struct ArgmaxLayout {
  size_t main, logits, total;
};
ArgmaxLayout argmax_layout(int64_t n, int64_t k, int64_t M) {
  ArgmaxLayout L{};
  L.main = round256(std::max(ws_bytes_kernels(n, k, M, W12_OP_GEMM), ws_bytes_kernels(n, k, M, W12_OP_LMHEAD_ARGMAX)));
  L.logits = L.main;
  L.total = L.logits + round256((size_t)M * (size_t)n * sizeof(float));
  return L;
}

// Every path a GEMM op may take for this shape fits in this much workspace.
size_t ws_bytes_any(int64_t n, int64_t k, int64_t M, int op) {
  if (op == W12_OP_LMHEAD_ARGMAX)
    return M > kFusedArgmaxMaxM ? argmax_layout(n, k, M).total : ws_bytes_kernels(n, k, M, op);
  return dense_layout(n, k, M, op).total;
}

int run_mx(const w12_matrix* m, const uint16_t* x, int64_t M, int64_t ldx, void* y, int64_t ldy, int y_dtype,
           int op, bool fix, void* ws, size_t ws_bytes, void* stream) {
  const MxPlan pl = plan_mx(m->n, m->k, M, g_tune_grid);
  const size_t need = mx_ws_bytes(pl);
  if (!ws || ws_bytes < need) return W12_E_WORKSPACE;
  MxParams p{};
  p.rec = m->records;
  p.e_top = m->e_top;
  p.row_ptr = m->esc_row_ptr;
  p.esc = reinterpret_cast<const uint2*>(m->esc);
  p.x = x;
  p.ldx = ldx;
  p.y = y;
  p.ldy = ldy;
  char* wsb = reinterpret_cast<char*>(ws);
  p.ctr = reinterpret_cast<uint32_t*>(wsb);
  p.part = reinterpret_cast<float*>(wsb + round256(kCounterBytes));
  p.n = (int)m->n;
  p.k = (int)m->k;
  p.kb = (int)(m->k / W12_REC_COLS);
  p.m = (int)M;
  p.y_f32 = y_dtype == W12_F32;
  p.fix = fix && m->n_esc > 0;
  p.q = op == W12_OP_GEMM_Q8;
  const hipError_t e = launch_mx(pl, p, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  return W12_OK;
}

int run_gemm(const w12_matrix* m, const uint16_t* x, int64_t M, int64_t ldx, void* y, int64_t ldy, int y_dtype,
             int op, bool fix, void* ws, size_t ws_bytes, int32_t* idx, float* maxv, void* stream,
             const uint32_t* gate = nullptr, int force_kernel = 0, uint16_t* dense_xt = nullptr);

// Dense escapes: activations transposed for the fix-up, the GEMM without escape
// work into fp32 sums, then the fix-up kernel writes y.
int run_dense(const w12_matrix* m, const uint16_t* x, int64_t M, int64_t ldx, void* y, int64_t ldy, int y_dtype,
              int op, void* ws, size_t ws_bytes, void* stream) {
  const DenseLayout d = dense_layout(m->n, m->k, M, op);
  if (!ws || ws_bytes < d.total) return W12_E_WORKSPACE;
  char* wsb = reinterpret_cast<char*>(ws);
  float* a = reinterpret_cast<float*>(wsb + d.a);
  uint16_t* xt = reinterpret_cast<uint16_t*>(wsb + d.xt);
  const int mm = (int)(((M + 15) / 16) * 16);
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // the GEMM call also writes xT, in the same launch as its own copies of x
  const int r = run_gemm(m, x, M, ldx, a, m->n, W12_F32, op, false, ws, d.main, nullptr, nullptr, stream, nullptr, 0, xt);
  if (r != W12_OK) return r;
  FixParams p{};
  p.a = a;
  p.row_ptr = m->esc_row_ptr;
  p.esc = reinterpret_cast<const uint2*>(m->esc);
  p.xt = xt;
  p.y = y;
  p.ldy = ldy;
  p.n = (int)m->n;
  p.m = (int)M;
  p.mm = mm;
  p.y_f32 = y_dtype == W12_F32;
  p.q = op == W12_OP_GEMM_Q8;
  p.slices = fix_slices(m->n, m->n_esc, (int)M);
  const hipError_t e = launch_fix_dense(p, st);
  if (e != hipSuccess) return hip_fail(e, "dense escapes: fix-up launch");
  return W12_OK;
}

// The LM-head argmax above 16 activation rows, in two passes: the helper-wave
// kernel stores the fp32 logits (the same kernel and summation order as the
// fused argmax, so the same values), then k_rows_argmax folds each row.
int run_argmax_two_pass(const w12_matrix* m, const uint16_t* x, int64_t M, int64_t ldx, bool fix, void* ws,
                        size_t ws_bytes, int32_t* idx, float* maxv, void* stream, const uint32_t* gate) {
  const ArgmaxLayout L = argmax_layout(m->n, m->k, M);
  if (!ws || ws_bytes < L.total) return W12_E_WORKSPACE;
  char* wsb = reinterpret_cast<char*>(ws);
  float* logits = reinterpret_cast<float*>(wsb + L.logits);
  const int r = run_gemm(m, x, M, ldx, logits, m->n, W12_F32, W12_OP_GEMM, fix, ws, L.main, nullptr, nullptr, stream,
                         gate, W12_KERNEL_MFMA_HELPER);
  if (r != W12_OK) return r;
  const hipError_t e = launch_rows_argmax(logits, m->n, (int)m->n, (int)M,
                                          reinterpret_cast<unsigned long long*>(wsb + kArgmaxStateOffset),
                                          reinterpret_cast<uint32_t*>(wsb + kArgmaxStateOffset +
                                                                      W12_MAX_M * kArgmaxStateBytes),
                                          idx, maxv, gate,
                                          reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "argmax of the stored logits: launch");
  return W12_OK;
}

// gate: null, or a device word that a kernel on the stream writes before this
// call's kernels run; they do nothing when it is zero (helper-wave kernels only).
// force_kernel: 0, or the kernel to run whatever the usual choice.
int run_gemm(const w12_matrix* m, const uint16_t* x, int64_t M, int64_t ldx, void* y, int64_t ldy, int y_dtype,
             int op, bool fix, void* ws, size_t ws_bytes, int32_t* idx, float* maxv, void* stream,
             const uint32_t* gate, int force_kernel, uint16_t* dense_xt) {
  // dense_xt: the dense path's transposed copy of x ([K][mm], rows past M
  // zero), written by this call's activation pre-pass (a launch of its own
  // before the stream kernel, which has none)
  if (op == W12_OP_LMHEAD_ARGMAX && M > kFusedArgmaxMaxM)
    return run_argmax_two_pass(m, x, M, ldx, fix, ws, ws_bytes, idx, maxv, stream, gate);
  if (!gate && !force_kernel && dense_path(m, op, fix))
    return run_dense(m, x, M, ldx, y, ldy, y_dtype, op, ws, ws_bytes, stream);
  const GemmPlan pl = make_plan(m->n, m->k, M, op);
  const int kernel = force_kernel ? force_kernel
                     : gate     ? (pl.mfma ? W12_KERNEL_MFMA_HELPER : W12_KERNEL_GEMV)
                                : choose_kernel(m->n, m->k, m->n_esc, M, op, fix, pl);
  if (kernel == W12_KERNEL_MFMA_STREAM) {
    if (dense_xt) {
      const hipError_t ex = launch_xpose(x, ldx, (int)M, (int)(((M + 15) / 16) * 16), (int)m->k, dense_xt, nullptr,
                                         nullptr, reinterpret_cast<hipStream_t>(stream));
      if (ex != hipSuccess) return hip_fail(ex, "dense escapes: activation transpose launch");
    }
    return run_mx(m, x, M, ldx, y, ldy, y_dtype, op, fix, ws, ws_bytes, stream);
  }
  if (!pl.mfma && M > 16) return W12_E_M_RANGE;
  const size_t need = gemm_ws_bytes(pl);
  if (need > 0 && (!ws || ws_bytes < need)) return W12_E_WORKSPACE;
  GemmParams p{};
  p.rec = m->records;
  p.e_top = m->e_top;
  p.row_ptr = m->esc_row_ptr;
  p.esc = reinterpret_cast<const uint2*>(m->esc);
  p.x = x;
  p.ldx = ldx;
  p.y = y;
  p.ldy = ldy;
  char* wsb = reinterpret_cast<char*>(ws);
  p.ctr = reinterpret_cast<uint32_t*>(wsb);
  p.part = reinterpret_cast<float*>(wsb + round256(pl.ctr_bytes));
  p.keys = pl.key_bytes ? reinterpret_cast<unsigned long long*>(wsb + round256(pl.ctr_bytes) + round256(pl.part_bytes))
                        : nullptr;
  p.idx = idx;
  p.maxv = maxv;
  p.n = (int)m->n;
  p.k = (int)m->k;
  p.kb = (int)(m->k / W12_REC_COLS);
  p.m = (int)M;
  p.y_f32 = y_dtype == W12_F32;
  p.mode = op == W12_OP_LMHEAD_ARGMAX ? kModeArgmax : kModeStore;
  p.fix = fix && m->n_esc > 0;
  p.q = op == W12_OP_GEMM_Q8;
  p.gate = gate;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // the copies of x the helper-wave kernel reads (x_copies)
  p.xt = nullptr;
  p.xk = nullptr;
  const XCopies xc = x_copies(m, pl, M, p.fix != 0);
  if (xc.xt || xc.xk || dense_xt) {
    const int64_t mm = ((M + 15) / 16) * 16;
    char* xt_at = wsb + round256(pl.ctr_bytes) + round256(pl.part_bytes) + round256(pl.key_bytes);
    uint16_t* xt = xc.xt ? reinterpret_cast<uint16_t*>(xt_at) : nullptr;
    uint16_t* xk = xc.xk ? reinterpret_cast<uint16_t*>(xt_at + round256(pl.xt_bytes)) : nullptr;
    // the dense path's xT takes the place of the kernel's own, which it does not read (no escape work)
    const hipError_t ex = launch_xpose(x, ldx, (int)M, (int)mm, (int)m->k, dense_xt ? dense_xt : xt, xk, gate, st);
    if (ex != hipSuccess) return hip_fail(ex, "activation transpose launch");
    p.xt = xt;
    p.xk = xk;
  }
  int unsupported = 0;
  const hipError_t e = launch_gemm(pl, p, st, &unsupported);
  if (unsupported) return W12_E_M_RANGE;
  if (e != hipSuccess) return hip_fail(e, "gemm launch");
  return W12_OK;
}

// ---------------------------------------------------------------- static scratch
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_at[kMaxDevices];

// Clears the counter words with plain vector stores (a kernel, not a memset
// node, so the clear is safe inside a captured graph too).
__global__ __launch_bounds__(256) void k_zero_words(uint32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The scratch address on the current device. On a device's first call it is
// looked up and its counter words cleared on `st`, ahead of the GEMM there.
int scratch_on_device(void** out, hipStream_t st) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "gemm_noalloc: current device");
  if (dev < 0 || dev >= kMaxDevices) {
    g_last_error = "gemm_noalloc: device ordinal " + std::to_string(dev) + " beyond the scratch table";
    return W12_E_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_at[dev]) {
    void* at = nullptr;
    e = hipGetSymbolAddress(&at, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "gemm_noalloc: scratch address");
    constexpr int kWords = (int)(kCounterBytes / sizeof(uint32_t));
    hipLaunchKernelGGL(k_zero_words, dim3((kWords + 255) / 256), dim3(256), 0, st, reinterpret_cast<uint32_t*>(at),
                       kWords);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "gemm_noalloc: counter clear");
    g_scratch_at[dev] = at;
  }
  *out = g_scratch_at[dev];
  return W12_OK;
}

}  // namespace

extern "C" {

int w12_abi_version(void) { return W12_ABI_VERSION; }

const char* w12_status_str(int status) {
  switch (status) {
    case W12_OK: return "ok";
    case W12_E_INVALID_ARG: return "invalid argument";
    case W12_E_UNSUPPORTED_SHAPE: return "unsupported shape (need N % 16 == 0, K % 512 == 0)";
    case W12_E_M_RANGE: return "M out of range (1..64)";
    case W12_E_WORKSPACE: return "workspace missing or too small";
    case W12_E_VERSION: return "unsupported format version";
    case W12_E_HIP: return "HIP runtime error";
    case W12_E_NOT_IMPLEMENTED: return "not implemented";
    case W12_E_CORRUPT: return "corrupt descriptor";
    default: return "unknown status";
  }
}

const char* w12_last_error(void) { return g_last_error.c_str(); }

int64_t w12_set_tuning(int key, int64_t value) {
  int64_t old = 0;
  if (key == W12_TUNE_PATH) {
    old = g_tune_path;
    g_tune_path = (int)value;
  } else if (key == W12_TUNE_GRID) {
    old = g_tune_grid;
    g_tune_grid = value;
  }
  return old;
}

size_t w12_workspace_bytes(int op, int64_t n, int64_t k, int64_t m) {
  if (check_shape(n, k) != W12_OK) return 0;
  if (op == W12_OP_ENCODE_PLAN) return round256((size_t)n * sizeof(uint32_t));
  if (op != W12_OP_GEMM && op != W12_OP_GEMM_Q8 && op != W12_OP_LMHEAD_ARGMAX && op != W12_OP_LMHEAD_CERTIFIED)
    return 0;
  if (m < 1 || m > W12_MAX_M) return 0;
  if (op == W12_OP_LMHEAD_CERTIFIED) return cert_layout(n, k, m).total;
  return ws_bytes_any(n, k, m, op);
}

int w12_plan_info(const w12_matrix* m, int op, int64_t M, uint32_t flags, w12_plan* out) {
  if (!m || !out) return W12_E_INVALID_ARG;
  const int s = check_shape(m->n, m->k);
  if (s != W12_OK) return s;
  if (m->n_esc < 0 || m->n_esc > m->n * m->k) return W12_E_INVALID_ARG;
  if (op != W12_OP_GEMM && op != W12_OP_GEMM_Q8 && op != W12_OP_LMHEAD_ARGMAX) return W12_E_INVALID_ARG;
  if (M < 1 || M > W12_MAX_M) return W12_E_M_RANGE;
  if (flags & ~W12_Q8_APPLY_ESCAPES) return W12_E_INVALID_ARG;
  bool fix = op != W12_OP_GEMM_Q8 || (flags & W12_Q8_APPLY_ESCAPES);
  const bool dense = dense_path(m, op, fix);
  if (dense) fix = false;
  const GemmPlan pl = make_plan(m->n, m->k, M, op);
  w12_plan o{};
  o.kernel = choose_kernel(m->n, m->k, m->n_esc, M, op, fix, pl);
  if (o.kernel == W12_KERNEL_MFMA_STREAM) {
    const MxPlan px = plan_mx(m->n, m->k, M, g_tune_grid);
    o.grid = px.P;
    o.threads = px.threads;
    o.tile_rows = px.gb * 16;
    o.whole_tiles = px.dp;
    o.split_tiles = px.sk_tiles;
    o.split_tile_rows = px.tb * 16;
    o.unit_cols = px.unit_cols;
    o.split_units = px.sk_units;
    o.prepass = 0;
    o.workspace_bytes = mx_ws_bytes(px);
  } else {
    if (!pl.mfma && M > 16) return W12_E_M_RANGE;
    o.grid = pl.P;
    o.threads = 320;
    o.tile_rows = pl.gb * 16;
    o.whole_tiles = pl.dp;
    o.split_tiles = pl.sk_tiles;
    o.split_tile_rows = pl.tile_rows;
    o.unit_cols = 256;
    o.split_units = pl.sk_units;
    const XCopies xc = x_copies(m, pl, M, fix);
    o.prepass = xc.xt || xc.xk ? 1 : 0;
    o.workspace_bytes = gemm_ws_bytes(pl);
  }
  if (dense) {
    o.fixup = 1;
    o.prepass = 1;
    o.workspace_bytes = dense_layout(m->n, m->k, M, op).total;
  }
  if (op == W12_OP_LMHEAD_ARGMAX && M > kFusedArgmaxMaxM) o.workspace_bytes = argmax_layout(m->n, m->k, M).total;
  *out = o;
  return W12_OK;
}

int w12_encode_plan(const uint16_t* w, int64_t n, int64_t k, uint8_t* e_top, uint32_t* esc_row_ptr,
                    int64_t* n_esc_host, void* ws, size_t ws_bytes, void* stream) {
  const int s = check_shape(n, k);
  if (s != W12_OK) return s;
  if (!w || !e_top || !esc_row_ptr || !n_esc_host || !aligned16(w)) return W12_E_INVALID_ARG;
  if (!ws || ws_bytes < (size_t)n * sizeof(uint32_t)) return W12_E_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(ws);
  hipError_t e = launch_plan(w, (int)n, (int)k, e_top, cnt, st);
  if (e != hipSuccess) return hip_fail(e, "encode_plan: window kernel");
  e = launch_scan(cnt, (int)n, esc_row_ptr, st);
  if (e != hipSuccess) return hip_fail(e, "encode_plan: scan kernel");
  uint32_t total = 0;
  e = hipMemcpyAsync(&total, esc_row_ptr + n, sizeof(uint32_t), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return hip_fail(e, "encode_plan: copy escape count");
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "encode_plan: synchronize");
  *n_esc_host = (int64_t)total;
  return W12_OK;
}

int w12_encode(const uint16_t* w, int64_t n, int64_t k, const uint8_t* e_top, const uint32_t* esc_row_ptr,
               uint8_t* records, w12_escape* esc, int64_t esc_capacity, void* stream) {
  const int s = check_shape(n, k);
  if (s != W12_OK) return s;
  if (!w || !e_top || !esc_row_ptr || !records || !aligned16(w) || !aligned16(records)) return W12_E_INVALID_ARG;
  if (esc_capacity < 0 || esc_capacity > n * k || (esc_capacity > 0 && !esc)) return W12_E_INVALID_ARG;
  const hipError_t e = launch_pack(w, (int)n, (int)k, e_top, esc_row_ptr, records, esc, (uint32_t)esc_capacity,
                                   reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "encode: pack kernel");
  return W12_OK;
}

int w12_decode(const w12_matrix* m, uint16_t* w_out, void* stream) {
  const int s = check_matrix(m);
  if (s != W12_OK) return s;
  if (!w_out || !aligned16(w_out)) return W12_E_INVALID_ARG;
  const hipError_t e = launch_decode(m, w_out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode kernel");
  return W12_OK;
}

int w12_gemm(const w12_matrix* m, const uint16_t* x, int64_t M, int64_t ldx, void* y, int64_t ldy, int y_dtype,
             void* ws, size_t ws_bytes, void* stream) {
  const int s = check_gemm_args(m, x, M, ldx, y, ldy, y_dtype);
  if (s != W12_OK) return s;
  return run_gemm(m, x, M, ldx, y, ldy, y_dtype, W12_OP_GEMM, true, ws, ws_bytes, nullptr, nullptr, stream);
}

int w12_gemm_noalloc(const w12_matrix* m, const uint16_t* x, int64_t M, int64_t ldx, void* y, int64_t ldy,
                     int y_dtype, void* stream) {
  const int s = check_gemm_args(m, x, M, ldx, y, ldy, y_dtype);
  if (s != W12_OK) return s;
  const size_t need = ws_bytes_any(m->n, m->k, M, W12_OP_GEMM);
  if (need > W12_NOALLOC_SCRATCH_BYTES) {
    g_last_error = "gemm_noalloc: this shape needs " + std::to_string(need) + " bytes of workspace, the static " +
                   "scratch holds " + std::to_string((size_t)W12_NOALLOC_SCRATCH_BYTES) + "; use w12_gemm";
    return W12_E_WORKSPACE;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  const int r = scratch_on_device(&ws, st);
  if (r != W12_OK) return r;
  return run_gemm(m, x, M, ldx, y, ldy, y_dtype, W12_OP_GEMM, true, ws, W12_NOALLOC_SCRATCH_BYTES, nullptr, nullptr,
                  stream);
}

int w12_gemm_q8(const w12_matrix* m, const uint16_t* x, int64_t M, int64_t ldx, void* y, int64_t ldy,
                int y_dtype, uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  const int s = check_gemm_args(m, x, M, ldx, y, ldy, y_dtype);
  if (s != W12_OK) return s;
  if (flags & ~W12_Q8_APPLY_ESCAPES) return W12_E_INVALID_ARG;
  return run_gemm(m, x, M, ldx, y, ldy, y_dtype, W12_OP_GEMM_Q8, (flags & W12_Q8_APPLY_ESCAPES) != 0, ws,
                  ws_bytes, nullptr, nullptr, stream);
}

int w12_lmhead_argmax(const w12_matrix* m, const uint16_t* x, int64_t M, int64_t ldx, int32_t* idx,
                      float* max_logit, void* ws, size_t ws_bytes, void* stream) {
  const int s = check_gemm_args(m, x, M, ldx, idx, m ? m->n : 0, W12_F32);
  if (s != W12_OK) return s;
  return run_gemm(m, x, M, ldx, nullptr, 0, W12_F32, W12_OP_LMHEAD_ARGMAX, true, ws, ws_bytes, idx, max_logit,
                  stream);
}

int w12_certify_bounds(const w12_matrix* m, float* bounds, void* stream) {
  const int s = check_matrix(m);
  if (s != W12_OK) return s;
  if (!bounds || (reinterpret_cast<uintptr_t>(bounds) & 7u) != 0) return W12_E_INVALID_ARG;
  const hipError_t e = launch_cert_bounds(m, bounds, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "certify bounds kernel");
  return W12_OK;
}

int w12_lmhead_argmax_certified(const w12_matrix* m, const float* bounds, const uint16_t* x, int64_t M,
                                int64_t ldx, int32_t* idx, float* max_logit, int32_t* survivors, void* ws,
                                size_t ws_bytes, void* stream) {
  const int s = check_gemm_args(m, x, M, ldx, idx, m ? m->n : 0, W12_F32);
  if (s != W12_OK) return s;
  if (!bounds) return W12_E_INVALID_ARG;
  const CertLayout c = cert_layout(m->n, m->k, M);
  if (!ws || ws_bytes < c.total) return W12_E_WORKSPACE;
  char* wsb = reinterpret_cast<char*>(ws);
  CertZero* z = reinterpret_cast<CertZero*>(wsb + kCertZeroOffset);
  CertCall* cc = reinterpret_cast<CertCall*>(wsb + c.state);
  float* lq = reinterpret_cast<float*>(wsb + c.logits);
  // 1. Q-copy logits: the view with the escapes applied, fp32
  int r = run_gemm(m, x, M, ldx, lq, m->n, W12_F32, W12_OP_GEMM_Q8, true, ws, c.gemm, nullptr, nullptr, stream);
  if (r != W12_OK) return r;
  // 2. bounds, survivors, exact rescoring, indices
  float* ub = reinterpret_cast<float*>(wsb + c.ub);
  const hipError_t e = launch_cert(m, x, ldx, (int)M, lq, bounds, z, cc, ub, ub + M * cert_chunks(m->n),
                                   reinterpret_cast<uint32_t*>(wsb + c.list), idx, max_logit, survivors,
                                   reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "certified head kernels");
  // 3. the full fused head, which does nothing unless the fallback flag is up
  return run_gemm(m, x, M, ldx, nullptr, 0, W12_F32, W12_OP_LMHEAD_ARGMAX, true, ws, c.gemm, idx, max_logit, stream,
                  &cc->flag);
}

int w12_validate(const w12_matrix* m, void* ws, size_t ws_bytes, void* stream) {
  const int s = check_matrix(m);
  if (s != W12_OK) return s;
  if (!ws || ws_bytes < sizeof(uint32_t)) return W12_E_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint32_t* flag = reinterpret_cast<uint32_t*>(ws);
  hipError_t e = launch_validate(m, flag, st);
  if (e != hipSuccess) return hip_fail(e, "validate kernel");
  uint32_t bad = 0;
  e = hipMemcpyAsync(&bad, flag, sizeof(uint32_t), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return hip_fail(e, "validate: copy flag");
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "validate: synchronize");
  return bad ? W12_E_CORRUPT : W12_OK;
}

}  // extern "C"

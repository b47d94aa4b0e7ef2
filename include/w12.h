/*
 * w12.h - C ABI of libw12, the MI355X (gfx950) implementation of the W12
 * lossless 12-bit weight format and its weight-read-bound skinny GEMM.
 *
 * Source of the method: "SpecPilot: Autonomous Algorithm Discovery and Systems
 * Optimization for Speculative Decoding" (arXiv 2611.02501), section 4.1
 * "W12: A Lossless 12-bit Weight Format" and Figure 5 (format, escapes, the
 * decode-in-register GEMM, deterministic stream-K), section 4.3 "Two-Level
 * Verification" (the Q pass over the nested 8-bit view), Appendix E "W12
 * Details" (the W12 LM head).
 *
 * ---------------------------------------------------------------- FORMAT v1
 * A weight matrix W is BF16 [N, K], row-major, one output channel per row
 * (y = x W^T). N % 16 == 0 and K % 512 == 0.
 *
 * Per row n the encoder picks E_n, the top of the 16-binade exponent window
 * [E_n - 15, E_n] holding the most normal weights (exponent field 1..254).
 * Ties go to the largest such top not above the row's largest normal exponent;
 * a row with no normal weight gets 16. E_n is in [16, 254]; it is stored as
 * e_top[n] (uint8).
 *
 * An in-window weight with sign s, exponent field e and mantissa m keeps
 *     off = e - (E_n - 15)   (4 bits, plane E)
 *     mh  = m >> 4           (3 bits, plane A together with s)
 *     ml  = m & 15           (4 bits, plane B)
 * and its 8-bit view byte is  v = s << 7 | off << 3 | mh.
 * Every other weight (below or above the window, +-0, subnormal, inf, NaN) is
 * an ESCAPE: its planes hold a placeholder, the in-window value nearest to it
 * with its sign - (s,15,7,15) above the window and for inf/NaN, (s,0,0,0)
 * otherwise - and the escape list keeps its exact bits.
 *
 * Records: 12288 bytes for 16 rows x 512 columns, stored in (row block
 * n / 16, column block k / 512) row-major order. Inside a record, row r and
 * column c = 16 G + t (G in 0..31, t in 0..15):
 *     view byte  at  (G*16 + r)*16 + t                         bytes [0, 8192)
 *     B nibble   in  8192 + (G*16 + r)*8 + (t/8)*4 + (t%4)     bytes [8192, 12288)
 *                    high nibble when t%8 < 4, low nibble otherwise.
 * The view (planes A and E) is therefore the first two thirds of every record
 * and the Q pass reads only it.
 *
 * Escapes: CSR by row. esc_row_ptr[N+1] (uint32) and 8-byte entries
 * { uint32 col; uint16 bits (original BF16); uint16 ph (placeholder BF16) },
 * columns ascending within a row.
 *
 * Encoded size: 1.5 N K + N + 4 (N + 1) + 8 n_esc bytes.
 *
 * ---------------------------------------------------------------- CONVENTIONS
 * - Every tensor pointer is a DEVICE pointer owned by the caller. Host pointers
 *   are the w12_matrix descriptor itself and n_esc_host. The library never
 *   allocates, frees or retains memory, apart from the static scratch that
 *   w12_gemm_noalloc uses (W12_NOALLOC_SCRATCH_BYTES per device).
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls
 *   are asynchronous on it, except w12_encode_plan and w12_validate, which
 *   synchronize it. Inputs must stay valid until the stream work completes.
 * - Every argument is checked before any launch; on error nothing is launched
 *   and a negative status is returned. No C++ exception crosses the ABI.
 * - Results are deterministic: the same inputs and shape give the same bits
 *   (the K reduction is split over workgroups in a fixed order that depends
 *   only on N, K and M).
 * - Concurrent calls need distinct workspaces. The first W12_WS_COUNTER_BYTES
 *   of a GEMM workspace (W12_OP_GEMM, _GEMM_Q8, _LMHEAD_ARGMAX,
 *   _LMHEAD_CERTIFIED) are counter
 *   words that must be zero before the workspace's first use (allocate it
 *   zero-filled once); every call leaves them zero again, so one workspace
 *   serves any sequence of GEMM calls, ops, matrices and sizes that fit in
 *   it. The rest of a workspace carries nothing from one call to the next.
 * - W12_E_HIP: a HIP call failed; w12_last_error() names it (thread-local).
 */
#ifndef W12_H
#define W12_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W12_ABI_VERSION 2
#define W12_FORMAT_VERSION 1

#define W12_REC_ROWS 16
#define W12_REC_COLS 512
#define W12_REC_BYTES 12288
#define W12_REC_VIEW_BYTES 8192
#define W12_MAX_M 64
#define W12_WS_COUNTER_BYTES 50432 /* counter words at the start of a GEMM workspace */
#define W12_NOALLOC_SCRATCH_BYTES (16u << 20) /* static scratch of w12_gemm_noalloc, per device */

/* status codes */
#define W12_OK 0
#define W12_E_INVALID_ARG (-1)       /* null pointer, bad dtype, bad leading dimension */
#define W12_E_UNSUPPORTED_SHAPE (-2) /* N % 16, K % 512, N, K <= 0, K > 2^23, N*K >= 2^32 */
#define W12_E_M_RANGE (-3)           /* M outside 1..64                                */
#define W12_E_WORKSPACE (-4)         /* workspace missing or smaller than required     */
#define W12_E_VERSION (-5)           /* descriptor format_version != W12_FORMAT_VERSION */
#define W12_E_HIP (-6)               /* a HIP runtime call failed                      */
#define W12_E_NOT_IMPLEMENTED (-7)
#define W12_E_CORRUPT (-8)           /* w12_validate found a broken descriptor         */

/* output dtypes */
#define W12_BF16 0 /* y[m, n] = RNE_bf16(fp32 accumulation) */
#define W12_F32 1  /* y[m, n] = fp32 accumulation           */

/* workspace queries */
#define W12_OP_ENCODE_PLAN 1
#define W12_OP_GEMM 2
#define W12_OP_GEMM_Q8 3
#define W12_OP_LMHEAD_ARGMAX 4
#define W12_OP_LMHEAD_CERTIFIED 5

#define W12_CERT_MAX_SURVIVORS 256 /* rows rescored per activation row before the full head runs */

/* w12_gemm_q8 flags */
#define W12_Q8_APPLY_ESCAPES 1u

typedef struct {
  uint32_t col;  /* column k of the escape                    */
  uint16_t bits; /* its original BF16 bits                    */
  uint16_t ph;   /* the placeholder BF16 its planes decode to */
} w12_escape;

typedef struct {
  int64_t n, k;                /* out features (N % 16 == 0), in features (K % 512 == 0) */
  const uint8_t* records;      /* (N/16)*(K/512)*12288 bytes, 16-byte aligned            */
  const uint8_t* e_top;        /* [N], values 16..254                                    */
  const uint32_t* esc_row_ptr; /* [N+1], esc_row_ptr[0] == 0, nondecreasing              */
  const w12_escape* esc;       /* [n_esc], may be NULL when n_esc == 0                   */
  int64_t n_esc;
  uint32_t format_version;     /* W12_FORMAT_VERSION                                     */
} w12_matrix;

int w12_abi_version(void);
const char* w12_status_str(int status);
/* Text of the last W12_E_HIP failure on the calling thread ("" if none). */
const char* w12_last_error(void);

/* Bytes of workspace `op` needs for an N x K matrix and M activation rows
 * (M is ignored for W12_OP_ENCODE_PLAN). 0 means no workspace is needed.
 * Returns 0 as well for arguments the op would reject. */
size_t w12_workspace_bytes(int op, int64_t n, int64_t k, int64_t m);

/* Encode, step 1 (section 4.1: per-channel window choice). Reads w (BF16
 * [N, K], device, 16-byte aligned, row-major), writes e_top[N] and
 * esc_row_ptr[N+1] (device), and stores the total number of escapes in
 * *n_esc_host (host). SYNCHRONIZES the stream (the escape count sizes the
 * escape buffer). ws: w12_workspace_bytes(W12_OP_ENCODE_PLAN, n, k, 0). */
int w12_encode_plan(const uint16_t* w, int64_t n, int64_t k, uint8_t* e_top, uint32_t* esc_row_ptr,
                    int64_t* n_esc_host, void* ws, size_t ws_bytes, void* stream);

/* Encode, step 2 (section 4.1 and Figure 5: split into planes, pack records,
 * list escapes). Inputs w, e_top, esc_row_ptr as produced by w12_encode_plan;
 * outputs records ((N/16)*(K/512)*12288 bytes, 16-byte aligned) and esc, a
 * buffer of esc_capacity entries (pass the count w12_encode_plan returned;
 * esc may be NULL only when esc_capacity is 0). Entries past esc_capacity are
 * never written: a smaller capacity than the count truncates the list.
 * W12_E_INVALID_ARG for a negative capacity, one above N*K, or a NULL esc
 * with a nonzero capacity. */
int w12_encode(const uint16_t* w, int64_t n, int64_t k, const uint8_t* e_top, const uint32_t* esc_row_ptr,
               uint8_t* records, w12_escape* esc, int64_t esc_capacity, void* stream);

/* Exact decode (section 4.1: the load-time bit-for-bit check): writes the
 * original BF16 matrix [N, K] (row-major, 16-byte aligned) to w_out. */
int w12_decode(const w12_matrix* m, uint16_t* w_out, void* stream);

/* Exact W12 GEMM (section 4.1, Figure 5b): y[M, N] = x[M, K] W^T with fp32
 * accumulation, escapes fixed up exactly before the output rounding.
 * x: BF16, row stride ldx >= K elements (a multiple of 8, at most 2^25),
 *    16-byte aligned rows.
 * y: BF16 or fp32 (y_dtype), row stride ldy >= N elements (below 2^31).
 * 1 <= M <= 64: M <= 2 runs the lane-per-row GEMV kernel, M >= 3 an MFMA
 * kernel (M padded to a multiple of 16); w12_plan_info names the kernel.
 * ws: w12_workspace_bytes(W12_OP_GEMM, n, k, M) bytes (device). */
int w12_gemm(const w12_matrix* m, const uint16_t* x, int64_t M, int64_t ldx, void* y, int64_t ldy,
             int y_dtype, void* ws, size_t ws_bytes, void* stream);

/* w12_gemm without a workspace argument, for callers that cannot allocate
 * device memory (code under graph capture, serving loops and harnesses that
 * forbid hipMalloc). Same arguments, kernels and results as w12_gemm; the
 * workspace is a static device array of W12_NOALLOC_SCRATCH_BYTES that each
 * device holds until the process ends. A device's first call looks up its
 * address and clears its counter words (a small kernel on `stream`); no call
 * allocates or frees anything. W12_E_WORKSPACE when
 * w12_workspace_bytes(W12_OP_GEMM, n, k, M) exceeds the scratch (nothing is
 * launched). All calls on one device share its scratch: calls that may
 * overlap on one device (different streams, or graphs replayed concurrently)
 * race and give wrong results; serialize them or use w12_gemm. */
int w12_gemm_noalloc(const w12_matrix* m, const uint16_t* x, int64_t M, int64_t ldx, void* y, int64_t ldy,
                     int y_dtype, void* stream);

/* Q pass (section 4.3, zero-copy Q pass): the same product over the 8-bit
 * view only - the first 8 KB of each record - with the four dropped mantissa
 * bits set to their midpoint (binary 1000). Escapes keep their placeholders
 * unless flags has W12_Q8_APPLY_ESCAPES. Arguments as w12_gemm;
 * ws: w12_workspace_bytes(W12_OP_GEMM_Q8, n, k, M). */
int w12_gemm_q8(const w12_matrix* m, const uint16_t* x, int64_t M, int64_t ldx, void* y, int64_t ldy,
                int y_dtype, uint32_t flags, void* ws, size_t ws_bytes, void* stream);

/* W12 LM head fused with a per-row argmax (Appendix E: the LM head converted
 * to W12): idx[i] = the lowest n attaining max_n (x W^T)[i, n], computed on
 * the fp32 logits after the escape fix-up. max_logit (nullable) receives
 * that fp32 maximum. idx and max_logit are device arrays of M entries.
 * ws: w12_workspace_bytes(W12_OP_LMHEAD_ARGMAX, n, k, M). */
int w12_lmhead_argmax(const w12_matrix* m, const uint16_t* x, int64_t M, int64_t ldx, int32_t* idx,
                      float* max_logit, void* ws, size_t ws_bytes, void* stream);

/* Certified argmax LM head (section 4.1, the certified LM head paragraph;
 * section 4.3, zero-copy Q pass), step 1, once per matrix: per-row bounds
 * for the Q copy, which is the 8-bit view with the escapes applied.
 * bounds: device float[2 N] (8-byte aligned): bounds[2n] = r_n =
 * ||w_n - q_n||_2 and bounds[2n+1] = a_n = ||w_n||_2 + ||v_n||_2 (w exact
 * weights, q the Q copy, v the view with its placeholders), both summed in
 * float64 and rounded up; +inf for a row holding inf or NaN. */
int w12_certify_bounds(const w12_matrix* m, float* bounds, void* stream);

/* Certified argmax LM head, per call: the same idx (and max_logit) contract as
 * w12_lmhead_argmax. A Q pass (w12_gemm_q8 with W12_Q8_APPLY_ESCAPES) gives
 * fp32 logits lq; with c = 4 K u / (1 - K u), u = 2^-24, row n is ruled out
 * when lq_n + ||x|| (r_n + c a_n) < max_j (lq_j - ||x|| (r_j + c a_j)), which
 * no row holding the largest exact logit can meet. The rows left are rescored
 * exactly (fp32 sums of the exact weights, placeholders swapped for the
 * escapes' values); the lowest index wins equal values. When any activation
 * row keeps more than W12_CERT_MAX_SURVIVORS rows, the full fused head
 * (w12_lmhead_argmax) runs for the call instead; it is always enqueued and
 * does nothing otherwise, so the call never synchronizes. max_logit is the
 * rescored fp32 logit (its summation order differs from the full head's).
 * survivors (nullable): M int32 counts of rows kept per activation row (above
 * the cap: the full head ran). bounds: from w12_certify_bounds.
 * ws: w12_workspace_bytes(W12_OP_LMHEAD_CERTIFIED, n, k, M), zero before its
 * first use; every call leaves it ready for the next. */
int w12_lmhead_argmax_certified(const w12_matrix* m, const float* bounds, const uint16_t* x, int64_t M,
                                int64_t ldx, int32_t* idx, float* max_logit, int32_t* survivors, void* ws,
                                size_t ws_bytes, void* stream);

/* Checks a descriptor's device arrays: e_top in [16, 254], esc_row_ptr
 * starting at 0, nondecreasing and ending at n_esc, escape columns < K and
 * strictly ascending within each row. SYNCHRONIZES the stream.
 * ws: 4 bytes of device memory. Returns W12_OK or W12_E_CORRUPT. */
int w12_validate(const w12_matrix* m, void* ws, size_t ws_bytes, void* stream);

/* The GEMM kernels (w12_plan.kernel and W12_TUNE_PATH values).
 * GEMV: one lane per matrix row, activations as scalar operands (M <= 2 by
 *   default; any M <= 16 when forced).
 * MFMA_HELPER: v_mfma_f32_16x16x32_bf16 with four streaming waves and a
 *   helper wave that applies the escape corrections; an activation transpose
 *   kernel runs first beyond 16 activation rows, and up to 16 only for
 *   matrices with many escapes per workgroup (w12_plan.prepass). The default
 *   from M = 3 where the stream kernel is not, and always for the LM-head
 *   argmax (fused up to 16 activation rows; above, it stores fp32 logits and
 *   a row-argmax kernel follows) and for K > 2^20.
 * MFMA_STREAM: v_mfma_f32_16x16x32_bf16 with eight streaming waves, escapes
 *   substituted into the decoded weights in registers, activations read
 *   from x through LDS; no pre-pass. The default from M = 3 when the matrix
 *   has fewer 64-row tiles than the GPU has compute units (N <= 16320),
 *   except up to 16 activation rows on matrices with K > 8192 or fewer than
 *   32 tiles (N <= 1984).
 * With more than 8 escapes per row on average, the exact GEMM and the Q pass
 * with escapes run the chosen kernel without escape work into fp32 sums and
 * a fix-up kernel applies the escapes (w12_plan.fixup). */
#define W12_KERNEL_GEMV 1
#define W12_KERNEL_MFMA_HELPER 2
#define W12_KERNEL_MFMA_STREAM 3

/* The plan of one GEMM call (host-side description; nothing is launched). */
typedef struct {
  int32_t kernel;          /* W12_KERNEL_*                                             */
  int32_t grid;            /* workgroups of the GEMM kernel                            */
  int32_t threads;         /* threads per workgroup                                    */
  int32_t tile_rows;       /* rows of a whole tile                                     */
  int32_t whole_tiles;     /* whole tiles per workgroup                                */
  int32_t split_tiles;     /* tiles whose columns several workgroups share (stream-K)  */
  int32_t split_tile_rows; /* rows of a split tile                                     */
  int32_t unit_cols;       /* columns of a stream-K unit                               */
  int64_t split_units;     /* units of the split tiles                                 */
  int32_t prepass;         /* 1: an activation transpose kernel runs before the GEMM   */
  int32_t fixup;           /* 1: dense escapes: the GEMM runs without escape work and  */
                           /*    a fix-up kernel applies the escapes after it          */
  size_t workspace_bytes;  /* what this plan uses (w12_workspace_bytes covers them all) */
} w12_plan;

/* The plan w12_gemm (op W12_OP_GEMM), w12_gemm_q8 (W12_OP_GEMM_Q8, with its
 * flags) or w12_lmhead_argmax (W12_OP_LMHEAD_ARGMAX) would run for matrix m
 * and M activation rows. Host-only: reads m->n, m->k and m->n_esc, touches no
 * device memory. Returns W12_OK or the status the call would return for
 * these arguments. */
int w12_plan_info(const w12_matrix* m, int op, int64_t M, uint32_t flags, w12_plan* out);

/* Test hooks, per calling thread (other threads' calls are unaffected).
 * W12_TUNE_PATH: 0 = the library's choice, 1 = the GEMV kernel (M <= 16),
 *   2 = the MFMA helper-wave kernel, 3 = the MFMA stream kernel (where it
 *   applies; the fused argmax always runs the helper-wave kernel), 4 = the
 *   dense-escape path (GEMM without escape work, then the fix-up kernel) for
 *   any matrix with escapes (the library's choice above 8 escapes per row).
 * W12_TUNE_GRID: workgroup count for the GEMM kernels (0 = the library's
 *   choice: 256, or c * T for a matrix of T < 256 tiles; at most 4096 and at
 *   most the number of work units are used).
 * A hook changes which kernel runs or how K is split, so the fp32 summation
 * order and the workspace size; query w12_workspace_bytes after setting it.
 * With the hooks at 0, results depend only on the matrix, x, N, K and M.
 * Returns the old value. */
#define W12_TUNE_PATH 1
#define W12_TUNE_GRID 2
int64_t w12_set_tuning(int key, int64_t value);

#ifdef __cplusplus
}
#endif
#endif /* W12_H */

/*
 * msign.h - C ABI of libmsign, a HIP/CDNA4 (gfx950) library that computes
 * msign(M) = (M M^T)^{-1/2} M = U V^T by Newton-Schulz iteration.
 *
 * Sources (cited by page title and section):
 *   [KX] "msign算子的Newton-Schulz迭代（上）" (kexue.fm/archives/10922):
 *        §写在前面 definition of msign; §迭代计算 the quintic iteration,
 *        Frobenius normalisation and the constants (3.4445, -4.7750, 2.0315),
 *        T = 5; §参考实现 batching over the last two dims, transpose when
 *        rows > cols, eps = 1e-20; §解开约束 per-step coefficients.
 *   [GR] "Gram Newton-Schulz" (zifeng-mai.github.io/2026/04/05/GramNewtonSchulz):
 *        §2.3 Algorithm 1, §3.2 restarting, §3.3 fp16 and the a_t terms kept
 *        out of Z, §3.4 Algorithm 2, §4 symmetric GEMM C <- aAB + bC + gI.
 *   [NB] nil9.net, flash-muon excerpt: the X X^T operator that computes only
 *        upper-triangle tiles and stores each tile's transpose into the
 *        mirrored lower-triangle tile; NS applied to the gradient or its
 *        momentum.
 *   [MS] the Mousse page (anti-entrophic.github.io/posts/10054.html),
 *        §标准 Muon 算法: the Muon update is -msign of the matrix.
 *
 * Conventions shared by every entry point:
 *   - Layout: contiguous row-major [batch, rows, cols]; matrix b starts at
 *     element b*rows*cols.  Pointers are DEVICE pointers unless stated.
 *   - Ownership: the caller owns every buffer (inputs, outputs, workspace).
 *     The library never allocates or frees device memory and keeps no
 *     pointer after a call returns.  All work is queued on `stream` (0 is
 *     the null stream); no call synchronises the host.
 *   - Errors: arguments are validated on the host before anything is
 *     launched; a non-OK status means nothing was launched and nothing
 *     written.  MSIGN_ERR_HIP reports a failed launch; msign_last_error()
 *     then holds the HIP message (thread-local).  No call aborts.
 *   - Degenerate sizes: batch, rows or cols equal to 0 is a successful no-op.
 *     NaN/Inf in the input propagate; an all-zero matrix maps to zero.
 *   - Bit stability: results do not depend on timing (no atomics, fixed
 *     reduction orders); the same call on the same device gives the same bits.
 *     The launch layout (tile size, K split of the last round of tiles)
 *     depends on the problem's shape including `batch`, so one matrix may
 *     differ in the last bits between calls with different batch sizes.
 *   - Concurrency: calls are thread-safe and may run on different streams as
 *     long as they do not share output or workspace buffers.
 */
#ifndef MSIGN_H_
#define MSIGN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSIGN_F32 = 0,
  MSIGN_BF16 = 1,
  MSIGN_F16 = 2
} msign_dtype_t;

typedef enum {
  MSIGN_OK = 0,
  MSIGN_ERR_ARG = 1,        /* null pointer, bad steps/eps/restart list   */
  MSIGN_ERR_DTYPE = 2,      /* unknown dtype or unsupported combination   */
  MSIGN_ERR_SHAPE = 3,      /* negative or too large size                  */
  MSIGN_ERR_WORKSPACE = 4,  /* workspace null or smaller than required     */
  MSIGN_ERR_ALIAS = 5,      /* output partially overlaps input/workspace   */
  MSIGN_ERR_HIP = 6         /* a HIP launch failed                         */
} msign_status_t;

/* Largest number of iteration steps accepted (coefficient tables). */
#define MSIGN_MAX_STEPS 64

/*
 * Bytes of device workspace msign_ns needs for this problem.  Returns 0 for
 * empty problems and (size_t)-1 for invalid sizes or dtypes.
 */
size_t msign_ns_workspace_bytes(int64_t batch, int64_t rows, int64_t cols,
                                int32_t compute_dtype);

/*
 * msign_ns - standard quintic Newton-Schulz ([KX] §迭代计算, §参考实现).
 *
 * For each matrix M (rows x cols) of the batch: X = M, or M^T when
 * rows > cols (n = min(rows, cols), m = max); X0 = X / sqrt(sum X^2 + eps);
 * then for t = 1..steps with (a_t, b_t, c_t):
 *     A = X X^T;  B = b_t A + c_t A A;  X <- a_t X + B X
 * and the result (transposed back when rows > cols) is written to y.
 *
 *   x, y           device, [batch, rows, cols] in io_dtype.  y == x (in place)
 *                  is allowed; any other overlap of y with x or workspace is
 *                  MSIGN_ERR_ALIAS.
 *   io_dtype       MSIGN_F32, MSIGN_BF16 or MSIGN_F16 (input and output).
 *   compute_dtype  operand dtype of the matrix products: MSIGN_BF16 or
 *                  MSIGN_F16 (MFMA with fp32 accumulation) or MSIGN_F32 (fp32
 *                  MFMA).  The iterate X itself is carried in fp32 between
 *                  steps; A and B are stored in compute_dtype.  Matrices
 *                  with n = min(rows, cols) <= 64 fit one 64-wide tile, where
 *                  the iteration is bound by launch latency: their products
 *                  always run in fp32 (no slower; 16-bit operands would miss
 *                  2e-2 on vector-like inputs, where a_t + b_t + c_t is a
 *                  cancellation).  In a grouped call such matrices form an
 *                  fp32 sub-call of their own.
 *   steps          1..MSIGN_MAX_STEPS.
 *   coeffs         HOST pointer to steps*3 floats (a_t, b_t, c_t per row,
 *                  [KX] §解开约束), or NULL for (3.4445, -4.7750, 2.0315)
 *                  at every step.  Read before the call returns.  A step
 *                  with c_t == 0 (cubic, [KX] §迭代计算) skips the A A
 *                  product: X <- a_t X + b_t A X.
 *   eps            >= 0, added to sum X^2 before the square root (1e-20 in
 *                  [KX] §参考实现).
 *   workspace      device, at least msign_ns_workspace_bytes(...) bytes,
 *                  256-byte aligned, contents on entry irrelevant.
 */
msign_status_t msign_ns(const void* x, void* y, int64_t batch, int64_t rows,
                        int64_t cols, int32_t io_dtype, int32_t compute_dtype,
                        int32_t steps, const float* coeffs, float eps,
                        void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * msign_ns_ex - msign_ns with option flags (msign_ns is msign_ns_ex with
 * flags = 0; both use msign_ns_workspace_bytes).
 *
 *   MSIGN_NS_IMPROVED_INIT  improved initial normalisation ([KX] §改良初值):
 *       on the first step, with A = X X^T and A2 = A A of the Frobenius-
 *       normalised X0, the iterate is further divided by
 *       s = (sum A2^2 + eps)^(1/8) = ||(X0 X0^T)^2||_F^(1/4) <= ||X0||_F,
 *       i.e. X1 = a X0/s + (b A/s^2 + c A2/s^4) X0/s.  A2 is formed even when
 *       c_1 = 0.  Later steps are unchanged.
 */
#define MSIGN_NS_IMPROVED_INIT 1u
/*
 *   MSIGN_NS_DENSE_PRODUCTS  measurement comparator: X X^T and c A A + b A
 *       are computed on every tile (plain products, no triangle), so their
 *       cost can be set against the triangle products' ([NB] flash-muon:
 *       the symmetric X X^T operator and its end-to-end NS saving).  Same
 *       arithmetic per element; the stored A and B are then symmetric only
 *       up to rounding.  One non-empty group only; not with
 *       MSIGN_NS_IMPROVED_INIT (MSIGN_ERR_ARG).
 *   Other bits are MSIGN_ERR_ARG.
 */
#define MSIGN_NS_DENSE_PRODUCTS 2u
msign_status_t msign_ns_ex(const void* x, void* y, int64_t batch, int64_t rows,
                           int64_t cols, int32_t io_dtype, int32_t compute_dtype,
                           int32_t steps, const float* coeffs, float eps,
                           uint32_t flags, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * msign_ns_noalloc - msign_ns without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same computation, kernels and
 * results (bit for bit) as msign_ns with the same arguments.
 *
 * Its workspace is a fixed scratch array of MSIGN_NOALLOC_SCRATCH_BYTES that
 * the library holds in device memory, one per device it runs on, until the
 * process ends; its device address is looked up once per device, on the
 * first call with that device current.  The call allocates and frees
 * nothing and creates no events (kernel timing does not apply to it).
 *   - A problem whose msign_ns_workspace_bytes(...) exceeds
 *     MSIGN_NOALLOC_SCRATCH_BYTES gets MSIGN_ERR_WORKSPACE, nothing launched
 *     (e.g. 1 x 1024 x 4096 bf16 fits; 1 x 2048 x 4096 does not).
 *   - Nothing in the scratch must start at zero: every region is written
 *     before it is read, so the contents a previous call left are harmless.
 *   - All calls on one device share its scratch: calls that may overlap in
 *     time on one device (different streams, or host threads without
 *     ordering) race and give wrong results.  Order them on one stream.
 *   - Other arguments, errors and aliasing rules as msign_ns.
 */
#define MSIGN_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
msign_status_t msign_ns_noalloc(const void* x, void* y, int64_t batch, int64_t rows,
                                int64_t cols, int32_t io_dtype, int32_t compute_dtype,
                                int32_t steps, const float* coeffs, float eps,
                                hipStream_t stream);

/* Bytes of device workspace msign_gram_ns needs; see msign_ns_workspace_bytes. */
size_t msign_gram_ns_workspace_bytes(int64_t batch, int64_t rows, int64_t cols,
                                     int32_t compute_dtype);

/*
 * msign_gram_ns - Gram Newton-Schulz ([GR] §3.4 Algorithm 2; with no restart
 * it is §2.3 Algorithm 1).
 *
 * X0 as in msign_ns, rounded to compute_dtype ([GR] §3.4 step 2).  Then
 *     R = X X^T, Q = I; for t = 1..steps:
 *         Z = b_t R + c_t R^2;  Q <- Q Z + a_t Q;
 *         RZ = R Z + a_t R;     R <- Z RZ + a_t RZ    (skipped when unused)
 *         after t in restart_after (t < steps): X <- Q X, R = X X^T, Q = I
 *     y = Q X  (transposed back when rows > cols).
 * Q, R, Z and RZ are n x n, kept exactly symmetric (upper-triangle tiles,
 * mirrored).  The a_t terms are applied in fp32 epilogues ([GR] §3.3); the
 * first Q of each block is Z + a_t I, added on the diagonal in registers.
 *
 *   compute_dtype   MSIGN_F16 (the pages' choice, [GR] §3.3), MSIGN_BF16 or
 *                   MSIGN_F32; as in msign_ns, matrices with n <= 64 always
 *                   use fp32 products.
 *   restart_after   HOST array of n_restarts step indices, strictly
 *                   increasing, each in 1..steps-1; NULL iff n_restarts == 0.
 *                   Algorithm 2 uses {2}.
 *   other arguments as in msign_ns.
 */
msign_status_t msign_gram_ns(const void* x, void* y, int64_t batch,
                             int64_t rows, int64_t cols, int32_t io_dtype,
                             int32_t compute_dtype, int32_t steps,
                             const float* coeffs, float eps,
                             const int32_t* restart_after, int32_t n_restarts,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * Grouped calls: one msign over several batches of different shapes at once
 * (the parameter list of an optimizer step holds a few shape groups, e.g.
 * the square and the 3.5x-wide matrices of a transformer block).  Every
 * matrix product of the iteration is ONE kernel launch over the tiles of
 * all groups (longest contraction first), so a small group fills the CUs
 * that a large group's last round of tiles leaves idle, and the launch
 * count does not grow with the number of groups.  Each matrix gets the
 * result of a call on its group alone up to rounding: a launch's tile size
 * and K split depend on all of its groups, which changes the order of the
 * fp32 sums, and the iteration carries such last-bit differences through
 * its rounded operands (both results stay within the same error of the
 * exact iteration).  A grouped call is itself bit-stable.
 *
 * Group g: x, y device [batch, rows, cols] in io_dtype, as in msign_ns (y ==
 * x allowed).  Groups with batch, rows or cols equal to 0 are skipped.  An
 * output may not overlap any other group's input or output (MSIGN_ERR_ALIAS);
 * inputs may overlap each other.  io_dtype, compute_dtype, steps, coeffs,
 * eps (and flags or the restart list) are shared by all groups.
 *   groups    HOST array of ngroups descriptors, read before the call returns.
 *   ngroups   1..MSIGN_MAX_GROUPS; with 1 these are msign_ns_ex and
 *             msign_gram_ns, workspace size included.
 * An invalid group is reported with its index in msign_last_error().
 */
#define MSIGN_MAX_GROUPS 4

typedef struct {
  const void* x;
  void* y;
  int64_t batch, rows, cols;
} msign_group_t;

/* Workspace of a grouped call; 0 if every group is empty, (size_t)-1 for an
 * invalid count, size or dtype. */
size_t msign_ns_grouped_workspace_bytes(const msign_group_t* groups, int32_t ngroups,
                                        int32_t compute_dtype);
size_t msign_gram_ns_grouped_workspace_bytes(const msign_group_t* groups, int32_t ngroups,
                                             int32_t compute_dtype);

msign_status_t msign_ns_grouped(const msign_group_t* groups, int32_t ngroups,
                                int32_t io_dtype, int32_t compute_dtype,
                                int32_t steps, const float* coeffs, float eps,
                                uint32_t flags, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

msign_status_t msign_gram_ns_grouped(const msign_group_t* groups, int32_t ngroups,
                                     int32_t io_dtype, int32_t compute_dtype,
                                     int32_t steps, const float* coeffs, float eps,
                                     const int32_t* restart_after, int32_t n_restarts,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/*
 * muon_step - one Muon optimizer step over up to MSIGN_MAX_GROUPS parameter
 * groups ([GR] §1.1 names the momentum coefficient mu, the learning rate
 * eta and M_0 = 0, its formula is lost in the text; [MS] §标准 Muon 算法:
 * the update is -msign; [NB]: NS acts on the gradient or its momentum).
 * Read as, for every matrix of every group:
 *     M <- mu M + G;   W <- W - lr msign(M)
 * with msign by standard NS (MUON_NS, as msign_ns_grouped with `flags`) or
 * Gram NS (MUON_GRAM, as msign_gram_ns_grouped; flags must be 0), all groups'
 * products in grouped launches.  The step is fused into the msign call: the
 * sum-of-squares pass that starts msign updates M in place (fp32, fmaf(mu,
 * M, G)) and the epilogue of the last product updates W in place (msign(M)
 * in fp32, W rounded once to io_dtype); there is no other pass and no buffer
 * for msign(M), so the workspace is that of the msign call alone.
 *
 * Group g: w (parameters, updated in place) and g (gradient), device
 * [batch, rows, cols] in io_dtype; m (momentum, updated in place), device
 * [batch, rows, cols] fp32, 16-byte alignment recommended.  Empty groups
 * are skipped.  w and m may overlap no other buffer of the step and no
 * buffer may overlap the workspace (MSIGN_ERR_ALIAS).
 *   mu, lr      finite.
 *   method      MUON_NS or MUON_GRAM.
 *   other arguments as in msign_ns_grouped / msign_gram_ns_grouped.
 * A non-OK status from argument checks means nothing was launched.
 */
#define MUON_NS 0
#define MUON_GRAM 1

typedef struct {
  void* w;
  const void* g;
  float* m;
  int64_t batch, rows, cols;
} muon_group_t;

/* Workspace of muon_step; 0 if every group is empty, (size_t)-1 for an
 * invalid count, size, method or dtype. */
size_t muon_step_workspace_bytes(const muon_group_t* groups, int32_t ngroups,
                                 int32_t method, int32_t compute_dtype);

msign_status_t muon_step(const muon_group_t* groups, int32_t ngroups,
                         int32_t io_dtype, float mu, float lr, int32_t method,
                         int32_t compute_dtype, int32_t steps,
                         const float* coeffs, float eps, uint32_t flags,
                         const int32_t* restart_after, int32_t n_restarts,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * syrk_xxt - C = alpha X X^T + beta D + gamma I for each matrix of a batch
 * ([NB] X X^T operator; [GR] §4 fused form C <- aAB + bC + gI with A = X,
 * B = X^T).
 *
 * Only upper-triangle tiles are computed; each is stored and its transpose
 * is stored into the mirrored tile, so C is exactly (bitwise) symmetric.
 *   x      device, [batch, n, k] in dtype (row pitch k).
 *   c      device, [batch, n, n] in dtype.  Must not overlap x or d.
 *   dtype  MSIGN_BF16 or MSIGN_F16 (MFMA, fp32 accumulation, one rounding on
 *          store) or MSIGN_F32.
 *   d      device, [batch, n, n] in dtype, or NULL (then beta is ignored).
 *          D must be symmetric; its upper triangle is what is read.
 *   workspace, workspace_bytes  device scratch, 256-byte aligned.
 *          syrk_xxt_workspace_bytes() is the size for the fastest path: a
 *          zero-padded copy of x (needed only when k is not a multiple of 64
 *          or x is not 16-byte aligned; then it is required) followed by
 *          scratch for splitting the last round of tiles along K (optional:
 *          with less, or NULL, those tiles are computed whole).
 */
size_t syrk_xxt_workspace_bytes(int64_t batch, int64_t n, int64_t k, int32_t dtype);

msign_status_t syrk_xxt(const void* x, void* c, int64_t batch, int64_t n,
                        int64_t k, int32_t dtype, float alpha, const void* d,
                        float beta, float gamma, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * syrk_xxt_ex - syrk_xxt with option flags (flags = 0 is syrk_xxt).
 *   MSIGN_SYRK_FULL_TILES  measurement comparator: every tile of X X^T is
 *       computed (a plain product, no triangle) and C is symmetric only up
 *       to rounding.  Same workspace rules as syrk_xxt.
 *   Other bits are MSIGN_ERR_ARG.
 */
#define MSIGN_SYRK_FULL_TILES 1u
msign_status_t syrk_xxt_ex(const void* x, void* c, int64_t batch, int64_t n, int64_t k, int32_t dtype,
                           float alpha, const void* d, float beta, float gamma, uint32_t flags,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static description of a status code; never NULL. */
const char* msign_status_string(msign_status_t status);

/* Detail of the last non-OK status on the calling thread ("" if none). */
const char* msign_last_error(void);

/* Library version string, e.g. "msign 0.1.0 gfx950". */
const char* msign_version(void);

/*
 * Per-kernel-class timing with HIP events, for measurement only.
 * While enabled for a class, every launch of that class made by the calls
 * above is bracketed by a pair of events recorded on the call's stream;
 * msign_kernel_timing_read() waits for them, adds their durations to
 * per-class totals and clears the queue.
 * Classes: 0 = normalise (sum of squares + scale/cast) and the other
 * elementwise passes, 1 = X X^T (triangle),
 * 2 = n x n triangle products (A^2 / Gram R, Q, Z, RZ updates), 3 = the
 * rectangular product (B X, Q X), 4 = the whole-iteration kernel of small
 * matrices (msign_ns with 64 < n <= 128 and m <= 256 after padding to 64,
 * 16-bit products: every step in one launch, one workgroup per matrix).
 *   msign_kernel_timing_enable   mask of classes to time (bit k = class k,
 *                                MSIGN_KCLASS_ALL for all; a nonzero mask also
 *                                resets the totals); 0 disables (and frees
 *                                events).  Bits beyond the classes give
 *                                MSIGN_ERR_ARG.
 *   msign_kernel_timing_read     fills total_ms[MSIGN_KCLASS_COUNT] and
 *                                launches[MSIGN_KCLASS_COUNT] (HOST).
 */
#define MSIGN_KCLASS_COUNT 5
#define MSIGN_KCLASS_ALL 0x1F
msign_status_t msign_kernel_timing_enable(int32_t enable);
msign_status_t msign_kernel_timing_read(double* total_ms, int64_t* launches);

/*
 * msign_mfma_probe - measurement only: one launch of a kernel that issues
 * nothing but 16x16x32 MFMAs (bf16 or fp16 operands, fp32 accumulation)
 * from registers, MSIGN_PROBE_BLOCKS blocks of MSIGN_PROBE_THREADS threads
 * (8 waves per CU, 2 per SIMD, 8 independent accumulator chains per wave),
 * `iters` rounds of 8 MFMAs per wave.  Timing it gives the matrix rate the
 * chip sustains (its clock under load), the denominator beside the
 * published peak.  Flops per launch: MSIGN_PROBE_FLOPS_PER_ITER * iters.
 *   dtype  MSIGN_BF16 or MSIGN_F16.
 *   out    device, MSIGN_PROBE_BLOCKS * MSIGN_PROBE_THREADS floats (one
 *          per thread; keeps the result alive, values meaningless).
 */
#define MSIGN_PROBE_BLOCKS 512
#define MSIGN_PROBE_THREADS 256
#define MSIGN_PROBE_FLOPS_PER_ITER (512.0 * 4 * 8 * 16 * 16 * 32 * 2)
msign_status_t msign_mfma_probe(int32_t dtype, int32_t iters, float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MSIGN_H_ */

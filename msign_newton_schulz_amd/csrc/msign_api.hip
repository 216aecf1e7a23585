// libmsign host side: argument checks, workspace planning and the launch
// sequences of standard and Gram Newton-Schulz on one HIP stream.
//
// Internal buffers live in the caller's workspace, one [batch][rows][cols]
// region each, with rows and columns padded to multiples of 64 and the
// padding kept at exactly zero (the normalise pass writes zero padding, every
// product of zero-padded operands is zero there, and diagonal terms stop at
// the true size), so the product kernel needs no K tail handling.
//
// Standard NS ("msign算子的Newton-Schulz迭代（上）" §迭代计算, §参考实现;
// the A = X X^T reuse of the flash-muon excerpt on nil9.net), per step:
//   A  = X X^T                 triangle product, K = m
//   B  = c A A + b A           triangle product, K = n, D = A
//   X' = B X + a X             full product, Q operand = X^T, D = X (fp32)
// X is carried in fp32 between steps (X32t, stored transposed so the
// epilogue reads four consecutive values per lane), together with two
// compute-dtype copies that feed the products: Xh (n x m) and Xht (m x n).
// Rounding only the product operands, not the iterate, keeps the small
// singular directions of spiked (momentum-like) matrices intact.
//
// Gram NS ("Gram Newton-Schulz" §3.4 Algorithm 2, §2.3 Algorithm 1) keeps
// everything in the compute dtype as the page does (§3.3), with the a_t
// terms applied in fp32 epilogues.
#include "../../include/msign.h"
#include "common.hpp"
#include "gemm_nt.hpp"
#include "normalize.hpp"

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

using namespace msign;

namespace {

thread_local std::string g_err;

msign_status_t fail(msign_status_t st, const std::string& msg) {
  g_err = msg;
  return st;
}

// Default coefficients: "msign算子的Newton-Schulz迭代（上）" §迭代计算.
constexpr float kKeller[3] = {3.4445f, -4.7750f, 2.0315f};

constexpr int64_t kPad = 64;
constexpr int64_t kMaxDim = int64_t(1) << 20;
constexpr int64_t kMaxBatch = 65535;

int64_t pad_up(int64_t v) { return (v + kPad - 1) / kPad * kPad; }
size_t dt_size(int32_t dt) { return dt == MSIGN_F32 ? 4 : 2; }
bool dt_valid(int32_t dt) { return dt == MSIGN_F32 || dt == MSIGN_BF16 || dt == MSIGN_F16; }
size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct Shape {
  int64_t n, m, np, mp;
  bool tall;
};

Shape canon(int64_t rows, int64_t cols) {
  Shape s;
  s.tall = rows > cols;
  s.n = s.tall ? cols : rows;
  s.m = s.tall ? rows : cols;
  s.np = pad_up(s.n);
  s.mp = pad_up(s.m);
  return s;
}

// K-split scratch of the products of one NS or Gram call, and the acc^2
// slots of the first A A product (defined below).
size_t split_scratch(const Shape& s, int64_t batch, int32_t cdt);
size_t init_sumsq_floats(const Shape& s, int64_t batch, int32_t cdt);

int32_t norm_blocks(int64_t count) {
  int64_t nb = (count + 16383) / 16384;
  if (nb < 1) nb = 1;
  if (nb > 1024) nb = 1024;
  return (int32_t)nb;
}

struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  }
};

struct NsPlan {
  Shape s;
  int32_t nblk;
  size_t x32[2], xh[2], a, b, partial, sumsq, scales, split, split_bytes, total;
};

NsPlan plan_ns(int64_t batch, int64_t rows, int64_t cols, int32_t cdt) {
  NsPlan p;
  p.s = canon(rows, cols);
  p.nblk = norm_blocks(rows * cols);
  const size_t cs = dt_size(cdt);
  const size_t nm = (size_t)batch * p.s.np * p.s.mp, nn = (size_t)batch * p.s.np * p.s.np;
  Carver c;
  for (int i = 0; i < 2; ++i) {
    p.x32[i] = c.take(nm * 4);
    p.xh[i] = c.take(nm * cs);
  }
  p.a = c.take(nn * cs);
  p.b = c.take(nn * cs);
  p.partial = c.take((size_t)batch * p.nblk * 4);
  p.sumsq = c.take(init_sumsq_floats(p.s, batch, cdt) * 4);
  p.scales = c.take((size_t)batch * 4 * 4);
  p.split_bytes = split_scratch(p.s, batch, cdt);
  p.split = c.take(p.split_bytes);
  p.total = c.off;
  return p;
}

struct GramPlan {
  Shape s;
  int32_t nblk;
  size_t xh[2], r, z, rz, q[2], partial, split, split_bytes, total;
};

GramPlan plan_gram(int64_t batch, int64_t rows, int64_t cols, int32_t cdt) {
  GramPlan p;
  p.s = canon(rows, cols);
  p.nblk = norm_blocks(rows * cols);
  const size_t cs = dt_size(cdt);
  const size_t nm = (size_t)batch * p.s.np * p.s.mp, nn = (size_t)batch * p.s.np * p.s.np;
  Carver c;
  for (int i = 0; i < 2; ++i) {
    p.xh[i] = c.take(nm * cs);
  }
  p.r = c.take(nn * cs);
  p.z = c.take(nn * cs);
  p.rz = c.take(nn * cs);
  p.q[0] = c.take(nn * cs);
  p.q[1] = c.take(nn * cs);
  p.partial = c.take((size_t)batch * p.nblk * 4);
  p.split_bytes = split_scratch(p.s, batch, cdt);
  p.split = c.take(p.split_bytes);
  p.total = c.off;
  return p;
}

// ---------------------------------------------------------------- timing --

struct Pending {
  int kclass;
  hipEvent_t start, stop;
};

struct Timing {
  std::mutex mu;
  std::atomic<uint32_t> mask{0};  // classes being timed (bit k = class k)
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  double total_ms[MSIGN_KCLASS_COUNT] = {0, 0, 0, 0};
  int64_t launches[MSIGN_KCLASS_COUNT] = {0, 0, 0, 0};
};

Timing& timing() {
  static Timing t;
  return t;
}

hipEvent_t pool_event(Timing& t) {
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one launch with events when timing is enabled.
struct TimedLaunch {
  int kclass;
  hipStream_t stream;
  hipEvent_t start = nullptr, stop = nullptr;
  TimedLaunch(int kc, hipStream_t s) : kclass(kc), stream(s) {
    Timing& t = timing();
    if (!((t.mask.load() >> kc) & 1u)) return;
    std::lock_guard<std::mutex> g(t.mu);
    start = pool_event(t);
    stop = pool_event(t);
    if (start && stop) (void)hipEventRecord(start, stream);
  }
  ~TimedLaunch() {
    if (!start || !stop) return;
    Timing& t = timing();
    (void)hipEventRecord(stop, stream);
    std::lock_guard<std::mutex> g(t.mu);
    t.pending.push_back({kclass, start, stop});
  }
};

enum KClass { KC_NORM = 0, KC_SYRK = 1, KC_SQUARE = 2, KC_RECT = 3 };

// --------------------------------------------------------------- launches --

// Tile configurations (measured on MI355X, 8192^2 bf16): 256 x 256 tiles
// with 16 waves of 64 x 64 (4 waves per SIMD hide LDS and MFMA latency; the
// 64 accumulators per lane stay in VGPRs; one block per CU) when the problem
// has at least one full round of such tiles for the 256 CUs, with 128-byte
// K slices (half the barriers of 64-byte slices) loaded straight into a
// 2-stage LDS ring (buffer_load ... lds); otherwise 128 x 128 tiles
// with 4 waves of 64 x 64 (two blocks per CU; 64-byte K slices, loaded the
// same way) if those fill the CUs, else 64 x 64 tiles shared along K by
// four waves (latency-bound problems; 64-byte K slices with two slices of
// register prefetch).
constexpr int kCUs = 256;
constexpr int kSplitMax = 8;

int tri_blocks(int tiles) {
  const int tv = tiles + (tiles & 1);
  return tv / 2 * (tv + 1);
}

// How one product launch is laid out: tile configuration, tiles, and the
// K split of the tiles past the last full round of resident blocks.
struct LaunchPlan {
  int bm;  // tile edge: 256, 128 or 64
  int32_t tiles_m, tiles_n, tpm;
  int64_t nt, nfull, tail;
  int32_t split;
  size_t partial_bytes;
};

LaunchPlan plan_launch(int64_t M, int64_t N, int64_t K, int64_t batch, bool tri, int32_t cdt) {
  LaunchPlan l;
  auto tiles_at = [&](int64_t e) {
    const int64_t tm = (M + e - 1) / e, t = tm * ((N + e - 1) / e);
    return (tri ? (t + tm) / 2 : t) * batch;
  };
  // the largest tile that still gives every CU a tile; 64 x 64 tiles (one
  // wave) when even 128 x 128 tiles leave CUs idle
  const int64_t kslices = K / (cdt == MSIGN_F32 ? 16 : 32);
  const int64_t t256 = tiles_at(256);
  bool big = t256 >= kCUs;
  if (!big && t256 > 0 && K >= 2048) {
    // long K: a K split of the big tiles that fills most CUs beats smaller
    // tiles (which would leave some CUs with two long tiles)
    int64_t sp = kCUs / t256;
    if (sp > kSplitMax) sp = kSplitMax;
    if (sp > kslices / 4) sp = kslices / 4;
    big = t256 * sp >= kCUs * 3 / 4;
  }
  l.bm = big ? 256 : (tiles_at(128) >= kCUs ? 128 : 64);
  // Blocks per CU that splitting the last round aims for (measured): one
  // 16-wave block of 256 x 256 keeps a CU busy; 4-wave 128 x 128 blocks
  // gain from two per CU.  A 64 x 64 tile is already shared along K by its
  // four waves.
  const int per_cu = l.bm == 128 ? 2 : 1;
  const int kwaves = l.bm == 64 ? 4 : 1;
  l.tiles_m = (int32_t)((M + l.bm - 1) / l.bm);
  l.tiles_n = (int32_t)((N + l.bm - 1) / l.bm);
  l.tpm = tri ? tri_blocks(l.tiles_m) : l.tiles_m * l.tiles_n;
  l.nt = (int64_t)l.tpm * batch;
  l.nfull = l.nt;
  l.tail = 0;
  l.split = 1;
  const int64_t slots = (int64_t)kCUs * per_cu;
  const int64_t rem = l.nt % slots;
  if (rem > 0) {
    int64_t sp = slots / rem;
    if (sp > kSplitMax) sp = kSplitMax;     // bounds the partial-sum traffic
    if (sp > kslices / (4 * kwaves)) sp = kslices / (4 * kwaves);  // >= 4 K slices per wave
    if (sp >= 2) {
      l.split = (int32_t)sp;
      l.tail = rem;
      l.nfull = l.nt - rem;
    }
  }
  l.partial_bytes = (size_t)l.tail * l.split * l.bm * l.bm * 4;
  return l;
}

template <typename T, int BM, int BN, int WGM, int WGN, int BKB, int NST, bool TRI, int KW, bool AT>
hipError_t launch_cfg(GemmParams q, const LaunchPlan& l, hipStream_t st) {
  q.tiles_m = l.tiles_m;
  q.tiles_n = l.tiles_n;
  q.tpm = l.tpm;
  q.nfull = (int32_t)l.nfull;
  q.split = l.split;
  const int64_t blocks = l.nfull + l.tail * l.split;
  if (blocks == 0) return hipSuccess;
  gemm_nt_kernel<T, BM, BN, WGM, WGN, BKB, NST, TRI, KW, AT>
      <<<dim3((unsigned)blocks), WGM * WGN * KW * 64, 0, st>>>(q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || l.tail == 0) return e;
  gemm_nt_reduce_kernel<T, BM, BN, WGM, WGN, TRI>
      <<<dim3((unsigned)(l.tail * WGM * WGN)), BM / WGM / 16 * 64, 0, st>>>(q);
  return hipGetLastError();
}

template <typename T, bool TRI>
hipError_t launch_nt_t(const GemmParams& q, const LaunchPlan& l, hipStream_t st) {
  static_assert(TRI, "rectangular products go through launch_nt_at");
  if (l.bm == 256) return launch_cfg<T, 256, 256, 4, 4, 128, 0, TRI, 1, false>(q, l, st);
  if (l.bm == 128) return launch_cfg<T, 128, 128, 2, 2, 64, 0, TRI, 1, false>(q, l, st);
  return launch_cfg<T, 64, 64, 1, 1, 64, 2, TRI, 4, false>(q, l, st);
}

// Rectangular products with P stored K-major (the iterate X, n x m, read
// as X^T).
template <typename T>
hipError_t launch_nt_at(const GemmParams& q, const LaunchPlan& l, hipStream_t st) {
  if (l.bm == 256) return launch_cfg<T, 256, 256, 4, 4, 128, 0, false, 1, true>(q, l, st);
  if (l.bm == 128) return launch_cfg<T, 128, 128, 2, 2, 64, 0, false, 1, true>(q, l, st);
  return launch_cfg<T, 64, 64, 1, 1, 64, 2, false, 4, true>(q, l, st);
}

// Launch one product: a triangle product (both operands read along K, P == Q
// symmetric or P Q^T symmetric) or a rectangular one with P stored K-major.
// `partial`/`partial_cap` is workspace for the K-split tail; with too little
// of it the tail is computed whole instead.
enum ProductKind { TRIANGLE, RECT_KMAJOR };

hipError_t launch_nt(int32_t cdt, ProductKind kind, GemmParams q, int64_t batch, hipStream_t st,
                     void* partial = nullptr, size_t partial_cap = 0) {
  const bool tri = kind == TRIANGLE;
  LaunchPlan l = plan_launch(q.M, q.N, q.K, batch, tri, cdt);
  if (l.tail > 0 && (partial == nullptr || partial_cap < l.partial_bytes)) {
    l.nfull = l.nt;
    l.tail = 0;
    l.split = 1;
  }
  q.partial = static_cast<float*>(partial);
  switch (cdt) {
    case MSIGN_BF16: return tri ? launch_nt_t<bf16_t, true>(q, l, st) : launch_nt_at<bf16_t>(q, l, st);
    case MSIGN_F16: return tri ? launch_nt_t<f16_t, true>(q, l, st) : launch_nt_at<f16_t>(q, l, st);
    default: return tri ? launch_nt_t<float, true>(q, l, st) : launch_nt_at<float>(q, l, st);
  }
}

// acc^2 slots (one per tile, wave and fragment row) of the A A launch.
int32_t sumsq_slots_per_tile(int bm) { return bm == 256 ? 16 * 4 : (bm == 128 ? 4 * 4 : 4); }

size_t init_sumsq_floats(const Shape& s, int64_t batch, int32_t cdt) {
  const LaunchPlan l = plan_launch(s.np, s.np, s.np, batch, true, cdt);
  return (size_t)l.nt * sumsq_slots_per_tile(l.bm);
}

// Largest K-split scratch any product of an NS or Gram call needs.
size_t split_scratch(const Shape& s, int64_t batch, int32_t cdt) {
  size_t b = 0;
  const LaunchPlan ls[3] = {plan_launch(s.np, s.np, s.mp, batch, true, cdt),
                            plan_launch(s.np, s.np, s.np, batch, true, cdt),
                            plan_launch(s.mp, s.np, s.np, batch, false, cdt)};
  for (const LaunchPlan& l : ls) b = l.partial_bytes > b ? l.partial_bytes : b;
  return b;
}

msign_status_t hip_fail(hipError_t e, const char* what) {
  return fail(MSIGN_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

GemmParams gemm_base(const void* P, int64_t ldp, int64_t sp, const void* Q, int64_t ldq, int64_t sq,
                     int64_t M, int64_t N, int64_t K, float alpha) {
  GemmParams g;
  std::memset(&g, 0, sizeof(g));
  g.P = P; g.ldp = ldp; g.sp = sp;
  g.Q = Q; g.ldq = ldq; g.sq = sq;
  g.M = (int32_t)M; g.N = (int32_t)N; g.K = (int32_t)K;
  g.alpha = alpha;
  g.beta = 0.f;
  g.Dt = nullptr;
  g.nout = 0;
  return g;
}

void set_d(GemmParams& g, const void* Dt, int64_t ldd, int64_t sd, int32_t dt, float beta, bool vec_ok) {
  g.Dt = Dt; g.ldd = ldd; g.sd = sd; g.d_dtype = dt; g.beta = beta; g.d_vec_ok = vec_ok ? 1 : 0;
}

void add_out(GemmParams& g, void* ptr, int64_t ld, int64_t bstride, int32_t dt, bool transposed,
             int64_t rows_lim, int64_t cols_lim, float diag, int64_t diag_lim, bool vec_ok) {
  OutSpec& o = g.out[g.nout++];
  o.ptr = ptr; o.ld = ld; o.bstride = bstride; o.dtype = dt; o.transposed = transposed ? 1 : 0;
  o.rows_lim = (int32_t)rows_lim; o.cols_lim = (int32_t)cols_lim;
  o.diag = diag; o.diag_lim = (int32_t)diag_lim; o.vec_ok = vec_ok ? 1 : 0;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + bn && pb < pa + an;
}

// Shared checks of msign_ns / msign_gram_ns.
msign_status_t check_common(const void* x, void* y, int64_t batch, int64_t rows, int64_t cols,
                            int32_t io_dtype, int32_t compute_dtype, int32_t steps,
                            const float* coeffs, float eps, bool* empty) {
  *empty = false;
  if (!dt_valid(io_dtype)) return fail(MSIGN_ERR_DTYPE, "io_dtype must be MSIGN_F32, MSIGN_BF16 or MSIGN_F16");
  if (!dt_valid(compute_dtype)) return fail(MSIGN_ERR_DTYPE, "compute_dtype must be MSIGN_F32, MSIGN_BF16 or MSIGN_F16");
  if (batch < 0 || rows < 0 || cols < 0) return fail(MSIGN_ERR_SHAPE, "batch, rows and cols must be >= 0");
  if (batch > kMaxBatch) return fail(MSIGN_ERR_SHAPE, "batch must be <= 65535");
  if (rows > kMaxDim || cols > kMaxDim) return fail(MSIGN_ERR_SHAPE, "rows and cols must be <= 2^20");
  if (steps < 1 || steps > MSIGN_MAX_STEPS) return fail(MSIGN_ERR_ARG, "steps must be in 1..64");
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(MSIGN_ERR_ARG, "eps must be finite and >= 0");
  if (coeffs) {
    for (int i = 0; i < 3 * steps; ++i)
      if (!std::isfinite(coeffs[i])) return fail(MSIGN_ERR_ARG, "coefficients must be finite");
  }
  if (batch == 0 || rows == 0 || cols == 0) {
    *empty = true;
    return MSIGN_OK;
  }
  const Shape s = canon(rows, cols);
  if ((double)batch * (double)s.np * (double)s.mp > 4.0e12)
    return fail(MSIGN_ERR_SHAPE, "problem too large");
  if (!x || !y) return fail(MSIGN_ERR_ARG, "x and y must be non-null");
  if (!aligned(x, dt_size(io_dtype)) || !aligned(y, dt_size(io_dtype)))
    return fail(MSIGN_ERR_ARG, "x and y must be aligned to their element size");
  return MSIGN_OK;
}

msign_status_t check_ws_alias(const void* x, void* y, size_t io_bytes, void* ws, size_t ws_bytes, size_t need) {
  if (!ws || ws_bytes < need)
    return fail(MSIGN_ERR_WORKSPACE, "workspace is null or smaller than the required " + std::to_string(need) + " bytes");
  if (!aligned(ws, 256)) return fail(MSIGN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (overlap(y, io_bytes, ws, need) || overlap(x, io_bytes, ws, need))
    return fail(MSIGN_ERR_ALIAS, "x or y overlaps the workspace");
  if (x != y && overlap(x, io_bytes, y, io_bytes))
    return fail(MSIGN_ERR_ALIAS, "y partially overlaps x (only y == x is allowed)");
  return MSIGN_OK;
}

// Sum of squares + scaled copies.  outs[k].transposed is relative to X
// (the wide orientation); converted here to the input's orientation.
msign_status_t launch_normalize(const void* x, int32_t io_dtype, int64_t batch, int64_t rows, int64_t cols,
                                const Shape& s, float* partial, int32_t nblk, float eps,
                                const NormOut* outs_x, int nout, hipStream_t st) {
  {
    TimedLaunch tl(KC_NORM, st);
    dim3 g1((unsigned)nblk, (unsigned)batch);
    sumsq_partial_kernel<256><<<g1, 256, 0, st>>>(x, io_dtype, rows * cols, nblk, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "sumsq_partial_kernel");
  }
  NormParams p;
  std::memset(&p, 0, sizeof(p));
  p.x = x;
  p.x_dtype = io_dtype;
  p.rows = rows;
  p.cols = cols;
  p.rows_pad = (int32_t)(s.tall ? s.mp : s.np);
  p.cols_pad = (int32_t)(s.tall ? s.np : s.mp);
  p.partial = partial;
  p.nblk = nblk;
  p.eps = eps;
  p.nout = nout;
  for (int k = 0; k < nout; ++k) {
    p.out[k] = outs_x[k];
    p.out[k].transposed = s.tall ? !outs_x[k].transposed : outs_x[k].transposed;
  }
  TimedLaunch tl(KC_NORM, st);
  dim3 g2((unsigned)((p.cols_pad + 63) / 64), (unsigned)((p.rows_pad + 63) / 64), (unsigned)batch);
  normalize_kernel<<<g2, 256, 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "normalize_kernel");
  return MSIGN_OK;
}

void coeff_at(const float* coeffs, int t, float* a, float* b, float* c) {
  const float* r = coeffs ? coeffs + 3 * t : kKeller;
  *a = r[0]; *b = r[1]; *c = r[2];
}

// Final output y (io dtype, user layout) of a product C' = X^T Z (m x n, C'
// [i][j] = X'[j][i]): wide -> y[j][i] (y is n x m, a transposed store),
// tall -> y[i][j] (y is m x n).
void add_final_out(GemmParams& g, void* y, const Shape& s, int32_t io_dtype) {
  const int64_t ld = s.tall ? s.n : s.m;
  const bool vec = !s.tall && (s.m % 4 == 0) && aligned(y, 4 * dt_size(io_dtype));
  add_out(g, y, ld, s.n * s.m, io_dtype, !s.tall, s.m, s.n, 0.f, 0, vec);
}

}  // namespace

extern "C" {

size_t msign_ns_workspace_bytes(int64_t batch, int64_t rows, int64_t cols, int32_t compute_dtype) {
  if (batch < 0 || rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim || batch > kMaxBatch ||
      !dt_valid(compute_dtype))
    return (size_t)-1;
  if (batch == 0 || rows == 0 || cols == 0) return 0;
  return plan_ns(batch, rows, cols, compute_dtype).total;
}

size_t msign_gram_ns_workspace_bytes(int64_t batch, int64_t rows, int64_t cols, int32_t compute_dtype) {
  if (batch < 0 || rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim || batch > kMaxBatch ||
      !dt_valid(compute_dtype))
    return (size_t)-1;
  if (batch == 0 || rows == 0 || cols == 0) return 0;
  return plan_gram(batch, rows, cols, compute_dtype).total;
}

msign_status_t msign_ns(const void* x, void* y, int64_t batch, int64_t rows, int64_t cols,
                        int32_t io_dtype, int32_t compute_dtype, int32_t steps, const float* coeffs,
                        float eps, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return msign_ns_ex(x, y, batch, rows, cols, io_dtype, compute_dtype, steps, coeffs, eps, 0u, workspace,
                     workspace_bytes, stream);
}

msign_status_t msign_ns_ex(const void* x, void* y, int64_t batch, int64_t rows, int64_t cols,
                           int32_t io_dtype, int32_t compute_dtype, int32_t steps, const float* coeffs,
                           float eps, uint32_t flags, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  g_err.clear();
  if (flags & ~(uint32_t)MSIGN_NS_IMPROVED_INIT) return fail(MSIGN_ERR_ARG, "unknown flag");
  const bool improved = (flags & MSIGN_NS_IMPROVED_INIT) != 0;
  bool empty = false;
  msign_status_t st = check_common(x, y, batch, rows, cols, io_dtype, compute_dtype, steps, coeffs, eps, &empty);
  if (st != MSIGN_OK || empty) return st;
  const NsPlan pl = plan_ns(batch, rows, cols, compute_dtype);
  const size_t io_bytes = (size_t)batch * rows * cols * dt_size(io_dtype);
  st = check_ws_alias(x, y, io_bytes, workspace, workspace_bytes, pl.total);
  if (st != MSIGN_OK) return st;

  const Shape& s = pl.s;
  const int32_t cdt = compute_dtype;
  const int64_t nm = s.np * s.mp, nn = s.np * s.np;
  void* x32[2] = {at(workspace, pl.x32[0]), at(workspace, pl.x32[1])};
  void* xh[2] = {at(workspace, pl.xh[0]), at(workspace, pl.xh[1])};
  void* A = at(workspace, pl.a);
  void* B = at(workspace, pl.b);
  float* partial = reinterpret_cast<float*>(at(workspace, pl.partial));
  float* sumsq = reinterpret_cast<float*>(at(workspace, pl.sumsq));
  float* scales = reinterpret_cast<float*>(at(workspace, pl.scales));
  void* split = at(workspace, pl.split);

  // X0 (n x m): in the compute dtype (the X X^T operand, also read K-major
  // as X^T by the update) and the fp32 master
  NormOut outs[2] = {
      {xh[0], s.mp, nm, cdt, 0},
      {x32[0], s.mp, nm, MSIGN_F32, 0},
  };
  st = launch_normalize(x, io_dtype, batch, rows, cols, s, partial, pl.nblk, eps, outs, 2, stream);
  if (st != MSIGN_OK) return st;

  for (int t = 0; t < steps; ++t) {
    float a, b, c;
    coeff_at(coeffs, t, &a, &b, &c);
    const int cur = t & 1, nxt = cur ^ 1;
    hipError_t e;
    {  // A = X X^T
      GemmParams g = gemm_base(xh[cur], s.mp, nm, xh[cur], s.mp, nm, s.np, s.np, s.mp, 1.f);
      add_out(g, A, s.np, nn, cdt, false, s.np, s.np, 0.f, 0, true);
      TimedLaunch tl(KC_SYRK, stream);
      e = launch_nt(cdt, TRIANGLE, g, batch, stream, split, pl.split_bytes);
      if (e != hipSuccess) return hip_fail(e, "X X^T");
    }
    // Improved initial normalisation (§改良初值), first step only: A2 = A A
    // into B with its acc^2 sums, s from them, B = (b/s^2) A + (c/s^4) A2,
    // and the update below scaled by 1/s.
    const bool rescale = improved && t == 0;
    if (rescale) {
      GemmParams g = gemm_base(A, s.np, nn, A, s.np, nn, s.np, s.np, s.np, 1.f);
      add_out(g, B, s.np, nn, cdt, false, s.np, s.np, 0.f, 0, true);
      g.sumsq = sumsq;
      {
        TimedLaunch tl(KC_SQUARE, stream);
        e = launch_nt(cdt, TRIANGLE, g, batch, stream, split, pl.split_bytes);
        if (e != hipSuccess) return hip_fail(e, "A A (first step)");
      }
      const LaunchPlan l = plan_launch(s.np, s.np, s.np, batch, true, cdt);
      g.tiles_m = l.tiles_m;
      g.tiles_n = l.tiles_n;
      g.tpm = l.tpm;
      TimedLaunch tl(KC_NORM, stream);
      init_scale_kernel<<<dim3((unsigned)batch), 256, 0, stream>>>(g, sumsq_slots_per_tile(l.bm), eps, scales);
      e = hipGetLastError();
      if (e != hipSuccess) return hip_fail(e, "init_scale_kernel");
      const unsigned nb = (unsigned)((nn / 4 + 255) / 256);
      init_combine_kernel<<<dim3(nb, (unsigned)batch), 256, 0, stream>>>(A, B, nn, cdt, b, c, scales);
      e = hipGetLastError();
      if (e != hipSuccess) return hip_fail(e, "init_combine_kernel");
    }
    // A cubic step (c = 0, "msign算子的Newton-Schulz迭代（上）" §迭代计算) has
    // B = b A: no A A product, and the next product takes A scaled by b.
    const bool cubic = (c == 0.f) && !rescale;
    if (!cubic && !rescale) {  // B = c A A + b A
      GemmParams g = gemm_base(A, s.np, nn, A, s.np, nn, s.np, s.np, s.np, c);
      set_d(g, A, s.np, nn, cdt, b, true);
      add_out(g, B, s.np, nn, cdt, false, s.np, s.np, 0.f, 0, true);
      TimedLaunch tl(KC_SQUARE, stream);
      e = launch_nt(cdt, TRIANGLE, g, batch, stream, split, pl.split_bytes);
      if (e != hipSuccess) return hip_fail(e, "c A A + b A");
    }
    {  // X' = B X + a X, as C' = X^T B + a X^T (m x n) with X read K-major;
       // C'[i][j] is stored at X'[j][i], four consecutive i per store
      GemmParams g = gemm_base(xh[cur], s.mp, nm, cubic ? A : B, s.np, nn, s.mp, s.np, s.np,
                               cubic ? b : 1.f);
      if (rescale) g.vscale = scales;
      set_d(g, x32[cur], s.mp, nm, MSIGN_F32, a, true);
      if (t + 1 < steps) {
        add_out(g, x32[nxt], s.mp, nm, MSIGN_F32, true, s.mp, s.np, 0.f, 0, true);
        add_out(g, xh[nxt], s.mp, nm, cdt, true, s.mp, s.np, 0.f, 0, true);
      } else {
        add_final_out(g, y, s, io_dtype);
      }
      TimedLaunch tl(KC_RECT, stream);
      e = launch_nt(cdt, RECT_KMAJOR, g, batch, stream, split, pl.split_bytes);
      if (e != hipSuccess) return hip_fail(e, "B X + a X");
    }
  }
  return MSIGN_OK;
}

msign_status_t msign_gram_ns(const void* x, void* y, int64_t batch, int64_t rows, int64_t cols,
                             int32_t io_dtype, int32_t compute_dtype, int32_t steps, const float* coeffs,
                             float eps, const int32_t* restart_after, int32_t n_restarts, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  if (n_restarts < 0 || (n_restarts > 0 && !restart_after) || (n_restarts == 0 && restart_after))
    return fail(MSIGN_ERR_ARG, "restart_after must be non-null exactly when n_restarts > 0");
  bool restart_at[MSIGN_MAX_STEPS + 1] = {false};
  if (steps >= 1 && steps <= MSIGN_MAX_STEPS) {
    int prev = 0;
    for (int i = 0; i < n_restarts; ++i) {
      const int r = restart_after[i];
      if (r <= prev || r >= steps)
        return fail(MSIGN_ERR_ARG, "restart_after must be strictly increasing within 1..steps-1");
      restart_at[r] = true;
      prev = r;
    }
  }
  bool empty = false;
  msign_status_t st = check_common(x, y, batch, rows, cols, io_dtype, compute_dtype, steps, coeffs, eps, &empty);
  if (st != MSIGN_OK || empty) return st;
  const GramPlan pl = plan_gram(batch, rows, cols, compute_dtype);
  const size_t io_bytes = (size_t)batch * rows * cols * dt_size(io_dtype);
  st = check_ws_alias(x, y, io_bytes, workspace, workspace_bytes, pl.total);
  if (st != MSIGN_OK) return st;

  const Shape& s = pl.s;
  const int32_t cdt = compute_dtype;
  const int64_t nm = s.np * s.mp, nn = s.np * s.np;
  void* xh[2] = {at(workspace, pl.xh[0]), at(workspace, pl.xh[1])};
  void* R = at(workspace, pl.r);
  void* Z = at(workspace, pl.z);
  void* RZ = at(workspace, pl.rz);
  void* Qb[2] = {at(workspace, pl.q[0]), at(workspace, pl.q[1])};
  float* partial = reinterpret_cast<float*>(at(workspace, pl.partial));
  void* split = at(workspace, pl.split);

  NormOut outs[1] = {{xh[0], s.mp, nm, cdt, 0}};
  st = launch_normalize(x, io_dtype, batch, rows, cols, s, partial, pl.nblk, eps, outs, 1, stream);
  if (st != MSIGN_OK) return st;

  hipError_t e;
  int cur = 0, qc = 0;
  auto gram_xxt = [&]() -> msign_status_t {
    GemmParams g = gemm_base(xh[cur], s.mp, nm, xh[cur], s.mp, nm, s.np, s.np, s.mp, 1.f);
    add_out(g, R, s.np, nn, cdt, false, s.np, s.np, 0.f, 0, true);
    TimedLaunch tl(KC_SYRK, stream);
    e = launch_nt(cdt, TRIANGLE, g, batch, stream, split, pl.split_bytes);
    return e == hipSuccess ? MSIGN_OK : hip_fail(e, "R = X X^T");
  };
  // tri product: out = P Q^T + beta D  (all n x n, symmetric)
  auto square = [&](const void* P, const void* Q, float alpha, const void* D, float beta, void* out,
                    void* out2, float diag2, const char* what) -> msign_status_t {
    GemmParams g = gemm_base(P, s.np, nn, Q, s.np, nn, s.np, s.np, s.np, alpha);
    if (D) set_d(g, D, s.np, nn, cdt, beta, true);
    add_out(g, out, s.np, nn, cdt, false, s.np, s.np, 0.f, 0, true);
    if (out2) add_out(g, out2, s.np, nn, cdt, false, s.np, s.np, diag2, s.n, true);
    TimedLaunch tl(KC_SQUARE, stream);
    e = launch_nt(cdt, TRIANGLE, g, batch, stream, split, pl.split_bytes);
    return e == hipSuccess ? MSIGN_OK : hip_fail(e, what);
  };

  st = gram_xxt();
  if (st != MSIGN_OK) return st;
  bool fresh = true;  // Q == I
  for (int t = 1; t <= steps; ++t) {
    float a, b, c;
    coeff_at(coeffs, t - 1, &a, &b, &c);
    const bool block_end = (t == steps) || restart_at[t];
    // Z = c R R + b R; on the first step of a block also Q = Z + a I
    st = square(R, R, c, R, b, Z, fresh ? Qb[qc] : nullptr, a, "Z = b R + c R^2");
    if (st != MSIGN_OK) return st;
    if (!fresh) {  // Q <- Q Z + a Q
      st = square(Qb[qc], Z, 1.f, Qb[qc], a, Qb[qc ^ 1], nullptr, 0.f, "Q <- Q Z + a Q");
      if (st != MSIGN_OK) return st;
      qc ^= 1;
    }
    fresh = false;
    if (!block_end) {
      st = square(R, Z, 1.f, R, a, RZ, nullptr, 0.f, "RZ <- R Z + a R");
      if (st != MSIGN_OK) return st;
      st = square(Z, RZ, 1.f, RZ, a, R, nullptr, 0.f, "R <- Z RZ + a RZ");
      if (st != MSIGN_OK) return st;
    }
    if (restart_at[t]) {  // X <- Q X, R = X X^T, Q = I
      // as C' = X^T Q (Q symmetric), stored transposed into the other X
      GemmParams g = gemm_base(xh[cur], s.mp, nm, Qb[qc], s.np, nn, s.mp, s.np, s.np, 1.f);
      add_out(g, xh[cur ^ 1], s.mp, nm, cdt, true, s.mp, s.np, 0.f, 0, true);
      {
        TimedLaunch tl(KC_RECT, stream);
        e = launch_nt(cdt, RECT_KMAJOR, g, batch, stream, split, pl.split_bytes);
        if (e != hipSuccess) return hip_fail(e, "restart X <- Q X");
      }
      cur ^= 1;
      st = gram_xxt();
      if (st != MSIGN_OK) return st;
      fresh = true;
    }
  }
  {  // y = Q X
    GemmParams g = gemm_base(xh[cur], s.mp, nm, Qb[qc], s.np, nn, s.mp, s.np, s.np, 1.f);
    add_final_out(g, y, s, io_dtype);
    TimedLaunch tl(KC_RECT, stream);
    e = launch_nt(cdt, RECT_KMAJOR, g, batch, stream, split, pl.split_bytes);
    if (e != hipSuccess) return hip_fail(e, "y = Q X");
  }
  return MSIGN_OK;
}

namespace {
// syrk_xxt workspace: [zero-padded copy of x, only when k is not a multiple
// of 64][K-split scratch for the last round of tiles, optional]
size_t syrk_pad_bytes(int64_t batch, int64_t n, int64_t k, int32_t dtype) {
  if (k % kPad == 0) return 0;
  return align256((size_t)batch * pad_up(n) * pad_up(k) * dt_size(dtype));
}
size_t syrk_split_bytes(int64_t batch, int64_t n, int64_t k, int32_t dtype) {
  return align256(plan_launch(n, n, pad_up(k), batch, true, dtype).partial_bytes);
}
}  // namespace

size_t syrk_xxt_workspace_bytes(int64_t batch, int64_t n, int64_t k, int32_t dtype) {
  if (batch < 0 || n < 0 || k < 0 || n > kMaxDim || k > kMaxDim || batch > kMaxBatch || !dt_valid(dtype))
    return (size_t)-1;
  if (batch == 0 || n == 0 || k == 0) return 0;
  return syrk_pad_bytes(batch, n, k, dtype) + syrk_split_bytes(batch, n, k, dtype);
}

msign_status_t syrk_xxt(const void* x, void* c, int64_t batch, int64_t n, int64_t k, int32_t dtype,
                        float alpha, const void* d, float beta, float gamma, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  if (!dt_valid(dtype)) return fail(MSIGN_ERR_DTYPE, "dtype must be MSIGN_F32, MSIGN_BF16 or MSIGN_F16");
  if (batch < 0 || n < 0 || k < 0) return fail(MSIGN_ERR_SHAPE, "batch, n and k must be >= 0");
  if (batch > kMaxBatch) return fail(MSIGN_ERR_SHAPE, "batch must be <= 65535");
  if (n > kMaxDim || k > kMaxDim) return fail(MSIGN_ERR_SHAPE, "n and k must be <= 2^20");
  if (!std::isfinite(alpha) || !std::isfinite(beta) || !std::isfinite(gamma))
    return fail(MSIGN_ERR_ARG, "alpha, beta and gamma must be finite");
  if (batch == 0 || n == 0) return MSIGN_OK;
  if (!c) return fail(MSIGN_ERR_ARG, "c must be non-null");
  const size_t es = dt_size(dtype);
  const size_t c_bytes = (size_t)batch * n * n * es;
  if (k > 0 && !x) return fail(MSIGN_ERR_ARG, "x must be non-null");
  if (!aligned(c, es) || (x && !aligned(x, es)) || (d && !aligned(d, es)))
    return fail(MSIGN_ERR_ARG, "buffers must be aligned to their element size");
  if (x && k > 0 && overlap(x, (size_t)batch * n * k * es, c, c_bytes))
    return fail(MSIGN_ERR_ALIAS, "c overlaps x");
  if (d && overlap(d, c_bytes, c, c_bytes)) return fail(MSIGN_ERR_ALIAS, "c overlaps d");
  // the product kernel reads K in whole 64-element slices from 16-byte
  // aligned rows; other inputs are first copied into a padded buffer
  const bool direct = (k % kPad == 0) && aligned(x, 16);
  const size_t pad_need = direct ? 0 : align256((size_t)batch * pad_up(n) * pad_up(k) * es);
  if (!direct && k > 0) {
    if (!workspace || workspace_bytes < pad_need)
      return fail(MSIGN_ERR_WORKSPACE, "workspace is null or smaller than the required " + std::to_string(pad_need) + " bytes");
  }
  if (workspace) {
    if (!aligned(workspace, 256)) return fail(MSIGN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (overlap(workspace, workspace_bytes, c, c_bytes) ||
        (x && k > 0 && overlap(workspace, workspace_bytes, x, (size_t)batch * n * k * es)) ||
        (d && overlap(workspace, workspace_bytes, d, c_bytes)))
      return fail(MSIGN_ERR_ALIAS, "workspace overlaps x, c or d");
  }
  // K-split scratch (optional): whatever workspace follows the padded copy
  void* split = nullptr;
  size_t split_cap = 0;
  if (workspace && workspace_bytes > pad_need) {
    split = at(workspace, pad_need);
    split_cap = workspace_bytes - pad_need;
  }

  const void* P = x;
  int64_t ldp = k, sp = n * k, K = k;
  if (k == 0) {
    P = c;  // never read: K = 0 means no K slices
    ldp = 0; sp = 0;
  } else if (!direct) {
    // copy into a zero-padded [batch][n][pad(k)] buffer (scale 1)
    const int64_t kp = pad_up(k), np = pad_up(n);
    NormParams p;
    std::memset(&p, 0, sizeof(p));
    p.x = x; p.x_dtype = dtype; p.rows = n; p.cols = k;
    p.rows_pad = (int32_t)np; p.cols_pad = (int32_t)kp;
    p.partial = nullptr; p.nblk = 0; p.eps = 0.f;
    p.out[0] = NormOut{workspace, kp, np * kp, dtype, 0};
    p.nout = 1;
    TimedLaunch tl(KC_NORM, stream);
    dim3 g2((unsigned)(kp / 64), (unsigned)(np / 64), (unsigned)batch);
    normalize_kernel<<<g2, 256, 0, stream>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "pad copy");
    P = workspace; ldp = kp; sp = np * kp; K = kp;
  }
  GemmParams g = gemm_base(P, ldp, sp, P, ldp, sp, n, n, K, alpha);
  const bool vec_c = (n % 4 == 0) && aligned(c, 4 * es);
  if (d && beta != 0.f) set_d(g, d, n, n * n, dtype, beta, (n % 4 == 0) && aligned(d, 4 * es));
  add_out(g, c, n, n * n, dtype, false, n, n, gamma, n, vec_c);
  TimedLaunch tl(KC_SYRK, stream);
  hipError_t e = launch_nt(dtype, TRIANGLE, g, batch, stream, split, split_cap);
  if (e != hipSuccess) return hip_fail(e, "syrk_xxt");
  return MSIGN_OK;
}

const char* msign_status_string(msign_status_t status) {
  switch (status) {
    case MSIGN_OK: return "ok";
    case MSIGN_ERR_ARG: return "invalid argument";
    case MSIGN_ERR_DTYPE: return "invalid or unsupported dtype";
    case MSIGN_ERR_SHAPE: return "invalid shape";
    case MSIGN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MSIGN_ERR_ALIAS: return "output overlaps input or workspace";
    case MSIGN_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* msign_last_error(void) { return g_err.c_str(); }

const char* msign_version(void) { return "msign 0.1.0 gfx950"; }

msign_status_t msign_kernel_timing_enable(int32_t enable) {
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  const uint32_t mask = (uint32_t)enable & ((1u << MSIGN_KCLASS_COUNT) - 1u);
  if (enable < 0 || (uint32_t)enable != mask) return fail(MSIGN_ERR_ARG, "unknown kernel class in mask");
  if (mask) {
    for (int k = 0; k < MSIGN_KCLASS_COUNT; ++k) {
      t.total_ms[k] = 0;
      t.launches[k] = 0;
    }
    t.mask.store(mask);
    return MSIGN_OK;
  }
  t.mask.store(0);
  for (auto& p : t.pending) {
    (void)hipEventSynchronize(p.stop);
    t.pool.push_back(p.start);
    t.pool.push_back(p.stop);
  }
  t.pending.clear();
  for (hipEvent_t e : t.pool) (void)hipEventDestroy(e);
  t.pool.clear();
  return MSIGN_OK;
}

msign_status_t msign_kernel_timing_read(double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return fail(MSIGN_ERR_ARG, "total_ms and launches must be non-null");
  Timing& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  for (auto& p : t.pending) {
    hipError_t e = hipEventSynchronize(p.stop);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.start, p.stop);
    if (e != hipSuccess) {
      g_err = std::string("event timing: ") + hipGetErrorString(e);
      return MSIGN_ERR_HIP;
    }
    t.total_ms[p.kclass] += ms;
    t.launches[p.kclass] += 1;
    t.pool.push_back(p.start);
    t.pool.push_back(p.stop);
  }
  t.pending.clear();
  for (int k = 0; k < MSIGN_KCLASS_COUNT; ++k) {
    total_ms[k] = t.total_ms[k];
    launches[k] = t.launches[k];
  }
  return MSIGN_OK;
}

}  // extern "C"

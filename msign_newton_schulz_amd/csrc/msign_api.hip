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
//   X' = B X + a X             rectangular product, computed as X^T B + a X^T
//                              with X read K-major, D = X (fp32)
// X is carried in fp32 between steps (X32, n x m), together with a
// compute-dtype copy Xh (n x m) that feeds the products (both ping-pong).
// Rounding only the product operands, not the iterate, keeps the small
// singular directions of spiked (momentum-like) matrices intact.
//
// Gram NS ("Gram Newton-Schulz" §3.4 Algorithm 2, §2.3 Algorithm 1) keeps
// everything in the compute dtype as the page does (§3.3), with the a_t
// terms applied in fp32 epilogues.
#include "../../include/msign.h"
#include "common.hpp"
#include "gemm_nt.hpp"
#include "init_scale.hpp"
#include "launch.hpp"
#include "mfma_probe.hpp"
#include "normalize.hpp"
#include "small_ns.hpp"

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

struct Prob;
// K-split scratch of the products of one NS or Gram call, and the acc^2
// slots of the first A A product (defined below).
size_t split_scratch(const Prob* pr, int ng, int32_t cdt);
size_t init_sumsq_floats(const Shape& s, int64_t batch);

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

// A Muon step fused around msign (see muon_run): the msign input x is the
// fp32 momentum M, which the sum-of-squares pass updates in place to
// fmaf(mu, M, G) before normalising it; the output y is the parameter W,
// which the last product's epilogue updates in place, W <- W - lr msign(M).
struct Fuse {
  const void* g;
  int32_t g_dtype;
  float mu, lr;
};

// One problem of a (grouped) call: batch matrices of rows x cols; y in
// y_dtype (the io dtype, except in a fused Muon step).
struct Prob {
  const void* x;
  void* y;
  int64_t batch, rows, cols;
  Shape s;
  int32_t y_dtype;
  const Fuse* fuse;  // null: a plain msign
};

// Workspace regions of one problem of an NS call (offsets from the call's
// workspace base).  `split` is the K-split scratch of the call's launches:
// the problem's own when it is alone, else one region shared by all.
struct NsPlan {
  int32_t nblk;
  size_t x32[2], xh[2], a, b, partial, sumsq, scales, nscales;
};

struct GramPlan {
  int32_t nblk;
  size_t xh[2], r, z, rz, q[2], partial, scales;
};

template <typename P>
struct CallPlan {
  int ng;
  P p[MSIGN_MAX_GROUPS];
  size_t split, split_bytes, total;
};

void plan_ns_regions(const Prob& pr, int32_t cdt, Carver& c, NsPlan& p) {
  p.nblk = norm_blocks(pr.rows * pr.cols);
  const size_t cs = dt_size(cdt);
  const size_t nm = (size_t)pr.batch * pr.s.np * pr.s.mp, nn = (size_t)pr.batch * pr.s.np * pr.s.np;
  for (int i = 0; i < 2; ++i) {
    p.x32[i] = c.take(nm * 4);
    p.xh[i] = c.take(nm * cs);
  }
  p.a = c.take(nn * cs);
  p.b = c.take(nn * cs);
  p.partial = c.take((size_t)pr.batch * p.nblk * 4);
  p.sumsq = c.take(init_sumsq_floats(pr.s, pr.batch) * 4);
  p.scales = c.take((size_t)pr.batch * 4 * 4);
  p.nscales = c.take((size_t)pr.batch * 4 * 4);
}

void plan_gram_regions(const Prob& pr, int32_t cdt, Carver& c, GramPlan& p) {
  p.nblk = norm_blocks(pr.rows * pr.cols);
  const size_t cs = dt_size(cdt);
  const size_t nm = (size_t)pr.batch * pr.s.np * pr.s.mp, nn = (size_t)pr.batch * pr.s.np * pr.s.np;
  for (int i = 0; i < 2; ++i) p.xh[i] = c.take(nm * cs);
  p.r = c.take(nn * cs);
  p.z = c.take(nn * cs);
  p.rz = c.take(nn * cs);
  p.q[0] = c.take(nn * cs);
  p.q[1] = c.take(nn * cs);
  p.partial = c.take((size_t)pr.batch * p.nblk * 4);
  p.scales = c.take((size_t)pr.batch * 4 * 4);
}

// Every problem's regions, one after the other, then the K-split scratch.
template <typename P, typename F>
CallPlan<P> plan_call(const Prob* pr, int ng, int32_t cdt, F regions) {
  CallPlan<P> cp;
  cp.ng = ng;
  Carver c;
  for (int i = 0; i < ng; ++i) regions(pr[i], cdt, c, cp.p[i]);
  cp.split_bytes = split_scratch(pr, ng, cdt);
  cp.split = c.take(cp.split_bytes);
  cp.total = c.off;
  return cp;
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
  double total_ms[MSIGN_KCLASS_COUNT] = {};
  int64_t launches[MSIGN_KCLASS_COUNT] = {};
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
// Set while a call that may allocate nothing runs on this thread: its
// launches are never bracketed by (created) events.
thread_local bool g_untimed = false;

struct TimedLaunch {
  int kclass;
  hipStream_t stream;
  hipEvent_t start = nullptr, stop = nullptr;
  TimedLaunch(int kc, hipStream_t s) : kclass(kc), stream(s) {
    Timing& t = timing();
    if (g_untimed || !((t.mask.load() >> kc) & 1u)) return;
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

enum KClass { KC_NORM = 0, KC_SYRK = 1, KC_SQUARE = 2, KC_RECT = 3, KC_SMALL = 4 };

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

// Sizes of one group of a product launch: C (M x N per matrix) over
// `batch` matrices, K the padded contraction length.
struct Dims {
  int64_t M, N, K, batch;
};

GroupPlan plan_groups(const Dims* d, int ng, bool tri, int32_t cdt) {
  GroupPlan l;
  std::memset(&l, 0, sizeof(l));
  l.ng = ng;
  for (int i = 0; i < ng; ++i) l.order[i] = i;
  for (int i = 1; i < ng; ++i)  // stable: equal K keeps the caller's order
    for (int j = i; j > 0 && d[l.order[j]].K > d[l.order[j - 1]].K; --j) std::swap(l.order[j], l.order[j - 1]);
  auto tiles_at = [&](const Dims& x, int64_t e) {
    const int64_t tm = (x.M + e - 1) / e, t = tm * ((x.N + e - 1) / e);
    return (tri ? (t + tm) / 2 : t) * x.batch;
  };
  int64_t t256 = 0, t128 = 0;
  for (int i = 0; i < ng; ++i) {
    t256 += tiles_at(d[i], 256);
    t128 += tiles_at(d[i], 128);
  }
  const Dims& last = d[l.order[ng - 1]];  // shortest K
  // the largest tile that still gives every CU a tile; 64 x 64 tiles (one
  // wave) when even 128 x 128 tiles leave CUs idle
  const int64_t kslices = last.K / (cdt == MSIGN_F32 ? 16 : 32);
  bool big = t256 >= kCUs;
  if (!big && t256 > 0 && last.K >= 2048) {
    // long K: a K split of the big tiles that fills most CUs beats smaller
    // tiles (which would leave some CUs with two long tiles)
    int64_t sp = kCUs / t256;
    if (sp > kSplitMax) sp = kSplitMax;
    if (sp > kslices / 4) sp = kslices / 4;
    big = t256 * sp >= kCUs * 3 / 4;
  }
  l.bm = big ? 256 : (t128 >= kCUs ? 128 : 64);
  // Blocks per CU that splitting the last round aims for (measured): one
  // 16-wave block of 256 x 256 keeps a CU busy; 4-wave 128 x 128 blocks
  // gain from two per CU.  A 64 x 64 tile is already shared along K by its
  // four waves.
  const int per_cu = l.bm == 128 ? 2 : 1;
  const int kwaves = l.bm == 64 ? 4 : 1;
  int64_t ntot = 0;
  for (int i = 0; i < ng; ++i) {
    l.tiles_m[i] = (int32_t)((d[i].M + l.bm - 1) / l.bm);
    l.tiles_n[i] = (int32_t)((d[i].N + l.bm - 1) / l.bm);
    l.tpm[i] = tri ? tri_blocks(l.tiles_m[i]) : l.tiles_m[i] * l.tiles_n[i];
    l.nt[i] = (int64_t)l.tpm[i] * d[i].batch;
    ntot += l.nt[i];
  }
  l.tail = 0;
  l.split = 1;
  const int64_t slots = (int64_t)kCUs * per_cu;
  const int64_t rem = ntot % slots;
  const int64_t nlast = l.nt[l.order[ng - 1]];
  if (rem > 0 && nlast > 0) {
    // the last round: rem tiles, of which the last group's are split into
    // the slots the whole tiles before them leave free
    const int64_t tail = rem < nlast ? rem : nlast;
    int64_t sp = (slots - (rem - tail)) / tail;
    if (sp > kSplitMax) sp = kSplitMax;     // bounds the partial-sum traffic
    if (sp > kslices / (4 * kwaves)) sp = kslices / (4 * kwaves);  // >= 4 K slices per wave
    if (sp >= 2) {
      l.split = (int32_t)sp;
      l.tail = tail;
    }
  }
  l.partial_bytes = (size_t)l.tail * l.split * l.bm * l.bm * 4;
  return l;
}

// The one-group view of a launch (workspace sizing of single problems).
struct LaunchPlan {
  int bm;
  int32_t tiles_m, tiles_n, tpm;
  int64_t nt, tail;
  int32_t split;
  size_t partial_bytes;
};

LaunchPlan plan_launch(int64_t M, int64_t N, int64_t K, int64_t batch, bool tri, int32_t cdt) {
  const Dims d{M, N, K, batch};
  const GroupPlan g = plan_groups(&d, 1, tri, cdt);
  LaunchPlan l;
  l.bm = g.bm;
  l.tiles_m = g.tiles_m[0];
  l.tiles_n = g.tiles_n[0];
  l.tpm = g.tpm[0];
  l.nt = g.nt[0];
  l.tail = g.tail;
  l.split = g.split;
  l.partial_bytes = g.partial_bytes;
  return l;
}

static_assert(kMaxGroups == MSIGN_MAX_GROUPS, "group table size");

// Launch one product over ng groups (1..MSIGN_MAX_GROUPS, each with its own
// operands, sizes and batch): a triangle product (both operands read along
// K, P == Q symmetric or P Q^T symmetric) or a rectangular one with P stored
// K-major.  `partial`/`partial_cap` is workspace for the K-split tail; with
// too little of it the tail is computed whole instead.
// DENSE: every tile of P Q^T with both operands read along K (the
// measurement comparator of the triangle products; one group only).
enum ProductKind { TRIANGLE, RECT_KMAJOR, DENSE };

Dims dims_of(const GemmParams& q, int64_t batch) { return Dims{q.M, q.N, q.K, batch}; }

hipError_t launch_grouped(int32_t cdt, ProductKind kind, GemmParams* qs, const int64_t* batches, int ng,
                          hipStream_t st, void* partial, size_t partial_cap, GroupPlan* used = nullptr) {
  const bool tri = kind == TRIANGLE;
  Dims d[MSIGN_MAX_GROUPS];
  for (int i = 0; i < ng; ++i) d[i] = dims_of(qs[i], batches[i]);
  GroupPlan l = plan_groups(d, ng, tri, cdt);
  if (l.tail > 0 && (partial == nullptr || partial_cap < l.partial_bytes)) {
    l.tail = 0;
    l.split = 1;
  }
  for (int i = 0; i < ng; ++i) qs[i].partial = static_cast<float*>(partial);
  if (used) *used = l;
  if (kind == DENSE) return launch_products_dense(cdt, qs, l, st);
  return ng == 1 ? launch_products_single(cdt, tri, qs, l, st) : launch_products_grouped(cdt, tri, qs, l, st);
}

hipError_t launch_nt(int32_t cdt, ProductKind kind, GemmParams q, int64_t batch, hipStream_t st,
                     void* partial = nullptr, size_t partial_cap = 0) {
  return launch_grouped(cdt, kind, &q, &batch, 1, st, partial, partial_cap);
}

// acc^2 slots (one per tile, wave and fragment row) of the A A launch.
int32_t sumsq_slots_per_tile(int bm) { return bm == 256 ? 16 * 4 : (bm == 128 ? 4 * 4 : 4); }

// Room for the acc^2 slots of an A A launch at any tile size (a grouped
// launch may pick another tile size than the problem alone would).
size_t init_sumsq_floats(const Shape& s, int64_t batch) {
  size_t most = 0;
  for (int bm = 64; bm <= 256; bm *= 2) {
    const size_t n = (size_t)tri_blocks((int)((s.np + bm - 1) / bm)) * batch * sumsq_slots_per_tile(bm);
    most = n > most ? n : most;
  }
  return most;
}

// Largest K-split scratch any product of an NS or Gram call over these
// problems needs (X X^T, the n x n products and the update).
size_t split_scratch(const Prob* pr, int ng, int32_t cdt) {
  Dims d[3][MSIGN_MAX_GROUPS];
  for (int i = 0; i < ng; ++i) {
    const Shape& s = pr[i].s;
    d[0][i] = Dims{s.np, s.np, s.mp, pr[i].batch};
    d[1][i] = Dims{s.np, s.np, s.np, pr[i].batch};
    d[2][i] = Dims{s.mp, s.np, s.np, pr[i].batch};
  }
  size_t b = 0;
  for (int k = 0; k < 3; ++k) {
    const size_t v = plan_groups(d[k], ng, k < 2, cdt).partial_bytes;
    b = v > b ? v : b;
  }
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
                            int32_t io_dtype, int32_t y_dtype, int32_t compute_dtype, int32_t steps,
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
  if (!aligned(x, dt_size(io_dtype)) || !aligned(y, dt_size(y_dtype)))
    return fail(MSIGN_ERR_ARG, "x and y must be aligned to their element size");
  return MSIGN_OK;
}

msign_status_t check_ws_alias(const void* x, size_t x_bytes, void* y, size_t y_bytes, void* ws, size_t ws_bytes,
                              size_t need) {
  if (!ws || ws_bytes < need)
    return fail(MSIGN_ERR_WORKSPACE, "workspace is null or smaller than the required " + std::to_string(need) + " bytes");
  if (!aligned(ws, 256)) return fail(MSIGN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (overlap(y, y_bytes, ws, need) || overlap(x, x_bytes, ws, need))
    return fail(MSIGN_ERR_ALIAS, "x or y overlaps the workspace");
  if (x != y && overlap(x, x_bytes, y, y_bytes))
    return fail(MSIGN_ERR_ALIAS, "y partially overlaps x (only y == x is allowed)");
  return MSIGN_OK;
}

// The first products may read the input itself instead of normalised
// copies: a wide matrix (no transpose) already in the compute dtype, whose
// rows are whole 64-element K slices (cols a multiple of 64) starting on 16
// bytes.  The normalisation X0 = X / s then becomes per-matrix factors of
// those products' epilogues: 1/s^2 for the first X X^T and 1/s for the first
// product with X (the rectangular step, or Gram's Q X), applied in fp32 to
// the accumulated values.  Not with a fused Muon step (its input is the fp32
// momentum).  With the improved initial normalisation, its first-step factor
// for the update is multiplied by 1/s.
bool direct_input(const Prob& pr, int32_t io_dtype, int32_t cdt) {
  return !pr.s.tall && io_dtype == cdt && pr.s.m % kPad == 0 && aligned(pr.x, 16) && pr.fuse == nullptr;
}

// Sum of squares, then the per-matrix factors of a direct first step into
// nscale[4 b] (1/s^2) and nscale[4 b + 1] (1/s).
msign_status_t launch_norm_scale(const void* x, int32_t io_dtype, int64_t batch, int64_t count, float* partial,
                                 int32_t nblk, float eps, float* nscale, hipStream_t st) {
  TimedLaunch tl(KC_NORM, st);
  dim3 g1((unsigned)nblk, (unsigned)batch);
  sumsq_partial_kernel<256><<<g1, 256, 0, st>>>(x, io_dtype, count, nblk, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "sumsq_partial_kernel");
  norm_scale_kernel<<<dim3((unsigned)batch), 256, 0, st>>>(partial, nblk, eps, nscale);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "norm_scale_kernel");
  return MSIGN_OK;
}

// Sum of squares + scaled copies.  outs[k].transposed is relative to X
// (the wide orientation); converted here to the input's orientation.
msign_status_t launch_normalize(const void* x, int32_t io_dtype, int64_t batch, int64_t rows, int64_t cols,
                                const Shape& s, float* partial, int32_t nblk, float eps,
                                const NormOut* outs_x, int nout, hipStream_t st, const Fuse* fuse = nullptr) {
  {
    TimedLaunch tl(KC_NORM, st);
    dim3 g1((unsigned)nblk, (unsigned)batch);
    if (fuse)  // x is the fp32 momentum: M <- mu M + G first (Muon step)
      sumsq_partial_kernel<256, true>
          <<<g1, 256, 0, st>>>(x, io_dtype, rows * cols, nblk, partial, fuse->g, fuse->g_dtype, fuse->mu);
    else
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
  // no transposed output and whole 16-byte chunks per input row: the
  // direct kernel (no LDS tile), else the tiled one
  bool direct = (reinterpret_cast<uintptr_t>(x) & 15) == 0 && cols % (io_dtype == MSIGN_F32 ? 4 : 8) == 0 &&
                p.cols_pad % 8 == 0;
  for (int k = 0; k < nout; ++k)
    direct = direct && !p.out[k].transposed && p.out[k].ld % 8 == 0 && p.out[k].bstride % 8 == 0 &&
             aligned(p.out[k].ptr, 16);
  TimedLaunch tl(KC_NORM, st);
  if (direct) {
    dim3 g3((unsigned)((p.cols_pad + 255) / 256), (unsigned)((p.rows_pad + 63) / 64), (unsigned)batch);
    normalize_direct_kernel<<<g3, 256, 0, st>>>(p);
  } else {
    dim3 g2((unsigned)((p.cols_pad + 63) / 64), (unsigned)((p.rows_pad + 63) / 64), (unsigned)batch);
    normalize_kernel<<<g2, 256, 0, st>>>(p);
  }
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
// A fused Muon step updates y (the parameters) in place: y <- y - lr C.
void add_final_out(GemmParams& g, const Prob& pr) {
  const Shape& s = pr.s;
  const int64_t ld = s.tall ? s.n : s.m;
  const bool vec = !s.tall && (s.m % 4 == 0) && aligned(pr.y, 4 * dt_size(pr.y_dtype));
  add_out(g, pr.y, ld, s.n * s.m, pr.y_dtype, !s.tall, s.m, s.n, 0.f, 0, vec);
  if (pr.fuse) {
    g.out[g.nout - 1].update = 1;
    g.out[g.nout - 1].axpy = -pr.fuse->lr;
  }
}

}  // namespace

namespace {

// Non-empty problems of a call, checked one by one; `*ng` of them.
msign_status_t gather(const msign_group_t* groups, int32_t ngroups, int32_t io_dtype, int32_t cdt,
                      int32_t steps, const float* coeffs, float eps, Prob* pr, int* ng, int32_t y_dtype = -1,
                      const Fuse* fuse = nullptr) {
  *ng = 0;
  if (y_dtype < 0) y_dtype = io_dtype;
  if (ngroups < 1 || ngroups > MSIGN_MAX_GROUPS)
    return fail(MSIGN_ERR_ARG, "ngroups must be in 1.." + std::to_string(MSIGN_MAX_GROUPS));
  if (!groups) return fail(MSIGN_ERR_ARG, "groups must be non-null");
  for (int i = 0; i < ngroups; ++i) {
    const msign_group_t& g = groups[i];
    bool empty = false;
    msign_status_t st =
        check_common(g.x, g.y, g.batch, g.rows, g.cols, io_dtype, y_dtype, cdt, steps, coeffs, eps, &empty);
    if (st != MSIGN_OK) return ngroups > 1 ? fail(st, "group " + std::to_string(i) + ": " + g_err) : st;
    if (empty) continue;
    Prob& p = pr[(*ng)++];
    p.x = g.x; p.y = g.y; p.batch = g.batch; p.rows = g.rows; p.cols = g.cols;
    p.s = canon(g.rows, g.cols);
    p.y_dtype = y_dtype;
    p.fuse = fuse ? &fuse[i] : nullptr;
  }
  return MSIGN_OK;
}

// Workspace size and alignment, no input or output inside it, y == x or
// apart within a problem, and no problem's output overlapping another
// problem's input or output.
msign_status_t check_call_ws(const Prob* pr, int ng, int32_t io_dtype, void* ws, size_t ws_bytes, size_t need) {
  auto bytes = [&](const Prob& p, int32_t dt) { return (size_t)p.batch * p.rows * p.cols * dt_size(dt); };
  for (int i = 0; i < ng; ++i) {
    const size_t xi = bytes(pr[i], io_dtype), yi = bytes(pr[i], pr[i].y_dtype);
    msign_status_t st = check_ws_alias(pr[i].x, xi, pr[i].y, yi, ws, ws_bytes, need);
    if (st != MSIGN_OK) return st;
    for (int j = 0; j < ng; ++j) {
      if (j == i) continue;
      if (overlap(pr[i].y, yi, pr[j].x, bytes(pr[j], io_dtype)) ||
          overlap(pr[i].y, yi, pr[j].y, bytes(pr[j], pr[j].y_dtype)))
        return fail(MSIGN_ERR_ALIAS, "the output of one group overlaps the input or output of another");
    }
  }
  return MSIGN_OK;
}

// Matrices with n <= 64 fit one 64-wide tile along n.  Their iteration is
// bound by launch latency, not by the products, so their products run in
// fp32 whatever the compute dtype: at no cost in time, and with 16-bit
// operands the iteration misses its tolerance on vector-like inputs (a 1 x m
// matrix is the scalar map x <- (a + b + c) x at x = 1, where a + b + c =
// 0.70 is a cancellation of 3.44 against -2.74 that magnifies the rounding
// of B).
constexpr int64_t kFp32MaxN = 64;

// The problems of a call, split by the dtype their products use: sub-call 0
// in the compute dtype, sub-call 1 (n <= 64) in fp32, each a grouped call of
// its own with its own workspace region (sub-call 0's first).
struct SubCalls {
  int n[2];
  Prob p[2][MSIGN_MAX_GROUPS];
  int32_t cdt[2];
  size_t off[2], total;
};

template <typename P, typename F>
SubCalls split_call(const Prob* pr, int ng, int32_t cdt, F regions) {
  SubCalls sc;
  sc.n[0] = sc.n[1] = 0;
  sc.cdt[0] = cdt;
  sc.cdt[1] = MSIGN_F32;
  for (int i = 0; i < ng; ++i) {
    const int k = (cdt != MSIGN_F32 && pr[i].s.n <= kFp32MaxN) ? 1 : 0;
    sc.p[k][sc.n[k]++] = pr[i];
  }
  size_t off = 0;
  for (int k = 0; k < 2; ++k) {
    sc.off[k] = off;
    if (sc.n[k] > 0) off = align256(off + plan_call<P>(sc.p[k], sc.n[k], sc.cdt[k], regions).total);
  }
  sc.total = off;
  return sc;
}

size_t call_workspace(const msign_group_t* groups, int32_t ngroups, int32_t cdt, bool gram) {
  if (ngroups < 1 || ngroups > MSIGN_MAX_GROUPS || !groups || !dt_valid(cdt)) return (size_t)-1;
  Prob pr[MSIGN_MAX_GROUPS];
  int ng = 0;
  for (int i = 0; i < ngroups; ++i) {
    const msign_group_t& g = groups[i];
    if (g.batch < 0 || g.rows < 0 || g.cols < 0 || g.rows > kMaxDim || g.cols > kMaxDim || g.batch > kMaxBatch)
      return (size_t)-1;
    if (g.batch == 0 || g.rows == 0 || g.cols == 0) continue;
    Prob& p = pr[ng++];
    p.batch = g.batch; p.rows = g.rows; p.cols = g.cols;
    p.s = canon(g.rows, g.cols);
  }
  if (ng == 0) return 0;
  return gram ? split_call<GramPlan>(pr, ng, cdt, plan_gram_regions).total
              : split_call<NsPlan>(pr, ng, cdt, plan_ns_regions).total;
}

// The launches of standard NS over checked problems pr[0..ng), all of whose
// products use compute dtype `cdt`, in a workspace laid out by plan_call.
// The whole iteration of each matrix in one workgroup (small_ns_kernel),
// for problems that fit it: 64 < n <= 128, m padded <= 256, 16-bit products.
bool small_fits(const Prob& pr, int32_t cdt) {
  return (cdt == MSIGN_BF16 || cdt == MSIGN_F16) && pr.s.np == kSmallN && pr.s.mp <= kSmallMaxM &&
         pr.fuse == nullptr;
}

msign_status_t launch_small(const Prob& pr, int32_t io_dtype, int32_t cdt, int32_t steps, const float* coeffs,
                            float eps, hipStream_t stream) {
  SmallNsParams q;
  std::memset(&q, 0, sizeof(q));
  q.x = pr.x;
  q.y = pr.y;
  q.rows = (int32_t)pr.rows;
  q.cols = (int32_t)pr.cols;
  q.n = (int32_t)pr.s.n;
  q.m = (int32_t)pr.s.m;
  q.mp = (int32_t)pr.s.mp;
  q.tall = pr.s.tall ? 1 : 0;
  q.io_dtype = io_dtype;
  q.steps = steps;
  q.eps = eps;
  for (int t = 0; t < steps; ++t) coeff_at(coeffs, t, &q.abc[t][0], &q.abc[t][1], &q.abc[t][2]);
  TimedLaunch tl(KC_SMALL, stream);
  if (cdt == MSIGN_BF16)
    small_ns_kernel<bf16_t><<<dim3((unsigned)pr.batch), kSmallThreads, 0, stream>>>(q);
  else
    small_ns_kernel<f16_t><<<dim3((unsigned)pr.batch), kSmallThreads, 0, stream>>>(q);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MSIGN_OK : hip_fail(e, "small_ns_kernel");
}

msign_status_t ns_exec(const Prob* pr, int ng, int32_t io_dtype, int32_t cdt, int32_t steps, const float* coeffs,
                       float eps, bool improved, bool dense, void* workspace, hipStream_t stream) {
  if (!improved && !dense) {
    // small problems run alone in one launch each; the others go on below
    Prob rest[MSIGN_MAX_GROUPS];
    int nr = 0;
    for (int i = 0; i < ng; ++i) {
      if (small_fits(pr[i], cdt)) {
        msign_status_t st = launch_small(pr[i], io_dtype, cdt, steps, coeffs, eps, stream);
        if (st != MSIGN_OK) return st;
      } else {
        rest[nr++] = pr[i];
      }
    }
    if (nr < ng) {
      return nr == 0 ? MSIGN_OK
                     : ns_exec(rest, nr, io_dtype, cdt, steps, coeffs, eps, improved, dense, workspace, stream);
    }
  }
  // symmetric n x n results: triangle products, or (dense) every tile with
  // the result stored through its transpose, the same matrix
  const ProductKind sym = dense ? DENSE : TRIANGLE;
  const CallPlan<NsPlan> cp = plan_call<NsPlan>(pr, ng, cdt, plan_ns_regions);
  msign_status_t st = MSIGN_OK;

  void* split = at(workspace, cp.split);
  struct G {
    Shape s;
    int64_t nm, nn;
    void *x32[2], *xh[2], *A, *B;
    float *partial, *sumsq, *scales;  // scales: the improved initial normalisation's
    float* nscales;  // 1/s^2, 1/s of a direct first step
    bool direct;     // the first products read the input itself
  } gv[MSIGN_MAX_GROUPS];
  int64_t batches[MSIGN_MAX_GROUPS];
  for (int i = 0; i < ng; ++i) {
    const NsPlan& pl = cp.p[i];
    G& v = gv[i];
    v.s = pr[i].s;
    v.nm = v.s.np * v.s.mp;
    v.nn = v.s.np * v.s.np;
    for (int k = 0; k < 2; ++k) {
      v.x32[k] = at(workspace, pl.x32[k]);
      v.xh[k] = at(workspace, pl.xh[k]);
    }
    v.A = at(workspace, pl.a);
    v.B = at(workspace, pl.b);
    v.partial = reinterpret_cast<float*>(at(workspace, pl.partial));
    v.sumsq = reinterpret_cast<float*>(at(workspace, pl.sumsq));
    v.scales = reinterpret_cast<float*>(at(workspace, pl.scales));
    v.nscales = reinterpret_cast<float*>(at(workspace, pl.nscales));
    batches[i] = pr[i].batch;
    v.direct = direct_input(pr[i], io_dtype, cdt);
    if (v.direct) {
      st = launch_norm_scale(pr[i].x, io_dtype, pr[i].batch, pr[i].rows * pr[i].cols, v.partial, pl.nblk, eps,
                             v.nscales, stream);
      if (st != MSIGN_OK) return st;
      continue;
    }
    // X0 (n x m): in the compute dtype (the X X^T operand, also read
    // K-major as X^T by the update) and the fp32 master
    NormOut outs[2] = {
        {v.xh[0], v.s.mp, v.nm, cdt, 0},
        {v.x32[0], v.s.mp, v.nm, MSIGN_F32, 0},
    };
    st = launch_normalize(pr[i].x, io_dtype, pr[i].batch, pr[i].rows, pr[i].cols, v.s, v.partial, pl.nblk, eps,
                          outs, 2, stream, pr[i].fuse);
    if (st != MSIGN_OK) return st;
  }

  GemmParams qs[MSIGN_MAX_GROUPS];
  for (int t = 0; t < steps; ++t) {
    float a, b, c;
    coeff_at(coeffs, t, &a, &b, &c);
    const int cur = t & 1, nxt = cur ^ 1;
    hipError_t e;
    {  // A = X X^T
      for (int i = 0; i < ng; ++i) {
        const G& v = gv[i];
        if (t == 0 && v.direct) {  // the input itself, n true rows, times 1/s^2
          const int64_t nm = v.s.n * v.s.m;
          qs[i] = gemm_base(pr[i].x, v.s.m, nm, pr[i].x, v.s.m, nm, v.s.n, v.s.n, v.s.mp, 1.f);
          qs[i].vscale = v.nscales;
        } else {
          qs[i] = gemm_base(v.xh[cur], v.s.mp, v.nm, v.xh[cur], v.s.mp, v.nm, v.s.np, v.s.np, v.s.mp, 1.f);
        }
        add_out(qs[i], v.A, v.s.np, v.nn, cdt, dense, v.s.np, v.s.np, 0.f, 0, true);
      }
      TimedLaunch tl(KC_SYRK, stream);
      e = launch_grouped(cdt, sym, qs, batches, ng, stream, split, cp.split_bytes);
      if (e != hipSuccess) return hip_fail(e, "X X^T");
    }
    // Improved initial normalisation (§改良初值), first step only: A2 = A A
    // into B with its acc^2 sums, s from them, B = (b/s^2) A + (c/s^4) A2,
    // and the update below scaled by 1/s.
    const bool rescale = improved && t == 0;
    if (rescale) {
      for (int i = 0; i < ng; ++i) {
        const G& v = gv[i];
        qs[i] = gemm_base(v.A, v.s.np, v.nn, v.A, v.s.np, v.nn, v.s.np, v.s.np, v.s.np, 1.f);
        add_out(qs[i], v.B, v.s.np, v.nn, cdt, false, v.s.np, v.s.np, 0.f, 0, true);
        qs[i].sumsq = v.sumsq;
      }
      GroupPlan used;
      {
        TimedLaunch tl(KC_SQUARE, stream);
        e = launch_grouped(cdt, TRIANGLE, qs, batches, ng, stream, split, cp.split_bytes, &used);
        if (e != hipSuccess) return hip_fail(e, "A A (first step)");
      }
      for (int i = 0; i < ng; ++i) {
        const G& v = gv[i];
        GemmParams q = qs[i];
        q.tiles_m = used.tiles_m[i];
        q.tiles_n = used.tiles_n[i];
        q.tpm = used.tpm[i];
        TimedLaunch tl(KC_NORM, stream);
        // a direct first step also folds its 1/s into the update's factor
        init_scale_kernel<<<dim3((unsigned)pr[i].batch), 256, 0, stream>>>(
            q, sumsq_slots_per_tile(used.bm), eps, v.scales, v.direct ? v.nscales : nullptr);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "init_scale_kernel");
        const unsigned nb = (unsigned)((v.nn / 4 + 255) / 256);
        init_combine_kernel<<<dim3(nb, (unsigned)pr[i].batch), 256, 0, stream>>>(v.A, v.B, v.nn, cdt, b, c,
                                                                                  v.scales);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "init_combine_kernel");
      }
    }
    // A cubic step (c = 0, "msign算子的Newton-Schulz迭代（上）" §迭代计算) has
    // B = b A: no A A product, and the next product takes A scaled by b.
    const bool cubic = (c == 0.f) && !rescale;
    if (!cubic && !rescale) {  // B = c A A + b A
      for (int i = 0; i < ng; ++i) {
        const G& v = gv[i];
        qs[i] = gemm_base(v.A, v.s.np, v.nn, v.A, v.s.np, v.nn, v.s.np, v.s.np, v.s.np, c);
        set_d(qs[i], v.A, v.s.np, v.nn, cdt, b, true);
        add_out(qs[i], v.B, v.s.np, v.nn, cdt, dense, v.s.np, v.s.np, 0.f, 0, true);
      }
      TimedLaunch tl(KC_SQUARE, stream);
      e = launch_grouped(cdt, sym, qs, batches, ng, stream, split, cp.split_bytes);
      if (e != hipSuccess) return hip_fail(e, "c A A + b A");
    }
    {  // X' = B X + a X, as C' = X^T B + a X^T (m x n) with X read K-major;
       // C'[i][j] is stored at X'[j][i], four consecutive i per store
      for (int i = 0; i < ng; ++i) {
        const G& v = gv[i];
        GemmParams& g = qs[i];
        if (t == 0 && v.direct) {
          // X = the input (n true rows, read K-major; D = the input in its
          // own dtype), every value times 1/s
          const int64_t nm = v.s.n * v.s.m;
          g = gemm_base(pr[i].x, v.s.m, nm, cubic ? v.A : v.B, v.s.np, v.nn, v.s.mp, v.s.n, v.s.np,
                        cubic ? b : 1.f);
          g.kvalid = (int32_t)v.s.n;
          // 1/s, or with the improved initial normalisation its factor times 1/s
          g.vscale = rescale ? v.scales : v.nscales + 1;
          set_d(g, pr[i].x, v.s.m, nm, io_dtype, a, true);
        } else {
          g = gemm_base(v.xh[cur], v.s.mp, v.nm, cubic ? v.A : v.B, v.s.np, v.nn, v.s.mp, v.s.np, v.s.np,
                        cubic ? b : 1.f);
          if (rescale) g.vscale = v.scales;
          set_d(g, v.x32[cur], v.s.mp, v.nm, MSIGN_F32, a, true);
        }
        if (t + 1 < steps) {
          add_out(g, v.x32[nxt], v.s.mp, v.nm, MSIGN_F32, true, v.s.mp, v.s.np, 0.f, 0, true);
          add_out(g, v.xh[nxt], v.s.mp, v.nm, cdt, true, v.s.mp, v.s.np, 0.f, 0, true);
        } else {
          add_final_out(g, pr[i]);
        }
      }
      TimedLaunch tl(KC_RECT, stream);
      e = launch_grouped(cdt, RECT_KMAJOR, qs, batches, ng, stream, split, cp.split_bytes);
      if (e != hipSuccess) return hip_fail(e, "B X + a X");
    }
  }
  return MSIGN_OK;
}

// Standard NS over ng problems: every product is one launch over all of
// them (a grouped launch), the normalise passes run per problem.  Arguments
// are checked; each sub-call (see split_call) runs with its own dtype.
msign_status_t ns_run(const msign_group_t* groups, int32_t ngroups, int32_t io_dtype, int32_t compute_dtype,
                      int32_t steps, const float* coeffs, float eps, uint32_t flags, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, int32_t y_dtype = -1,
                      const Fuse* fuse = nullptr) {
  g_err.clear();
  if (flags & ~(uint32_t)(MSIGN_NS_IMPROVED_INIT | MSIGN_NS_DENSE_PRODUCTS)) return fail(MSIGN_ERR_ARG, "unknown flag");
  const bool improved = (flags & MSIGN_NS_IMPROVED_INIT) != 0;
  const bool dense = (flags & MSIGN_NS_DENSE_PRODUCTS) != 0;
  if (dense && improved)
    return fail(MSIGN_ERR_ARG, "MSIGN_NS_DENSE_PRODUCTS does not combine with MSIGN_NS_IMPROVED_INIT");
  Prob pr[MSIGN_MAX_GROUPS];
  int ng = 0;
  msign_status_t st = gather(groups, ngroups, io_dtype, compute_dtype, steps, coeffs, eps, pr, &ng, y_dtype, fuse);
  if (st != MSIGN_OK || ng == 0) return st;
  if (dense && ng > 1) return fail(MSIGN_ERR_ARG, "MSIGN_NS_DENSE_PRODUCTS takes one non-empty group");
  const SubCalls sc = split_call<NsPlan>(pr, ng, compute_dtype, plan_ns_regions);
  st = check_call_ws(pr, ng, io_dtype, workspace, workspace_bytes, sc.total);
  if (st != MSIGN_OK) return st;
  for (int k = 0; k < 2; ++k) {
    if (sc.n[k] == 0) continue;
    st = ns_exec(sc.p[k], sc.n[k], io_dtype, sc.cdt[k], steps, coeffs, eps, improved, dense,
                 at(workspace, sc.off[k]), stream);
    if (st != MSIGN_OK) return st;
  }
  return MSIGN_OK;
}

// Restart list of Gram NS: strictly increasing step indices in 1..steps-1
// (steps itself is checked with the other arguments).
msign_status_t parse_restarts(int32_t steps, const int32_t* restart_after, int32_t n_restarts, bool* restart_at) {
  if (n_restarts < 0 || (n_restarts > 0 && !restart_after) || (n_restarts == 0 && restart_after))
    return fail(MSIGN_ERR_ARG, "restart_after must be non-null exactly when n_restarts > 0");
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
  return MSIGN_OK;
}

// The launches of Gram NS over checked problems pr[0..ng) with products in
// `cdt`, in a workspace laid out by plan_call; restart_at[t] marks a
// restart after step t.
msign_status_t gram_exec(const Prob* pr, int ng, int32_t io_dtype, int32_t cdt, int32_t steps,
                         const float* coeffs, float eps, const bool* restart_at, void* workspace,
                         hipStream_t stream) {
  const CallPlan<GramPlan> cp = plan_call<GramPlan>(pr, ng, cdt, plan_gram_regions);
  msign_status_t st = MSIGN_OK;
  void* split = at(workspace, cp.split);
  struct G {
    Shape s;
    int64_t nm, nn;
    void *xh[2], *R, *Z, *RZ, *Qb0, *Qb1;  // Q double-buffered
    float* scales;
    bool direct;  // X0 is the input itself until the first restart (scales: 1/s^2, 1/s)
  } gv[MSIGN_MAX_GROUPS];
  int64_t batches[MSIGN_MAX_GROUPS];
  for (int i = 0; i < ng; ++i) {
    const GramPlan& pl = cp.p[i];
    G& v = gv[i];
    v.s = pr[i].s;
    v.nm = v.s.np * v.s.mp;
    v.nn = v.s.np * v.s.np;
    v.xh[0] = at(workspace, pl.xh[0]);
    v.xh[1] = at(workspace, pl.xh[1]);
    v.R = at(workspace, pl.r);
    v.Z = at(workspace, pl.z);
    v.RZ = at(workspace, pl.rz);
    v.Qb0 = at(workspace, pl.q[0]);
    v.Qb1 = at(workspace, pl.q[1]);
    batches[i] = pr[i].batch;
    v.scales = reinterpret_cast<float*>(at(workspace, pl.scales));
    float* partial = reinterpret_cast<float*>(at(workspace, pl.partial));
    v.direct = direct_input(pr[i], io_dtype, cdt);
    if (v.direct) {
      st = launch_norm_scale(pr[i].x, io_dtype, pr[i].batch, pr[i].rows * pr[i].cols, partial, pl.nblk, eps,
                             v.scales, stream);
    } else {
      NormOut outs[1] = {{v.xh[0], v.s.mp, v.nm, cdt, 0}};
      st = launch_normalize(pr[i].x, io_dtype, pr[i].batch, pr[i].rows, pr[i].cols, v.s, partial, pl.nblk, eps,
                            outs, 1, stream, pr[i].fuse);
    }
    if (st != MSIGN_OK) return st;
  }

  hipError_t e;
  int cur = 0, qc = 0;
  bool raw = true;  // X is still X0 (the input itself for direct groups)
  GemmParams qs[MSIGN_MAX_GROUPS];
  auto gram_xxt = [&]() -> msign_status_t {
    for (int i = 0; i < ng; ++i) {
      const G& v = gv[i];
      if (raw && v.direct) {  // the input, n true rows, times 1/s^2
        const int64_t nm = v.s.n * v.s.m;
        qs[i] = gemm_base(pr[i].x, v.s.m, nm, pr[i].x, v.s.m, nm, v.s.n, v.s.n, v.s.mp, 1.f);
        qs[i].vscale = v.scales;
      } else {
        qs[i] = gemm_base(v.xh[cur], v.s.mp, v.nm, v.xh[cur], v.s.mp, v.nm, v.s.np, v.s.np, v.s.mp, 1.f);
      }
      add_out(qs[i], v.R, v.s.np, v.nn, cdt, false, v.s.np, v.s.np, 0.f, 0, true);
    }
    TimedLaunch tl(KC_SYRK, stream);
    e = launch_grouped(cdt, TRIANGLE, qs, batches, ng, stream, split, cp.split_bytes);
    return e == hipSuccess ? MSIGN_OK : hip_fail(e, "R = X X^T");
  };
  // tri product: out = P Q^T + beta D  (all n x n, symmetric); operands
  // named by their member in G
  using Buf = void* G::*;
  auto square = [&](Buf P, Buf Q, float alpha, Buf D, float beta, Buf out, Buf out2, float diag2,
                    const char* what) -> msign_status_t {
    for (int i = 0; i < ng; ++i) {
      G& v = gv[i];
      qs[i] = gemm_base(v.*P, v.s.np, v.nn, v.*Q, v.s.np, v.nn, v.s.np, v.s.np, v.s.np, alpha);
      if (D) set_d(qs[i], v.*D, v.s.np, v.nn, cdt, beta, true);
      add_out(qs[i], v.*out, v.s.np, v.nn, cdt, false, v.s.np, v.s.np, 0.f, 0, true);
      if (out2) add_out(qs[i], v.*out2, v.s.np, v.nn, cdt, false, v.s.np, v.s.np, diag2, v.s.n, true);
    }
    TimedLaunch tl(KC_SQUARE, stream);
    e = launch_grouped(cdt, TRIANGLE, qs, batches, ng, stream, split, cp.split_bytes);
    return e == hipSuccess ? MSIGN_OK : hip_fail(e, what);
  };
  // rect product: C' = X^T Q (Q symmetric, X read K-major), stored
  // transposed into the other X, or into y on the last one
  auto apply_q = [&](bool final_out, const char* what) -> msign_status_t {
    for (int i = 0; i < ng; ++i) {
      G& v = gv[i];
      if (raw && v.direct) {  // the input read K-major (n true rows), times 1/s
        const int64_t nm = v.s.n * v.s.m;
        qs[i] = gemm_base(pr[i].x, v.s.m, nm, qc ? v.Qb1 : v.Qb0, v.s.np, v.nn, v.s.mp, v.s.n, v.s.np, 1.f);
        qs[i].kvalid = (int32_t)v.s.n;
        qs[i].vscale = v.scales + 1;
      } else {
        qs[i] = gemm_base(v.xh[cur], v.s.mp, v.nm, qc ? v.Qb1 : v.Qb0, v.s.np, v.nn, v.s.mp, v.s.np, v.s.np, 1.f);
      }
      if (final_out) add_final_out(qs[i], pr[i]);
      else add_out(qs[i], v.xh[cur ^ 1], v.s.mp, v.nm, cdt, true, v.s.mp, v.s.np, 0.f, 0, true);
    }
    TimedLaunch tl(KC_RECT, stream);
    e = launch_grouped(cdt, RECT_KMAJOR, qs, batches, ng, stream, split, cp.split_bytes);
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
    st = square(&G::R, &G::R, c, &G::R, b, &G::Z, fresh ? (qc ? &G::Qb1 : &G::Qb0) : nullptr, a,
                "Z = b R + c R^2");
    if (st != MSIGN_OK) return st;
    if (!fresh) {  // Q <- Q Z + a Q
      const Buf q0 = qc ? &G::Qb1 : &G::Qb0, q1 = qc ? &G::Qb0 : &G::Qb1;
      st = square(q0, &G::Z, 1.f, q0, a, q1, nullptr, 0.f, "Q <- Q Z + a Q");
      if (st != MSIGN_OK) return st;
      qc ^= 1;
    }
    fresh = false;
    if (!block_end) {
      st = square(&G::R, &G::Z, 1.f, &G::R, a, &G::RZ, nullptr, 0.f, "RZ <- R Z + a R");
      if (st != MSIGN_OK) return st;
      st = square(&G::Z, &G::RZ, 1.f, &G::RZ, a, &G::R, nullptr, 0.f, "R <- Z RZ + a RZ");
      if (st != MSIGN_OK) return st;
    }
    if (restart_at[t]) {  // X <- Q X, R = X X^T, Q = I
      st = apply_q(false, "restart X <- Q X");
      if (st != MSIGN_OK) return st;
      cur ^= 1;
      raw = false;
      st = gram_xxt();
      if (st != MSIGN_OK) return st;
      fresh = true;
    }
  }
  return apply_q(true, "y = Q X");  // y = Q X
}

// Gram NS over ng problems, every product one grouped launch; arguments
// checked here, each sub-call (see split_call) run with its own dtype.
msign_status_t gram_run(const msign_group_t* groups, int32_t ngroups, int32_t io_dtype, int32_t compute_dtype,
                        int32_t steps, const float* coeffs, float eps, const int32_t* restart_after,
                        int32_t n_restarts, void* workspace, size_t workspace_bytes, hipStream_t stream,
                        int32_t y_dtype = -1, const Fuse* fuse = nullptr) {
  g_err.clear();
  bool restart_at[MSIGN_MAX_STEPS + 1] = {false};
  msign_status_t st0 = parse_restarts(steps, restart_after, n_restarts, restart_at);
  if (st0 != MSIGN_OK) return st0;
  Prob pr[MSIGN_MAX_GROUPS];
  int ng = 0;
  msign_status_t st = gather(groups, ngroups, io_dtype, compute_dtype, steps, coeffs, eps, pr, &ng, y_dtype, fuse);
  if (st != MSIGN_OK || ng == 0) return st;
  const SubCalls sc = split_call<GramPlan>(pr, ng, compute_dtype, plan_gram_regions);
  st = check_call_ws(pr, ng, io_dtype, workspace, workspace_bytes, sc.total);
  if (st != MSIGN_OK) return st;
  for (int k = 0; k < 2; ++k) {
    if (sc.n[k] == 0) continue;
    st = gram_exec(sc.p[k], sc.n[k], io_dtype, sc.cdt[k], steps, coeffs, eps, restart_at,
                   at(workspace, sc.off[k]), stream);
    if (st != MSIGN_OK) return st;
  }
  return MSIGN_OK;
}

// ------------------------------------------------------------ Muon step --

// msign groups of a Muon step: x = the fp32 momentum M, y = the parameters
// W; the step itself is fused into the msign call (see Fuse).
struct MuonCall {
  int ng;
  msign_group_t mg[MSIGN_MAX_GROUPS];
  const muon_group_t* src[MSIGN_MAX_GROUPS];
  size_t total;
};

bool muon_shape_ok(const muon_group_t& g) {
  return g.batch >= 0 && g.rows >= 0 && g.cols >= 0 && g.rows <= kMaxDim && g.cols <= kMaxDim &&
         g.batch <= kMaxBatch;
}

// Non-empty groups and the workspace size (that of the msign call).
msign_status_t plan_muon(const muon_group_t* groups, int32_t ngroups, int32_t method, int32_t cdt,
                         MuonCall* mc) {
  mc->ng = 0;
  if (ngroups < 1 || ngroups > MSIGN_MAX_GROUPS)
    return fail(MSIGN_ERR_ARG, "ngroups must be in 1.." + std::to_string(MSIGN_MAX_GROUPS));
  if (!groups) return fail(MSIGN_ERR_ARG, "groups must be non-null");
  if (method != MUON_NS && method != MUON_GRAM) return fail(MSIGN_ERR_ARG, "method must be MUON_NS or MUON_GRAM");
  if (!dt_valid(cdt)) return fail(MSIGN_ERR_DTYPE, "compute_dtype must be MSIGN_F32, MSIGN_BF16 or MSIGN_F16");
  for (int i = 0; i < ngroups; ++i) {
    const muon_group_t& g = groups[i];
    if (!muon_shape_ok(g)) return fail(MSIGN_ERR_SHAPE, "group " + std::to_string(i) + ": invalid shape");
    if (g.batch == 0 || g.rows == 0 || g.cols == 0) continue;
    const int k = mc->ng++;
    mc->src[k] = &g;
    mc->mg[k].x = g.m;
    mc->mg[k].y = g.w;
    mc->mg[k].batch = g.batch;
    mc->mg[k].rows = g.rows;
    mc->mg[k].cols = g.cols;
  }
  const size_t need = mc->ng == 0 ? 0 : call_workspace(mc->mg, mc->ng, cdt, method == MUON_GRAM);
  if (need == (size_t)-1) return fail(MSIGN_ERR_SHAPE, "invalid sizes");
  mc->total = need;
  return MSIGN_OK;
}

// One Muon step as one msign call: the sum-of-squares pass first forms
// M <- mu M + G in place (fp32), and the last product's epilogue writes
// W <- W - lr msign(M) in place (fp32 arithmetic, W rounded once).  No
// other pass and no buffer for msign(M).
msign_status_t muon_run(const muon_group_t* groups, int32_t ngroups, int32_t io_dtype, float mu, float lr,
                        int32_t method, int32_t compute_dtype, int32_t steps, const float* coeffs, float eps,
                        uint32_t flags, const int32_t* restart_after, int32_t n_restarts, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  if (!dt_valid(io_dtype)) return fail(MSIGN_ERR_DTYPE, "io_dtype must be MSIGN_F32, MSIGN_BF16 or MSIGN_F16");
  if (!std::isfinite(mu) || !std::isfinite(lr)) return fail(MSIGN_ERR_ARG, "mu and lr must be finite");
  if (method == MUON_GRAM && flags != 0) return fail(MSIGN_ERR_ARG, "flags apply to MUON_NS only");
  if (flags & ~(uint32_t)MSIGN_NS_IMPROVED_INIT) return fail(MSIGN_ERR_ARG, "unknown flag");
  if (method == MUON_GRAM) {
    bool restart_at[MSIGN_MAX_STEPS + 1] = {false};
    msign_status_t st0 = parse_restarts(steps, restart_after, n_restarts, restart_at);
    if (st0 != MSIGN_OK) return st0;
  }
  MuonCall mc;
  msign_status_t st = plan_muon(groups, ngroups, method, compute_dtype, &mc);
  if (st != MSIGN_OK || mc.ng == 0) return st;
  if (!workspace || workspace_bytes < mc.total)
    return fail(MSIGN_ERR_WORKSPACE, "workspace is null or smaller than the required " + std::to_string(mc.total) + " bytes");
  if (!aligned(workspace, 256)) return fail(MSIGN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const size_t es = dt_size(io_dtype);
  for (int k = 0; k < mc.ng; ++k) {
    const muon_group_t& g = *mc.src[k];
    if (!g.w || !g.g || !g.m) return fail(MSIGN_ERR_ARG, "w, g and m must be non-null");
    if (!aligned(g.w, es) || !aligned(g.g, es) || !aligned(g.m, 4))
      return fail(MSIGN_ERR_ARG, "w, g and m must be aligned to their element size");
  }
  // buffers: w and m written, g read; none may overlap the workspace, and a
  // written buffer may overlap no other buffer
  struct Buf { const void* p; size_t n; bool written; };
  Buf bufs[3 * MSIGN_MAX_GROUPS];
  int nb = 0;
  for (int k = 0; k < mc.ng; ++k) {
    const muon_group_t& g = *mc.src[k];
    const size_t cnt = (size_t)g.batch * g.rows * g.cols;
    bufs[nb++] = {g.w, cnt * es, true};
    bufs[nb++] = {g.g, cnt * es, false};
    bufs[nb++] = {g.m, cnt * 4, true};
  }
  for (int i = 0; i < nb; ++i) {
    if (overlap(bufs[i].p, bufs[i].n, workspace, mc.total))
      return fail(MSIGN_ERR_ALIAS, "w, g or m overlaps the workspace");
    for (int j = 0; j < nb; ++j)
      if (j != i && (bufs[i].written || bufs[j].written) && overlap(bufs[i].p, bufs[i].n, bufs[j].p, bufs[j].n))
        return fail(MSIGN_ERR_ALIAS, "w or m overlaps another buffer of the step");
  }
  Fuse fz[MSIGN_MAX_GROUPS];
  for (int k = 0; k < mc.ng; ++k) fz[k] = Fuse{mc.src[k]->g, io_dtype, mu, lr};
  // msign of the fp32 momentum into the io-dtype parameters, step fused;
  // its own checks all run before its first launch
  return method == MUON_NS
             ? ns_run(mc.mg, mc.ng, MSIGN_F32, compute_dtype, steps, coeffs, eps, flags, workspace,
                      workspace_bytes, stream, io_dtype, fz)
             : gram_run(mc.mg, mc.ng, MSIGN_F32, compute_dtype, steps, coeffs, eps, restart_after, n_restarts,
                        workspace, workspace_bytes, stream, io_dtype, fz);
}

// ------------------------------------------------- allocation-free calls --

// Scratch of msign_ns_noalloc, for callers that cannot allocate device
// memory.  Each device the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device array: its device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is
// passed to kernels.
static_assert(MSIGN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[MSIGN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on the first
// call on that device).
msign_status_t device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MSIGN_ERR_HIP, "device index out of range");
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr || !aligned(p, 256)) return fail(MSIGN_ERR_HIP, "scratch address is null or misaligned");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MSIGN_OK;
}

msign_group_t one_group(const void* x, void* y, int64_t batch, int64_t rows, int64_t cols) {
  msign_group_t g;
  g.x = x; g.y = y; g.batch = batch; g.rows = rows; g.cols = cols;
  return g;
}

}  // namespace

extern "C" {

size_t msign_ns_workspace_bytes(int64_t batch, int64_t rows, int64_t cols, int32_t compute_dtype) {
  const msign_group_t g = one_group(nullptr, nullptr, batch, rows, cols);
  return call_workspace(&g, 1, compute_dtype, false);
}

size_t msign_gram_ns_workspace_bytes(int64_t batch, int64_t rows, int64_t cols, int32_t compute_dtype) {
  const msign_group_t g = one_group(nullptr, nullptr, batch, rows, cols);
  return call_workspace(&g, 1, compute_dtype, true);
}

size_t msign_ns_grouped_workspace_bytes(const msign_group_t* groups, int32_t ngroups, int32_t compute_dtype) {
  return call_workspace(groups, ngroups, compute_dtype, false);
}

size_t msign_gram_ns_grouped_workspace_bytes(const msign_group_t* groups, int32_t ngroups,
                                             int32_t compute_dtype) {
  return call_workspace(groups, ngroups, compute_dtype, true);
}

msign_status_t msign_ns(const void* x, void* y, int64_t batch, int64_t rows, int64_t cols,
                        int32_t io_dtype, int32_t compute_dtype, int32_t steps, const float* coeffs,
                        float eps, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const msign_group_t g = one_group(x, y, batch, rows, cols);
  return ns_run(&g, 1, io_dtype, compute_dtype, steps, coeffs, eps, 0u, workspace, workspace_bytes, stream);
}

msign_status_t msign_ns_noalloc(const void* x, void* y, int64_t batch, int64_t rows, int64_t cols,
                                int32_t io_dtype, int32_t compute_dtype, int32_t steps, const float* coeffs,
                                float eps, hipStream_t stream) {
  g_err.clear();
  const msign_group_t g = one_group(x, y, batch, rows, cols);
  {  // the argument checks of msign_ns, before the device is touched
    Prob pr[1];
    int ng = 0;
    msign_status_t st = gather(&g, 1, io_dtype, compute_dtype, steps, coeffs, eps, pr, &ng);
    if (st != MSIGN_OK || ng == 0) return st;
  }
  const size_t need = call_workspace(&g, 1, compute_dtype, false);
  if (need == (size_t)-1) return fail(MSIGN_ERR_SHAPE, "invalid sizes");
  if (need > (size_t)MSIGN_NOALLOC_SCRATCH_BYTES)
    return fail(MSIGN_ERR_WORKSPACE, "problem needs " + std::to_string(need) +
                                         " bytes of scratch; msign_ns_noalloc holds " +
                                         std::to_string((size_t)MSIGN_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  msign_status_t st = device_scratch(&ws);
  if (st != MSIGN_OK) return st;
  g_untimed = true;
  st = ns_run(&g, 1, io_dtype, compute_dtype, steps, coeffs, eps, 0u, ws, need, stream);
  g_untimed = false;
  return st;
}

msign_status_t msign_ns_ex(const void* x, void* y, int64_t batch, int64_t rows, int64_t cols,
                           int32_t io_dtype, int32_t compute_dtype, int32_t steps, const float* coeffs,
                           float eps, uint32_t flags, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  const msign_group_t g = one_group(x, y, batch, rows, cols);
  return ns_run(&g, 1, io_dtype, compute_dtype, steps, coeffs, eps, flags, workspace, workspace_bytes, stream);
}

msign_status_t msign_ns_grouped(const msign_group_t* groups, int32_t ngroups, int32_t io_dtype,
                                int32_t compute_dtype, int32_t steps, const float* coeffs, float eps,
                                uint32_t flags, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return ns_run(groups, ngroups, io_dtype, compute_dtype, steps, coeffs, eps, flags, workspace, workspace_bytes,
                stream);
}

msign_status_t msign_gram_ns(const void* x, void* y, int64_t batch, int64_t rows, int64_t cols,
                             int32_t io_dtype, int32_t compute_dtype, int32_t steps, const float* coeffs,
                             float eps, const int32_t* restart_after, int32_t n_restarts, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  const msign_group_t g = one_group(x, y, batch, rows, cols);
  return gram_run(&g, 1, io_dtype, compute_dtype, steps, coeffs, eps, restart_after, n_restarts, workspace,
                  workspace_bytes, stream);
}

size_t muon_step_workspace_bytes(const muon_group_t* groups, int32_t ngroups, int32_t method,
                                 int32_t compute_dtype) {
  MuonCall mc;
  const std::string keep = g_err;
  const msign_status_t st = plan_muon(groups, ngroups, method, compute_dtype, &mc);
  g_err = keep;
  return st == MSIGN_OK ? mc.total : (size_t)-1;
}

msign_status_t muon_step(const muon_group_t* groups, int32_t ngroups, int32_t io_dtype, float mu, float lr,
                         int32_t method, int32_t compute_dtype, int32_t steps, const float* coeffs, float eps,
                         uint32_t flags, const int32_t* restart_after, int32_t n_restarts, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return muon_run(groups, ngroups, io_dtype, mu, lr, method, compute_dtype, steps, coeffs, eps, flags,
                  restart_after, n_restarts, workspace, workspace_bytes, stream);
}

msign_status_t msign_gram_ns_grouped(const msign_group_t* groups, int32_t ngroups, int32_t io_dtype,
                                     int32_t compute_dtype, int32_t steps, const float* coeffs, float eps,
                                     const int32_t* restart_after, int32_t n_restarts, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  return gram_run(groups, ngroups, io_dtype, compute_dtype, steps, coeffs, eps, restart_after, n_restarts,
                  workspace, workspace_bytes, stream);
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
  return syrk_xxt_ex(x, c, batch, n, k, dtype, alpha, d, beta, gamma, 0u, workspace, workspace_bytes, stream);
}

msign_status_t syrk_xxt_ex(const void* x, void* c, int64_t batch, int64_t n, int64_t k, int32_t dtype,
                           float alpha, const void* d, float beta, float gamma, uint32_t flags,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  if (flags & ~(uint32_t)MSIGN_SYRK_FULL_TILES) return fail(MSIGN_ERR_ARG, "unknown flag");
  const bool full = (flags & MSIGN_SYRK_FULL_TILES) != 0;
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
  // full tiles: C is stored through its transpose (the same matrix), which
  // takes the whole-line epilogue when there is no diagonal term
  add_out(g, c, n, n * n, dtype, full, n, n, gamma, gamma != 0.f ? n : 0, vec_c);
  TimedLaunch tl(KC_SYRK, stream);
  hipError_t e = launch_nt(dtype, full ? DENSE : TRIANGLE, g, batch, stream, split, split_cap);
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

msign_status_t msign_mfma_probe(int32_t dtype, int32_t iters, float* out, hipStream_t stream) {
  g_err.clear();
  static_assert(kProbeBlocks == MSIGN_PROBE_BLOCKS && kProbeThreads == MSIGN_PROBE_THREADS, "probe layout");
  if (dtype != MSIGN_BF16 && dtype != MSIGN_F16) return fail(MSIGN_ERR_DTYPE, "dtype must be MSIGN_BF16 or MSIGN_F16");
  if (iters < 1) return fail(MSIGN_ERR_ARG, "iters must be >= 1");
  if (!out || !aligned(out, 4)) return fail(MSIGN_ERR_ARG, "out must be a non-null float buffer");
  if (dtype == MSIGN_BF16)
    mfma_probe_kernel<bf16_t><<<kProbeBlocks, kProbeThreads, 0, stream>>>(iters, 0.5f, out);
  else
    mfma_probe_kernel<f16_t><<<kProbeBlocks, kProbeThreads, 0, stream>>>(iters, 0.5f, out);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MSIGN_OK : hip_fail(e, "mfma_probe_kernel");
}

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

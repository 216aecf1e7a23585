"""Plain fp64 CPU oracle for msign by Newton-Schulz iteration.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
this module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark use it.  It shares no code with the HIP library (no kernels, headers,
helpers or constant tables) and imports nothing from it.

Everything here is slow, obvious and in float64.  Each function names the
passage of the source pages it follows.  Page keys used below:

  [KX]  kexue.fm/archives/10922, "msign算子的Newton-Schulz迭代（上）"
        sections 写在前面 (definition), 迭代计算 (iteration, Keller constants),
        参考实现 (reference loop), 原理分析 (per-singular-value scalar map),
        解开约束 / 自己试试 / 其他解集 (per-step coefficient tables),
        改良初值 (improved initial normalisation).
  [GR]  zifeng-mai.github.io/2026/04/05/GramNewtonSchulz, "Gram Newton-Schulz"
        §1.2 (standard NS and its FLOP count), §2.2 (Proposition 1, Lemma 1,
        Theorem 1), §2.3 (Algorithm 1, naive Gram NS), §2.4 (FLOP count),
        §3.4 (Algorithm 2, stabilised Gram NS with restart), Appendix 1-2.
  [NB]  nil9.net blog index, flash-muon excerpt (the PyTorch loop that forms
        A = X X^T once and reuses it; the iterated matrix is the gradient or
        its momentum).
  [MS]  anti-entrophic.github.io/posts/10054.html, the Mousse page,
        §标准 Muon 算法 (the Muon update is -msign of the matrix).

Pins: every function here is checked by the not-gpu tests against closed forms,
invariants or values the pages print (tests/test_oracle_pins.py).  No function
is "parity unpinned".
"""

from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np

# [KX] §迭代计算: the coefficient choice of the Muon author, used for all T steps.
KELLER_ABC = (3.4445, -4.7750, 2.0315)
DEFAULT_STEPS = 5
# [KX] §参考实现: the reference loop adds eps = 1e-20 under the square root.
DEFAULT_EPS = 1e-20


# ---------------------------------------------------------------------------
# coefficient schedules
# ---------------------------------------------------------------------------

def coefficient_schedule(coeffs=None, steps: int = DEFAULT_STEPS):
    """Per-step (a_t, b_t, c_t) list of length `steps`.

    `coeffs=None` repeats the Keller triple ([KX] §迭代计算).  A single triple
    is repeated; a table of `steps` triples is used as given, one row per step
    ([KX] §解开约束: a different triple at each step costs nothing extra).
    """
    if steps < 1:
        raise ValueError("steps must be >= 1")
    if coeffs is None:
        return [tuple(float(v) for v in KELLER_ABC)] * steps
    arr = np.asarray(coeffs, dtype=np.float64)
    if arr.shape == (3,):
        return [tuple(float(v) for v in arr)] * steps
    if arr.ndim != 2 or arr.shape[1] != 3 or arr.shape[0] != steps:
        raise ValueError(f"coefficient table must be ({steps}, 3); got {arr.shape}")
    return [tuple(float(v) for v in row) for row in arr]


# ---------------------------------------------------------------------------
# exact definition
# ---------------------------------------------------------------------------

def svd_msign(m: np.ndarray) -> np.ndarray:
    """Exact msign of one matrix: U[:, :r] V[:, :r]^T ([KX] §写在前面, eq. 1).

    r is the numerical rank: singular values above sigma_1 * max(n, m) * 2^-52
    count as nonzero.  A zero matrix gives a zero matrix.
    """
    m = np.asarray(m, dtype=np.float64)
    u, s, vt = np.linalg.svd(m, full_matrices=False)
    if s.size == 0 or s[0] == 0.0:
        return np.zeros_like(m)
    tol = s[0] * max(m.shape) * np.finfo(np.float64).eps
    r = int(np.sum(s > tol))
    return u[:, :r] @ vt[:r, :]


def inverse_sqrt_msign(m: np.ndarray) -> np.ndarray:
    """msign(M) = (M M^T)^{-1/2} M for full-row-rank M ([KX] §写在前面, eq. 2).

    The inverse square root comes from the symmetric eigendecomposition of
    M M^T; this is a second, SVD-free route to the exact value.
    """
    m = np.asarray(m, dtype=np.float64)
    g = m @ m.T
    w, v = np.linalg.eigh(g)
    if np.any(w <= 0):
        raise ValueError("M M^T must be positive definite (full row rank)")
    return (v * (1.0 / np.sqrt(w))) @ v.T @ m


# ---------------------------------------------------------------------------
# scalar view of the iteration
# ---------------------------------------------------------------------------

def poly_step(x, a: float, b: float, c: float):
    """One quintic step on a singular value: a x + b x^3 + c x^5 ([KX] §原理分析)."""
    return a * x + b * x ** 3 + c * x ** 5


def phi(x, coeffs=None, steps: int = DEFAULT_STEPS):
    """T-fold composition of the per-step polynomials ([KX] §原理分析;
    [GR] §2.2 Proposition 1: p_{k+1} = a p_k + b p_k^3 + c p_k^5)."""
    y = np.asarray(x, dtype=np.float64)
    for a, b, c in coefficient_schedule(coeffs, steps):
        y = poly_step(y, a, b, c)
    return y


def theorem1_xq(x, coeffs=None, steps: int = DEFAULT_STEPS):
    """x * q_T(x^2) from the r/q recursion of [GR] §2.2 Theorem 1 (proof in
    Appendix 2).

    With h_t(y) = a_t + b_t y + c_t y^2 (Lemma 1: p_t(x) = x h_t(x^2)):
    r_0 = x^2, q_0 = 1, z_t = h_t(r_{t-1}), q_t = q_{t-1} z_t,
    r_t = r_{t-1} z_t^2.  The theorem states x q_T(x^2) = phi(x).
    """
    x = np.asarray(x, dtype=np.float64)
    r = x * x
    q = np.ones_like(x)
    for a, b, c in coefficient_schedule(coeffs, steps):
        z = a + b * r + c * r * r
        q = q * z
        r = r * z * z
    return x * q


# ---------------------------------------------------------------------------
# matrix iterations
# ---------------------------------------------------------------------------

def _as_wide(m: np.ndarray):
    """Work on the wide orientation: transpose when rows > cols ([KX] §参考实现)."""
    tall = m.shape[-2] > m.shape[-1]
    return (m.T if tall else m), tall


def frobenius_normalize(x: np.ndarray, eps: float = DEFAULT_EPS) -> np.ndarray:
    """X / sqrt(sum(X^2) + eps) ([KX] §迭代计算 X_0 = M/||M||_F, with the eps of
    §参考实现).  The Gram pages write ||X||_F + eps with eps = 1e-7 instead; the
    same normalisation is used for both iterations here so that the two agree
    exactly (see the readings listed in the design notes)."""
    return x / math.sqrt(float(np.sum(x * x)) + eps)


def ns_single(m: np.ndarray, coeffs=None, steps: int = DEFAULT_STEPS,
              eps: float = DEFAULT_EPS) -> np.ndarray:
    """Standard quintic Newton-Schulz on one matrix, fp64.

    [KX] §迭代计算 and §参考实现, with A = X X^T formed once per step and reused
    ([NB] flash-muon excerpt): X <- a X + (b A + c A A) X.
    """
    m = np.asarray(m, dtype=np.float64)
    x, tall = _as_wide(m)
    x = _quintic_steps(frobenius_normalize(x, eps), coefficient_schedule(coeffs, steps))
    return x.T if tall else x


def _quintic_steps(x: np.ndarray, sched) -> np.ndarray:
    """The NS steps X <- a X + (b A + c A A) X, A = X X^T, from a given X_0."""
    for a, b, c in sched:
        A = x @ x.T
        B = b * A + c * (A @ A)
        x = a * x + B @ x
    return x


def gram_ns_single(m: np.ndarray, coeffs=None, steps: int = DEFAULT_STEPS,
                   eps: float = DEFAULT_EPS,
                   restart_after: Iterable[int] = (2,)) -> np.ndarray:
    """Gram Newton-Schulz on one matrix, fp64.

    [GR] §3.4 Algorithm 2 (stabilised Gram NS) without the fp16 cast, which is
    a precision choice of the GPU path.  `restart_after` lists the steps t
    after which X <- Q X, R <- X X^T, Q <- I; Algorithm 2 restarts after t = 2.
    An empty list is [GR] §2.3 Algorithm 1 (naive Gram NS): Q_t = Q_{t-1} Z_t,
    R_t = Z_t R_{t-1} Z_t with Z_t = a_t I + b_t R + c_t R^2.  The update below
    is Algorithm 2's form, which keeps a_t out of Z:
      Z <- b R + c R^2;  Q <- Q Z + a Q;  RZ <- R Z + a R;  R <- Z RZ + a RZ.
    """
    m = np.asarray(m, dtype=np.float64)
    x, tall = _as_wide(m)
    x = frobenius_normalize(x, eps)
    sched = coefficient_schedule(coeffs, steps)
    restarts = set(int(t) for t in restart_after)
    n = x.shape[0]
    eye = np.eye(n)
    R = x @ x.T
    Q = eye.copy()
    for t, (a, b, c) in enumerate(sched, start=1):
        Z = b * R + c * (R @ R)
        Q = Q @ Z + a * Q
        RZ = R @ Z + a * R
        R = Z @ RZ + a * RZ
        if t in restarts and t < steps:
            x = Q @ x
            R = x @ x.T
            Q = eye.copy()
    y = Q @ x
    return y.T if tall else y


def spectral_ns_single(m: np.ndarray, coeffs=None, steps: int = DEFAULT_STEPS,
                       eps: float = DEFAULT_EPS) -> np.ndarray:
    """U diag(phi(sigma_i / sqrt(sum sigma^2 + eps))) V^T.

    [KX] §原理分析: the iteration leaves U and V alone and maps each normalised
    singular value through the scalar polynomial; [GR] §2.2 Proposition 1.
    The normalisation uses the singular values, not the entries.
    """
    m = np.asarray(m, dtype=np.float64)
    u, s, vt = np.linalg.svd(m, full_matrices=False)
    scale = math.sqrt(float(np.sum(s * s)) + eps)
    return (u * phi(s / scale, coeffs, steps)) @ vt


def _batched(fn, m, **kw):
    m = np.asarray(m, dtype=np.float64)
    if m.ndim < 2:
        raise ValueError("need at least 2 dims")
    if m.ndim == 2:
        return fn(m, **kw)
    flat = m.reshape((-1,) + m.shape[-2:])
    out = [fn(flat[i], **kw) for i in range(flat.shape[0])]
    shape = m.shape[:-2] + (out[0].shape if out else m.shape[-2:])
    return np.stack(out).reshape(shape) if out else np.zeros(shape)


def ns(m, coeffs=None, steps: int = DEFAULT_STEPS, eps: float = DEFAULT_EPS):
    """Batched standard NS over the last two dims ([KX] §参考实现)."""
    return _batched(ns_single, m, coeffs=coeffs, steps=steps, eps=eps)


def gram_ns(m, coeffs=None, steps: int = DEFAULT_STEPS, eps: float = DEFAULT_EPS,
            restart_after: Sequence[int] = (2,)):
    """Batched Gram NS over the last two dims ([GR] §3.4 Algorithm 2)."""
    return _batched(gram_ns_single, m, coeffs=coeffs, steps=steps, eps=eps,
                    restart_after=tuple(restart_after))


def spectral_ns(m, coeffs=None, steps: int = DEFAULT_STEPS, eps: float = DEFAULT_EPS):
    """Batched SVD form of the NS output ([KX] §原理分析)."""
    return _batched(spectral_ns_single, m, coeffs=coeffs, steps=steps, eps=eps)


def exact_msign(m):
    """Batched exact msign via SVD ([KX] §写在前面)."""
    return _batched(svd_msign, m)


def ns_improved_init_single(m: np.ndarray, coeffs=None, steps: int = DEFAULT_STEPS,
                            eps: float = DEFAULT_EPS) -> np.ndarray:
    """NS with the improved initial normalisation of [KX] §改良初值.

    The section bounds the largest singular value by the chain
    sigma_1 <= (sum sigma_i^8)^(1/8) <= (sum sigma_i^4)^(1/4) <= ||M||_F and
    proposes dividing by the eighth-root term, the fourth root of
    ||(M M^T)^2||_F, instead of by ||M||_F.  It notes that this factor is free
    inside the iteration because X_0 X_0^T and its square are formed anyway,
    so it is taken from the Frobenius-normalised X_0.  Written here from that
    definition: with lambda_i the eigenvalues of X_0 X_0^T (= sigma_i(X_0)^2),
        s = (sum_i lambda_i^4 + eps)^(1/8),
    then the plain NS steps run from X_0 / s.  eps sits where the Frobenius
    normalisation puts it (under the root; 1e-20 by default), which only
    matters for an all-zero input.
    """
    m = np.asarray(m, dtype=np.float64)
    x, tall = _as_wide(m)
    x0 = frobenius_normalize(x, eps)
    lam = np.linalg.eigvalsh(x0 @ x0.T)
    s = (float(np.sum(lam ** 4)) + eps) ** 0.125
    x = _quintic_steps(x0 / s, coefficient_schedule(coeffs, steps))
    return x.T if tall else x


def ns_improved_init(m, coeffs=None, steps: int = DEFAULT_STEPS, eps: float = DEFAULT_EPS):
    """Batched form of `ns_improved_init_single`."""
    return _batched(ns_improved_init_single, m, coeffs=coeffs, steps=steps, eps=eps)


# ---------------------------------------------------------------------------
# Muon step around msign
# ---------------------------------------------------------------------------

def muon_step(w, g, m, mu: float, lr: float, msign=None):
    """One Muon update of parameters w with gradient g and momentum m.

    [GR] §1.1 states the update rule with a momentum matrix M_k (M_0 = 0),
    a momentum coefficient mu and a learning rate eta, but the formula itself
    is lost in the text; [MS] §标准 Muon 算法 gives the update direction
    -msign; [NB] applies NS to the gradient or its momentum.  Read as
        M <- mu M + G,   W <- W - eta msign(M).
    `msign` is the map applied over the last two dims (default: this
    module's NS).  Returns (new w, new m), both float64.
    """
    w = np.asarray(w, dtype=np.float64)
    m_new = mu * np.asarray(m, dtype=np.float64) + np.asarray(g, dtype=np.float64)
    o = (ns if msign is None else msign)(m_new)
    return w - lr * o, m_new


# ---------------------------------------------------------------------------
# error measure used by the parity tests
# ---------------------------------------------------------------------------

def max_rel_fro_error(y, ref) -> float:
    """max over the batch of ||Y - O||_F / ||O||_F (absolute ||Y||_F when O = 0)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if y.shape != ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {ref.shape}")
    if y.size == 0:
        return 0.0
    yb = y.reshape((-1,) + y.shape[-2:])
    rb = ref.reshape((-1,) + ref.shape[-2:])
    worst = 0.0
    for yi, ri in zip(yb, rb):
        den = float(np.linalg.norm(ri))
        num = float(np.linalg.norm(yi - ri))
        worst = max(worst, num / den if den > 0 else num)
    return worst


# ---------------------------------------------------------------------------
# FLOP models ([GR] §1.2, §2.4, §3.4), X is n x m with n <= m, alpha = m / n
# ---------------------------------------------------------------------------

def dense_ns_flops(n: int, m: int, steps: int = DEFAULT_STEPS) -> float:
    """Per step: X X^T 2mn^2, A^2 2n^3, B X 2mn^2 ([GR] §1.2)."""
    return steps * (2.0 * m * n * n + 2.0 * n ** 3 + 2.0 * m * n * n)


def symmetric_ns_flops(n: int, m: int, steps: int = DEFAULT_STEPS) -> float:
    """Symmetric GEMMs halve X X^T and A^2: T (3 alpha + 1) n^3 ([GR] §2.4)."""
    return steps * (1.0 * m * n * n + 1.0 * n ** 3 + 2.0 * m * n * n)


def naive_gram_flops(n: int, m: int, steps: int = DEFAULT_STEPS) -> float:
    """[GR] §2.4: X X^T (mn^2) + T steps of R^2 (n^3), Q Z (n^3), Z R Z (2n^3)
    + Q X (2mn^2), minus the free Q_1 (n^3) and the unused R_T (2n^3)."""
    per_step = 4.0 * n ** 3
    return m * n * n + steps * per_step + 2.0 * m * n * n - n ** 3 - 2.0 * n ** 3


def restart_gram_flops(n: int, m: int, steps: int = DEFAULT_STEPS, restarts: int = 1) -> float:
    """[GR] §3.4: each restart adds Q X (2mn^2) and X X^T (mn^2) and saves the
    unused R update (2n^3) and the free first Q product of the new block (n^3)."""
    return naive_gram_flops(n, m, steps) + restarts * (3.0 * m * n * n - 3.0 * n ** 3)

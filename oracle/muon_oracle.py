"""Plain, slow, float64 CPU oracle for the Muon optimizer step and the
periodic-RowNorm step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import or call this module; only the tests, the
smoke check and the CPU-baseline leg of the benchmark do.  It shares no code
with the GPU path.

Every function works on float64 NumPy copies of exactly the values the
caller stored (fp32 or bf16 values are upcast without change), and follows
the pages' order of operations with no blocking, fusion or reordering.

Sources (page title, then section / equation):
  [Infra]  "Infra Optimizers" (a summary of "Muon is Scalable for LLM
           Training"): Background, eq. (1) momentum and update, the Nesterov
           remark, the Frobenius normalisation X0 = M/||M||_F, eq. (2) the
           quintic Newton-Schulz step and its coefficients a, b, c;
           "Scaling Up Muon": eq. (3) weight decay, Lemma 1 and eq. (4) the
           0.2*sqrt(max(A, B)) update scale, N = 5 and mu = 0.95.
  [DiT]    "Scaling Muon for Diffusion Transformers": section 2.1 (the
           decoupled update W <- (1 - eta*lambda) W - eta*s(W)*Phi_5(M)),
           section 3.1 (short-side orientation O(.), the polar factor and the
           row-normalisation operator R_eps).
  [DMuon]  "DMuon: Efficient Distributed Muon Training with Near-Adam
           Overhead": section 2.2 (Gram-space Newton-Schulz on G = X X^T).

Readings where the pages are silent (each is also listed in the design
notes):
  * Nesterov input is U = mu*M' + G with M' the updated momentum and no
    (1 - mu) dampening ([Infra] Background).
  * The Frobenius normalisation is applied to U, the quantity fed to NS.
  * No epsilon in that normalisation: if ||U||_F == 0 the NS output is 0.
  * A square matrix is not transposed (m <= n keeps M, [DiT] 3.1).
  * RowNorm normalises the r rows of the oriented r x c matrix, i.e. the
    columns of M when m > n ([DiT] 3.1); rows with norm < eps are divided by
    eps exactly as R_eps is written.
  * RowNorm input is the same U (Nesterov blend); the RowNorm update uses the
    same 0.2*sqrt(max(m, n)) scale (the page is cut off before stating one).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# Coefficients of the quintic f(x) = a x + b x^3 + c x^5 ([Infra] eq. (2)).
NS_A = 3.4445
NS_B = -4.7750
NS_C = 2.0315


@dataclass(frozen=True)
class Hyper:
    """Hyper-parameters of one step.  Defaults: [Infra] "Scaling Up Muon"
    (mu = 0.95, N = 5, the 0.2 RMS-matching factor) and eq. (2) (a, b, c)."""

    momentum: float = 0.95
    nesterov: bool = True
    ns_steps: int = 5
    a: float = NS_A
    b: float = NS_B
    c: float = NS_C
    scale_coeff: float = 0.2
    rownorm_eps: float = 1e-8


def _f64(x) -> np.ndarray:
    return np.array(x, dtype=np.float64, copy=True)


def momentum_update(M, G, mu: float) -> np.ndarray:
    """M_t = mu * M_{t-1} + grad  ([Infra] eq. (1), first line; M_0 = 0)."""
    return mu * _f64(M) + _f64(G)


def nesterov_input(M_new, G, mu: float, nesterov: bool = True) -> np.ndarray:
    """The matrix fed to Newton-Schulz: mu * M_t + grad with M_t already
    updated ([Infra] Background, Nesterov remark); M_t itself if disabled."""
    M_new = _f64(M_new)
    if not nesterov:
        return M_new
    return mu * M_new + _f64(G)


def orient(U) -> tuple[np.ndarray, bool]:
    """Short-side orientation O(.) of [DiT] 3.1: keep U when m <= n, else
    use its transpose, so the result is r x c with r = min(m, n).  Returns
    (X, transposed)."""
    U = _f64(U)
    m, n = U.shape
    if m <= n:
        return U, False
    return U.T.copy(), True


def unorient(X, transposed: bool) -> np.ndarray:
    """O^{-1}: map an r x c result back to the m x n parameter shape."""
    return X.T.copy() if transposed else X


def ns5_direct(X, hp: Hyper = Hyper()) -> np.ndarray:
    """Newton-Schulz in the textbook direct form ([Infra] Background).

    X_0 = X / ||X||_F, then N times
        X_k = a X_{k-1} + b (X_{k-1} X_{k-1}^T) X_{k-1}
              + c (X_{k-1} X_{k-1}^T)^2 X_{k-1}        (eq. (2)).
    A zero input returns zero (no epsilon is stated; see module notes).
    Works for any orientation; callers pass the short-side X."""
    X = _f64(X)
    nrm = math.sqrt(float(np.sum(X * X)))
    if nrm == 0.0:
        return np.zeros_like(X)
    X = X / nrm
    for _ in range(hp.ns_steps):
        A = X @ X.T
        X = hp.a * X + hp.b * (A @ X) + hp.c * ((A @ A) @ X)
    return X


def ns5_gram(X, hp: Hyper = Hyper()) -> np.ndarray:
    """Gram-space form of the same iteration ([DMuon] 2.2: iterate on
    G = X X^T instead of the r x c matrix).

    Written from the algebra of eq. (2): X_k = p(A_{k-1}) X_{k-1} with
    p(A) = a I + b A + c A^2 and A_{k-1} = X_{k-1} X_{k-1}^T.  p(A) is a
    polynomial in A, so it commutes with A and
        A_k = p(A_{k-1}) A_{k-1} p(A_{k-1}),
        X_N = p(A_{N-1}) ... p(A_0) X_0.
    Kept only as an independent cross-check of the Gram formulation."""
    X = _f64(X)
    nrm = math.sqrt(float(np.sum(X * X)))
    if nrm == 0.0:
        return np.zeros_like(X)
    X0 = X / nrm
    r = X0.shape[0]
    I = np.eye(r)
    A = X0 @ X0.T
    Q = I.copy()
    for k in range(hp.ns_steps):
        P = hp.a * I + hp.b * A + hp.c * (A @ A)
        Q = P @ Q
        if k + 1 < hp.ns_steps:
            A = P @ A @ P
    return Q @ X0


def update_scale(m: int, n: int, coeff: float = 0.2) -> float:
    """s(W) = 0.2 * sqrt(max(A, B)) ([Infra] Lemma 1 and eq. (4))."""
    return coeff * math.sqrt(max(m, n))


def rownorm(X, eps: float) -> np.ndarray:
    """R_eps(X)_{i:} = X_{i:} / max(||X_{i:}||_2, eps), i = 1..r
    ([DiT] 3.1), applied to the oriented r x c matrix."""
    X = _f64(X)
    out = np.empty_like(X)
    for i in range(X.shape[0]):
        nrm = math.sqrt(float(np.dot(X[i], X[i])))
        # max(nrm, eps); a NaN norm (a NaN in the row) is kept, so the row
        # stays NaN rather than being scaled by 1/eps
        den = eps if nrm < eps else nrm
        out[i] = X[i] / den
    return out


def apply_update(W, D, lr: float, wd: float, scale: float) -> np.ndarray:
    """W_t = (1 - eta*lambda) W_{t-1} - eta * s * D
    ([DiT] 2.1 update; [Infra] eq. (4) expanded)."""
    return (1.0 - lr * wd) * _f64(W) - lr * scale * _f64(D)


def muon_step(W, M, G, lr: float, wd: float, hp: Hyper = Hyper(), form: str = "direct"):
    """One Newton-Schulz (refresh) step for a single m x n matrix.

    Returns (W_new, M_new, O) where O = O^{-1}(NS5(O(U))) is the m x n
    orthogonalised direction before scaling.  form="gram" evaluates the same
    map through ns5_gram (pinned equal to the direct form), which is cheaper
    for very wide matrices."""
    m, n = np.shape(W)
    M_new = momentum_update(M, G, hp.momentum)
    U = nesterov_input(M_new, G, hp.momentum, hp.nesterov)
    X, tr = orient(U)
    ns = ns5_gram if form == "gram" else ns5_direct
    O = unorient(ns(X, hp), tr)
    W_new = apply_update(W, O, lr, wd, update_scale(m, n, hp.scale_coeff))
    return W_new, M_new, O


def rownorm_step(W, M, G, lr: float, wd: float, hp: Hyper = Hyper()):
    """One non-refresh step of periodic RowNorm Muon ([DiT] abstract and
    3.1): the same momentum and Nesterov input, then R_eps on the oriented
    matrix in place of NS5, then the same scaled, decayed update.

    Returns (W_new, M_new, R) with R the m x n normalised direction."""
    m, n = np.shape(W)
    M_new = momentum_update(M, G, hp.momentum)
    U = nesterov_input(M_new, G, hp.momentum, hp.nesterov)
    X, tr = orient(U)
    R = unorient(rownorm(X, hp.rownorm_eps), tr)
    W_new = apply_update(W, R, lr, wd, update_scale(m, n, hp.scale_coeff))
    return W_new, M_new, R

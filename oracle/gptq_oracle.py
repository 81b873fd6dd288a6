"""Float64 CPU oracle of the GPTQ-family layer-quantisation path.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import
this module.  The HIP library never calls it, and it shares no code with the HIP path: it is a plain, slow,
obviously correct restatement of what the method computes, written from the method pages.

Sources (cited by page title and section; the pages are web pages, not code):
  [T]  GPTQ tutorial page, "GPTQ：量化一个权重之后怎样补偿输出误差" (charlestar.github.io, 2026-10-15).
       Its sections are referred to by order:
         T1 calibration objective and Hessian      T2 the two-weight example
         T3 one constrained compensation           T4 why the Cholesky factor is not the inverse
         T5 shared order, layout and lazy blocks    T6 damping, dead coordinates, grouping parameters
         T7 the two-dimensional check               T8 the three-dimensional counterexample
         T9 grid values vs stored low-bit codes
  [R]  "Rethinking Residual Errors in Compensation-based LLM Quantization" notes (ICLR 2026), section
       "关键设计" items 1-3 (column objective, compensation-aware error, neuron decomposition).
  [A]  "GPTAQ: Efficient Finetuning-Free Quantization for Asymmetric Calibration" notes (ICML 2025),
       section "关键设计" (asymmetric objective, closed form, channel parallelisation).
  [G]  "G²PTQ: Improving LLM Post-Training Quantization with Generalized Gradient Compensation" digest,
       method paragraphs (output-channel groups with one Hessian each; symmetric per-channel weights).

Notation follows [T]: X is M x K (tokens x input features), W is K x N (one column per output channel),
H = 2 X^T X.  Everything is float64 unless a step is defined in another precision, and then that precision
is emulated exactly (the fp32 scale, bf16 rounding of row-scaled activations).

Readings where the pages are silent (each is listed with its reason in the design notes):
  * damping: H_d = H + percdamp * mean(diag H) * I, the mean taken after the dead fix            [T6]
  * dead coordinates: H_kk == 0 -> H_kk := 1 and weight row k := 0, before damping             [T6]
  * grid: symmetric per-channel, s = fp32(2*max|w| / (2^b - 1)), zero point z = 2^(b-1), codes 0..2^b-1,
    reconstruction s*(c - z), round half to even then clamp; s from W before dead rows are zeroed
  * GPTAQ mask strictly upper, L = U^T, Hessian of the quantised stream (damped), coefficient = the
    coordinate's pre-rounding value at its step.
  * CAE term: P2 from 2 X~^T X = H + A (no separate Gram, as [R] item 3 notes), same mask and L; its
    coefficient is w0_q - w_q with w0 the original weight after dead rows are zeroed.

Pins (tests/test_oracle_pins.py): the two- and three-weight worked examples of [T2]/[T7]/[T8] with their
printed values, explicit-inverse sequential compensation and exhaustive search on tiny inputs, the factor's
Schur property, lazy == eager blocks, the per-channel loss identity, invariance under H -> cH, dead
coordinates, P1 and P2 against per-step least-squares solves (and the CAE loop against an explicit per-step
solve of the r1 + r2 residual), Gram identities and bf16 rounding against torch.
The scale rule of channel_scales (s = 2*absmax/(2^b-1), zero point 2^(b-1)) is pinned to the symmetric min-max
grid that [T2] (a quantiser's grid normally comes from min-max, unlike its fixed teaching grid) and [G] (symmetric
per channel) describe, built from its definition in the tests.
Parity unpinned by the pages: the value 1 given to dead diagonals (and the MSE clipping candidates) are readings
the pages leave open; their implementation is pinned only to their own stated definition (properties in the
tests), not to a value the pages print.
"""
from __future__ import annotations

import itertools
from typing import Iterable, Optional

import numpy as np

__all__ = [
    "bf16_round", "gram", "gram_row_scaled", "cross_gram", "prepare", "channel_scales", "quantize_layer",
    "asym_correction", "asym_correction_by_definition", "cae_correction", "cae_correction_by_definition",
    "act_order_perm", "grid_scales", "MSE_SHRINK", "pack_codes", "unpack_codes", "sylvester", "hadamard_rotate_rows", "layer_objective", "asym_objective",
    "obq_sequential", "exhaustive_best", "fixed_grid_quantize", "dequantize_fp32",
]


# ----------------------------------------------------------------------------------------------------------
# bf16 rounding (needed where the method rounds an fp32 product to bf16 before the Gram)
# ----------------------------------------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value, ties to even; returns float32 holding bf16 values.

    bf16 keeps the top 16 bits of the fp32 encoding.  Rounding adds 0x7FFF plus the lowest kept bit, then
    truncates; NaN is passed through unchanged.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    out = r.view(np.float32).copy()
    nan = np.isnan(x)
    out[nan] = x[nan]
    return out


# ----------------------------------------------------------------------------------------------------------
# a1: Gram / Hessian.  [T1]: the layer objective ||X W_hat - X W||_F^2 splits into one quadratic per output
# column, 1/2 dw^T H dw, with H = 2 X^T X shared by every output channel and accumulated batch by batch.
# ----------------------------------------------------------------------------------------------------------
def gram(batches: Iterable[np.ndarray], K: Optional[int] = None) -> np.ndarray:
    """H = 2 * sum over batches of X_b^T X_b, exact inputs promoted to float64."""
    H = None
    for Xb in batches:
        Xb = np.asarray(Xb, dtype=np.float64)
        if H is None:
            H = np.zeros((Xb.shape[1], Xb.shape[1]))
        H += 2.0 * (Xb.T @ Xb)
    if H is None:
        H = np.zeros((K, K))
    return H


def gram_row_scaled(X: np.ndarray, rho: np.ndarray) -> np.ndarray:
    """[G] one Hessian per output-channel group: H_g = 2 X_g^T X_g with X_g = bf16(fp32(rho_t) * x_t).

    The token weight multiplies each activation row in fp32 and the product is rounded to bf16 (the
    activations stay a bf16 stream); the Gram of the rounded rows is then exact in float64.
    """
    prod = np.asarray(rho, np.float32)[:, None] * np.asarray(X, np.float32)   # fp32 products, RNE
    Xg = bf16_round(prod)
    return gram([Xg])


def cross_gram(X_float: np.ndarray, X: np.ndarray) -> np.ndarray:
    """[R] item 3 / [A]: asymmetric term A = 2 (X~ - X)^T X, with X~ the float stream and X the quantised
    stream (so that X~^T X = X^T X + dX^T X, which lets the method reuse the ordinary Gram)."""
    Xf = np.asarray(X_float, np.float64)
    Xq = np.asarray(X, np.float64)
    return 2.0 * ((Xf - Xq).T @ Xq)


# ----------------------------------------------------------------------------------------------------------
# a2 + a3: dead coordinates, damping, and the upper factor U of the inverse.  [T4], [T6]
# ----------------------------------------------------------------------------------------------------------
class NotPositiveDefinite(ValueError):
    pass


def prepare(H: np.ndarray, percdamp: float) -> dict:
    """Returns U (upper, H_d^{-1} = U^T U), the dead mask, damp and H_d.

    [T6] zero-diagonal (dead) coordinates get diagonal 1; then percdamp * mean(diag H) is added to the
    diagonal.  [T4] U is the upper Cholesky factor of the inverse: read row by row, U_qq^2 is the inverse of
    the remaining Hessian when q is the first free coordinate.
    """
    H = np.array(H, dtype=np.float64, copy=True)
    if not np.all(np.isfinite(H)):
        raise ValueError("non-finite Hessian")
    K = H.shape[0]
    d = np.diag(H).copy()
    dead = d == 0.0
    H[dead, dead] = 1.0
    damp = percdamp * float(np.mean(np.diag(H))) if K else 0.0
    Hd = H + damp * np.eye(K)
    try:
        np.linalg.cholesky(Hd)
    except np.linalg.LinAlgError as e:
        raise NotPositiveDefinite(str(e)) from None
    P = np.linalg.inv(Hd)
    P = 0.5 * (P + P.T)
    L = np.linalg.cholesky(P)          # P = L L^T, L lower
    U = L.T                            # P = U^T U, U upper
    return {"U": U, "dead": dead, "damp": damp, "Hd": Hd, "P": P}


# ----------------------------------------------------------------------------------------------------------
# a5: the per-channel grid.  [G] symmetric per-channel weights; [T2]/[T9] codes 0..2^b-1 with zero point and
# reconstruction s*(q - z).  The scale rule itself is not printed on the pages; this is the reading adopted.
# ----------------------------------------------------------------------------------------------------------
def channel_scales(W: np.ndarray, bits: int) -> np.ndarray:
    """s_n = fp32(2 * max_k |W_kn| / (2^b - 1)) in fp32 arithmetic; 1 for an all-zero channel."""
    Wf = np.asarray(W, dtype=np.float32)
    amax = np.max(np.abs(Wf), axis=0) if Wf.shape[0] else np.zeros(Wf.shape[1], np.float32)
    qmax = np.float32(2 ** bits - 1)
    s = (np.float32(2.0) * amax) / qmax
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    return s


def dequantize_fp32(codes: np.ndarray, scales: np.ndarray, bits: int) -> np.ndarray:
    """[T9] reconstruction s * (c - z) evaluated in fp32 (the value written back as a weight)."""
    z = np.float32(2 ** (bits - 1))
    return (np.asarray(scales, np.float32)[None, :] * (codes.astype(np.float32) - z)).astype(np.float32)


# ----------------------------------------------------------------------------------------------------------
# a6 + a7: the shared-order column loop.  [T3] one constrained compensation, [T4] its Cholesky form,
# [T5] shared order for all channels and lazy block updates; [R]/[A] the asymmetric correction term.
# ----------------------------------------------------------------------------------------------------------
MSE_SHRINK = np.array([1.0 - i / 100.0 for i in range(21)], np.float32)   # clipping factors 1.00 .. 0.80


def act_order_perm(H: np.ndarray) -> np.ndarray:
    """[T6] act-order: the coordinates by descending Hessian diagonal, a processing-order heuristic.  Reading:
    the dead fix comes first (a zero diagonal counts as 1), the sort is stable (equal diagonals keep their
    natural order)."""
    d = np.diag(np.asarray(H, np.float64)).copy()
    d[d == 0.0] = 1.0
    return np.argsort(-d, kind="stable")


def grid_scales(Wg: np.ndarray, bits: int, mse: bool = False, choice: Optional[np.ndarray] = None,
                band: float = 1e-4) -> np.ndarray:
    """Symmetric grid scale per column of Wg (rows x N): s = fp32(2 max|w| / (2^b - 1)), 1 for an all-zero column.

    mse=True (the weight-MSE clipping of [G]'s main experiments): candidates s_i = fp32(fp32(2 max|w| alpha_i)
    / (2^b - 1)) for alpha_i = 1.00, 0.99, .., 0.80, and the one with the smallest sum of squared rounding
    errors over the column is taken (the first on exact ties).  choice (N scales, optional): where another run
    picked a different candidate whose error is within `band` (relative) of the smallest, that candidate is
    taken (several results are correct when fp32 error sums decide).
    """
    Wf = np.asarray(Wg, np.float32)
    N = Wf.shape[1]
    amax = np.max(np.abs(Wf), axis=0) if Wf.shape[0] else np.zeros(N, np.float32)
    qmax = np.float32(2 ** bits - 1)
    base = np.float32(2.0) * amax
    if not mse:
        s = base / qmax
    else:
        z = 2 ** (bits - 1)
        cand = (base[None, :] * MSE_SHRINK[:, None]) / qmax                   # fp32 products and quotients
        w = Wf.astype(np.float64)
        err = np.zeros(cand.shape)
        for i in range(len(MSE_SHRINK)):
            ci = cand[i].astype(np.float64)
            safe = np.where(ci > 0, ci, 1.0)
            q = ci * (np.clip(np.rint(w / safe) + z, 0, 2 ** bits - 1) - z)
            err[i] = np.sum((w - q) ** 2, axis=0)
        best = np.argmin(err, axis=0)
        if choice is not None:
            choice = np.asarray(choice, np.float32)
            for n in range(N):
                hit = np.flatnonzero(cand[:, n] == choice[n])
                if hit.size and err[hit[0], n] <= err[best[n], n] * (1.0 + band):
                    best[n] = hit[0]
        s = cand[best, np.arange(N)]
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def quantize_layer(W: np.ndarray, U: np.ndarray, bits: int, dead: Optional[np.ndarray] = None,
                   scales: Optional[np.ndarray] = None, blocksize: Optional[int] = None,
                   P1: Optional[np.ndarray] = None, tie_codes: Optional[np.ndarray] = None,
                   band: float = 1e-4, record_trace: bool = False, P2: Optional[np.ndarray] = None,
                   groupsize: Optional[int] = None, static_groups: bool = False, mse: bool = False,
                   perm: Optional[np.ndarray] = None, scale_choice: Optional[np.ndarray] = None) -> dict:
    """Quantise every output channel of W (K x N), all channels sharing one coordinate order.

    For coordinate j in processing order (same j for every channel), with s the scale in force at j:
        v = w_j / s;  c = clamp(round_half_even(v) + z, 0, 2^b - 1);  q = s (c - z)
        E_j = (w_j - q) / U_jj
        w_k -= U_jk E_j                      for every still-free k > j            [T3], [T4]
        w_k += P1_jk * w_j(pre-rounding)     for every k > j, asymmetric variant   [R] item 3
        w_k += P2_jk * (w0_j - w_j(pre))     for every k > j, CAE term             [R] items 2, 3
        w_j  = q
    (w0 is the original weight, after dead rows are zeroed.)
    blocksize=None applies every update at once (the literal sequential reading).  blocksize=B applies the
    updates inside the current block at once and the rest for the whole block at its end (lazy batch,
    [T5]); the two are the same computation up to rounding order.

    Scales ([T6]: groupsize changes the representation, blocksize only the computation):
      groupsize=None   one scale per channel (grid_scales of W before dead rows are zeroed), or `scales`;
      groupsize=G      one scale per channel and group of G coordinates.  Default ("re-estimated during
                       compensation"): the groups are G consecutive coordinates of the processing order, and a
                       group's scale is taken from the current, already compensated weights when the loop
                       reaches its first coordinate.  static_groups=True: groups of G consecutive original
                       coordinates with scales from W before the loop.
      mse=True         weight-MSE clipping (grid_scales) of the scales that come from W before the loop
                       (per channel or static groups); scale_choice gives another run's choice for ties.
    perm (act-order, [T6]): processing order; U, P1, P2 and dead then belong to the permuted Hessian
    (H[perm][:, perm]).  Inputs and outputs (codes, Q, E, V, W_pre, tie_codes) are in the original row
    order; g_idx gives the group of each original coordinate.

    tie_codes (K x N ints, optional): where several results are correct - v within `band` of a rounding
    midpoint - take the given code if it is one of the two codes nearest to v, so that the remainder of a
    channel can be compared with a run that broke that tie the other way.  Anywhere else it is ignored.
    """
    W_in = np.asarray(W)
    K, N = W_in.shape
    order = np.arange(K) if perm is None else np.asarray(perm, np.int64)
    assert sorted(order.tolist()) == list(range(K))
    U = np.asarray(U, np.float64)
    z = 2 ** (bits - 1)
    qmax = 2 ** bits - 1
    if groupsize is None:
        ng = 1
        s32 = grid_scales(W_in, bits, mse, scale_choice) if scales is None else np.asarray(scales, np.float32)
        S = s32[None, :]
        grp = np.zeros(K, np.int64)                       # group of each processing position
    else:
        G = int(groupsize)
        assert scales is None
        ng = (K + G - 1) // G
        S = np.zeros((ng, N), np.float32)
        if static_groups:
            for g in range(ng):
                ch = None if scale_choice is None else np.asarray(scale_choice)[g]
                S[g] = grid_scales(W_in[g * G:(g + 1) * G], bits, mse, ch)
            grp = order // G
        else:
            assert not mse, "MSE clipping applies to scales taken from W before the loop"
            grp = np.arange(K) // G
    W0 = np.array(W_in, dtype=np.float64, copy=True)[order]
    if dead is not None:                                  # like U, the dead mask is in processing order
        W0[np.asarray(dead, bool), :] = 0.0
    tie_p = None if tie_codes is None else np.asarray(tie_codes)[order]
    Wk = W0.copy()
    codes = np.zeros((K, N), np.int64)
    E = np.zeros((K, N))
    V = np.zeros((K, N))
    Wpre = np.zeros((K, N))
    Q = np.zeros((K, N))
    n_inband = 0
    n_adopted = 0
    trace = []
    B = max(K, 1) if blocksize is None else int(blocksize)
    for b0 in range(0, K, B):
        b1 = min(b0 + B, K)
        for j in range(b0, b1):
            if groupsize is not None and not static_groups and j % G == 0:
                S[j // G] = grid_scales(Wk[j:j + G], bits)   # current (compensated) weights of the group
            s = S[grp[j]].astype(np.float64)
            w = Wk[j].copy()
            Wpre[j] = w
            v = w / s
            c = np.clip(np.rint(v) + z, 0, qmax)
            fl = np.floor(v)
            inband = np.abs(v - fl - 0.5) < band
            n_inband += int(inband.sum())
            if tie_p is not None and inband.any():
                lo = np.clip(fl + z, 0, qmax)
                hi = np.clip(fl + 1 + z, 0, qmax)
                t = np.asarray(tie_p[j], np.float64)
                take = inband & ((t == lo) | (t == hi)) & (t != c)
                n_adopted += int(take.sum())
                c = np.where(take, t, c)
            q = s * (c - z)
            e = (w - q) / U[j, j]
            codes[j] = c.astype(np.int64)
            V[j] = v
            E[j] = e
            Q[j] = q
            if blocksize is None:
                hi_k = K
            else:
                hi_k = b1
            if j + 1 < hi_k:
                Wk[j + 1:hi_k] -= np.outer(U[j, j + 1:hi_k], e)
                if P1 is not None:
                    Wk[j + 1:hi_k] += np.outer(P1[j, j + 1:hi_k], w)
                if P2 is not None:
                    Wk[j + 1:hi_k] += np.outer(P2[j, j + 1:hi_k], W0[j] - w)
            Wk[j] = q
            if record_trace:
                trace.append(Wk.copy())
        if blocksize is not None and b1 < K:
            Wk[b1:] -= U[b0:b1, b1:].T @ E[b0:b1]
            if P1 is not None:
                Wk[b1:] += P1[b0:b1, b1:].T @ Wpre[b0:b1]
            if P2 is not None:
                Wk[b1:] += P2[b0:b1, b1:].T @ (W0[b0:b1] - Wpre[b0:b1])
    losses = 0.5 * np.sum(E * E, axis=0)

    def orig(a):                                           # processing order -> original row order
        out = np.empty_like(a)
        out[order] = a
        return out

    g_idx = orig(grp)
    codes_o = orig(codes)
    W_hat = (S[g_idx].astype(np.float32) * (codes_o.astype(np.float32) - np.float32(z))).astype(np.float32)
    return {
        "codes": codes_o, "scales": S[0] if groupsize is None else S, "Q": orig(Q), "E": orig(E), "V": orig(V),
        "W_pre": orig(Wpre), "W0": orig(W0), "losses": losses, "W_hat_fp32": W_hat, "g_idx": g_idx,
        "n_inband": n_inband, "n_adopted": n_adopted, "trace": trace,
    }


# ----------------------------------------------------------------------------------------------------------
# a4: GPTAQ correction matrix P1.  [R] item 3 gives the precomputed form [(dX X^T L) (.) M_U] L^T with
# H~^{-1} = L L^T; in this layout L = U^T and dX X^T is A / 2 scaled like H.
# ----------------------------------------------------------------------------------------------------------
def asym_correction(U: np.ndarray, A: np.ndarray) -> np.ndarray:
    """P1 = [(A U^T) masked to the strictly upper triangle] U."""
    U = np.asarray(U, np.float64)
    T = np.asarray(A, np.float64) @ U.T
    return np.triu(T, 1) @ U


def asym_correction_by_definition(Hd: np.ndarray, A: np.ndarray) -> np.ndarray:
    """Row q of P1 is the ridge least-squares response of the free coordinates F = {q+1..K-1} to coordinate
    q's input mismatch:  P1[q, F] = A[q, F] (H_d[F, F])^{-1}  ([A] closed form, the r X^T H^{-1}_{-q} term,
    split per coordinate by [R]'s neuron decomposition)."""
    K = Hd.shape[0]
    P1 = np.zeros((K, K))
    for q in range(K - 1):
        F = slice(q + 1, K)
        P1[q, F] = np.linalg.solve(Hd[F, F], A[q, F])     # H_FF symmetric
    return P1


# ----------------------------------------------------------------------------------------------------------
# CAE term.  [R] item 2: aligning every step to the fixed float output W0 X~ splits the residual into
# r1 = w^(q)(X~ - X) (the GPTAQ term) and the compensation-aware error r2 = (w^(0) - w^(q)) X~; item 3 makes
# r2 a per-coordinate term with the precomputed P2 = [(X~ X^T L) (.) M_U] L^T and the extra update
# (W0_q - W^(q)_q) P2[q, q:].  In this layout L = U^T and X~^T X = X^T X + dX^T X, i.e. 2 X~^T X = H + A.
# ----------------------------------------------------------------------------------------------------------
def cae_correction(U: np.ndarray, H: np.ndarray, A: Optional[np.ndarray] = None) -> np.ndarray:
    """P2 = [((H + A) U^T) masked to the strictly upper triangle] U, H = 2 X^T X, A = 2 (X~ - X)^T X."""
    U = np.asarray(U, np.float64)
    G = np.asarray(H, np.float64) + (0.0 if A is None else np.asarray(A, np.float64))
    return np.triu(G @ U.T, 1) @ U


def cae_correction_by_definition(Hd: np.ndarray, G: np.ndarray) -> np.ndarray:
    """Row q of P2 is the ridge least-squares response of the free coordinates F = {q+1..K-1} to coordinate
    q's float-stream input X~_q:  P2[q, F] = G[q, F] (H_d[F, F])^{-1} with G = 2 X~^T X (the r2 part of the
    r X^T H^{-1}_{-q} term, split per coordinate)."""
    K = Hd.shape[0]
    P2 = np.zeros((K, K))
    for q in range(K - 1):
        F = slice(q + 1, K)
        P2[q, F] = np.linalg.solve(Hd[F, F], G[q, F])
    return P2


# ----------------------------------------------------------------------------------------------------------
# Randomised Hadamard rotation.  [G] (setup paragraph): a Hadamard rotation is applied before quantisation.
# Reading: rows x of length K = 2^n (activation rows, and weight rows in the nn.Linear N x K layout) become
# x' = (x * d) H_K / sqrt(K) with d a +-1 vector and H_K the Sylvester Hadamard matrix, an orthogonal map that
# keeps x W^T unchanged when both sides are rotated.
# ----------------------------------------------------------------------------------------------------------
def sylvester(K: int) -> np.ndarray:
    """H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]."""
    assert K >= 1 and K & (K - 1) == 0
    H = np.ones((1, 1))
    while H.shape[0] < K:
        H = np.block([[H, H], [H, -H]])
    return H


def hadamard_rotate_rows(x: np.ndarray, signs: Optional[np.ndarray] = None) -> np.ndarray:
    """Each row of x (R x K) -> (row * signs) H_K / sqrt(K), in float64."""
    x = np.asarray(x, np.float64)
    K = x.shape[1]
    d = np.ones(K) if signs is None else np.asarray(signs, np.float64)
    return (x * d[None, :]) @ sylvester(K) / np.sqrt(K)


# ----------------------------------------------------------------------------------------------------------
# Packing.  [T9]: the loop's results are grid values s(c - z); storing them means turning them into integer
# codes packed into a wider integer container together with scale, zero point and layout.  The pages fix no
# bit layout; the reading used here: each output channel's K codes form one little-endian bitstream, code k
# occupying stream bits [bits*k, bits*k + bits), stored as 32-bit words along K (bit i of the stream is bit
# i % 32 of word i // 32).  Written bit by bit so the layout can be read off the code.
# ----------------------------------------------------------------------------------------------------------
def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes (K x N ints in [0, 2^bits)) -> words (ceil(K*bits/32) x N uint32)."""
    codes = np.asarray(codes, np.int64)
    K, N = codes.shape
    assert codes.min(initial=0) >= 0 and codes.max(initial=0) < (1 << bits)
    nw = (K * bits + 31) // 32
    out = np.zeros((nw, N), np.uint64)
    for k in range(K):
        for t in range(bits):
            bit = k * bits + t
            out[bit // 32] |= ((codes[k] >> t) & 1).astype(np.uint64) << np.uint64(bit % 32)
    return out.astype(np.uint32)


def unpack_codes(words: np.ndarray, K: int, bits: int) -> np.ndarray:
    """Inverse of pack_codes: words (ceil(K*bits/32) x N) -> codes (K x N int64)."""
    words = np.asarray(words, np.uint64)
    N = words.shape[1]
    codes = np.zeros((K, N), np.int64)
    for k in range(K):
        for t in range(bits):
            bit = k * bits + t
            codes[k] |= (((words[bit // 32] >> np.uint64(bit % 32)) & np.uint64(1)).astype(np.int64)) << t
    return codes


# ----------------------------------------------------------------------------------------------------------
# objectives.  [T1] J = ||X (W_hat - W)||_F^2 = 1/2 tr(D^T H D);  [A] asymmetric ||X W_hat - X~ W||_F^2.
# ----------------------------------------------------------------------------------------------------------
def layer_objective(H: np.ndarray, W: np.ndarray, W_hat: np.ndarray) -> float:
    D = np.asarray(W_hat, np.float64) - np.asarray(W, np.float64)
    return float(0.5 * np.sum((np.asarray(H, np.float64) @ D) * D))


def layer_objective_per_channel(H: np.ndarray, W: np.ndarray, W_hat: np.ndarray) -> np.ndarray:
    D = np.asarray(W_hat, np.float64) - np.asarray(W, np.float64)
    return 0.5 * np.sum((np.asarray(H, np.float64) @ D) * D, axis=0)


def asym_objective(H: np.ndarray, A: np.ndarray, G_float: np.ndarray, W: np.ndarray,
                   W_hat: np.ndarray) -> float:
    """||X W_hat - X~ W||^2 from the three Grams: H = 2X^TX, A = 2(X~-X)^T X, G~ = 2 X~^T X~ (so that
    X^T X~ = (H + A^T) / 2)."""
    W = np.asarray(W, np.float64)
    Wh = np.asarray(W_hat, np.float64)
    return float(0.5 * np.sum(Wh * (H @ Wh)) - np.sum(Wh * ((H + A.T) @ W)) + 0.5 * np.sum(W * (G_float @ W)))


# ----------------------------------------------------------------------------------------------------------
# textbook references used to pin the loop on tiny inputs.
# ----------------------------------------------------------------------------------------------------------
def fixed_grid_quantize(v: np.ndarray, lo: int = -8, hi: int = 7) -> np.ndarray:
    """[T2] fixed teaching grid {lo..hi}, step 1, round half to even."""
    return np.clip(np.rint(v), lo, hi)


def obq_sequential(H: np.ndarray, w: np.ndarray, quant, order=None, A: Optional[np.ndarray] = None,
                   damp: float = 0.0, X_free_basis: Optional[np.ndarray] = None, cae: bool = False,
                   quant_at=None) -> dict:
    """Sequential constrained compensation with an explicit inverse of the free block at every step.

    [T3]: with free set F (current coordinate q first) and P_F = (H[F,F])^{-1}, fixing w_q to its grid
    value moves the free coordinates by delta_F = -r P_F[:, q] / P_F[q, q], r = w_q - Q(w_q); the added
    objective is r^2 / (2 P_F[q, q]).
    Asymmetric variant: additionally the coordinates after q absorb coordinate q's input mismatch by
    ridge least squares; X_free_basis = (X, dX) pairs it is solved from directly (lstsq), independent of
    the P1 closed form.  cae=True adds the compensation-aware residual of coordinate q, (w0_q - w_q) X~_q with
    X~ = X + dX and w0 the starting weights, to the same least-squares right-hand side ([R] items 2, 3).
    quant_at(i, w) (optional) returns the quantiser for step i given the current weights (grids that are
    re-estimated during compensation).
    """
    H = np.asarray(H, np.float64)
    K = H.shape[0]
    w = np.array(w, np.float64, copy=True)
    w0 = w.copy()
    order = list(range(K)) if order is None else list(order)
    added = []
    trace = []
    for i, q in enumerate(order):
        F = order[i:]
        PF = np.linalg.inv(H[np.ix_(F, F)])
        pre = w[q]
        target = (quant if quant_at is None else quant_at(i, w))(w[q])
        r = w[q] - target
        delta = -r * PF[:, 0] / PF[0, 0]
        added.append(r * r / (2.0 * PF[0, 0]))
        w[F] = w[F] + delta
        w[q] = target
        if X_free_basis is not None and len(F) > 1:
            Xq, dXq = X_free_basis
            rest = F[1:]
            Xr = Xq[:, rest]
            lam = np.sqrt(damp / 2.0)
            lhs = np.vstack([Xr, lam * np.eye(len(rest))])
            resid = dXq[:, q] * pre
            if cae:
                resid = resid + (Xq[:, q] + dXq[:, q]) * (w0[q] - pre)
            rhs = np.concatenate([resid, np.zeros(len(rest))])
            sol = np.linalg.lstsq(lhs, rhs, rcond=None)[0]
            w[rest] += sol
        trace.append(w.copy())
    return {"w": w, "added": np.array(added), "trace": trace}


def exhaustive_best(objective, K: int, grid: Iterable[float]):
    """Minimum of objective over every point of grid^K and all minimisers (brute force, tiny K)."""
    grid = list(grid)
    best, arg = None, []
    for cand in itertools.product(grid, repeat=K):
        val = objective(np.array(cand, np.float64))
        if best is None or val < best - 1e-12:
            best, arg = val, [cand]
        elif abs(val - best) <= 1e-12:
            arg.append(cand)
    return best, arg

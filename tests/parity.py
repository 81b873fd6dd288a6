"""Comparison helpers of the parity tests (GPU path vs float64 oracle).  Test infrastructure only.

Tolerances (the bar of the parity suite):
  * H, A: relative Frobenius error <= 1e-4.
  * codes: identical, except at coordinates where the oracle's pre-rounding value w/s lies within 1e-4 of a
    rounding midpoint; there both neighbouring codes are correct, and the oracle follows the GPU's choice
    (it must be one of the two nearest codes) so that the rest of the channel stays comparable.
  * per-channel losses sum 1/2 E^2 and the layer objective 1/2 tr(D^T H D): relative error <= 1e-3.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O

BAND = 1e-4
H_TOL = 1e-4
OBJ_TOL = 1e-3


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def rel_fro(a: np.ndarray, b: np.ndarray) -> float:
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


DYN_SCALE_TOL = 1e-4   # re-estimated group scales: max of fp32 vs float64 working weights


def check_codes(gpu: dict, W: np.ndarray, U_ref: np.ndarray, bits: int, dead=None, P1=None, scales=None,
                H_obj: np.ndarray | None = None, label: str = "", P2=None, **opts) -> dict:
    """Runs the oracle loop with tie-following and asserts the GPU codes, scales, losses and objective.

    opts go to the oracle loop (groupsize, static_groups, mse, perm).  Scales taken from W before the loop are
    compared exactly (the oracle follows the GPU's pick among MSE candidates of equal error within the band);
    scales re-estimated from the working weights within DYN_SCALE_TOL.
    """
    codes = gpu["codes"].cpu().numpy().astype(np.int64)
    s_gpu = gpu["scales"].cpu().numpy()
    dynamic = opts.get("groupsize") and not opts.get("static_groups")
    if opts.get("mse"):
        opts["scale_choice"] = s_gpu
    ref = O.quantize_layer(W, U_ref, bits, dead=dead, scales=scales, blocksize=128, P1=P1, tie_codes=codes,
                           band=BAND, P2=P2, **opts)
    if dynamic:
        rel = np.abs(s_gpu.astype(np.float64) - ref["scales"]) / ref["scales"]
        assert rel.max() <= DYN_SCALE_TOL, f"{label}: re-estimated scales differ by {rel.max():.2e}"
    else:
        assert np.array_equal(s_gpu, ref["scales"]), f"{label}: scales differ"
    bad = codes != ref["codes"]
    n_bad = int(bad.sum())
    if n_bad:
        k, n = np.argwhere(bad)[0]
        v = ref["V"][k, n]
        raise AssertionError(f"{label}: {n_bad} code mismatches outside the tie band; first at (k={k}, n={n}) "
                             f"gpu={codes[k, n]} oracle={ref['codes'][k, n]} v={v!r}")
    info = {"n_inband": ref["n_inband"], "n_adopted": ref["n_adopted"], "ref": ref}
    if gpu.get("losses") is not None:
        lg = gpu["losses"].cpu().double().numpy()
        lr = ref["losses"]
        err = np.abs(lg - lr) / np.maximum(np.abs(lr), 1e-30)
        live = lr > 1e-30 * max(1.0, lr.max())
        assert (err[live] <= OBJ_TOL).all(), f"{label}: loss rel err max {err[live].max():.3e}"
        info["loss_rel_max"] = float(err[live].max()) if live.any() else 0.0
    if H_obj is not None:
        # the layer objective 1/2 tr(D^T H D) and, since it splits into one quadratic per output channel, each
        # channel's 1/2 d_n^T H d_n, both within OBJ_TOL of the oracle's
        z = 2 ** (bits - 1)
        W_hat = _gpu_values(codes, s_gpu, bits, ref)
        jg = O.layer_objective_per_channel(H_obj, W, W_hat)
        jr = O.layer_objective_per_channel(H_obj, W, ref["Q"])
        Jg, Jr = float(jg.sum()), float(jr.sum())
        assert abs(Jg - Jr) <= OBJ_TOL * abs(Jr), f"{label}: objective {Jg} vs {Jr}"
        live = jr > 1e-30 * max(1.0, float(jr.max()))
        cerr = np.abs(jg - jr)[live] / jr[live]
        assert (cerr <= OBJ_TOL).all(), f"{label}: per-channel objective rel err max {cerr.max():.3e}"
        info["J_gpu"], info["J_ref"] = Jg, Jr
        info["J_channel_rel_max"] = float(cerr.max()) if cerr.size else 0.0
    return info


def _gpu_values(codes: np.ndarray, s_gpu: np.ndarray, bits: int, ref: dict) -> np.ndarray:
    """Grid values s (c - z) of the GPU's codes in float64, with the scale in force at each original row
    (per channel, or per group through the oracle's group index of every row)."""
    z = 2 ** (bits - 1)
    s = np.asarray(s_gpu, np.float64)
    if s.ndim == 1:
        return s[None, :] * (codes - z)
    return s[ref["g_idx"]] * (codes - z)


def inverse_factor_residual(H32: np.ndarray, U_rows: np.ndarray, rows: np.ndarray, dead: np.ndarray,
                            damp: float, chunk: int = 2048) -> np.ndarray:
    """(U H_d U^T)[rows, rows] - I in float64, from the full fp32 Hessian and the sampled rows of U.

    H_d is H with dead diagonal entries set to 1 and damp added to the diagonal.  UᵀU = H_d⁻¹ with U upper
    is equivalent to U H_d Uᵀ = I (U invertible), a property that holds at any size, so sampled rows of U
    can be checked without a full-size reference factorisation.  H is streamed in row chunks.
    """
    K = H32.shape[0]
    Us = np.asarray(U_rows, np.float64)                      # len(rows) x K
    Y = np.empty((K, Us.shape[0]))
    for r0 in range(0, K, chunk):
        Y[r0:r0 + chunk] = H32[r0:r0 + chunk].astype(np.float64) @ Us.T
    fix = np.full(K, float(damp))
    d = np.asarray(dead, bool)
    fix[d] += 1.0 - H32[np.flatnonzero(d), np.flatnonzero(d)].astype(np.float64)
    Y += fix[:, None] * Us.T
    return Us @ Y - np.eye(len(rows))

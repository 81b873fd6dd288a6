"""Parity at the benchmark's full size and launch configuration (LLaMA-8B q_proj: K = N = 4096,
M = 1024 x 2048 tokens, bf16 Hadamard-rotated activations, 3-bit), on outputs the oracle can compute one by
one: a sampled principal block of H (exact float64 sums over all 2,097,152 tokens), and the column loop on
sampled channels after a full-size prepare of an oracle-computed Hessian.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads
from tests.parity import BAND, H_TOL, check_codes, inverse_factor_residual, np64, rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import post_weight_quantization_09_amd as pkg
    pkg.load()
    return pkg


@pytest.fixture(scope="module")
def c2(g):
    cfg = workloads.CONFIGS["c2_q_proj_8b"]
    X = torch.empty(cfg.M, cfg.K, dtype=torch.bfloat16, device=DEV)
    workloads.ActivationSource(cfg, DEV).fill(X)
    W = workloads.make_weights(cfg, device=DEV)
    torch.cuda.synchronize()
    print(f"generated c2 X {tuple(X.shape)}", flush=True)
    yield cfg, X, W
    del X


def test_c2_gram_sampled_block(g, c2):
    cfg, X, W = c2
    H = torch.zeros(cfg.K, cfg.K, device=DEV)
    g.gptq_accumulate_hessian(H, X)
    rng = np.random.default_rng(2024)
    S = np.sort(rng.choice(cfg.K, size=48, replace=False))
    S = np.unique(np.concatenate([S, [0, cfg.K - 1]]))
    idx = torch.tensor(S, device=DEV)
    Xs = X.index_select(1, idx).float().cpu().numpy()
    ref = O.gram([Xs])
    got = np64(H)[np.ix_(S, S)]
    err = rel_fro(got, ref)
    scale = np.sqrt(np.outer(np.diag(ref), np.diag(ref)))
    emax = float(np.max(np.abs(got - ref) / scale))
    print(f"c2 Gram sampled {len(S)}x{len(S)} block: rel fro {err:.3e}, max |dH|/sqrt(HiiHjj) {emax:.3e}", flush=True)
    assert err <= H_TOL
    Hn = np64(H)
    assert np.array_equal(Hn, Hn.T)


def test_c2_prepare_and_quantize_sampled_channels(g, c2):
    """The whole q_proj layer as the bench runs it: the GPU Gram over all 2,097,152 tokens, prepare and the column
    loop over all 4096 channels; the oracle factorises the same Hessian in float64 (its own U) and runs its loop on
    64 sampled channels: codes, per-channel and layer objectives, and the pre-rounding drift."""
    cfg, X, W = c2
    H = torch.zeros(cfg.K, cfg.K, device=DEV)
    g.gptq_accumulate_hessian(H, X)
    H32 = H.cpu().numpy()
    H64 = H32.astype(np.float64)
    ref = O.prepare(H64, cfg.percdamp)
    dead, damp, n_dead = g.gptq_prepare(H, cfg.percdamp)
    Ug = np64(H)
    uerr = float(np.abs(Ug - ref["U"]).max() / np.abs(ref["U"]).max())
    print(f"c2 prepare K={cfg.K}: U max rel err {uerr:.3e}, damp {damp:.6e} vs {ref['damp']:.6e}", flush=True)
    assert uerr <= 1e-3
    chans = np.sort(np.random.default_rng(7).choice(cfg.N, size=64, replace=False))
    _loop_check(g, W, H, dead, cfg.bits, chans, "c2 full layer (oracle's own U)", U_ref=ref["U"],
                dead_ref=ref["dead"], H_obj=H64)


# ------------------------------------------------------------------------------------------------------------
# The other layer workloads at full size: C3 (down_proj 8B, K = 14336, four output-channel groups with their
# own token-weighted Hessians), C4 (up_proj 8B with asymmetric calibration), C5 (70B down_proj, K = 28672, with
# 287 dead input channels).  Gram blocks are checked exactly on sampled coordinates; U through the
# U H_d U^T = I property on sampled rows; the column loop on sampled channels against the oracle, with the
# oracle's own float64 factor wherever the host finishes it in about a minute (K = 4096, 14336) and with the
# library's U at K = 28672 (the float64 inverse and two Cholesky factorisations of a 28672 x 28672 matrix take
# several minutes of host time), every time with the layer objective of the full-size Hessian.
# ------------------------------------------------------------------------------------------------------------
RESID_TOL = 1e-4   # |U H_d U^T - I| on sampled rows: fp32 rounding gives ~1e-6 here; a 1% damping error gives ~1e-2


def _make(cfg):
    W = workloads.make_weights(cfg, device=DEV)
    X = torch.empty(cfg.M, cfg.K, dtype=cfg.torch_x_dtype, device=DEV)
    Xf = torch.empty_like(X) if cfg.asym_noise > 0 else None
    workloads.ActivationSource(cfg, DEV).fill(X, Xf)
    rho = workloads.make_group_row_weights(cfg, device=DEV)
    torch.cuda.synchronize()
    print(f"generated {cfg.name}: X {tuple(X.shape)}", flush=True)
    return W, X, Xf, rho


def _sample(K, n, seed, extra=()):
    rng = np.random.default_rng(seed)
    S = rng.choice(K, size=min(n, K), replace=False)
    return np.unique(np.concatenate([S, [0, K - 1], np.asarray(extra, np.int64)])).astype(np.int64)


def _cols(T, S):
    return T.index_select(1, torch.tensor(S, device=T.device)).float().cpu().numpy()


def _block_err(Hg, ref, S, label):
    got = np64(Hg)[np.ix_(S, S)] if isinstance(Hg, torch.Tensor) else Hg
    err = rel_fro(got, ref)
    print(f"{label}: sampled {len(S)}x{len(S)} block rel fro {err:.3e}", flush=True)
    return err


def _factor_check(U, H32, dead, damp, percdamp, label, rows_seed):
    """Dead set and damping exactly, and U H_d U^T = I on sampled rows of the library's U (device, in place of H)."""
    K = H32.shape[0]
    diag = np.diag(H32).astype(np.float64)
    dead_ref = diag == 0.0
    damp_ref = percdamp * np.where(dead_ref, 1.0, diag).mean()
    assert np.array_equal(dead.cpu().numpy().astype(bool), dead_ref)
    assert abs(damp - damp_ref) <= 1e-6 * damp_ref
    rows = _sample(K, 24, rows_seed, extra=np.flatnonzero(dead_ref)[:2])
    Ur = U.index_select(0, torch.tensor(rows, device=U.device)).cpu().numpy()
    for i, r in enumerate(rows):
        assert np.count_nonzero(Ur[i, :r]) == 0, f"{label}: row {r} of U not upper triangular"
    R = inverse_factor_residual(H32, Ur, rows, dead_ref, damp)
    print(f"{label}: prepare n_dead={int(dead_ref.sum())} damp={damp:.6e} |U H_d U^T - I| max on {len(rows)} rows "
          f"{np.abs(R).max():.3e}", flush=True)
    assert np.abs(R).max() <= RESID_TOL
    return dead_ref


def _prepare_and_check(g, H, cfg, label, rows_seed):
    """Full-size prepare on the GPU; returns (dead device mask, dead reference, fp32 Hessian copied before)."""
    H32 = H.cpu().numpy()
    dead, damp, n_dead = g.gptq_prepare(H, cfg.percdamp)
    dead_ref = _factor_check(H, H32, dead, damp, cfg.percdamp, label, rows_seed)
    assert n_dead == int(dead_ref.sum())
    return dead, dead_ref, H32


def _drift_and_print(label, info, pre_sub, extra=""):
    drift = float(np.abs(pre_sub - info["ref"]["V"]).max())
    print(f"{label}: {info['ref']['V'].shape[1]} channels: codes equal outside the band; inband={info['n_inband']} "
          f"adopted={info['n_adopted']} pre_round drift max={drift:.2e} loss rel max={info.get('loss_rel_max', 0):.2e}"
          f" objective rel max per channel={info.get('J_channel_rel_max', 0):.2e} "
          f"J={info.get('J_gpu', 0):.6e}/{info.get('J_ref', 0):.6e}{extra}", flush=True)
    assert drift < BAND
    return drift


def _loop_check(g, W, U, dead, bits, chans, label, U_ref=None, dead_ref=None, P1=None, P1_ref=None, P2=None,
                H_obj=None):
    """The column loop over all of W's channels (the bench's launch), checked on `chans` against the oracle with
    U_ref (default: the library's U) and P1_ref (default: the library's P1).  P2 given: the loop runs with
    GPTQ_FLAG_CAE and the oracle with that P2.  Returns the check info and the pre-rounding drift."""
    K, N = W.shape
    pre = torch.empty(K, N, device=DEV)
    out = g.gptq_quantize_layer(W, U, bits, dead=dead, P1=P1, losses=torch.empty(N, device=DEV), pre_round=pre,
                                cae=P2 is not None)
    C = torch.tensor(chans, device=DEV)
    sub = {"codes": out["codes"][:, C], "scales": out["scales"][C], "losses": out["losses"][C]}
    U64 = np64(U) if U_ref is None else U_ref
    P64 = (np64(P1) if P1 is not None else None) if P1_ref is None else P1_ref
    dref = dead.cpu().numpy().astype(bool) if dead_ref is None else dead_ref
    info = check_codes(sub, W.float().cpu().numpy()[:, chans], U64, bits, dead=dref, P1=P64, P2=P2, H_obj=H_obj,
                       label=label)
    drift = _drift_and_print(label, info, pre[:, C].cpu().double().numpy())
    return info, drift


def test_c3_groups_full_size_end_to_end(g):
    """The down_proj layer with four output-channel groups as the bench runs it: four token-weighted Grams,
    gptq_prepare_groups and gptq_quantize_layer_groups over all 4096 channels.  Group 2 against the oracle's own
    float64 factor of its Hessian (32 sampled channels); every group's factor by the U H_d U^T = I property and
    8 channels of each group against the oracle fed that group's library U; objectives of each group's Hessian."""
    cfg = workloads.CONFIGS["c3_down_proj_8b_g4"]
    W, X, _, rho = _make(cfg)
    Hs = torch.zeros(cfg.groups, cfg.K, cfg.K, device=DEV)
    for gi in range(cfg.groups):
        g.gptq_accumulate_hessian(Hs[gi], X, row_scale=rho[gi].contiguous())
    S = _sample(cfg.K, 40, 31)
    ref_blk = O.gram_row_scaled(_cols(X, S), rho[2].cpu().numpy())
    assert _block_err(Hs[2], ref_blk, S, "c3 group 2 Gram") <= H_TOL
    del X
    torch.cuda.empty_cache()
    H32 = [Hs[gi].cpu().numpy() for gi in range(cfg.groups)]
    dead, damps, n_dead = g.gptq_prepare_groups(Hs, cfg.percdamp)
    for gi in range(cfg.groups):
        _factor_check(Hs[gi], H32[gi], dead[gi], damps[gi], cfg.percdamp, f"c3 group {gi}", 32 + gi)
    K, N, gs = cfg.K, cfg.N, cfg.N // cfg.groups
    pre = torch.empty(K, N, device=DEV)
    out = g.gptq_quantize_layer_groups(W, Hs, cfg.bits, dead=dead, losses=torch.empty(N, device=DEV), pre_round=pre)
    Wn = W.float().cpu().numpy()

    def check(gi, chans, U_ref, dead_ref, label):
        cols = gi * gs + chans
        C = torch.tensor(cols, device=DEV)
        sub = {"codes": out["codes"][:, C], "scales": out["scales"][C], "losses": out["losses"][C]}
        H64 = H32[gi].astype(np.float64)
        info = check_codes(sub, Wn[:, cols], U_ref, cfg.bits, dead=dead_ref, H_obj=H64, label=label)
        _drift_and_print(label, info, pre[:, C].cpu().double().numpy())

    rng = np.random.default_rng(33)
    for gi in range(cfg.groups):
        chans = np.sort(rng.choice(gs, 8, replace=False))
        check(gi, chans, np64(Hs[gi]), dead[gi].cpu().numpy().astype(bool), f"c3 group {gi} (library U)")
    ref = O.prepare(H32[2].astype(np.float64), cfg.percdamp)
    uerr = float(np.abs(np64(Hs[2]) - ref["U"]).max() / np.abs(ref["U"]).max())
    print(f"c3 group 2: float64 factor K={K}; library U max rel err {uerr:.3e}", flush=True)
    check(2, np.sort(rng.choice(gs, 32, replace=False)), ref["U"], ref["dead"], "c3 group 2 (oracle's own U)")
    # wider grids on the same factor: 5 and 6 bits (the band is relatively tighter as |w / s| grows)
    chans = np.sort(rng.choice(gs, 16, replace=False))
    for bits in (5, 6):
        Wg = W[:, 2 * gs:3 * gs]
        pre_b = torch.empty(K, gs, device=DEV)
        out_b = g.gptq_quantize_layer(Wg, Hs[2], bits, dead=dead[2], losses=torch.empty(gs, device=DEV),
                                      pre_round=pre_b)
        C = torch.tensor(chans, device=DEV)
        sub = {"codes": out_b["codes"][:, C], "scales": out_b["scales"][C], "losses": out_b["losses"][C]}
        label = f"c3 group 2 at {bits} bits (oracle's own U)"
        info = check_codes(sub, Wn[:, 2 * gs + chans], ref["U"], bits, dead=ref["dead"],
                           H_obj=H32[2].astype(np.float64), label=label)
        _drift_and_print(label, info, pre_b[:, C].cpu().double().numpy())


def test_c3_prepare_groups_full_size(g):
    """The four group Hessians of the down_proj workload (K = 14336) factorised in one grouped call, as the
    bench's groups driver does: bit-identical to one gptq_prepare per group (the batched launches include the
    128 x 128-tile triangular products of the two top levels)."""
    cfg = workloads.CONFIGS["c3_down_proj_8b_g4"]
    _, X, _, rho = _make(cfg)
    Hs = torch.zeros(cfg.groups, cfg.K, cfg.K, device=DEV)
    for gi in range(cfg.groups):
        g.gptq_accumulate_hessian(Hs[gi], X, row_scale=rho[gi].contiguous())
    del X
    torch.cuda.empty_cache()
    single = Hs.clone()
    dead, damps, n_dead = g.gptq_prepare_groups(Hs, cfg.percdamp)
    for gi in range(cfg.groups):
        d1, damp1, nd1 = g.gptq_prepare(single[gi], cfg.percdamp)
        assert torch.equal(Hs[gi], single[gi]), f"group {gi}: U differs from the single-Hessian call"
        assert torch.equal(dead[gi], d1) and damps[gi] == damp1 and n_dead[gi] == nd1
    print(f"c3 grouped prepare: {cfg.groups} x K={cfg.K} identical to single calls; damps {damps}", flush=True)


def test_c4_gptaq_gram_prepare_asym_loop(g):
    cfg = workloads.CONFIGS["c4_up_proj_8b_gptaq"]
    W, X, Xf, _ = _make(cfg)
    H = torch.zeros(cfg.K, cfg.K, device=DEV)
    A = torch.zeros(cfg.K, cfg.K, device=DEV)
    g.gptq_accumulate_hessian(H, X, X_float=Xf, A=A)
    S = _sample(cfg.K, 40, 41)
    Xs, Xfs = _cols(X, S), _cols(Xf, S)
    assert _block_err(H, O.gram([Xs]), S, "c4 Gram") <= H_TOL
    assert _block_err(A, O.cross_gram(Xfs, Xs), S, "c4 cross Gram") <= H_TOL
    del X, Xf
    torch.cuda.empty_cache()
    H64 = np64(H)
    A64 = np64(A)
    dead, damp, n_dead = g.gptq_prepare(H, cfg.percdamp)
    ref = O.prepare(H64, cfg.percdamp)
    U64 = np64(H)
    uerr = float(np.abs(U64 - ref["U"]).max() / np.abs(ref["U"]).max())
    print(f"c4 prepare K={cfg.K}: U max rel err {uerr:.3e}", flush=True)
    assert uerr <= 1e-3
    P1 = g.gptq_asym_correction(H, A)
    P1_lib = O.asym_correction(U64, A64)
    perr = rel_fro(np64(P1), P1_lib)
    print(f"c4 P1 (full {cfg.K}x{cfg.K}) rel fro {perr:.3e}", flush=True)
    assert perr <= 1e-4
    P1_ref = O.asym_correction(ref["U"], A64)          # from the oracle's own factor
    chans = np.sort(np.random.default_rng(43).choice(cfg.N, 32, replace=False))
    _loop_check(g, W, H, dead, cfg.bits, chans, "c4 (oracle's own U and P1)", U_ref=ref["U"], dead_ref=ref["dead"],
                P1=P1, P1_ref=P1_ref, H_obj=H64)
    P2 = O.cae_correction(ref["U"], H64, A64)           # the CAE term from the oracle's U, H and A
    _loop_check(g, W, H, dead, cfg.bits, chans, "c4 with the CAE term (oracle's own U, P1, P2)", U_ref=ref["U"],
                dead_ref=ref["dead"], P1=P1, P1_ref=P1_ref, P2=P2, H_obj=H64)


def test_c5_gram_prepare_loop(g):
    cfg = workloads.CONFIGS["c5_down_proj_70b"]
    W, X, _, _ = _make(cfg)
    dead_idx = workloads.dead_channels(cfg)
    assert len(dead_idx) == round(0.01 * cfg.K)
    H = torch.zeros(cfg.K, cfg.K, device=DEV)
    g.gptq_accumulate_hessian(H, X)
    S = _sample(cfg.K, 40, 51, extra=dead_idx[:3])
    assert _block_err(H, O.gram([_cols(X, S)]), S, "c5 Gram") <= H_TOL
    del X
    torch.cuda.empty_cache()
    dead, dead_ref, H32 = _prepare_and_check(g, H, cfg, "c5", 52)
    assert np.array_equal(np.flatnonzero(dead_ref), dead_idx)
    chans = np.sort(np.random.default_rng(53).choice(cfg.N, 32, replace=False))
    H64 = H32.astype(np.float64)
    _loop_check(g, W, H, dead, cfg.bits, chans, "c5 (library U)", dead_ref=dead_ref, H_obj=H64)
    _loop_check(g, W, H, dead, 6, chans[::2], "c5 at 6 bits (library U)", dead_ref=dead_ref, H_obj=H64)


def test_c5_pack_codes_full_size(g):
    """Codes of the 70B down_proj shape (K = 28672, N = 8192, 4-bit) packed and read back; sampled channels
    against the oracle's bitstream."""
    cfg = workloads.CONFIGS["c5_down_proj_70b"]
    gen = torch.Generator(device=DEV)
    gen.manual_seed(55)
    codes = torch.randint(0, 1 << cfg.bits, (cfg.K, cfg.N), generator=gen, device=DEV, dtype=torch.int32).to(torch.uint8)
    packed = g.gptq_pack_codes(codes, cfg.bits)
    assert packed.shape == (cfg.K * cfg.bits // 32, cfg.N)
    chans = np.sort(np.random.default_rng(56).choice(cfg.N, 16, replace=False))
    C = torch.tensor(chans, device=DEV)
    ref = O.pack_codes(codes[:, C].cpu().numpy().astype(np.int64), cfg.bits)
    assert np.array_equal(packed[:, C].cpu().numpy().view(np.uint32), ref)
    back = g.gptq_unpack_codes(packed, cfg.K, cfg.bits)
    assert torch.equal(back["codes"], codes)
    print(f"c5 packing: {cfg.K}x{cfg.N} {cfg.bits}-bit codes -> {tuple(packed.shape)} words, round trip exact",
          flush=True)


def test_c2_hadamard_rotation_full_size(g):
    """The rotation step of the q_proj workload at full size (2,097,152 bf16 rows of K = 4096, in place) on
    sampled rows against the exact rotation of the same unrotated rows."""
    cfg = workloads.CONFIGS["c2_q_proj_8b"].scaled(hadamard=False)
    X = torch.empty(cfg.M, cfg.K, dtype=torch.bfloat16, device=DEV)
    workloads.ActivationSource(cfg, DEV).fill(X)
    rows = np.sort(np.random.default_rng(61).choice(cfg.M, 64, replace=False))
    R = torch.tensor(rows, device=DEV)
    before = X.index_select(0, R).float().cpu().numpy().astype(np.float64)
    d = workloads.hadamard_signs(workloads.CONFIGS["c2_q_proj_8b"]).astype(np.int8)
    g.gptq_hadamard_rotate(X, torch.tensor(d, device=DEV), out=X)
    after = X.index_select(0, R).float().cpu().numpy().astype(np.float64)
    ref = O.hadamard_rotate_rows(before, d)
    n = int(np.log2(cfg.K))
    bound = 2.0 * (n + 2) * 2.0 ** -24 * np.abs(before).sum(axis=1, keepdims=True) / np.sqrt(cfg.K)
    rel = np.abs(after - ref) - np.abs(ref) * 2.0 ** -8      # bf16 half-ulp of the result
    assert (rel <= bound).all()
    print(f"c2 rotation: {cfg.M} rows of {cfg.K} in place; 64 sampled rows within half a bf16 ulp + the fp32 bound",
          flush=True)

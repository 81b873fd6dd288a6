"""The C-ABI library loads and exports every symbol include/gptq.h declares; host-side validation paths
(no GPU needed: arguments are checked before any HIP call)."""
import ctypes
import os
import re

import pytest

import post_weight_quantization_09_amd as g
from post_weight_quantization_09_amd import _binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(gptq_[a-z_0-9]+)\s*\(", text))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(g.LIB_PATH):
        pytest.fail("libgptq_hip.so is not built (run __graft_entry__.build())")
    return g.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"gptq_accumulate_hessian", "gptq_prepare", "gptq_asym_correction", "gptq_quantize_layer"} <= names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert g.version().count(".") == 2
    for s in range(6):
        assert g.status_string(s)
    assert g.status_string(0) == "ok"


def test_workspace_sizes(lib):
    acc_small = g.gptq_workspace_bytes(g.GPTQ_CALL_ACCUMULATE_HESSIAN, 512, 0, 4096)
    acc_cross = g.gptq_workspace_bytes(g.GPTQ_CALL_ACCUMULATE_HESSIAN, 512, 0, 4096, 1)
    assert acc_small >= 256 and acc_cross >= acc_small
    assert g.gptq_workspace_bytes(g.GPTQ_CALL_PREPARE, 4096) >= 4096 * 4096
    q = g.gptq_workspace_bytes(g.GPTQ_CALL_QUANTIZE_LAYER, 4096, 4096)
    qa = g.gptq_workspace_bytes(g.GPTQ_CALL_QUANTIZE_LAYER, 4096, 4096, 0, 2)
    assert q >= 4096 * 4096 * 5 and qa > q
    for v in (acc_small, acc_cross, q, qa):
        assert v % 256 == 0
    assert lib.gptq_workspace_bytes(17, 10, 10, 10, 0) == 0


FAKE = ctypes.c_void_p(0x100000)   # never dereferenced: validation fails first


def test_accumulate_validation(lib):
    ws = ctypes.c_void_p(0x100000)
    assert lib.gptq_accumulate_hessian(None, 8, FAKE, 1, 4, 8, None, None, 8, None, ws, 1 << 20, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_accumulate_hessian(FAKE, 0, FAKE, 1, 4, 8, None, None, 8, None, ws, 1 << 20, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_accumulate_hessian(FAKE, 8, FAKE, 1, 4, 7, None, None, 8, None, ws, 1 << 20, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_accumulate_hessian(FAKE, 8, FAKE, 5, 4, 8, None, None, 8, None, ws, 1 << 20, None) == b.GPTQ_ERR_ARG
    # row scale needs bf16; cross term needs A
    assert lib.gptq_accumulate_hessian(FAKE, 8, FAKE, 0, 4, 8, FAKE, None, 8, None, ws, 1 << 20, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_accumulate_hessian(FAKE, 8, FAKE, 1, 4, 8, None, FAKE, 8, None, ws, 1 << 20, None) == b.GPTQ_ERR_ARG
    # workspace too small or misaligned
    assert lib.gptq_accumulate_hessian(FAKE, 8, FAKE, 1, 4, 8, None, None, 8, None, ws, 16, None) == b.GPTQ_ERR_WORKSPACE
    assert lib.gptq_accumulate_hessian(FAKE, 8, FAKE, 1, 4, 8, None, None, 8, None, ctypes.c_void_p(0x100010),
                                       1 << 20, None) == b.GPTQ_ERR_WORKSPACE


def test_prepare_validation(lib):
    d, n = ctypes.c_float(0), ctypes.c_int64(0)
    ws = ctypes.c_void_p(0x100000)
    assert lib.gptq_prepare(None, 8, 0.01, FAKE, ctypes.byref(d), ctypes.byref(n), ws, 1 << 20, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_prepare(FAKE, 8, -0.5, FAKE, ctypes.byref(d), ctypes.byref(n), ws, 1 << 20, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_prepare(FAKE, 8, float("nan"), FAKE, None, None, ws, 1 << 20, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_prepare(FAKE, 8, 0.01, None, None, None, ws, 1 << 20, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_prepare(FAKE, 4096, 0.01, FAKE, None, None, ws, 1024, None) == b.GPTQ_ERR_WORKSPACE


def test_prepare_groups_validation(lib):
    ws = ctypes.c_void_p(0x100000)
    big = 1 << 30
    assert lib.gptq_prepare_groups(None, 8, 2, 64, 0.01, FAKE, None, None, ws, big, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_prepare_groups(FAKE, 8, 0, 64, 0.01, FAKE, None, None, ws, big, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_prepare_groups(FAKE, 8, 65536, 64, 0.01, FAKE, None, None, ws, big, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_prepare_groups(FAKE, 8, 2, 63, 0.01, FAKE, None, None, ws, big, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_prepare_groups(FAKE, 8, 2, 64, -1.0, FAKE, None, None, ws, big, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_prepare_groups(FAKE, 8, 2, 64, 0.01, None, None, None, ws, big, None) == b.GPTQ_ERR_ARG
    one = lib.gptq_workspace_bytes(b.GPTQ_CALL_PREPARE, 4096, 1, 0, 0)
    four = lib.gptq_workspace_bytes(b.GPTQ_CALL_PREPARE, 4096, 4, 0, 0)
    assert four > 3 * one and one == lib.gptq_workspace_bytes(b.GPTQ_CALL_PREPARE, 4096, 0, 0, 0)
    assert lib.gptq_prepare_groups(FAKE, 4096, 4, 4096 * 4096, 0.01, FAKE, None, None, ws, four - 256,
                                   None) == b.GPTQ_ERR_WORKSPACE


def test_quantize_validation(lib):
    ws = ctypes.c_void_p(0x100000)
    big = 1 << 30

    def call(**kw):
        a = dict(W=FAKE, dt=1, K=64, N=64, wrs=64, wcs=1, U=FAKE, dead=None, P1=None, bits=4, bsz=128, flags=0,
                 codes=FAKE, crs=64, ccs=1, scales=FAKE, ws=ws, wsb=big)
        a.update(kw)
        return lib.gptq_quantize_layer(a["W"], a["dt"], a["K"], a["N"], a["wrs"], a["wcs"], a["U"], a["dead"],
                                       a["P1"], a["bits"], a["bsz"], a["flags"], a["codes"], a["crs"], a["ccs"],
                                       a["scales"], None, None, None, a.get("perm"), a.get("G", 0), None, a["ws"],
                                       a["wsb"], None)

    assert call(bits=1) == b.GPTQ_ERR_ARG
    assert call(bits=9) == b.GPTQ_ERR_ARG
    assert call(bits=7) == b.GPTQ_ERR_ARG and call(bits=8) == b.GPTQ_ERR_ARG   # beyond the fp32 drift bound
    assert call(bsz=64) == b.GPTQ_ERR_ARG
    assert call(W=None) == b.GPTQ_ERR_ARG
    assert call(dt=7) == b.GPTQ_ERR_ARG
    assert call(K=0) == b.GPTQ_ERR_ARG
    assert call(flags=8) == b.GPTQ_ERR_ARG
    assert call(wcs=0) == b.GPTQ_ERR_ARG
    assert call(wsb=100) == b.GPTQ_ERR_WORKSPACE
    # the CAE term keeps a copy of the original weights in the workspace
    plain = lib.gptq_workspace_bytes(b.GPTQ_CALL_QUANTIZE_LAYER, 64, 64, 0, 0)
    cae = lib.gptq_workspace_bytes(b.GPTQ_CALL_QUANTIZE_LAYER, 64, 64, 0, b.GPTQ_FLAG_CAE)
    assert cae >= plain + 64 * 128 * 4
    assert call(flags=b.GPTQ_FLAG_CAE, wsb=plain) == b.GPTQ_ERR_WORKSPACE
    # group sizes and the flags that go with them
    assert call(G=48) == b.GPTQ_ERR_ARG and call(G=256) == b.GPTQ_ERR_ARG
    assert call(flags=b.GPTQ_FLAG_STATIC_GROUPS) == b.GPTQ_ERR_ARG              # static groups need a size
    assert call(flags=b.GPTQ_FLAG_MSE, G=64) == b.GPTQ_ERR_ARG                  # MSE only on scales from W
    assert call(flags=b.GPTQ_FLAG_SCALES_GIVEN, G=64) == b.GPTQ_ERR_ARG
    assert call(flags=b.GPTQ_FLAG_SCALES_GIVEN | b.GPTQ_FLAG_MSE) == b.GPTQ_ERR_ARG
    assert call(flags=32) == b.GPTQ_ERR_ARG


def test_quantize_groups_validation(lib):
    ws = ctypes.c_void_p(0x100000)
    big = 1 << 30

    def call(**kw):
        a = dict(K=64, N=64, groups=2, u_stride=64 * 64)
        a.update(kw)
        return lib.gptq_quantize_layer_groups(FAKE, 1, a["K"], a["N"], a["N"], 1, a["groups"], FAKE, a["u_stride"],
                                              None, None, 4, 128, 0, FAKE, a["N"], 1, FAKE, None, None, None, None, 0,
                                              None, ws, big, None)

    assert call(groups=0) == b.GPTQ_ERR_ARG
    assert call(groups=65536) == b.GPTQ_ERR_ARG
    assert call(groups=3) == b.GPTQ_ERR_ARG                 # 64 channels do not split into 3 equal groups
    assert call(N=96, groups=4) == b.GPTQ_ERR_ARG           # 24 channels per group: not a multiple of 16
    assert call(u_stride=64 * 64 - 1) == b.GPTQ_ERR_ARG
    assert call(K=0) == b.GPTQ_ERR_ARG
    assert lib.gptq_quantize_layer_groups(FAKE, 1, 64, 64, 64, 1, 2, FAKE, 4096, None, None, 4, 128, 0, FAKE, 64, 1,
                                          FAKE, None, None, None, None, 0, None, ws, 100, None) == b.GPTQ_ERR_WORKSPACE


def test_asym_validation(lib):
    ws = ctypes.c_void_p(0x100000)
    assert lib.gptq_asym_correction(None, FAKE, FAKE, 8, ws, 1 << 20, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_asym_correction(FAKE, FAKE, FAKE, 0, ws, 1 << 20, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_asym_correction(FAKE, FAKE, FAKE, 64, ws, 100, None) == b.GPTQ_ERR_WORKSPACE


def test_binding_refuses_missing_library(tmp_path):
    with pytest.raises(RuntimeError):
        b.load(str(tmp_path / "missing.so"))


def test_pack_validation(lib):
    assert lib.gptq_packed_words(32, 3) == 3 and lib.gptq_packed_words(33, 3) == 4 and lib.gptq_packed_words(5, 2) == 1
    assert lib.gptq_packed_words(8, 0) < 0 and lib.gptq_packed_words(8, 9) < 0
    assert lib.gptq_pack_codes(FAKE, 8, 1, 16, 8, 0, FAKE, 8, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_pack_codes(FAKE, 8, 1, 16, 8, 9, FAKE, 8, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_pack_codes(None, 8, 1, 16, 8, 3, FAKE, 8, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_pack_codes(FAKE, 8, 1, 16, 8, 3, FAKE, 4, None) == b.GPTQ_ERR_ARG      # ldp < N
    assert lib.gptq_pack_codes(FAKE, 0, 1, 16, 8, 3, FAKE, 8, None) == b.GPTQ_ERR_ARG
    un = lib.gptq_unpack_codes
    assert un(None, 8, 16, 8, 3, None, FAKE, 8, 1, None, 0, 0, 0, None) == b.GPTQ_ERR_ARG
    assert un(FAKE, 8, 16, 8, 3, None, FAKE, 8, 1, FAKE, 0, 8, 1, None) == b.GPTQ_ERR_ARG  # W_hat without scales
    assert un(FAKE, 8, 16, 8, 3, FAKE, None, 0, 0, FAKE, 7, 8, 1, None) == b.GPTQ_ERR_ARG  # bad dtype
    assert un(FAKE, 8, 0, 8, 3, None, FAKE, 8, 1, None, 0, 0, 0, None) == b.GPTQ_ERR_ARG


def test_hadamard_validation(lib):
    h = lib.gptq_hadamard_rotate
    assert h(FAKE, 64, FAKE, 64, 0, 4, 48, None, None) == b.GPTQ_ERR_ARG          # K not a power of two
    assert h(FAKE, 16, FAKE, 16, 0, 4, 8, None, None) == b.GPTQ_ERR_ARG           # K < 16
    assert h(FAKE, 32768, FAKE, 32768, 0, 4, 32768, None, None) == b.GPTQ_ERR_ARG  # K > 16384
    assert h(FAKE, 32, FAKE, 64, 7, 4, 64, None, None) == b.GPTQ_ERR_ARG          # ld < K, bad dtype
    assert h(FAKE, 64, FAKE, 128, 0, 4, 64, None, None) == b.GPTQ_ERR_ARG         # in place with different ld
    assert h(None, 64, FAKE, 64, 0, 4, 64, None, None) == b.GPTQ_ERR_ARG
    assert h(FAKE, 64, FAKE, 64, 0, 0, 64, None, None) == b.GPTQ_OK                # no rows: nothing to do


def test_act_order_validation(lib):
    ws = ctypes.c_void_p(0x100000)
    need = lib.gptq_workspace_bytes(b.GPTQ_CALL_ACT_ORDER, 64, 0, 0, 0)
    assert need >= 64 * 64 * 4
    assert lib.gptq_act_order(None, None, 64, FAKE, ws, need, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_act_order(FAKE, None, 64, None, ws, need, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_act_order(FAKE, None, 0, FAKE, ws, need, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_act_order(FAKE, None, 64, FAKE, ws, need - 1, None) == b.GPTQ_ERR_WORKSPACE


def test_device_status_and_timer_host_paths(lib):
    """gptq_device_status refuses a NULL or misaligned workspace before any HIP call; the kernel timer turns on and
    off and reads zeros when nothing was launched (no device work is needed for either)."""
    assert lib.gptq_device_status(None, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_device_status(ctypes.c_void_p(0x100010), None) == b.GPTQ_ERR_ARG
    assert lib.gptq_timer_read(None, None) == b.GPTQ_ERR_ARG
    assert lib.gptq_timer_enable(1) == b.GPTQ_OK
    t = g.gptq_timer_read()
    assert set(t) == set(g.GPTQ_TIMER_CLASSES) and all(v == (0.0, 0) for v in t.values())
    assert lib.gptq_timer_enable(0) == b.GPTQ_OK


def _al(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("K", [1, 8, 255, 256, 257, 300, 520, 1000, 1024, 4096, 7936, 7937, 11264, 11265, 14336,
                               28672])
def test_gram_plans_fit_the_workspace(lib, K):
    """Host-side check of every Gram plan against the workspace gptq_workspace_bytes sizes (symmetric, row-weighted
    and cross term, ragged K and M, every split count the planner picks): the split partials the launches write
    (split, tile, wave) for the symmetric plan and, with X_float, the cross plan that reuses the same region; the
    staging of a transformed operand; the token ranges of the splits (inside [0, M), covering every token)."""
    for M in (0, 1, 31, 32, 33, 1000, 2500, 4096, 8200, 20000, 65536, 65537, 196608, 327680, 524288, 2097152):
        for cross, scaled in ((False, False), (False, True), (True, False)):
            flags = (1 if cross else 0) | (2 if scaled else 0)
            ws = g.gptq_workspace_bytes(g.GPTQ_CALL_ACCUMULATE_HESSIAN, K, 0, M, flags)
            plans = [g.gptq_gram_plan(K, M, False, cross or scaled)]
            if cross:
                plans.append(g.gptq_gram_plan(K, M, True, True))
            region = 0
            for c, pl in zip((False, True), plans):
                nb = -(-K // 256)
                assert pl["nb"] == nb
                assert pl["ntiles"] == (nb * nb if c else nb * (nb + 1) // 2)
                assert pl["tokens_per_split"] % 32 == 0 and pl["splits"] >= 1
                assert pl["splits"] * pl["tokens_per_split"] >= M, (K, M, c, pl)
                # highest float a workgroup writes: ((split * ntiles + tile) * 4 + wave) * 16384 + 16383
                top = ((pl["splits"] - 1) * pl["ntiles"] + pl["ntiles"] - 1) * 4 + 3
                assert (top + 1) * 16384 == pl["partial_floats"]
                region = max(region, pl["partial_floats"])
                for s in range(pl["splits"]):
                    t0 = s * pl["tokens_per_split"]
                    t1 = min(M, t0 + pl["tokens_per_split"])
                    assert t0 >= 0 and (t1 <= t0 or t1 <= M)
            staging = plans[0]["staging_elems"]
            if (cross or scaled) and K % 256 == 0 and M % 32 == 0:
                assert staging == M * K
            else:
                assert staging == 0
            need = 256 + _al(4 * region) + _al(2 * staging)
            assert ws >= need, (K, M, cross, scaled, ws, need)

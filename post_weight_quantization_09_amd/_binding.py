"""ctypes binding of libgptq_hip.so (the C ABI declared in include/gptq.h).

Argument marshalling only: every step of the path runs in the library's HIP kernels.  torch supplies
device memory (tensors, workspace) and the current HIP stream.  The functions carry the C names.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libgptq_hip.so")

GPTQ_OK, GPTQ_ERR_ARG, GPTQ_ERR_NONFINITE, GPTQ_ERR_NOT_PD, GPTQ_ERR_WORKSPACE, GPTQ_ERR_HIP = range(6)
GPTQ_DTYPE_F32, GPTQ_DTYPE_BF16 = 0, 1
GPTQ_CALL_ACCUMULATE_HESSIAN, GPTQ_CALL_PREPARE, GPTQ_CALL_ASYM_CORRECTION, GPTQ_CALL_QUANTIZE_LAYER, GPTQ_CALL_ACT_ORDER = range(5)
GPTQ_FLAG_SCALES_GIVEN = 1
GPTQ_FLAG_CAE = 4
GPTQ_FLAG_STATIC_GROUPS = 8
GPTQ_FLAG_MSE = 16

_i64, _f32, _u32, _ptr, _size = ctypes.c_int64, ctypes.c_float, ctypes.c_uint, ctypes.c_void_p, ctypes.c_size_t

_SIGNATURES = {
    "gptq_version": (ctypes.c_char_p, []),
    "gptq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gptq_workspace_bytes": (_size, [ctypes.c_int, _i64, _i64, _i64, _u32]),
    "gptq_accumulate_hessian": (ctypes.c_int, [_ptr, _i64, _ptr, ctypes.c_int, _i64, _i64, _ptr, _ptr, _i64, _ptr,
                                               _ptr, _size, _ptr]),
    "gptq_prepare": (ctypes.c_int, [_ptr, _i64, _f32, _ptr, ctypes.POINTER(_f32), ctypes.POINTER(_i64), _ptr,
                                    _size, _ptr]),
    "gptq_prepare_groups": (ctypes.c_int, [_ptr, _i64, _i64, _i64, _f32, _ptr, ctypes.POINTER(_f32),
                                           ctypes.POINTER(_i64), _ptr, _size, _ptr]),
    "gptq_asym_correction": (ctypes.c_int, [_ptr, _ptr, _ptr, _i64, _ptr, _size, _ptr]),
    "gptq_quantize_layer": (ctypes.c_int, [_ptr, ctypes.c_int, _i64, _i64, _i64, _i64, _ptr, _ptr, _ptr,
                                           ctypes.c_int, ctypes.c_int, _u32, _ptr, _i64, _i64, _ptr, _ptr, _ptr,
                                           _ptr, _ptr, _i64, _ptr, _ptr, _size, _ptr]),
    "gptq_quantize_layer_groups": (ctypes.c_int, [_ptr, ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _ptr, _i64, _ptr,
                                                  _ptr, ctypes.c_int, ctypes.c_int, _u32, _ptr, _i64, _i64, _ptr,
                                                  _ptr, _ptr, _ptr, _ptr, _i64, _ptr, _ptr, _size, _ptr]),
    "gptq_act_order": (ctypes.c_int, [_ptr, _ptr, _i64, _ptr, _ptr, _size, _ptr]),
    "gptq_packed_words": (_i64, [_i64, ctypes.c_int]),
    "gptq_hadamard_rotate": (ctypes.c_int, [_ptr, _i64, _ptr, _i64, ctypes.c_int, _i64, _i64, _ptr, _ptr]),
    "gptq_pack_codes": (ctypes.c_int, [_ptr, _i64, _i64, _i64, _i64, ctypes.c_int, _ptr, _i64, _ptr]),
    "gptq_unpack_codes": (ctypes.c_int, [_ptr, _i64, _i64, _i64, ctypes.c_int, _ptr, _ptr, _i64, _i64, _ptr,
                                         ctypes.c_int, _i64, _i64, _ptr]),
    "gptq_device_status": (ctypes.c_int, [_ptr, _ptr]),
    "gptq_quantize_layer_noalloc": (ctypes.c_int, [_ptr, ctypes.c_int, _i64, _i64, _i64, _i64, _ptr, _ptr, _ptr,
                                                   ctypes.c_int, ctypes.c_int, _u32, _ptr, _i64, _i64, _ptr, _ptr, _ptr,
                                                   _ptr, _ptr, _i64, _ptr, _ptr]),
    "gptq_gram_plan": (ctypes.c_int, [_i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.POINTER(_i64)]),
    "gptq_timer_enable": (ctypes.c_int, [ctypes.c_int]),
    "gptq_timer_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
}

GPTQ_TIMER_CLASSES = ("gram", "gram_reduce", "factor_diag", "factor_gemm", "loop", "trailing", "other")

_lib = None


class GptqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Loads the in-tree library; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m post_weight_quantization_09_amd.build` "
                           "(or __graft_entry__.build()); there is no CPU fallback")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().gptq_status_string(int(status)).decode()


def version() -> str:
    return load().gptq_version().decode()


def gptq_workspace_bytes(call: int, K: int, N: int = 0, M: int = 0, flags: int = 0) -> int:
    return int(load().gptq_workspace_bytes(int(call), int(K), int(N), int(M), int(flags)))


def _check(status: int, where: str):
    if status != GPTQ_OK:
        raise GptqError(status, where)


def _dptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device, stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(call, K, N, M, flags, device, workspace):
    need = gptq_workspace_bytes(call, K, N, M, flags)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace, ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def _contig(t: Optional[torch.Tensor], name: str, dtype=None):
    """Matrices and vectors cross the C ABI as plain row-major pointers: refuse other layouts."""
    if t is None:
        return
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")


def _square(t: torch.Tensor, name: str, K: Optional[int] = None):
    if t.dim() != 2 or t.shape[0] != t.shape[1] or (K is not None and t.shape[0] != K):
        raise ValueError(f"{name} must be a square K x K matrix")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GPTQ_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return GPTQ_DTYPE_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def gptq_device_status(workspace: torch.Tensor, stream=None, check: bool = False) -> int:
    """Synchronises the stream and returns the status latched in `workspace` by the latest prepare / quantize call
    that used it (GPTQ_OK, GPTQ_ERR_NONFINITE or GPTQ_ERR_NOT_PD); check=True raises GptqError instead of
    returning an error status."""
    st = load().gptq_device_status(_dptr(workspace), _stream(workspace.device, stream))
    if check:
        _check(st, "gptq_device_status")
    return int(st)


def gptq_gram_plan(K: int, M: int, cross: bool = False, transformed: bool = False) -> dict:
    """How gptq_accumulate_hessian splits K features x M tokens (host-side query)."""
    out = (_i64 * 6)()
    _check(load().gptq_gram_plan(int(K), int(M), int(cross), int(transformed), out), "gptq_gram_plan")
    keys = ("nb", "ntiles", "splits", "tokens_per_split", "partial_floats", "staging_elems")
    return {k: int(out[i]) for i, k in enumerate(keys)}


def gptq_timer_enable(on: bool = True) -> None:
    """Turns the library's per-class kernel timer on or off (drops unread records)."""
    _check(load().gptq_timer_enable(1 if on else 0), "gptq_timer_enable")


def gptq_timer_read() -> dict:
    """{class: (ms, launches)} for the launches recorded since the last enable or read."""
    n = len(GPTQ_TIMER_CLASSES)
    ms = (ctypes.c_double * n)()
    cnt = (_i64 * n)()
    _check(load().gptq_timer_read(ms, cnt), "gptq_timer_read")
    return {c: (float(ms[i]), int(cnt[i])) for i, c in enumerate(GPTQ_TIMER_CLASSES)}


def gptq_accumulate_hessian(H: torch.Tensor, X: torch.Tensor, row_scale: Optional[torch.Tensor] = None,
                            X_float: Optional[torch.Tensor] = None, A: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """H += 2 Xs^T Xs (and A += 2 (X_float - X)^T X).  X: M x K with unit column stride."""
    K = H.shape[0]
    M = X.shape[0]
    _square(H, "H")
    _contig(H, "H", torch.float32)
    _contig(A, "A", torch.float32)
    _contig(row_scale, "row_scale", torch.float32)
    if X.dim() != 2 or X.shape[1] != K or X.stride(1) != 1:
        raise ValueError("X must be M x K with contiguous rows")
    if X_float is not None and (X_float.shape != X.shape or X_float.stride(1) != 1):
        raise ValueError("X_float must match X")
    flags = (1 if X_float is not None else 0) | (2 if row_scale is not None else 0)
    workspace, wp, wb = _workspace(GPTQ_CALL_ACCUMULATE_HESSIAN, K, 0, M, flags, H.device, workspace)
    st = load().gptq_accumulate_hessian(
        _dptr(H), K, _dptr(X), _dtype_code(X), M, X.stride(0) if M > 0 else K, _dptr(row_scale), _dptr(X_float),
        X_float.stride(0) if X_float is not None and M > 0 else K, _dptr(A), wp, wb, _stream(H.device, stream))
    _check(st, "gptq_accumulate_hessian")


def gptq_prepare(H: torch.Tensor, percdamp: float, dead: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None, sync: bool = True):
    """In place H -> U.  Returns (dead uint8[K], damp, n_dead).  sync=False passes no host outputs: the call then
    returns after enqueueing with damp and n_dead None, and device errors are read with gptq_device_status."""
    K = H.shape[0]
    _square(H, "H")
    _contig(H, "H", torch.float32)
    _contig(dead, "dead", torch.uint8)
    if dead is None:
        dead = torch.empty(K, dtype=torch.uint8, device=H.device)
    workspace, wp, wb = _workspace(GPTQ_CALL_PREPARE, K, 0, 0, 0, H.device, workspace)
    damp = _f32(0.0)
    n_dead = _i64(0)
    st = load().gptq_prepare(_dptr(H), K, float(percdamp), _dptr(dead), ctypes.byref(damp) if sync else None,
                             ctypes.byref(n_dead) if sync else None, wp, wb, _stream(H.device, stream))
    _check(st, "gptq_prepare")
    if not sync:
        return dead, None, None
    return dead, float(damp.value), int(n_dead.value)


def gptq_prepare_groups(H: torch.Tensor, percdamp: float, dead: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None, sync: bool = True):
    """In place H[g] -> U[g] for every group g of H (groups x K x K, each K x K matrix contiguous).
    Returns (dead uint8[groups, K], damps list, n_dead list); sync=False as for gptq_prepare (lists None)."""
    if H.dim() != 3 or H.shape[1] != H.shape[2]:
        raise ValueError("H must be groups x K x K")
    Gn, K = H.shape[0], H.shape[1]
    if H.dtype != torch.float32 or H.stride(2) != 1 or H.stride(1) != K or H.stride(0) < K * K:
        raise ValueError("H must be float32 with contiguous K x K matrices")
    if dead is None:
        dead = torch.empty(Gn, K, dtype=torch.uint8, device=H.device)
    _contig(dead, "dead", torch.uint8)
    if dead.numel() != Gn * K:
        raise ValueError("dead must hold groups x K entries")
    workspace, wp, wb = _workspace(GPTQ_CALL_PREPARE, K, Gn, 0, 0, H.device, workspace)
    damps = (_f32 * Gn)()
    n_dead = (_i64 * Gn)()
    st = load().gptq_prepare_groups(_dptr(H), K, Gn, H.stride(0), float(percdamp), _dptr(dead),
                                    damps if sync else None, n_dead if sync else None, wp, wb,
                                    _stream(H.device, stream))
    _check(st, "gptq_prepare_groups")
    if not sync:
        return dead, None, None
    return dead, [float(x) for x in damps], [int(x) for x in n_dead]


def gptq_asym_correction(U: torch.Tensor, A: torch.Tensor, P1: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    K = U.shape[0]
    for t, nm in ((U, "U"), (A, "A"), (P1, "P1")):
        if t is not None:
            _square(t, nm, K)
    _contig(U, "U", torch.float32)
    _contig(A, "A", torch.float32)
    _contig(P1, "P1", torch.float32)
    if P1 is None:
        P1 = torch.empty(K, K, dtype=torch.float32, device=U.device)
    workspace, wp, wb = _workspace(GPTQ_CALL_ASYM_CORRECTION, K, 0, 0, 0, U.device, workspace)
    st = load().gptq_asym_correction(_dptr(U), _dptr(A), _dptr(P1), K, wp, wb, _stream(U.device, stream))
    _check(st, "gptq_asym_correction")
    return P1


def gptq_quantize_layer(W: torch.Tensor, U: torch.Tensor, bits: int, dead: Optional[torch.Tensor] = None,
                        P1: Optional[torch.Tensor] = None, blocksize: int = 128,
                        scales: Optional[torch.Tensor] = None, codes: Optional[torch.Tensor] = None,
                        W_hat: Optional[torch.Tensor] = None, losses: Optional[torch.Tensor] = None,
                        pre_round: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        stream=None, cae: bool = False, perm: Optional[torch.Tensor] = None, groupsize: int = 0,
                        static_groups: bool = False, mse: bool = False, g_idx: Optional[torch.Tensor] = None,
                        check: bool = True) -> dict:
    """Quantises W (K x N view, any strides) with U; given `scales` are used as the grid (fixed-grid mode);
    cae=True adds the compensation-aware error term (GPTQ_FLAG_CAE); perm (from gptq_act_order) runs the loop in
    act-order; groupsize > 0 gives group-wise scales (ceil(K/groupsize) x N), re-estimated during the loop or
    static_groups; mse clips the scales taken from W before the loop.
    The C call is stream-ordered; check=True then reads the latched device status (gptq_device_status, which
    synchronises) and raises on an error, check=False leaves that to the caller.

    Returns dict(codes uint8 K x N, scales fp32[N], W_hat, losses, pre_round) with the tensors written.
    """
    K = W.shape[0]
    _square(U, "U", K)
    if P1 is not None:
        _square(P1, "P1", K)
    _contig(U, "U", torch.float32)
    _contig(P1, "P1", torch.float32)
    _contig(dead, "dead", torch.uint8)
    _contig(perm, "perm", torch.int32)
    _contig(g_idx, "g_idx", torch.int32)
    return _quantize(W, 1, U, 0, bits, dead, P1, blocksize, scales, codes, W_hat, losses, pre_round, workspace,
                     stream, cae, perm, groupsize, static_groups, mse, g_idx, check)


def gptq_quantize_layer_groups(W: torch.Tensor, U: torch.Tensor, bits: int, dead: Optional[torch.Tensor] = None,
                               P1: Optional[torch.Tensor] = None, blocksize: int = 128,
                               scales: Optional[torch.Tensor] = None, codes: Optional[torch.Tensor] = None,
                               W_hat: Optional[torch.Tensor] = None, losses: Optional[torch.Tensor] = None,
                               pre_round: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                               stream=None, cae: bool = False, perm: Optional[torch.Tensor] = None,
                               groupsize: int = 0, static_groups: bool = False, mse: bool = False,
                               g_idx: Optional[torch.Tensor] = None, check: bool = True) -> dict:
    """gptq_quantize_layer for output-channel groups: U (and P1) are groups x K x K (each K x K contiguous, the same
    group stride), dead, perm and g_idx groups x K; the N channels of W split into `groups` equal contiguous
    groups, group g quantised against U[g].  Same outputs as gptq_quantize_layer."""
    if U.dim() != 3 or U.shape[1] != U.shape[2]:
        raise ValueError("U must be groups x K x K")
    Gn, K = U.shape[0], U.shape[1]
    if W.shape[0] != K:
        raise ValueError("W must be K x N")
    for t, nm in ((U, "U"), (P1, "P1")):
        if t is not None and (t.shape != U.shape or t.dtype != torch.float32 or t.stride(2) != 1 or t.stride(1) != K
                              or t.stride(0) != U.stride(0)):
            raise ValueError(f"{nm} must be float32 groups x K x K with contiguous matrices and U's group stride")
    for t, nm, dt in ((dead, "dead", torch.uint8), (perm, "perm", torch.int32), (g_idx, "g_idx", torch.int32)):
        if t is not None and (t.dtype != dt or not t.is_contiguous() or t.numel() != Gn * K):
            raise ValueError(f"{nm} must be a contiguous {dt} tensor of groups x K entries")
    return _quantize(W, Gn, U, U.stride(0), bits, dead, P1, blocksize, scales, codes, W_hat, losses, pre_round,
                     workspace, stream, cae, perm, groupsize, static_groups, mse, g_idx, check)


def _quantize(W, groups, U, u_stride, bits, dead, P1, blocksize, scales, codes, W_hat, losses, pre_round, workspace,
              stream, cae, perm, groupsize, static_groups, mse, g_idx, check) -> dict:
    K, N = W.shape
    dev = W.device
    _contig(scales, "scales", torch.float32)
    _contig(losses, "losses", torch.float32)
    flags = 0
    ng = (K + groupsize - 1) // groupsize if groupsize > 0 else 0
    if scales is None:
        scales = torch.empty((ng, N) if ng else (N,), dtype=torch.float32, device=dev)
    else:
        flags |= GPTQ_FLAG_SCALES_GIVEN
    if cae:
        flags |= GPTQ_FLAG_CAE
    if static_groups:
        flags |= GPTQ_FLAG_STATIC_GROUPS
    if mse:
        flags |= GPTQ_FLAG_MSE
    if codes is None:
        codes = torch.empty(K, N, dtype=torch.uint8, device=dev)
    if W_hat is not None and (W_hat.shape != W.shape or W_hat.stride() != W.stride() or W_hat.dtype != W.dtype):
        raise ValueError("W_hat must have W's shape, strides and dtype")
    if pre_round is not None and (pre_round.shape != (K, N) or not pre_round.is_contiguous()):
        raise ValueError("pre_round must be a contiguous K x N fp32 tensor")
    ws_flags = flags | (2 if P1 is not None else 0)
    workspace, wp, wb = _workspace(GPTQ_CALL_QUANTIZE_LAYER, K, N, groups, ws_flags, dev, workspace)
    common = (int(bits), int(blocksize), flags, _dptr(codes), codes.stride(0), codes.stride(1), _dptr(scales),
              _dptr(W_hat), _dptr(losses), _dptr(pre_round), _dptr(perm), int(groupsize), _dptr(g_idx), wp, wb,
              _stream(dev, stream))
    if groups == 1:
        st = load().gptq_quantize_layer(_dptr(W), _dtype_code(W), K, N, W.stride(0), W.stride(1), _dptr(U),
                                        _dptr(dead), _dptr(P1), *common)
        _check(st, "gptq_quantize_layer")
    else:
        st = load().gptq_quantize_layer_groups(_dptr(W), _dtype_code(W), K, N, W.stride(0), W.stride(1), int(groups),
                                               _dptr(U), int(u_stride), _dptr(dead), _dptr(P1), *common)
        _check(st, "gptq_quantize_layer_groups")
    if check:
        _check(load().gptq_device_status(wp, _stream(dev, stream)),
               "gptq_quantize_layer" if groups == 1 else "gptq_quantize_layer_groups")
    return {"codes": codes, "scales": scales, "W_hat": W_hat, "losses": losses, "pre_round": pre_round,
            "g_idx": g_idx}


def gptq_packed_words(K: int, bits: int) -> int:
    return int(load().gptq_packed_words(int(K), int(bits)))


def gptq_pack_codes(codes: torch.Tensor, bits: int, packed: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """codes: K x N uint8 view (any strides) -> packed words, ceil(K*bits/32) x N, held as int32 (bit patterns of
    the uint32 words)."""
    if codes.dtype != torch.uint8 or codes.dim() != 2:
        raise ValueError("codes must be a 2-D uint8 tensor")
    K, N = codes.shape
    nw = gptq_packed_words(K, bits)
    if packed is None:
        packed = torch.empty(nw, N, dtype=torch.int32, device=codes.device)
    if packed.shape != (nw, N) or packed.dtype != torch.int32 or packed.stride(1) != 1:
        raise ValueError(f"packed must be int32 of shape ({nw}, {N}) with unit column stride")
    st = load().gptq_pack_codes(_dptr(codes), codes.stride(0), codes.stride(1), K, N, int(bits), _dptr(packed),
                                packed.stride(0), _stream(codes.device, stream))
    _check(st, "gptq_pack_codes")
    return packed


def gptq_unpack_codes(packed: torch.Tensor, K: int, bits: int, scales: Optional[torch.Tensor] = None,
                      codes: Optional[torch.Tensor] = None, W_hat: Optional[torch.Tensor] = None,
                      stream=None) -> dict:
    """Inverse of gptq_pack_codes; with `scales` (and W_hat, or a new fp32 K x N) also s (c - z)."""
    if packed.dtype != torch.int32 or packed.dim() != 2 or packed.stride(1) != 1:
        raise ValueError("packed must be a 2-D int32 tensor with unit column stride")
    N = packed.shape[1]
    dev = packed.device
    if codes is None:
        codes = torch.empty(K, N, dtype=torch.uint8, device=dev)
    if scales is not None:
        _contig(scales, "scales", torch.float32)
        if W_hat is None:
            W_hat = torch.empty(K, N, dtype=torch.float32, device=dev)
    if W_hat is not None and scales is None:
        raise ValueError("W_hat needs scales")
    st = load().gptq_unpack_codes(_dptr(packed), packed.stride(0), K, N, int(bits), _dptr(scales), _dptr(codes),
                                  codes.stride(0), codes.stride(1), _dptr(W_hat),
                                  _dtype_code(W_hat) if W_hat is not None else 0,
                                  W_hat.stride(0) if W_hat is not None else 0,
                                  W_hat.stride(1) if W_hat is not None else 0, _stream(dev, stream))
    _check(st, "gptq_unpack_codes")
    return {"codes": codes, "W_hat": W_hat}


def gptq_hadamard_rotate(x: torch.Tensor, signs: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """Rows of x (R x K, unit column stride, fp32 or bf16) -> (row * signs) H_K / sqrt(K); out=x rotates in place."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    R, K = x.shape
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or out.stride(1) != 1:
        raise ValueError("out must match x")
    if signs is not None and (signs.dtype != torch.int8 or signs.numel() != K or not signs.is_contiguous()):
        raise ValueError("signs must be a contiguous int8 tensor of K entries")
    st = load().gptq_hadamard_rotate(_dptr(x), x.stride(0), _dptr(out), out.stride(0), _dtype_code(x), R, K,
                                     _dptr(signs), _stream(x.device, stream))
    _check(st, "gptq_hadamard_rotate")
    return out


def gptq_act_order(H: torch.Tensor, A: Optional[torch.Tensor] = None, perm: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Act-order: returns perm (int32[K]) and permutes H (and A) in place to H[perm][:, perm]."""
    K = H.shape[0]
    _square(H, "H", K)
    _contig(H, "H", torch.float32)
    if A is not None:
        _square(A, "A", K)
        _contig(A, "A", torch.float32)
    if perm is None:
        perm = torch.empty(K, dtype=torch.int32, device=H.device)
    _contig(perm, "perm", torch.int32)
    workspace, wp, wb = _workspace(GPTQ_CALL_ACT_ORDER, K, 0, 0, 0, H.device, workspace)
    st = load().gptq_act_order(_dptr(H), _dptr(A), K, _dptr(perm), wp, wb, _stream(H.device, stream))
    _check(st, "gptq_act_order")
    return perm

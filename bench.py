"""Layer-quantisation benchmark on one MI355X.

One step = the whole hot path for one K x N linear layer with its calibration activations already resident
in HBM:  H = 0;  H += 2 X^T X over all M tokens (gptq_accumulate_hessian);  dead/damp + U (gptq_prepare);
[GPTAQ: P1 (gptq_asym_correction)];  shared-order column loop with lazy trailing GEMMs (gptq_quantize_layer).
Output groups (G2PTQ-style workloads): one Gram per group, then the groups' factorisations and column loops
together (gptq_prepare_groups, gptq_quantize_layer_groups).

Prints one JSON line: layer time (ms, lower is better) plus the Gram's MFMA roofline fraction, the trailing
products' fp32 MFMA fraction and the column loop's HBM fraction, and the float64 oracle timed on a bounded sample
of the same workload on the host cores.  The default workload is the largest that fits one GPU: the 70B-shaped
down_proj layer (K = 28672, N = 8192, 524,288 calibration tokens).

    python bench.py [--gpus 1] [--steps 5] [--warmup 1] [--config c5_down_proj_70b] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import post_weight_quantization_09_amd as G  # noqa: E402
import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gram_flops(cfg) -> float:
    """Algorithmic work of one Gram launch: the upper triangle incl. diagonal, M multiply-adds each."""
    per = float(cfg.M) * cfg.K * (cfg.K + 1)
    if cfg.asym_noise > 0:
        per += 2.0 * cfg.M * cfg.K * cfg.K          # the cross term is a full K x K product
    return per


def trailing_flops(cfg) -> float:
    """Lazy-batch GEMMs of the column loop: N * K * (K - B) multiply-adds x2 (x2 again with the P1 term)."""
    n = cfg.N
    f = 0.0
    for b0 in range(0, cfg.K, cfg.blocksize):
        b1 = min(b0 + cfg.blocksize, cfg.K)
        f += 2.0 * n * (b1 - b0) * (cfg.K - b1)
    return f * (2 if cfg.asym_noise > 0 else 1)


def loop_bytes(cfg) -> float:
    """Algorithmic HBM bytes of the column loop (every block kernel of one layer): the working weights read and
    written once in fp32 (8 bytes per coordinate and channel), the codes written (1 byte); 4 more bytes per
    coordinate and channel for the pre-rounding values the asymmetric term keeps."""
    return (13.0 if cfg.asym_noise > 0 else 9.0) * cfg.K * cfg.N


STEP_CHAIN_NS = 20.0   # one coordinate step's dependent chain: a broadcast and about six dependent fp32 operations


def loop_rounds(cfg) -> int:
    """Rounds of the column loop's workgroups (16 channels each, one per CU at a time): every channel in flight at
    once when N / 16 <= 256."""
    return -(-(cfg.N // 16) // 256)


def chain_floor_ms(cfg) -> float:
    """Latency floor of the column loop: K dependent coordinate steps per channel, once per round of workgroups."""
    return loop_rounds(cfg) * cfg.K * STEP_CHAIN_NS * 1e-6


def factor_flops(cfg) -> float:
    """Cholesky factorisation plus triangular inverse: 2 K^3 / 3 per Hessian (x groups)."""
    return 2.0 * cfg.K ** 3 / 3.0 * cfg.groups


def source_hash(*names) -> str:
    """Hash of the code of the named sources (line comments and blank lines dropped, so that a comment edit
    does not disown the traffic measured on the same kernel)."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "post_weight_quantization_09_amd", "csrc", n)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary of this kernel on this workload, if it was
    taken on the current source (else None)."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("source_hash") != src_hash or d.get("workload") != workload:
        return None
    return d.get("bytes_per_launch")


class Layer:
    def __init__(self, cfg, dev):
        self.cfg, self.dev = cfg, dev
        t0 = time.time()
        self.W = workloads.make_weights(cfg, device=dev)
        self.X = torch.empty(cfg.M, cfg.K, dtype=cfg.torch_x_dtype, device=dev)
        self.Xf = torch.empty_like(self.X) if cfg.asym_noise > 0 else None
        workloads.ActivationSource(cfg, dev).fill(self.X, self.Xf)
        self.rho = workloads.make_group_row_weights(cfg, device=dev)
        torch.cuda.synchronize()
        log(f"generated {cfg.name}: X {tuple(self.X.shape)} {self.X.dtype} in {time.time() - t0:.1f}s")
        K, N, M = cfg.K, cfg.N, cfg.M
        # one Hessian per output-channel group (one for plain layers); self.H is the last group's
        if cfg.groups > 1 and cfg.asym_noise > 0:
            raise ValueError("asymmetric calibration with output groups is not a workload here")
        self.Hs = torch.empty(cfg.groups, K, K, dtype=torch.float32, device=dev)
        self.H = self.Hs[cfg.groups - 1]
        self.A = torch.empty(K, K, dtype=torch.float32, device=dev) if self.Xf is not None else None
        self.P1 = torch.empty(K, K, dtype=torch.float32, device=dev) if self.Xf is not None else None
        self.deads = torch.empty(cfg.groups, K, dtype=torch.uint8, device=dev)
        self.dead = self.deads[cfg.groups - 1]
        gs = N // cfg.groups
        self.gs = gs
        self.codes = torch.empty(K, N, dtype=torch.uint8, device=dev)
        self.scales = torch.empty(N, dtype=torch.float32, device=dev)
        self.losses = torch.empty(N, dtype=torch.float32, device=dev)
        flags = (1 if self.Xf is not None else 0) | (2 if self.rho is not None else 0)
        ws = max(G.gptq_workspace_bytes(G.GPTQ_CALL_ACCUMULATE_HESSIAN, K, 0, M, flags),
                 G.gptq_workspace_bytes(G.GPTQ_CALL_PREPARE, K, cfg.groups),
                 G.gptq_workspace_bytes(G.GPTQ_CALL_ASYM_CORRECTION, K),
                 G.gptq_workspace_bytes(G.GPTQ_CALL_QUANTIZE_LAYER, K, N, cfg.groups, 2 if self.Xf is not None else 0))
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev)
        self.ws_cae = torch.empty(G.gptq_workspace_bytes(G.GPTQ_CALL_QUANTIZE_LAYER, K, gs, 0,
                                                         G.GPTQ_FLAG_CAE | (2 if self.Xf is not None else 0)),
                                  dtype=torch.uint8, device=dev)
        self.ev = []

    def step(self, record: bool, sync_prepare: bool = False):
        """One pass of the hot path; with record=True returns HIP events (current stream) at the starts and ends of
        the three stages: every group's Gram, the factorisation(s), every group's column loop."""
        cfg = self.cfg
        evs = []

        def mark():
            if record:
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                evs.append(e)

        mark()
        for gi in range(cfg.groups):
            Hg = self.Hs[gi]
            Hg.zero_()
            if self.A is not None:
                self.A.zero_()
            rs = self.rho[gi].contiguous() if self.rho is not None else None
            G.gptq_accumulate_hessian(Hg, self.X, row_scale=rs, X_float=self.Xf, A=self.A, workspace=self.ws)
        mark()
        # stream-ordered unless sync_prepare (then damping and dead counts come back to the host, one
        # synchronisation after the factorisation); device errors are read from the latch after the timed steps
        if cfg.groups == 1:
            d, damp, nd = G.gptq_prepare(self.H, cfg.percdamp, dead=self.dead, workspace=self.ws, sync=sync_prepare)
            self.damps, self.n_deads = [damp], [nd]
        else:   # the groups' Hessians factorised together, every step one launch over all groups
            _, self.damps, self.n_deads = G.gptq_prepare_groups(self.Hs, cfg.percdamp, dead=self.deads,
                                                               workspace=self.ws, sync=sync_prepare)
        P1 = None
        if self.A is not None:
            P1 = G.gptq_asym_correction(self.H, self.A, self.P1, workspace=self.ws)
        mark()
        # stream-ordered: no host synchronisation; the latched status is read after the timed steps
        if cfg.groups == 1:
            G.gptq_quantize_layer(self.W, self.H, cfg.bits, dead=self.dead, P1=P1, blocksize=cfg.blocksize,
                                  scales=None, codes=self.codes, losses=None, workspace=self.ws, check=False)
        else:   # every group's column loop in the same launches
            G.gptq_quantize_layer_groups(self.W, self.Hs, cfg.bits, dead=self.deads, blocksize=cfg.blocksize,
                                         scales=None, codes=self.codes, losses=None, workspace=self.ws,
                                         check=False)
        mark()
        return evs


def cpu_baseline(layer: Layer) -> dict:
    """The float64 oracle on a bounded sample of the same workload (about 10-20 s of host time), projected to the
    full layer: the Gram on Ms tokens of all K features (scaled by M / Ms); prepare on the leading Ks x Ks block of
    that Hessian (scaled by (K / Ks)^3); the blocked loop on Ks coordinates x Ns channels with that factor (scaled
    by (K / Ks)^2 x gs / Ns).  Per output-channel group, times the groups."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count()
    cfg = layer.cfg
    cores = len(os.sched_getaffinity(0))
    Ms = min(cfg.M, max(1024, (16384 * 4096 * 4096) // (cfg.K * cfg.K) // 1024 * 1024))
    Ks = min(cfg.K, 4096)
    Xs = layer.X[:Ms].float().cpu().numpy()
    t0 = time.perf_counter()
    H = O.gram([Xs])
    if layer.Xf is not None:
        O.cross_gram(layer.Xf[:Ms].float().cpu().numpy(), Xs)
    t_gram = (time.perf_counter() - t0) * (cfg.M / Ms)
    Hk = H[:Ks, :Ks]
    del H
    t0 = time.perf_counter()
    prep = O.prepare(Hk, cfg.percdamp)
    t_prep = (time.perf_counter() - t0) * (cfg.K / Ks) ** 3
    Ns = min(layer.gs, 128)
    Wsub = layer.W[:Ks, :Ns].float().cpu().numpy()
    t0 = time.perf_counter()
    O.quantize_layer(Wsub, prep["U"], cfg.bits, dead=prep["dead"], blocksize=cfg.blocksize)
    t_loop = (time.perf_counter() - t0) * (cfg.K / Ks) ** 2 * (layer.gs / Ns)
    per_group = t_gram + t_prep + t_loop
    total_ms = 1e3 * per_group * cfg.groups
    return {"value": round(total_ms, 1), "unit": "ms", "cores": int(min(cores, threads or cores)), "kind": "oracle",
            "sample": f"float64 numpy/BLAS oracle on a bounded sample, projected: Gram on {Ms} of {cfg.M} tokens x "
                      f"{cfg.K} features (x{cfg.M / Ms:.0f}); prepare on the leading {Ks}x{Ks} block "
                      f"(x(K/{Ks})^3); blocked loop on {Ks} coordinates x {Ns} of {layer.gs} channels "
                      f"(x(K/{Ks})^2 x {layer.gs / Ns:.0f}); projected stage seconds gram={t_gram:.1f} "
                      f"prepare={t_prep:.1f} loop={t_loop:.1f} per group, x{cfg.groups} groups",
            "host_cores_visible": cores}


def kernel_breakdown(layer: Layer) -> dict:
    """One more step of the path with the library's kernel timer on (HIP events around every launch, on the
    stream the kernel runs on): GPU time per kernel class, and the rates of the classes the metric names."""
    cfg = layer.cfg
    G.gptq_timer_enable(True)
    try:
        layer.step(record=False)
        t = G.gptq_timer_read()
    finally:
        G.gptq_timer_enable(False)
    ms = {k: round(v[0], 3) for k, v in t.items()}
    launches = {k: v[1] for k, v in t.items()}
    tf = trailing_flops(cfg)
    lb = loop_bytes(cfg)
    ff = factor_flops(cfg)
    loop_ms, tr_ms = t["loop"][0], t["trailing"][0]
    steps = cfg.K   # dependent coordinate steps of every channel (the loop's latency chain)
    out = {
        "ms": ms, "launches": launches,
        "trailing_gemm": {"ms": round(tr_ms, 3), "flop": tf,
                          "TFLOP/s": round(tf / (tr_ms * 1e-3) / 1e12, 1) if tr_ms > 0 else None,
                          "peak": PEAK_FP32_MFMA_TFLOPS,
                          "frac": round(tf / (tr_ms * 1e-3) / 1e12 / PEAK_FP32_MFMA_TFLOPS, 4) if tr_ms > 0 else None,
                          "floor_ms": round(tf / (PEAK_FP32_MFMA_TFLOPS * 1e12) * 1e3, 3)},
        "column_loop": {"ms": round(loop_ms, 3), "bytes": lb,
                        "GB/s": round(lb / (loop_ms * 1e-3) / 1e9, 1) if loop_ms > 0 else None,
                        "peak": PEAK_HBM_GBS,
                        "frac": round(lb / (loop_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) if loop_ms > 0 else None,
                        "hbm_floor_ms": round(lb / (PEAK_HBM_GBS * 1e9) * 1e3, 3),
                        "chain_floor_ms": round(chain_floor_ms(cfg), 3),
                        "ns_per_step": round(loop_ms * 1e6 / steps, 1) if loop_ms > 0 else None,
                        "workgroup_rounds": loop_rounds(cfg),
                        "ns_per_step_per_round": round(loop_ms * 1e6 / steps / loop_rounds(cfg), 1)
                        if loop_ms > 0 else None},
        "factorisation": {"ms": round(t["factor_diag"][0] + t["factor_gemm"][0], 3), "flop": ff,
                          "TFLOP/s": round(ff / ((t["factor_diag"][0] + t["factor_gemm"][0]) * 1e-3) / 1e12, 1)
                          if t["factor_gemm"][0] > 0 else None},
    }
    return out


def _time_ms(fn, reps: int = 3) -> float:
    """Average HIP-event time of fn() on the current stream, after one untimed call."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def extras(layer: "Layer") -> dict:
    """The rows beyond the layer path, on the same resident data: the CAE term in the column loop, act-order with
    re-estimated groups, MSE-clipped scales, packing the layer's codes (and unpacking them with dequantisation),
    and the Hadamard rotation of the activations.
    HBM-bound ones report bytes moved / time against the 8 TB/s peak."""
    cfg, out = layer.cfg, {}
    gs = layer.gs
    sl = slice((cfg.groups - 1) * gs, cfg.groups * gs)          # H holds the last group's U after a step
    Wg = layer.W[:, sl]

    def quant(cae):
        return lambda: G.gptq_quantize_layer(Wg, layer.H, cfg.bits, dead=layer.dead, P1=layer.P1 if layer.A is not None
                                             else None, codes=layer.codes[:, sl], workspace=layer.ws_cae, cae=cae,
                                             check=False)
    q_plain = _time_ms(quant(False))
    q_cae = _time_ms(quant(True))
    out["cae_term"] = {"quantize_ms": round(q_cae, 3), "quantize_ms_without": round(q_plain, 3),
                       "channels": gs, "asymmetric": layer.A is not None}
    # act-order on a K x K matrix (here a copy of the factor), then the loop with its permutation and
    # re-estimated groups of 128; per-channel weight-MSE clipping
    Hc = layer.H.clone()
    ws_ao = torch.empty(G.gptq_workspace_bytes(G.GPTQ_CALL_ACT_ORDER, cfg.K), dtype=torch.uint8, device=layer.dev)
    perm = G.gptq_act_order(Hc, workspace=ws_ao)
    t_ao = _time_ms(lambda: G.gptq_act_order(Hc, perm=perm, workspace=ws_ao))
    q_grp = _time_ms(lambda: G.gptq_quantize_layer(Wg, layer.H, cfg.bits, dead=layer.dead, codes=layer.codes[:, sl],
                                                   workspace=layer.ws_cae, perm=perm, groupsize=128, check=False))
    q_mse = _time_ms(lambda: G.gptq_quantize_layer(Wg, layer.H, cfg.bits, dead=layer.dead, codes=layer.codes[:, sl],
                                                   workspace=layer.ws_cae, mse=True, check=False))
    out["act_order"] = {"ms": round(t_ao, 3), "K": cfg.K}
    out["quantize_act_order_groups128_ms"] = round(q_grp, 3)
    out["quantize_mse_clipped_ms"] = round(q_mse, 3)
    K, N, b = cfg.K, cfg.N, cfg.bits
    packed = G.gptq_pack_codes(layer.codes, b)
    t_pack = _time_ms(lambda: G.gptq_pack_codes(layer.codes, b, packed=packed))
    words = G.gptq_packed_words(K, b) * N * 4
    W_hat = torch.empty(K, N, dtype=torch.bfloat16, device=layer.dev)
    scales = torch.full((N,), 0.01, dtype=torch.float32, device=layer.dev)
    t_unpack = _time_ms(lambda: G.gptq_unpack_codes(packed, K, b, scales=scales, codes=layer.codes, W_hat=W_hat))
    for name, t, byt in (("pack_codes", t_pack, K * N + words), ("unpack_dequant_bf16", t_unpack, words + 3 * K * N)):
        out[name] = {"ms": round(t, 4), "GB/s": round(byt / (t * 1e-3) / 1e9, 1),
                     "frac_hbm": round(byt / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 3), "bytes": byt}
    if K & (K - 1) == 0 and 16 <= K <= 16384:
        d = torch.tensor(workloads.hadamard_signs(cfg).astype("int8"), device=layer.dev)
        t_rot = _time_ms(lambda: G.gptq_hadamard_rotate(layer.X, d, out=layer.X), reps=2)
        byt = 2 * layer.X.numel() * layer.X.element_size()
        out["hadamard_rotate_X"] = {"ms": round(t_rot, 3), "GB/s": round(byt / (t_rot * 1e-3) / 1e9, 1),
                                    "frac_hbm": round(byt / (t_rot * 1e-3) / 1e9 / PEAK_HBM_GBS, 3), "bytes": byt,
                                    "rows": layer.X.shape[0], "K": K, "dtype": str(layer.X.dtype)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="c5_down_proj_70b", choices=sorted(workloads.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the timings of the rows beyond the layer path")
    ap.add_argument("--only", choices=["gram", "copy", "hadamard"], default=None,
                    help="profiling aids: run only the Gram launch per step, only the in-place Hadamard rotation of "
                         "the activations per step, or a 1 GiB device copy (the reference for scaling HBM byte "
                         "counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer path is single-GPU here",
              file=sys.stderr)
        sys.exit(2)
    cfg = workloads.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    G.load()
    if args.only == "copy":
        a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(args.warmup + args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": a.numel() * 4, "copy_bytes_written": b.numel() * 4,
                          "launches": args.warmup + args.steps}), flush=True)
        return
    layer = Layer(cfg, dev)
    if args.only == "gram":
        for i in range(args.warmup + args.steps):
            layer.H.zero_()
            G.gptq_accumulate_hessian(layer.H, layer.X, workspace=layer.ws)
        torch.cuda.synchronize()
        log(f"gram-only: {args.warmup + args.steps} launches")
        return
    if args.only == "hadamard":
        d = torch.tensor(workloads.hadamard_signs(cfg).astype("int8"), device=dev)
        for i in range(args.warmup + args.steps):
            G.gptq_hadamard_rotate(layer.X, d, out=layer.X)
        torch.cuda.synchronize()
        log(f"hadamard-only: {args.warmup + args.steps} rotations of {tuple(layer.X.shape)}")
        return
    for i in range(args.warmup):
        layer.step(record=False)
        log(f"warmup step {i} done")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    stage = {"gram": 0.0, "prepare": 0.0, "quantize": 0.0}
    ev_all = []
    for i in range(args.steps):
        ev_all.append(layer.step(record=True))
        log(f"timed step {i} enqueued/done")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    status = G.gptq_device_status(layer.ws)   # the latched device status of the last step's calls
    if status != G.GPTQ_OK:
        raise G.GptqError(status, "bench step")
    for e in ev_all:
        stage["gram"] += e[0].elapsed_time(e[1])
        stage["prepare"] += e[1].elapsed_time(e[2])
        stage["quantize"] += e[2].elapsed_time(e[3])
    for k in stage:
        stage[k] /= args.steps
    ms = 1e3 * wall / args.steps
    gflop = gram_flops(cfg) * cfg.groups
    gram_launch_ms = stage["gram"] / cfg.groups
    achieved = gram_flops(cfg) / (gram_launch_ms * 1e-3) / 1e12
    src = source_hash("gram.hip")
    traffic = measured_traffic("gram_bf16", cfg.name, src)
    out = {
        "metric": "layer quantize time (ms) + Gram/trailing TFLOP/s vs MFMA peak, KxN layer",
        "value": round(ms, 3),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+f32",   # bf16 MFMA products with fp32 accumulation (Gram); fp32 factorisation and loop
        "data": "synthetic",
        "config": {"workload": cfg.name, "K": cfg.K, "N": cfg.N, "M": cfg.M, "x_dtype": cfg.x_dtype,
                   "w_dtype": cfg.w_dtype, "bits": cfg.bits, "blocksize": cfg.blocksize, "percdamp": cfg.percdamp,
                   "groups": cfg.groups, "hadamard": cfg.hadamard, "asymmetric": cfg.asym_noise > 0,
                   "dead_frac": cfg.dead_frac},
        "stages_ms": {k: round(v, 3) for k, v in stage.items()},
        "gram_tflops": round(gflop / (stage["gram"] * 1e-3) / 1e12, 1),
        "roofline": {"bound": "mfma", "kernel": "gram_bf16_lds_kernel + gram_reduce_kernel (one accumulate call)",
                     "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "algorithmic_flop_per_launch": gram_flops(cfg), "launch_ms": round(gram_launch_ms, 3)},
    }
    log("kernel classes: one more step with the kernel timer on ...")
    out["kernels"] = kernel_breakdown(layer)
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on a bounded sample ...")
        out["cpu_baseline"] = cpu_baseline(layer)
    if not args.no_extras:   # last: the rotation timing rotates the resident activations in place
        log("timing the CAE term, act-order, groups, MSE clipping, packing and the Hadamard rotation ...")
        out["extras"] = extras(layer)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

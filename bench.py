"""Benchmark: one cube block-sparse attention layer (forward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 720p]

A step is one pass of the whole layer on inputs already resident in HBM:
permute Q, K, V (cube means of Q and K pooled in the same pass) -> coarse
stage (block scores, top-k) -> fine block-sparse attention -> (linear
branch, hybrid workload) -> unpermute.  The default workload is the largest
one-GPU layer, 720P video (81 frames at 720x1280: latent 21x45x80, padded to
24x48x80, 1440 cubes, 40 heads, head_dim 128, sparsity 0.9 -> k = 144).
The others (wan1.3b, wan14b, hybrid, sta, tiny) are selected with --workload.

Prints one JSON line.  `value` is the effective throughput of the whole
layer: the flops of the computed 64x64 blocks (4 * 64 * 64 * D each, QK^T
plus PV) divided by the layer time.  `roofline` reports the fine-stage kernel
alone (the dominant kernel), timed with HIP events on the stream it runs on.
`cpu_baseline` times the fp64 oracle on a bounded sample of the same layer on
the host cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_FP8_TFLOPS = 5033.2  # dense fp8 MFMA: twice the bf16 rate
PEAK_HBM_GBS = 8000.0
METRIC = "ms/layer + effective TFLOPS (frac of bf16 MFMA peak), block-sparse attn fwd"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="720p")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    ap.add_argument("--k-raster", action="store_true",
                    help="let the fine stage gather K tiles from raster rows too (no K permute)")
    ap.add_argument("--unpacked", action="store_true",
                    help="the unpacked fine stage (one 64-key tile per selected cube, K token-major, V "
                         "cube-transposed) instead of the packed one (cubes with few valid keys share tiles); "
                         "with --fp8 the unpacked fp8 stage")
    ap.add_argument("--one-stream", action="store_true",
                    help="every launch on one stream (the V permute otherwise runs on a second stream beside the "
                         "coarse stage); for per-kernel traces whose durations no other kernel shares")
    ap.add_argument("--backward", action="store_true",
                    help="also time the backward of the fine stage (dQ, dK, dV) after the forward steps; "
                         "reported under 'backward', not in 'value'")
    ap.add_argument("--fused-linear", action="store_true",
                    help="hybrid layer: the fine stage and the linear branch in one fused pass "
                         "(vsa_sparse_attn_linear_fwd) instead of two calls with fp32 O_sparse in between")
    ap.add_argument("--linear-tiles", action="store_true",
                    help="hybrid layer: the linear branch as total minus selected blocks on K/V tiles "
                         "(vsa_linear_state + vsa_linear_apply after the fine stage's fp32 output) instead of "
                         "summed per-cube states applied in the fine stage's epilogue")
    ap.add_argument("--fp8", action="store_true",
                    help="low-precision layer: Q, K, V quantized to fp8 E4M3 in the step, fine stage on the "
                         "fp8 matrix cores (roofline against the fp8 peak)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes (3 times) and exit; "
                         "used to calibrate the FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def copy_calibration(nbytes: int) -> None:
    import torch

    src = torch.ones(nbytes // 2, dtype=torch.int16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": src.numel() * 2, "copies": 3}))


KERNEL_SOURCES = {
    "attn_fwd": ("attn_fwd.hip", "attn_core.h", "tile_pipeline.h", "device.h"),
    "attn_fwd_fp8": ("attn_fp8.hip", "tile_pipeline.h", "device.h"),
}


def kernel_source_hash(kernel: str = "attn_fwd") -> str:
    """sha256 (first 16 hex digits) of a fine-stage kernel's sources: the kernel and the headers it includes."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, "block_sparse_video_cube_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str = "attn_fwd"):
    """HBM bytes per fine-stage launch from committed rocprofv3 counters, if current."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sha256_16") != kernel_source_hash(kernel):
        return None  # the kernel changed since the counters were taken
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(wl, budget_s: float):
    """Time the fp64 oracle on whole heads of the layer and scale to the layer."""
    import oracle
    import workloads

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    valid = oracle.valid_rows(wl.grid)
    scale = wl.softmax_scale
    n_heads = wl.batch * wl.heads
    # Whole heads in order, each: permute + pool + score + top-k of all rows,
    # then its query cubes one by one, until the time budget is spent (the
    # last head may stop part-way; its remaining cubes are estimated from its
    # own per-cube time).
    head_s, cubes_total, t0 = [], 0, time.perf_counter()
    for bh in range(n_heads):
        b, h = divmod(bh, wl.heads)
        sub = {n: workloads.make_head(wl, n, b, h)[None, :, None, :] for n in ("q", "k", "v")}
        th = time.perf_counter()
        qc, kc, vc = (oracle.cube_permute(sub[n], wl.grid) for n in ("q", "k", "v"))
        if wl.pattern == "sta":
            idx = oracle.sta_index(wl.grid, wl.window)[None, None]
        else:
            idx = oracle.select_topk(qc, kc, valid, wl.topk)
        states = oracle.vsa_oracle._cube_states(kc[0, 0], vc[0, 0], valid) if wl.linear else None
        fixed = time.perf_counter() - th
        t1, done = time.perf_counter(), 0
        for i in range(wl.n_cubes):
            oracle.attention_cube(qc[0, 0, 64 * i:64 * i + 64], kc[0, 0], vc[0, 0], valid, idx[0, 0, i], scale)
            if wl.linear:
                oracle.linear_cube(qc[0, 0, 64 * i:64 * i + 64], states, idx[0, 0, i])
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        head_s.append(fixed + wl.n_cubes * (time.perf_counter() - t1) / done)
        cubes_total += done
        if time.perf_counter() - t0 > budget_s:
            break
    t_total = time.perf_counter() - t0
    layer_s = n_heads * float(np.mean(head_s))
    return {
        "value": wl.fine_flops / layer_s / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle on {len(head_s)} of {n_heads} heads of {wl.name} (each: permute+"
                   f"{'sliding-tile lists' if wl.pattern == 'sta' else 'pool+score+top-k'} of all "
                   f"{wl.n_cubes} rows, then its query cubes; {cubes_total} query cubes in all, "
                   f"{t_total:.1f} s), scaled to {n_heads} heads"),
        "ms_per_layer": layer_s * 1e3,
        "host_cpus": os.cpu_count(),
        "cpu_model": platform.processor() or platform.machine(),
    }


def mfma_probe(vsa, torch, blocks=2048, iters=2000):
    """Sustained bf16 matrix-core rate and shader clock (vsa_mfma_probe): a
    measured denominator beside the published peak."""
    vsa.mfma_probe(blocks, iters)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3
    e0.record()
    for _ in range(reps):
        _, clk = vsa.mfma_probe(blocks, iters)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tflops = blocks * 4 * iters * 8 * 32768 / (ms * 1e-3) / 1e12
    c = clk.cpu().numpy().astype(np.float64)
    ghz = float(np.median(c[:, 0] / (c[:, 1] / 100e6))) / 1e9
    return {"kernel": "v_mfma_f32_32x32x16_bf16, 8 independent chains per wavefront",
            "tflops": round(tflops, 1), "frac_of_published_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "shader_clock_ghz": round(ghz, 3), "ms": round(ms, 4)}


def hbm_probe(vsa, torch, nbytes=1 << 30, reps=10):
    """Rates of plain HBM streams (vsa_hbm_probe: copy, read, write over 1 GiB):
    a measured denominator beside the published 8 TB/s for the memory-bound
    steps (the permutes and pooling)."""
    a = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    out = {}
    for kind, moved in (("copy", 2), ("read", 1), ("write", 1)):
        def f():
            vsa.hbm_probe(kind, a if kind != "write" else None, b if kind != "read" else None)
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[f"{kind}_tbps"] = round(moved * nbytes / (ms * 1e-3) / 1e12, 3)
    del a, b
    return {"kernel": "hbm_stream (vsa_hbm_probe): 16384 x 256 threads, four 16-byte words per thread per round, "
                      "nontemporal stores", "bytes": nbytes, **out,
            "frac_of_published": {k[:-5]: round(v / (PEAK_HBM_GBS / 1e3), 4) for k, v in out.items()}}


def valid_fine_flops(wl, idx, torch):
    """Flops of the computed blocks over valid query and key tokens only
    (4 D n_valid(i) n_valid(j) per block), from the block lists."""
    (t, h, w), (tp, hp, wp) = wl.grid, wl.padded_grid
    nt = np.minimum(4, t - 4 * np.arange(tp // 4))
    ny = np.minimum(4, h - 4 * np.arange(hp // 4))
    nx = np.minimum(4, w - 4 * np.arange(wp // 4))
    nv = (nt[:, None, None] * ny[None, :, None] * nx[None, None, :]).reshape(-1)
    nvt = torch.from_numpy(nv.astype(np.float64)).to(idx.device)
    per_row = nvt[idx.long()].sum(-1) * nvt  # [B, H, Nc]
    return float(4 * wl.head_dim * per_row.sum().item())


def time_backward(vsa, wl, q, k, v, o, qc, kc, vt, idx, args, dev):
    """Backward of the fine stage on the layer's last forward state.

    One backward step: the layouts it reads (Q, K, V and dO cube-major,
    token-major), the forward's O and lse (one fine-stage call), then
    vsa_sparse_attn_bwd and the three unpermutes to raster gradients.
    Flops are counted as 2.5x the forward's (five 64x64xD products per block:
    the usual accounting; the kernels recompute S and dP in both passes).
    """
    import torch

    rng = np.random.default_rng(7)
    do = torch.from_numpy(rng.standard_normal(tuple(q.shape), dtype=np.float32)).to(dev).to(torch.bfloat16)
    B, H, D = wl.batch, wl.heads, wl.head_dim
    qc = vsa.cube_permute(q, wl.grid, out=qc)
    kc = vsa.cube_permute(k, wl.grid, out=kc)
    oc, _, lse = vsa.sparse_attn_fwd(qc, kc, vt, idx, wl.grid, wl.softmax_scale, want_lse=True)
    ws = torch.empty(max(16, vsa._lib.load().vsa_attn_bwd_workspace_bytes(
        vsa.make_geom(B, H, D, wl.grid), wl.topk)), dtype=torch.uint8, device=dev)

    def layouts():
        # The raster forward keeps no cube-major Q, K: the backward makes every layout it reads.
        vsa.cube_permute(q, wl.grid, out=qc)
        vsa.cube_permute(k, wl.grid, out=kc)
        return vsa.cube_permute(v, wl.grid), vsa.cube_permute(do, wl.grid)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        vc, doc = layouts()
        if ev is not None:
            ev[1].record()
        dq, dk, dv = vsa.sparse_attn_bwd(qc, kc, vc, oc, doc, lse, idx, wl.grid, wl.softmax_scale, workspace=ws)
        if ev is not None:
            ev[2].record()
        outs = [vsa.cube_unpermute(x, wl.grid) for x in (dq, dk, dv)]
        if ev is not None:
            ev[3].record()
        return outs

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for s_ in range(args.steps):
        outs = step(evs[s_])
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    kern = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    lay = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    unp = float(np.median([e[2].elapsed_time(e[3]) for e in evs]))
    finite = all(bool(torch.isfinite(x.float()).all()) for x in outs)
    flops = 2.5 * wl.fine_flops
    lin = None
    if wl.linear:
        # The linear branch's own gradients, from the forward's saved O_lin and 1/den
        # (as the autograd node runs it), and recomputing them.
        vc, doc = layouts()
        _, of, _ = vsa.sparse_attn_fwd(qc, kc, vt, idx, wl.grid, wl.softmax_scale, want_f32=True)
        _, saved = vsa.linear_branch(qc, kc, vt, idx, of, wl.grid, save=True)
        wsl = torch.empty(max(16, vsa._lib.load().vsa_linear_bwd_workspace_bytes(
            vsa.make_geom(B, H, D, wl.grid), wl.topk)), dtype=torch.uint8, device=dev)
        lin = {}
        for key, sv in (("ms", saved), ("ms_recomputing", None)):
            for _ in range(max(1, args.warmup)):
                vsa.linear_branch_bwd(qc, kc, vc, vt, idx, doc, wl.grid, workspace=wsl, saved=sv)
            torch.cuda.synchronize()
            l0, l1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            l0.record()
            for _ in range(args.steps):
                lo = vsa.linear_branch_bwd(qc, kc, vc, vt, idx, doc, wl.grid, workspace=wsl, saved=sv)
            l1.record()
            torch.cuda.synchronize()
            lin[key] = round(l0.elapsed_time(l1) / args.steps, 4)
            lin["finite"] = lin.get("finite", True) and all(bool(torch.isfinite(x.float()).all()) for x in lo)
    return {
        "ms_per_layer": round(ms, 4),
        "stage_ms": {"layouts": round(lay, 4), "bwd_kernels": round(kern, 4), "unpermute": round(unp, 4)},
        "bwd_kernels_tflops": round(flops / (kern * 1e-3) / 1e12, 2),
        "frac_of_bf16_peak": round(flops / (kern * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "flops": flops,
        "finite": finite,
        **({"linear_branch_bwd": lin} if lin is not None else {}),
    }


def main():
    args = parse()
    if args.copy_bytes:
        copy_calibration(args.copy_bytes)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): every step of the "
              "layer is independent per (batch, head), so several GPUs would each run this same "
              "kernel on their share of the heads.", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_video_cube_amd as vsa
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = workloads.workload(args.workload)
    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    inp = workloads.make_inputs(wl)
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    del inp
    g = vsa.make_geom(wl.batch, wl.heads, wl.head_dim, wl.grid)
    d = vsa.geom_dims(g)
    B, H, D = wl.batch, wl.heads, wl.head_dim
    bufs = vsa.LayerBuffers(B, H, D, wl.grid, wl.topk, linear=wl.linear, device=dev)
    qc, kc, vt, qbar, kbar, idx = bufs.qc, bufs.kc, bufs.vt, bufs.qbar, bufs.kbar, bufs.idx
    ws_sel = bufs.ws_sel
    o = torch.empty_like(q)

    # The layer's chain (vsa.layer_forward; the full-size GPU tests run the
    # same function): without the linear branch the fine stage reads Q and
    # writes the output in raster order, Q is only pooled, K is pooled and
    # permuted in one pass (contiguous 16 KB tiles stream faster than tiles
    # gathered from 64 raster rows; --k-raster gathers them instead), V is
    # permuted into the cube-transposed layout.  The hybrid layer permutes K
    # (the linear branch's state reads cube-major keys); its two calls read
    # raster Q and write the raster output (the fused pass keeps the
    # permute / unpermute pair).
    linear_mode = "tiles" if args.linear_tiles else "states"
    stages = vsa.layer_stages(wl.linear, args.fused_linear, linear_mode)
    if args.fp8:
        if wl.linear:
            print("--fp8 covers the fine stage without the linear branch", file=sys.stderr)
            sys.exit(2)
        # Q, K quantized per cube and V per channel in the step; the fp8 fine
        # stage writes the raster-order output itself.
        stages = ["quant", "select", "fine"]
        # On grids with partial cubes the packed fp8 stage (edge cubes share
        # tiles; K codes in compact rows, V codes in 16-key slots), as the bf16
        # layer does; full grids keep the unpacked one.
        fp8_packed = any(int(x) % 4 for x in wl.grid) and not args.unpacked
        fp8_bufs = (torch.empty((B, H, d.rows, D), dtype=torch.uint8, device=dev),
                    torch.empty((B, H, d.n_cubes), dtype=torch.float32, device=dev),
                    torch.empty((B, H, d.rows, D), dtype=torch.uint8, device=dev),
                    torch.empty((B, H, d.n_cubes), dtype=torch.float32, device=dev),
                    torch.empty((B, H, d.n_cubes, 4, D, 16) if fp8_packed else (B, H, d.n_cubes, D, 64),
                                dtype=torch.uint8, device=dev),
                    torch.empty((B, H, D), dtype=torch.float32, device=dev),
                    qbar if wl.pattern != "sta" else None, kbar if wl.pattern != "sta" else None)
        ws_q = torch.empty(vsa.quant_fp8_workspace_bytes(g), dtype=torch.uint8, device=dev)
        nplan = vsa.packed_workspace_bytes(g, wl.topk) if fp8_packed else 0
        ws_plan8 = torch.empty(nplan, dtype=torch.uint8, device=dev) if nplan else None

    def step_fp8(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()

        mark(0)
        # One pass over Q, K, V: codes, scales, the cube means of Q and K for the
        # coarse stage, V's channel maxima; a second pass for V's codes.
        q8, qs, k8, ks, v8t, vs, _, _ = vsa.quant_fp8(q, k, v, wl.grid, out=fp8_bufs, workspace=ws_q,
                                                      packed=fp8_packed)
        mark(1)
        if wl.pattern == "sta":
            vsa.sta_index(wl.grid, wl.window, B, H, head_dim=D, out=idx)
        else:
            vsa.select_topk_pooled(qbar, kbar, wl.grid, wl.topk, out=idx, workspace=ws_sel)
        mark(2)
        if fp8_packed:
            vsa.sparse_attn_fwd_fp8_packed(q8, qs, k8, ks, v8t, vs, idx, wl.grid, wl.softmax_scale, out=o,
                                           raster=True, workspace=ws_plan8)
        else:
            vsa.sparse_attn_fwd_fp8(q8, qs, k8, ks, v8t, vs, idx, wl.grid, wl.softmax_scale, out=o, raster=True)
        mark(3)

    def step(ev=None):
        if args.fp8:
            step_fp8(ev)
            return
        vsa.layer_forward(q, k, v, wl.grid, wl.topk, wl.softmax_scale, linear=wl.linear,
                          fused_linear=args.fused_linear, k_raster=args.k_raster,
                          window=wl.window if wl.pattern == "sta" else None, bufs=bufs, out=o,
                          mark=(lambda i: ev[i].record()) if ev is not None else None,
                          packed=not args.unpacked, overlap=not args.one_stream, linear_mode=linear_mode)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: exactly K steps, synchronised on both sides.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for s in range(args.steps):
        step(evs[s])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    per_stage = {name: [] for name in stages}
    for s in range(args.steps):
        for i, name in enumerate(stages):
            per_stage[name].append(evs[s][i].elapsed_time(evs[s][i + 1]))
    stage_ms = {name: float(np.median(vals)) for name, vals in per_stage.items()}
    fine_key = "fine+linear" if "fine+linear" in per_stage else "fine"
    fine_ms = float(np.mean(per_stage[fine_key]))
    if not torch.isfinite(o.float()).all():
        print("non-finite output", file=sys.stderr)
        sys.exit(1)

    flops = wl.fine_flops
    value = flops / (ms_step * 1e-3) / 1e12
    fine_tflops = flops / (fine_ms * 1e-3) / 1e12
    step_ms = [evs[s][0].elapsed_time(evs[s][len(stages)]) for s in range(args.steps)]
    vflops = valid_fine_flops(wl, idx, torch)
    probe = mfma_probe(vsa, torch)
    hbm = hbm_probe(vsa, torch)
    # Algorithmic bytes of one fine-stage launch: Q, K, V read once, O written
    # once (bf16; fp8 codes are one byte, plus their scales).
    alg_bytes = 4 * B * H * d.rows * D * 2
    peak, kname = PEAK_BF16_TFLOPS, "attn_fwd"
    traffic = measured_traffic(wl.name)
    if wl.linear and args.fused_linear:
        kname = "attn_lin_fwd (stage includes lin_state, lin_reduce)"
        traffic = None
    elif wl.linear and linear_mode == "states":
        kname = "attn_fwd with the linear branch's epilogue"
        traffic = None
    if args.fp8:
        alg_bytes = B * H * d.rows * D * (1 + 1 + 1 + 2) + 4 * B * H * (2 * d.n_cubes + D)
        peak, kname = PEAK_FP8_TFLOPS, "attn_fwd_fp8"
        traffic = measured_traffic(wl.name, "attn_fwd_fp8")
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 (fp32 softmax)" if args.fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "batch": B, "heads": H, "head_dim": D,
            "latent_grid": list(wl.grid), "padded_grid": list(wl.padded_grid),
            "tokens": wl.tokens, "n_cubes": wl.n_cubes, "topk": wl.topk,
            "sparsity": wl.sparsity, "linear_branch": wl.linear, "pattern": wl.pattern,
            **({"linear_branch_form": ("fused pass" if args.fused_linear else
                                       ("tiles: total minus selected blocks" if linear_mode == "tiles" else
                                        "summed per-cube states, applied in the fine stage's epilogue"))}
               if wl.linear else {}),
            "layout": (("cube-major q/k/o (permute, unpermute), cube-transposed v" if args.fused_linear else
                        "raster q/o; cube-major k, cube-transposed v") if wl.linear else ("raster q, k, v in; fp8 cube-major codes" +
                                                     ("; packed tiles: compact k, slot-layout v" if args.fp8 and
                                                      fp8_packed else "") + "; raster o")
                       if args.fp8 else ("raster q/k/o" if args.k_raster else
                                         "raster q/o" + ("" if args.unpacked else
                                                         "; packed tiles: compact k, slot-layout v"))),
            **({"precision": "fp8 e4m3: Q, K per cube, V per channel; P e4m3"} if args.fp8 else {}),
            **({"window_cubes": list(wl.window)} if wl.window else {}),
            "streams": 1 if (args.one_stream or args.fp8) else 2,
            "computed_blocks": wl.blocks, "fine_flops": flops,
        },
        "ms_per_layer": round(ms_step, 4),
        "step_ms_median_p10_p90": [round(float(np.percentile(step_ms, p)), 4) for p in (50, 10, 90)],
        "stage_ms_median": {kname: round(x, 4) for kname, x in stage_ms.items()},
        "fine_stage_tflops": round(fine_tflops, 2),
        "frac_of_bf16_peak_layer": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": {
            "kernel": kname,
            "bound": "mfma",
            "achieved": round(fine_tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(fine_tflops / peak, 4),
            "traffic": traffic,
            "algorithmic_bytes": alg_bytes,
            "avg_launch_ms": round(fine_ms, 4),
            **({} if args.fp8 else {"frac_of_measured_peak": round(fine_tflops / probe["tflops"], 4)}),
        },
        "valid_tokens_only": {
            "fine_flops": vflops,
            "value": round(vflops / (ms_step * 1e-3) / 1e12, 3),
            "fine_stage_tflops": round(vflops / (fine_ms * 1e-3) / 1e12, 2),
        },
        "mfma_probe": probe,
        "hbm_probe": hbm,
        "wall_s_timed": round(wall, 3),
        "device": torch.cuda.get_device_name(0),
    }
    if args.backward and not args.fp8:
        res["backward"] = time_backward(vsa, wl, q, k, v, o, qc, kc, vt, idx, args, dev)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()

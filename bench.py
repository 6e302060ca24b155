#!/usr/bin/env python3
"""Throughput of the block-sparse attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one full forward (``bsattn_forward``: every non-zero 64x64 tile of
the layout, the split of the dense global rows and their log-sum-exp merge)
over one batch of the workload, inputs already resident in HBM.  With
``--pass backward`` a step is one full backward (``bsattn_backward``: delta,
the dQ pass, the dK/dV pass and the sums of split rows and columns) on the
forward's outputs and a seeded upstream gradient; with ``--pass layer`` a
step is one ``bsattn_layer_forward`` (qkv projection, head split, attention,
head concatenation, output projection; no CPU baseline).  W untimed
steps, then exactly K timed steps bracketed by device synchronisation; three
copies of the inputs are rotated so that consecutive steps do not hit the
256 MB last-level cache with the previous step's tensors.

Prints ONE JSON line with the metric, ``roofline`` (the main attention
kernel timed by HIP events that its own dispatch records, on one step in
``--event-every`` of the timed region, priced against the bf16 dense MFMA
peak) and ``cpu_baseline`` (the fp64 oracle on a bounded sample of the same
workload, on the host cores).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "block-sparse attn fwd tokens/s and effective TFLOP/s (% bf16 MFMA peak), L=8192"
METRIC_BWD = "block-sparse attn bwd tokens/s and effective TFLOP/s (% bf16 MFMA peak), L=8192"
METRIC_LAYER = "block-sparse attn layer fwd tokens/s and effective TFLOP/s (% bf16 MFMA peak), L=8192"
# MI355X published dense bf16 MFMA peak: 256 CUs x 2.4 GHz x 4096 flop/clk/CU.
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12
KERNEL_SOURCE = os.path.join(ROOT, "block_sparse_transformer_amd", "csrc", "kernels", "fwd_bf16.hip")
BWD_KERNEL_SOURCE = os.path.join(ROOT, "block_sparse_transformer_amd", "csrc", "kernels", "bwd_bf16.hip")
# the attention kernel that dominates a bf16 forward: one for D = 64, one for D = 128
def main_kernel(head_dim: int) -> str:
    return "fwd_bf16_d64_kernel" if head_dim == 64 else "fwd_bf16_kernel"


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=None, help="default: the L=8192 BigBird workload")
    p.add_argument("--rotate", type=int, default=3, help="input copies rotated across steps")
    p.add_argument("--event-every", type=int, default=8,
                   help="time the main kernel with HIP events on one timed step in this many")
    p.add_argument("--pass", dest="which", choices=("forward", "backward", "layer"), default="forward",
                   help="time the forward (default), the backward, or the whole attention layer")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="the CPU baseline runs whole (batch, head) pairs until this much time has passed")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="instead of the benchmark, run plain device copies of MIB MiB (counter calibration)")
    return p.parse_args()


def tile_stats(wl, row_ptr, col, valid_len=None):
    """Non-zero 64x64 tiles computed per step (padding-aware when valid_len is given)."""
    import numpy as np
    per_head = np.diff(row_ptr).reshape(wl.heads, wl.seq_len // 64)   # rows of 64-token tiles
    if valid_len is None:
        return int(per_head.sum()) * wl.batch
    total = 0
    for b in range(wl.batch):
        nvb = -(-int(valid_len[b]) // 64)
        total += int((col < nvb).sum())
    return total


def traffic_from_profile(workload: str, kernel: str, source: str = KERNEL_SOURCE):
    """HBM bytes per launch of the main kernel from the committed counter summary, or None
    when the summary is missing or the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b:
        return None
    sha = hashlib.sha256(open(source, "rb").read()).hexdigest()
    if sha != m_sha.group(1):
        return None
    return float(m_b.group(1))


def calibrate_copy(mib: int) -> None:
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n * 4, "bytes_written": n * 4, "launches": 5}))


def cpu_baseline(wl, inp, layout_o, seconds: float):
    """The oracle as it stands, on whole (batch, head) pairs (all query rows) taken in order
    until ``seconds`` have passed, scaled to the whole job."""
    from threadpoolctl import threadpool_info

    from oracle import attention as OA
    all_pairs = [(b, h) for b in range(wl.batch) for h in range(wl.heads)]
    vl = inp.get("valid_len")
    pairs = []
    t0 = time.perf_counter()
    for b, h in all_pairs:
        OA.attention_forward(inp["q"], inp["k"], inp["v"], layout_o, wl.scale,
                             valid_len=None if vl is None else vl.tolist(), heads=[h], batches=[b])
        pairs.append((b, h))
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    full_s = dt * (wl.batch * wl.heads) / len(pairs)
    return {"value": wl.batch * wl.seq_len / full_s, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(pairs)} of {wl.batch * wl.heads} (batch, head) pairs, all {wl.seq_len} query rows, "
                      f"dense fp64 masked attention; {dt:.2f} s measured, scaled to the whole job",
            "seconds": round(dt, 3)}


def cpu_baseline_adaptive(wl, inp, seconds: float):
    """The oracle's adaptive forward (block sums, scores, selection, dense masked attention) on
    whole (batch, head) pairs taken in order until ``seconds`` have passed, scaled to the job."""
    from threadpoolctl import threadpool_info

    from oracle import adaptive as OD
    all_pairs = [(b, h) for b in range(wl.batch) for h in range(wl.heads)]
    pairs = []
    t0 = time.perf_counter()
    for b, h in all_pairs:
        rows = [[None] * wl.heads for _ in range(wl.batch)]
        rows[b][h] = OD.adaptive_rows(inp["q"][b:b + 1, h:h + 1], inp["k"][b:b + 1, h:h + 1], wl.keep_blocks)[0][0]
        OD.adaptive_attention_forward(inp["q"], inp["k"], inp["v"], wl.keep_blocks, wl.scale, rows=rows,
                                      pairs=[(b, h)])
        pairs.append((b, h))
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    full_s = dt * (wl.batch * wl.heads) / len(pairs)
    return {"value": wl.batch * wl.seq_len / full_s, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(pairs)} of {wl.batch * wl.heads} (batch, head) pairs, all {wl.seq_len} query rows, "
                      f"block selection and dense fp64 masked attention; {dt:.2f} s measured, scaled to the whole job",
            "seconds": round(dt, 3)}


def cpu_baseline_bwd(wl, inp, do, layout_o, seconds: float):
    """The oracle backward as it stands, on whole (batch, head) pairs taken in order until
    ``seconds`` have passed, scaled to the whole job."""
    from threadpoolctl import threadpool_info

    from oracle import attention_grad as OG
    all_pairs = [(b, h) for b in range(wl.batch) for h in range(wl.heads)]
    vl = inp.get("valid_len")
    pairs = []
    t0 = time.perf_counter()
    for b, h in all_pairs:
        OG.attention_backward(inp["q"], inp["k"], inp["v"], do, layout_o, wl.scale,
                              valid_len=None if vl is None else vl.tolist(), heads=[h], batches=[b])
        pairs.append((b, h))
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    full_s = dt * (wl.batch * wl.heads) / len(pairs)
    return {"value": wl.batch * wl.seq_len / full_s, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(pairs)} of {wl.batch * wl.heads} (batch, head) pairs, all {wl.seq_len} query rows, "
                      f"dense fp64 masked attention gradients; {dt:.2f} s measured, scaled to the whole job",
            "seconds": round(dt, 3)}


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "each (batch, head) pair is independent, so more GPUs would shard heads with no collective.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_transformer_amd as bs
    from workloads import THROUGHPUT_WORKLOAD, WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    wl = WORKLOADS[args.workload or THROUGHPUT_WORKLOAD]
    if wl.routed:
        print("bench.py times the block-layout forward; routed workloads are parity cases", file=sys.stderr)
        sys.exit(2)
    inp = make_inputs(wl)

    if (wl.adaptive and args.which != "forward") or (wl.token and args.which == "backward"):
        print("adaptive workloads are timed in the forward only, token-pattern workloads in the forward and "
              "the layer", file=sys.stderr)
        sys.exit(2)
    t0 = time.perf_counter()
    if wl.band:
        lay = bs.bsattn_make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens)
    elif wl.token:
        lay = bs.bsattn_make_token_layout(wl.heads, wl.seq_len, wl.band_tokens, wl.num_global, wl.random_tokens,
                                          wl.layout_seed)
    elif wl.adaptive:
        lay = bs.bsattn_make_adaptive_layout(wl.heads, wl.seq_len, wl.keep_blocks)
    else:
        lay = bs.bsattn_make_layout(wl.heads, wl.seq_len, wl.block, wl.window_blocks, list(wl.global_blocks),
                                    wl.random_blocks, wl.layout_seed)
    layout_host_us = (time.perf_counter() - t0) * 1e6
    bs.bsattn_layout_upload(lay)
    row_ptr, col = bs.bsattn_layout_csr(lay)
    vl_host = inp.get("valid_len")
    tiles = tile_stats(wl, row_ptr, col, None if vl_host is None else vl_host.tolist())
    if wl.token:
        # the global rows' tiles: ceil(n_global / 64) gathered-row tiles over every key block
        tiles += wl.batch * wl.heads * (-(-wl.num_global // 64)) * (wl.seq_len // 64)
    stored_tiles = tiles
    masks = bs.bsattn_layout_tile_masks(lay)
    if masks is not None:
        # 32-token blocks: the work is the layout's 32 x 32 blocks (a quarter of a
        # stored tile each), not the whole tiles the kernels compute
        tiles = wl.batch * int(np.unpackbits(masks).sum()) / 4.0
    flops_per_step = tiles * 4.0 * 64 * 64 * wl.head_dim
    elem = 2 if wl.dtype == "bf16" else 4
    alg_bytes = wl.batch * wl.heads * wl.seq_len * (4 * wl.head_dim * elem + 4)

    dev = torch.device("cuda:0")
    sets = []
    base = {k: v.to(dev) for k, v in inp.items()}
    for r in range(max(1, args.rotate)):
        sets.append({k: (v if r == 0 else v.clone()) for k, v in base.items()})
    B, H, L, D = wl.batch, wl.heads, wl.seq_len, wl.head_dim
    outs = [torch.empty((B, H, L, D), dtype=base["q"].dtype, device=dev) for _ in sets]
    lses = [torch.empty((B, H, L), dtype=torch.float32, device=dev) for _ in sets]
    ws_bytes = bs.bsattn_workspace_size(lay, B, D)
    ws = torch.empty(max(1, (ws_bytes + 255) // 4), dtype=torch.float32, device=dev)

    # Pre-marshalled C calls: the timed loop pays only the ctypes call itself.
    L_ = bs.lib()
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    dtype_code = 1 if wl.dtype == "bf16" else 0
    calls = []
    for s, o, l in zip(sets, outs, lses):
        vl = s.get("valid_len")
        calls.append((lay.handle, dtype_code, B, H, L, D, s["q"].data_ptr(), s["k"].data_ptr(),
                      s["v"].data_ptr(), o.data_ptr(), l.data_ptr(), None if vl is None else vl.data_ptr(),
                      ctypes.c_float(wl.scale), ws.data_ptr(), ctypes.c_size_t(ws_bytes), sh))
    fwd = L_.bsattn_forward
    backward = args.which == "backward"
    if backward:
        from workloads import make_grad_output
        for c in calls:                          # the forward's outputs, once, untimed
            st = fwd(*c)
            if st != 0:
                raise bs.BsattnError("bsattn_forward", st)
        do_host = make_grad_output(wl)
        dos = [do_host.to(dev) if r == 0 else do_host.to(dev).clone() for r in range(len(sets))]
        grads = [[torch.empty((B, H, L, D), dtype=base["q"].dtype, device=dev) for _ in range(3)] for _ in sets]
        wsb_bytes = bs.bsattn_backward_workspace_size(lay, B, D)
        wsb = torch.empty(max(1, (wsb_bytes + 255) // 4), dtype=torch.float32, device=dev)
        bcalls = []
        for s, o, l, g, dd in zip(sets, outs, lses, grads, dos):
            vl = s.get("valid_len")
            bcalls.append((lay.handle, dtype_code, B, H, L, D, s["q"].data_ptr(), s["k"].data_ptr(),
                           s["v"].data_ptr(), o.data_ptr(), l.data_ptr(), dd.data_ptr(), g[0].data_ptr(),
                           g[1].data_ptr(), g[2].data_ptr(), None if vl is None else vl.data_ptr(),
                           ctypes.c_float(wl.scale), wsb.data_ptr(), ctypes.c_size_t(wsb_bytes), sh))
        bwd = L_.bsattn_backward
        torch.cuda.synchronize()
        # algorithmic work: the five products of a backward that recomputes P
        # (S, dP, dV, dK, dQ), 2 * 64 * 64 * D flop each per tile; the dK/dV
        # kernel does the first four of them
        flops_per_step = tiles * 10.0 * 64 * 64 * wl.head_dim
        kernel_flops = tiles * 8.0 * 64 * 64 * wl.head_dim
        alg_bytes = wl.batch * wl.heads * wl.seq_len * (8 * wl.head_dim * elem + 4)

        def step(i):
            st = bwd(*bcalls[i % len(bcalls)])
            if st != 0:
                raise bs.BsattnError("bsattn_backward", st)
    elif args.which == "layer":
        from workloads import make_layer_params
        C = H * D
        lp = make_layer_params(wl)
        lsets = [{k: v.to(dev) for k, v in lp.items()}]
        for _ in range(1, len(sets)):
            lsets.append({k: (v if k != "x" else v.clone()) for k, v in lsets[0].items()})
        louts = [torch.empty((B, L, C), dtype=torch.bfloat16, device=dev) for _ in lsets]
        wsl_bytes = bs.bsattn_layer_workspace_size(lay, B, D)
        wsl = torch.empty(max(1, (wsl_bytes + 255) // 4), dtype=torch.float32, device=dev)
        lcalls = []
        for ls_, lo, s in zip(lsets, louts, sets):
            vl = s.get("valid_len")
            lcalls.append((lay.handle, B, H, L, D, ls_["x"].data_ptr(), ls_["w_qkv"].data_ptr(),
                           ls_["b_qkv"].data_ptr(), ls_["w_proj"].data_ptr(), ls_["b_proj"].data_ptr(),
                           lo.data_ptr(), None if vl is None else vl.data_ptr(), ctypes.c_float(wl.scale),
                           wsl.data_ptr(), ctypes.c_size_t(wsl_bytes), sh))
        lfwd = L_.bsattn_layer_forward
        # the two projections (2 * rows * C * 4C flop) plus the attention's tiles
        kernel_flops = flops_per_step
        flops_per_step = flops_per_step + 2.0 * B * L * C * 4 * C
        alg_bytes = alg_bytes + B * L * C * 2 * 2 + 4 * C * C * 2

        def step(i):
            st = lfwd(*lcalls[i % len(lcalls)])
            if st != 0:
                raise bs.BsattnError("bsattn_layer_forward", st)
    else:
        kernel_flops = flops_per_step

        def step(i):
            st = fwd(*calls[i % len(calls)])
            if st != 0:
                raise bs.BsattnError("bsattn_forward", st)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    ev = bs.HipEvents(len(range(0, K, max(1, args.event_every))))
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    set_ev = L_.bsattn_set_profile_events
    # The main kernel is timed by events its own dispatch records, on one step in
    # `event_every` of the timed region: an instrumented step runs a few
    # microseconds slower, and timing every step would charge that to the step.
    every = max(1, args.event_every)
    timed = list(range(0, K, every))
    torch.cuda.synchronize()
    t_start.record(stream)
    j = 0
    for i in range(K):
        if i % every == 0:
            set_ev(ev.before[j], ev.after[j])
            step(i)
            set_ev(None, None)
            j += 1
        else:
            step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / K
    kern_ms = [ev.elapsed_ms(n) for n in range(len(timed))]
    ev.destroy()
    kern_avg_ms = float(np.mean(kern_ms))

    tokens = B * L
    value = tokens / (ms_step / 1e3)
    eff_tflops = flops_per_step / (ms_step / 1e3) / 1e12
    kern_tflops = kernel_flops / (kern_avg_ms / 1e3) / 1e12
    kname = "bwd_dkdv_kernel" if backward else main_kernel(D)
    traffic = traffic_from_profile(wl.name, kname, BWD_KERNEL_SOURCE if backward else KERNEL_SOURCE)

    result = {
        "metric": METRIC_BWD if backward else (METRIC_LAYER if args.which == "layer" else METRIC),
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": ("synthetic (seeded Gaussian x and layer weights of the workload's shape)" if args.which == "layer"
                 else "synthetic (seeded Gaussian Q/K/V" + (" and dO" if backward else "") + " of the workload's shape)"),
        "config": {
            "workload": wl.name, "pass": args.which, "batch": B, "heads": H, "seq_len": L, "head_dim": D, "block": wl.block,
            "window_blocks": wl.window_blocks, "global_blocks": list(wl.global_blocks),
            "random_blocks": wl.random_blocks, "layout_seed": wl.layout_seed, "band_tokens": wl.band_tokens,
            "nonzero_tiles": stored_tiles, "layout_density": round(tiles / (B * H * (L // 64) ** 2), 5),
            **({"num_global": wl.num_global, "random_tokens": wl.random_tokens} if wl.token else {}),
            **({"keep_blocks": wl.keep_blocks} if wl.adaptive else {}),
        },
        "eff_tflops": round(eff_tflops, 2),
        "pct_bf16_peak": round(100 * eff_tflops / PEAK_BF16_TFLOPS, 2),
        "hbm_alg_gbps": round(alg_bytes / (ms_step / 1e3) / 1e9, 1),
        "layout_build_host_us": round(layout_host_us, 1),
        "roofline": {
            "bound": "mfma",
            "kernel": kname,
            "achieved": round(kern_tflops, 2),
            "peak": round(PEAK_BF16_TFLOPS, 1),
            "unit": "TFLOP/s",
            "frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel_avg_us": round(kern_avg_ms * 1e3, 3),
            "kernel_timed_steps": len(kern_ms),
            "flop_per_launch": kernel_flops,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and args.which != "layer":
        from oracle import layout as OL
        if wl.band:
            olay = OL.make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens)
        elif wl.token:
            olay = OL.make_token_layout(wl.heads, wl.seq_len, wl.band_tokens, wl.num_global, wl.random_tokens,
                                        wl.layout_seed)
        elif wl.adaptive:
            olay = None   # chosen from the data, per (batch, head)
        else:
            olay = OL.make_layout(wl.heads, wl.seq_len, wl.block, wl.window_blocks, list(wl.global_blocks),
                                  wl.random_blocks, wl.layout_seed)
        if wl.adaptive:
            result["cpu_baseline"] = cpu_baseline_adaptive(wl, inp, args.cpu_seconds)
        elif backward:
            result["cpu_baseline"] = cpu_baseline_bwd(wl, inp, do_host, olay, args.cpu_seconds)
        else:
            result["cpu_baseline"] = cpu_baseline(wl, inp, olay, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

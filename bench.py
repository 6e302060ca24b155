#!/usr/bin/env python3
"""Throughput of the block-sparse attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one full forward (``bsattn_forward``: every non-zero 64x64 tile of
the layout, the split of the dense global rows and their log-sum-exp merge)
over one batch of the workload, inputs already resident in HBM.  For the
routed workload a step is the router (``bsattn_route_topk``: fp64 scores and
the per-head top-k) followed by ``bsattn_forward_routed`` (the band forward,
the routed rows' tiles over every key and their merge).  With
``--pass backward`` a step is one full backward (``bsattn_backward``: delta,
the dQ pass, the dK/dV pass and the sums of split rows and columns) on the
forward's outputs and a seeded upstream gradient; with ``--pass layer`` a
step is one ``bsattn_layer_forward`` (qkv projection, head split, attention,
head concatenation, output projection; no CPU baseline).  W untimed
steps, then exactly K timed steps bracketed by device synchronisation; four
sets of inputs and outputs (about 406 MB at bigbird-L8192) are rotated so that
a step does not find the previous step's tensors in the 256 MB last-level
cache.

Prints ONE JSON line with the metric, ``roofline`` (the main attention
kernel timed by HIP events that its own dispatch records -- on every timed
step when K <= 25, else on one in K // 25 -- mean and median over the timed
region, priced against the bf16 dense MFMA peak or the HBM bandwidth, whichever
floor is larger for the kernel's algorithmic flops and bytes; then the median of
25 warm launches on one input set) and ``cpu_baseline`` (the fp64 oracle on a
bounded sample of the same workload, on the host cores, with the CPU model
and the cores the process may use).
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
PEAK_HBM_GBPS = 8000.0   # MI355X published HBM3E bandwidth
# MI355X published fp32 vector peak (256 CUs x 4 SIMDs x 16 lanes x 2 flop x 2 for packed
# FMA x 2.4 GHz); code built without packed fp32 instructions can reach half of it
PEAK_F32_VECTOR_TFLOPS = 157.3
KERNEL_SOURCE = os.path.join(ROOT, "block_sparse_transformer_amd", "csrc", "kernels", "fwd_bf16.hip")
BWD_KERNEL_SOURCE = os.path.join(ROOT, "block_sparse_transformer_amd", "csrc", "kernels", "bwd_bf16.hip")
TOPR_KERNEL_SOURCE = os.path.join(ROOT, "block_sparse_transformer_amd", "csrc", "kernels", "topr.hip")
CAND_KERNEL_SOURCE = os.path.join(ROOT, "block_sparse_transformer_amd", "csrc", "kernels", "candidates.hip")
# the attention kernel that dominates a bf16 forward: one for D = 64, one for D = 128
def main_kernel(head_dim: int) -> str:
    return "fwd_bf16_d64_kernel" if head_dim == 64 else "fwd_bf16_kernel"


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=None, help="default: the L=8192 BigBird workload")
    p.add_argument("--rotate", type=int, default=4,
                   help="input sets rotated across steps (4 bigbird-L8192 sets, inputs and outputs, hold "
                        "about 406 MB: more than the 256 MB last-level cache)")
    p.add_argument("--event-every", type=int, default=None,
                   help="time the main kernel with HIP events on one timed step in this many "
                        "(default: every step when K <= 25, else one in K // 25)")
    p.add_argument("--warm-launches", type=int, default=25,
                   help="after the timed region, launches on one input set (caches warm) timed by events")
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


def token_extra_pairs(bs, lay, wl):
    """(query, key) pairs of one batch entry that the token kernels add: every non-global
    row's global keys outside its band, and its random tokens."""
    import numpy as np
    g, links = bs.bsattn_layout_token_links(lay)
    g = np.asarray(g, dtype=np.int64)
    t = np.arange(wl.seq_len)
    nonglobal = ~np.isin(t, g)
    inside = np.searchsorted(g, t + wl.band_tokens, side="right") - np.searchsorted(g, t - wl.band_tokens, side="left")
    per_row = (len(g) - inside) * nonglobal
    total = int(per_row.sum()) * wl.heads
    if links is not None and links.size:
        total += int(((links >= 0) & nonglobal[None, :, None]).sum())
    return total


def cpu_baseline_candidates(wl, inp, seconds: float):
    """The oracle as it stands on the candidate workload: the positions of batch entry 0,
    then whole heads of it until ``seconds`` have passed, scaled to the whole job."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import candidates as OC
    t0 = time.perf_counter()
    pos = OC.candidate_positions(inp["x"][:1], inp["w_conv"].permute(2, 1, 0).contiguous().numpy(),
                                 inp["b_conv"].numpy())
    t_conv = time.perf_counter() - t0
    pos_all = np.zeros((wl.batch,) + pos.shape[1:], dtype=np.int32)
    pos_all[0] = pos[0]
    heads = 0
    t1 = time.perf_counter()
    for h in range(wl.heads):
        OC.candidate_attention_forward(inp["q"], inp["k"], inp["v"], pos_all, wl.cand_keep, wl.scale,
                                       rows=[(0, h, t) for t in range(wl.seq_len)])
        heads += 1
        if time.perf_counter() - t0 >= seconds:
            break
    t_head = (time.perf_counter() - t1) / heads
    full_s = wl.batch * (t_conv + wl.heads * t_head)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": wl.batch * wl.seq_len / full_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the positions of 1 of {wl.batch} batch entries ({t_conv:.2f} s, fp64 fixed-order "
                      f"convolution) and {heads} of its {wl.heads} heads ({t_head:.2f} s each: fp32 ranking of "
                      f"the candidates and fp64 attention over the kept ones), scaled to the whole job",
            "seconds": round(time.perf_counter() - t0, 3), **host_info()}


def run_candidates(args, wl, inp, bs, torch, np):
    """Candidate-list attention: one step is the candidate positions of the hidden
    states followed by the attention over each query's kept candidates."""
    dev = torch.device("cuda:0")
    base = {k: v.to(dev) for k, v in inp.items()}
    sets = [{k: (v if r == 0 else v.clone()) for k, v in base.items()} for r in range(max(1, args.rotate))]
    B, H, L, D = wl.batch, wl.heads, wl.seq_len, wl.head_dim
    C, kc, keep = H * D, wl.num_candidates, wl.cand_keep
    poss = [torch.empty((B, L, kc), dtype=torch.int32, device=dev) for _ in sets]
    outs = [torch.empty((B, H, L, D), dtype=torch.bfloat16, device=dev) for _ in sets]
    lses = [torch.empty((B, H, L), dtype=torch.float32, device=dev) for _ in sets]
    rotation_bytes = sum(t.numel() * t.element_size() for st in sets for t in st.values()) + \
        sum(t.numel() * t.element_size() for lst in (poss, outs, lses) for t in lst)
    L_ = bs.lib()
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    calls = []
    for s_, p_, o_, l_ in zip(sets, poss, outs, lses):
        calls.append(((s_["x"].data_ptr(), s_["w_conv"].data_ptr(), s_["b_conv"].data_ptr(), B, L, C, kc,
                       p_.data_ptr(), sh),
                      (1, B, H, L, D, s_["q"].data_ptr(), s_["k"].data_ptr(), s_["v"].data_ptr(), p_.data_ptr(), kc,
                       keep, ctypes.c_float(wl.scale), o_.data_ptr(), l_.data_ptr(), None, sh)))
    posf, fwd = L_.bsattn_candidate_positions, L_.bsattn_candidate_forward

    def step(i):
        pc, fc = calls[i % len(calls)]
        st = posf(*pc)
        if st != 0:
            raise bs.BsattnError("bsattn_candidate_positions", st)
        st = fwd(*fc)
        if st != 0:
            raise bs.BsattnError("bsattn_candidate_forward", st)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    every = max(1, args.event_every if args.event_every is not None else (1 if K <= 25 else K // 25))
    timed = list(range(0, K, every))
    ev = bs.HipEvents(len(timed))
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    set_ev = L_.bsattn_set_profile_events
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
    ms_step = t_start.elapsed_time(t_end) / K
    kern_ms = [ev.elapsed_ms(n) for n in range(len(timed))]
    ev.destroy()
    warm_ms = []
    if args.warm_launches > 0:
        wev = bs.HipEvents(args.warm_launches)
        for n in range(args.warm_launches):
            set_ev(wev.before[n], wev.after[n])
            step(0)
        set_ev(None, None)
        torch.cuda.synchronize()
        warm_ms = [wev.elapsed_ms(n) for n in range(args.warm_launches)]
        wev.destroy()
    kern_avg_ms, kern_med_ms = float(np.mean(kern_ms)), float(np.median(kern_ms))
    # work: the convolution (2 x 3C flop per output), the candidates' scores (2 D per
    # candidate) and the attention over the kept keys (4 D per kept key)
    conv_flops = 2.0 * B * L * kc * 3 * C
    attn_flops = B * H * L * (2.0 * kc * D + 4.0 * keep * D)
    flops_per_step = conv_flops + attn_flops
    # the attention kernel's algorithmic bytes: Q, K, V read and O, LSE written once, the positions read
    kernel_bytes = B * H * L * (4 * D * 2 + 4) + B * L * kc * 4
    kern_gbps = kernel_bytes / (kern_avg_ms / 1e3) / 1e9
    kern_tflops = attn_flops / (kern_avg_ms / 1e3) / 1e12
    t_hbm = kernel_bytes / (PEAK_HBM_GBPS * 1e9)
    t_alu = attn_flops / (PEAK_F32_VECTOR_TFLOPS * 1e12)
    if t_hbm >= t_alu:
        bound, achieved, peak, unit = "hbm", kern_gbps, PEAK_HBM_GBPS, "GB/s"
    else:
        bound, achieved, peak, unit = "alu", kern_tflops, PEAK_F32_VECTOR_TFLOPS, "TFLOP/s"
    kname = "cand_attention2_kernel" if kc <= 32 else "cand_attention_kernel"   # two queries per wave up to k = 32
    traffic = traffic_from_profile(wl.name, kname, CAND_KERNEL_SOURCE)
    result = {
        "metric": METRIC, "value": round(B * L / (ms_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded Gaussian Q/K/V, hidden states and candidate-generator weights of the workload's "
                "shape)",
        "config": {"workload": wl.name, "pass": "forward", "batch": B, "heads": H, "seq_len": L, "head_dim": D,
                   "channels": C, "num_candidates": kc, "keep": keep},
        "eff_tflops": round(flops_per_step / (ms_step / 1e3) / 1e12, 2),
        "pct_bf16_peak": round(100 * flops_per_step / (ms_step / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "hbm_alg_gbps": round(kernel_bytes / (ms_step / 1e3) / 1e9, 1),
        "roofline": {
            "bound": bound, "kernel": kname, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "mfma_frac": 0.0, "hbm_frac": round(kern_gbps / PEAK_HBM_GBPS, 4),
            "kernel_avg_us": round(kern_avg_ms * 1e3, 3), "kernel_median_us": round(kern_med_ms * 1e3, 3),
            "kernel_timed_steps": len(kern_ms),
            "kernel_warm_median_us": round(float(np.median(warm_ms)) * 1e3, 3) if warm_ms else None,
            "input_sets": len(sets), "rotation_bytes": int(rotation_bytes),
            "flop_per_launch": attn_flops, "alg_bytes_per_launch": kernel_bytes,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_candidates(wl, inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


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
            "seconds": round(dt, 3), **host_info()}


def host_info():
    """The host the CPU baseline ran on: CPU model and the cores this process may use."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0))}


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
            "seconds": round(dt, 3), **host_info()}


def cpu_baseline_routed(wl, inp, seconds: float):
    """The oracle's routed path (fp64 scores, top-k, banded plus routed dense attention) on
    whole (batch, head) pairs taken in order until ``seconds`` have passed, scaled to the job."""
    from threadpoolctl import threadpool_info

    from oracle import attention as OA
    from oracle import router as OR
    all_pairs = [(b, h) for b in range(wl.batch) for h in range(wl.heads)]
    pairs = []
    t0 = time.perf_counter()
    for b, h in all_pairs:
        q, k, v = (inp[n][b:b + 1, h:h + 1] for n in ("q", "k", "v"))
        rr = OR.topk_rows(OR.router_scores(q, inp["w"]), wl.routed_k)
        OA.routed_attention_forward(q, k, v, rr, wl.band_tokens, wl.scale)
        pairs.append((b, h))
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    full_s = dt * (wl.batch * wl.heads) / len(pairs)
    return {"value": wl.batch * wl.seq_len / full_s, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(pairs)} of {wl.batch * wl.heads} (batch, head) pairs, all {wl.seq_len} query rows, "
                      f"router top-{wl.routed_k} and dense fp64 masked attention; {dt:.2f} s measured, scaled to "
                      "the whole job",
            "seconds": round(dt, 3), **host_info()}


def cpu_baseline_topr(wl, inp, seconds: float):
    """The oracle's top-keep forward (fp32 ranking scores, per-query selection, dense fp64
    masked attention) on whole (batch, head) pairs taken in order until ``seconds`` have
    passed, scaled to the job."""
    from threadpoolctl import threadpool_info

    from oracle import topr as OT
    all_pairs = [(b, h) for b in range(wl.batch) for h in range(wl.heads)]
    pairs = []
    t0 = time.perf_counter()
    for b, h in all_pairs:
        OT.topr_attention_forward(inp["q"][b:b + 1], inp["k"][b:b + 1], inp["v"][b:b + 1], wl.keep_tokens,
                                  wl.scale, heads=[h])
        pairs.append((b, h))
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    full_s = dt * (wl.batch * wl.heads) / len(pairs)
    return {"value": wl.batch * wl.seq_len / full_s, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{len(pairs)} of {wl.batch * wl.heads} (batch, head) pairs, all {wl.seq_len} query rows, "
                      f"fp32 ranking scores, top-{wl.keep_tokens} per query and dense fp64 masked attention; "
                      f"{dt:.2f} s measured, scaled to the whole job",
            "seconds": round(dt, 3), **host_info()}


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
            "seconds": round(dt, 3), **host_info()}


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
    inp = make_inputs(wl)

    if (wl.adaptive or wl.routed or wl.topr or wl.candidates) and args.which != "forward":
        print("adaptive, routed, top-keep and candidate workloads are timed in the forward only", file=sys.stderr)
        sys.exit(2)
    if wl.candidates:
        run_candidates(args, wl, inp, bs, torch, np)
        return
    t0 = time.perf_counter()
    if wl.band or wl.routed:
        lay = bs.bsattn_make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens)
    elif wl.token:
        lay = bs.bsattn_make_token_layout(wl.heads, wl.seq_len, wl.band_tokens, wl.num_global, wl.random_tokens,
                                          wl.layout_seed)
    elif wl.adaptive:
        lay = bs.bsattn_make_adaptive_layout(wl.heads, wl.seq_len, wl.keep_blocks)
    elif wl.topr:
        lay = bs.bsattn_make_topr_layout(wl.heads, wl.seq_len, wl.keep_tokens)
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
    if wl.routed:
        # the routed rows, gathered into ceil(k / 64) tiles per head, over every key block
        tiles += wl.batch * wl.heads * (-(-wl.routed_k // 64)) * (wl.seq_len // 64)
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
    rotation_bytes = sum(t.numel() * t.element_size() for st in sets for t in st.values()) + \
        sum(o.numel() * o.element_size() + l_.numel() * l_.element_size() for o, l_ in zip(outs, lses))
    ws_bytes = bs.bsattn_workspace_size(lay, B, D, wl.routed_k)
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
        bwd_tiles, extra_pairs = tiles, 0
        if wl.token:
            # the block passes walk the band tiles and the global rows' tiles; each
            # non-global row's global keys outside its band and its random tokens
            # are pairs of the token kernels (the same five products, 10 D flop a pair)
            bwd_tiles = tiles - wl.batch * (len(row_ptr) - 1) * (-(-wl.num_global // 64))   # less the gathered tiles
            extra_pairs = wl.batch * token_extra_pairs(bs, lay, wl)
        flops_per_step = bwd_tiles * 10.0 * 64 * 64 * wl.head_dim + extra_pairs * 10.0 * wl.head_dim
        kernel_flops = bwd_tiles * 8.0 * 64 * 64 * wl.head_dim
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
    elif wl.routed:
        # one step: the router's top-k, then the band forward with the routed
        # rows' tiles over every key and the merge of their split partials
        kernel_flops = flops_per_step
        k_r = wl.routed_k
        wsr_bytes = bs.bsattn_route_workspace_size(B, H, L, k_r)
        wsr = torch.empty(max(1, (wsr_bytes + 255) // 4), dtype=torch.float32, device=dev)
        rrs = [torch.empty((B, H, k_r), dtype=torch.int32, device=dev) for _ in sets]
        rcalls = []
        for s, o, l, rr in zip(sets, outs, lses, rrs):
            rcalls.append(((s["q"].data_ptr(), s["w"].data_ptr(), B, H, L, D, k_r, rr.data_ptr(), wsr.data_ptr(),
                            ctypes.c_size_t(wsr_bytes), sh),
                           (lay.handle, dtype_code, B, H, L, D, s["q"].data_ptr(), s["k"].data_ptr(),
                            s["v"].data_ptr(), rr.data_ptr(), k_r, o.data_ptr(), l.data_ptr(), ctypes.c_float(wl.scale),
                            ws.data_ptr(), ctypes.c_size_t(ws_bytes), sh)))
        route, fwd_r = L_.bsattn_route_topk, L_.bsattn_forward_routed

        def step(i):
            rc, fc = rcalls[i % len(rcalls)]
            st = route(*rc)
            if st != 0:
                raise bs.BsattnError("bsattn_route_topk", st)
            st = fwd_r(*fc)
            if st != 0:
                raise bs.BsattnError("bsattn_forward_routed", st)
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
    every = args.event_every if args.event_every is not None else (1 if K <= 25 else K // 25)
    every = max(1, every)
    ev = bs.HipEvents(len(range(0, K, every)))
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    set_ev = L_.bsattn_set_profile_events
    # The main kernel is timed by events its own dispatch records, on one step in
    # `every` of the timed region (timing-only events, recorded by the dispatch
    # itself, add no packets between kernels).
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
    kern_med_ms = float(np.median(kern_ms))
    # warm: the same launch on one input set, back to back, after the timed region
    warm_ms = []
    if args.warm_launches > 0:
        wev = bs.HipEvents(args.warm_launches)
        for n in range(args.warm_launches):
            set_ev(wev.before[n], wev.after[n])
            step(0)
        set_ev(None, None)
        torch.cuda.synchronize()
        warm_ms = [wev.elapsed_ms(n) for n in range(args.warm_launches)]
        wev.destroy()

    tokens = B * L
    value = tokens / (ms_step / 1e3)
    eff_tflops = flops_per_step / (ms_step / 1e3) / 1e12
    kern_tflops = kernel_flops / (kern_avg_ms / 1e3) / 1e12
    # the top-keep selection: key-stationary at D = 64, L <= 2048, else the LDS-tiled kernel
    topr_kernel = "topr_select_ks_kernel" if (D == 64 and L <= 2048) else "topr_select_kernel"
    kname = "bwd_dkdv_kernel" if backward else (topr_kernel if wl.topr else main_kernel(D))
    # the kernel's own algorithmic bytes: Q, K, V read and O, LSE written once (the
    # backward's dK/dV pass: Q, K, V, dO read, dK, dV written, LSE and delta read)
    kernel_bytes = wl.batch * wl.heads * wl.seq_len * ((6 if backward else 4) * wl.head_dim * elem + (8 if backward else 4))
    kern_gbps = kernel_bytes / (kern_avg_ms / 1e3) / 1e9
    # the roofline that bounds the kernel: the larger of its two floors at the
    # published peaks; where they are within 10% the contraction's peak is kept
    t_mfma = kernel_flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = kernel_bytes / (PEAK_HBM_GBPS * 1e9)
    if wl.topr:
        # the timed kernel is the selection: 2 L^2 D flop of in-order fp32 FMA
        # chains per (batch, head), bound by the vector ALU
        sel_flops = 2.0 * B * H * L * L * D
        kern_tflops = sel_flops / (kern_avg_ms / 1e3) / 1e12
        bound, achieved, peak, unit = "alu", kern_tflops, PEAK_F32_VECTOR_TFLOPS, "TFLOP/s"
        kernel_flops = sel_flops
        kernel_bytes = B * H * L * 2 * D * elem + B * H * L * (L // 64) * 8
        kern_gbps = kernel_bytes / (kern_avg_ms / 1e3) / 1e9
    elif t_hbm > 1.1 * t_mfma:
        bound, achieved, peak, unit = "hbm", kern_gbps, PEAK_HBM_GBPS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", kern_tflops, round(PEAK_BF16_TFLOPS, 1), "TFLOP/s"
    traffic = traffic_from_profile(wl.name, kname, BWD_KERNEL_SOURCE if backward else
                                   TOPR_KERNEL_SOURCE if wl.topr else KERNEL_SOURCE)

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
            **({"routed_k": wl.routed_k} if wl.routed else {}),
            **({"keep_tokens": wl.keep_tokens} if wl.topr else {}),
        },
        "eff_tflops": round(eff_tflops, 2),
        "pct_bf16_peak": round(100 * eff_tflops / PEAK_BF16_TFLOPS, 2),
        "hbm_alg_gbps": round(alg_bytes / (ms_step / 1e3) / 1e9, 1),
        "layout_build_host_us": round(layout_host_us, 1),
        "roofline": {
            "bound": bound,
            "kernel": kname,
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "mfma_frac": round(kern_tflops / PEAK_BF16_TFLOPS, 4),
            "hbm_frac": round(kern_gbps / PEAK_HBM_GBPS, 4),
            "kernel_avg_us": round(kern_avg_ms * 1e3, 3),
            "kernel_median_us": round(kern_med_ms * 1e3, 3),
            "kernel_timed_steps": len(kern_ms),
            "kernel_warm_median_us": round(float(np.median(warm_ms)) * 1e3, 3) if warm_ms else None,
            "input_sets": len(sets),
            "rotation_bytes": int(rotation_bytes),
            "flop_per_launch": kernel_flops,
            "alg_bytes_per_launch": kernel_bytes,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and args.which != "layer":
        from oracle import layout as OL
        if wl.band or wl.routed:
            olay = OL.make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens)
        elif wl.token:
            olay = OL.make_token_layout(wl.heads, wl.seq_len, wl.band_tokens, wl.num_global, wl.random_tokens,
                                        wl.layout_seed)
        elif wl.adaptive or wl.topr:
            olay = None   # chosen from the data, per (batch, head)
        else:
            olay = OL.make_layout(wl.heads, wl.seq_len, wl.block, wl.window_blocks, list(wl.global_blocks),
                                  wl.random_blocks, wl.layout_seed)
        if wl.adaptive:
            result["cpu_baseline"] = cpu_baseline_adaptive(wl, inp, args.cpu_seconds)
        elif wl.topr:
            result["cpu_baseline"] = cpu_baseline_topr(wl, inp, args.cpu_seconds)
        elif wl.routed:
            result["cpu_baseline"] = cpu_baseline_routed(wl, inp, args.cpu_seconds)
        elif backward:
            result["cpu_baseline"] = cpu_baseline_bwd(wl, inp, do_host, olay, args.cpu_seconds)
        else:
            result["cpu_baseline"] = cpu_baseline(wl, inp, olay, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

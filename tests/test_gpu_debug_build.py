"""The bounds-checking debug build (libbsattn_debug.so, -DBSATTN_DEBUG) on the GPU.

In that build the forward kernels check every schedule entry they read (list
lengths, unit records, tile entries), the backward kernels every item and block
list entry, and each forward and backward pass synchronises and fails if a check
did not hold.  Run as a script, this file computes forwards and backwards of
every schedule kind (D = 64 rows with split global rows, D = 128 with key
padding, the routed variant, the token pattern) with whichever library
BSATTN_LIBRARY selects and saves them; the test runs it once with each build,
in child processes one after the other, and requires the debug build's calls to
succeed and to give the release build's outputs bit for bit (the checks change
no arithmetic)."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "block_sparse_transformer_amd")


def _cases(out_path):
    sys.path.insert(0, ROOT)
    import torch

    import block_sparse_transformer_amd as bs
    from workloads import WORKLOADS, make_grad_output, make_inputs

    res = {}

    def say(*a):
        print("[gpu-case]", *a, file=sys.stderr, flush=True)

    # D = 64, split global rows merged inside the kernel
    wl = WORKLOADS["bigbird-L2048"].with_(batch=2, heads=3)
    say("debug-build", wl.name, "D=64 split rows")
    inp = {k: v.cuda() for k, v in make_inputs(wl).items()}
    lay = bs.bsattn_make_layout(wl.heads, wl.seq_len, 64, wl.window_blocks, list(wl.global_blocks),
                                wl.random_blocks, wl.layout_seed)
    bs.bsattn_layout_upload(lay)
    o, l = bs.forward(inp["q"], inp["k"], inp["v"], lay, scale=wl.scale)
    res["d64_o"], res["d64_l"] = o, l
    do = make_grad_output(wl).cuda()
    res["d64_dq"], res["d64_dk"], res["d64_dv"] = bs.backward(inp["q"], inp["k"], inp["v"], o, l, do, lay,
                                                              scale=wl.scale)
    # D = 128 with key padding (the two-wave kernel)
    wl = WORKLOADS["window-pad-L16384"].with_(batch=2, heads=2, seq_len=2048)
    say("debug-build", wl.name, "D=128 padded")
    inp = {k: v.cuda() for k, v in make_inputs(wl).items()}
    lay = bs.bsattn_make_layout(wl.heads, wl.seq_len, 64, wl.window_blocks, list(wl.global_blocks),
                                wl.random_blocks, wl.layout_seed)
    bs.bsattn_layout_upload(lay)
    o, l = bs.forward(inp["q"], inp["k"], inp["v"], lay, key_valid_len=inp["valid_len"], scale=wl.scale)
    res["pad_o"], res["pad_l"] = o, l
    do = make_grad_output(wl).cuda()
    res["pad_dq"], res["pad_dk"], res["pad_dv"] = bs.backward(inp["q"], inp["k"], inp["v"], o, l, do, lay,
                                                              key_valid_len=inp["valid_len"], scale=wl.scale)
    # routed rows over a token band
    wl = WORKLOADS["routed-L4096"].with_(heads=2, seq_len=1024, routed_k=70)
    say("debug-build", wl.name, "routed k=70")
    inp = {k: v.cuda() for k, v in make_inputs(wl).items()}
    rr = torch.empty((wl.batch, wl.heads, wl.routed_k), dtype=torch.int32, device="cuda")
    bs.bsattn_route_topk(inp["q"], inp["w"], wl.routed_k, rr)
    band = bs.bsattn_make_band_layout(wl.heads, wl.seq_len, 64, wl.band_tokens)
    bs.bsattn_layout_upload(band)
    o, l = bs.forward_routed(inp["q"], inp["k"], inp["v"], band, rr, scale=wl.scale)
    res["routed_o"], res["routed_l"] = o, l
    do = make_grad_output(wl).cuda()
    res["routed_dq"], res["routed_dk"], res["routed_dv"] = bs.backward_routed(
        inp["q"], inp["k"], inp["v"], o, l, do, band, rr, scale=wl.scale)
    # the token pattern (gathered global-key tiles, per-token random links)
    wl = WORKLOADS["bigbird-tok-L8192"].with_(batch=1, heads=2, seq_len=1536)
    say("debug-build", wl.name, "token pattern")
    inp = {k: v.cuda() for k, v in make_inputs(wl).items()}
    lay = bs.bsattn_make_token_layout(wl.heads, wl.seq_len, wl.band_tokens, wl.num_global, wl.random_tokens,
                                      wl.layout_seed)
    bs.bsattn_layout_upload(lay)
    o, l = bs.forward(inp["q"], inp["k"], inp["v"], lay, scale=wl.scale)
    res["tok_o"], res["tok_l"] = o, l
    do = make_grad_output(wl).cuda()
    res["tok_dq"], res["tok_dk"], res["tok_dv"] = bs.backward(inp["q"], inp["k"], inp["v"], o, l, do, lay,
                                                              scale=wl.scale)
    torch.cuda.synchronize()
    np.savez(out_path, **{k: (v.view(torch.int16) if v.dtype == torch.bfloat16 else v).cpu().numpy()
                          for k, v in res.items()})


def _run(lib, out_path):
    env = dict(os.environ)
    env.pop("BSATTN_LIBRARY", None)
    if lib:
        env["BSATTN_LIBRARY"] = lib
    r = subprocess.run([sys.executable, "-u", os.path.abspath(__file__), out_path], capture_output=True, text=True,
                       env=env, timeout=300)
    assert r.returncode == 0, f"{os.path.basename(lib or 'libbsattn.so')}: exit {r.returncode}\n{r.stderr[-4000:]}"
    return dict(np.load(out_path))


@pytest.mark.gpu
def test_debug_build_checks_pass_and_outputs_match(tmp_path):
    debug_lib = os.path.join(PKG, "libbsattn_debug.so")
    assert os.path.exists(debug_lib), f"{debug_lib} is missing: run __graft_entry__.build()"
    dbg = _run(debug_lib, str(tmp_path / "debug.npz"))
    rel = _run(None, str(tmp_path / "release.npz"))
    assert sorted(dbg) == sorted(rel)
    for k in rel:
        assert np.array_equal(dbg[k], rel[k], equal_nan=True), f"{k}: the debug build's output differs"


if __name__ == "__main__":
    _cases(sys.argv[1])

"""Schedule and workspace independence of the prefill and decode paths.

The kernels coordinate through atomics (routing records, dispatch cursors),
persistent workgroups and workspace buffers that no call clears in full.  A
result must not depend on what the workspace held before, on which stream a
call runs, or on other work sharing the GPU at the same time: every output
here must equal, bit for bit, the one of a plain call on the default stream
with a fresh workspace.
"""
from __future__ import annotations

import sys

import pytest
import torch

import content_routed_block_stats_amd as ssa
from synth_inputs import CONFIGS, make_decode, make_prefill

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


WL = CONFIGS["prefill_32k"].replace(n_q_heads=8, n_kv_heads=2, seq_len=64 * 97 + 13, block=64,
                                    top_k=8, window=64, plants=4)


def _params(wl, Q):
    b, hq, n, d = Q.shape
    return ssa.make_params(batch=b, n_q_heads=hq, n_kv_heads=wl.n_kv_heads, head_dim=d, seq_len=n,
                           block_size=wl.block, top_k=wl.top_k, window=wl.window, beta=wl.beta,
                           scale=wl.scale, in_dtype=Q.dtype)


def _prefill(wl, Q, K, V, ws_r=None, ws_a=None):
    mu, sigma = ssa.ssa_block_stats(K, wl.block)
    idx = ssa.ssa_route_topk(Q, mu, sigma, block_size=wl.block, top_k=wl.top_k, beta=wl.beta,
                             workspace=ws_r)
    O, lse = ssa.ssa_sparse_attn_fwd(Q, K, V, idx, block_size=wl.block, window=wl.window,
                                     scale=wl.scale, workspace=ws_a)
    return mu, sigma, idx, O, lse


def _same(a, b, what):
    for x, y, name in zip(a, b, ("mu", "sigma", "idx", "O", "lse")):
        assert torch.equal(x, y), f"{what}: {name} differs"


def test_prefill_independent_of_workspace_and_stream():
    data = make_prefill(WL, seed=3, device=DEV)
    Q, K, V = data["Q"], data["K"], data["V"]
    ref = _prefill(WL, Q, K, V)
    torch.cuda.synchronize()
    p = _params(WL, Q)
    nr, na = ssa.ssa_workspace_size(p, 1), ssa.ssa_workspace_size(p, 2)
    g = torch.Generator(device=DEV).manual_seed(11)
    for fill in ("ones", "random"):
        ws_r = torch.empty(nr, dtype=torch.uint8, device=DEV)
        ws_a = torch.empty(na, dtype=torch.uint8, device=DEV)
        if fill == "ones":
            ws_r.fill_(0xFF)
            ws_a.fill_(0xFF)
        else:
            ws_r.random_(0, 256, generator=g)
            ws_a.random_(0, 256, generator=g)
        say(f"  workspace filled with {fill}")
        _same(ref, _prefill(WL, Q, K, V, ws_r, ws_a), f"workspace {fill}")
        torch.cuda.synchronize()
    # on a side stream while other inputs run on the default stream
    other = make_prefill(WL, seed=4, device=DEV)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        got = _prefill(WL, Q, K, V)
    busy = _prefill(WL, other["Q"], other["K"], other["V"])
    torch.cuda.synchronize()
    _same(ref, got, "side stream")
    _same(_prefill(WL, other["Q"], other["K"], other["V"]), busy, "default stream beside it")
    # the same call twice in a row on one stream, with one workspace
    ws_r = torch.empty(nr, dtype=torch.uint8, device=DEV)
    ws_a = torch.empty(na, dtype=torch.uint8, device=DEV)
    first = _prefill(WL, Q, K, V, ws_r, ws_a)
    second = _prefill(WL, Q, K, V, ws_r, ws_a)
    torch.cuda.synchronize()
    _same(ref, first, "first of two")
    _same(ref, second, "second of two")


def test_decode_independent_of_workspace_and_stream():
    wl = CONFIGS["decode_256k"].replace(batch=3, n_q_heads=8, n_kv_heads=2, seq_len=64 * 40 + 63,
                                        block=64, top_k=8, window=64, plants=2)
    data = make_decode(wl, seed=5, capacity=wl.seq_len + 8)
    L = wl.seq_len

    def step(ws=None, stream=None):
        Kc, Vc = data["K_cache"].to(DEV), data["V_cache"].to(DEV)
        mu, sigma = ssa.ssa_block_stats(Kc, wl.block)
        cl = torch.full((wl.batch,), L, dtype=torch.int32, device=DEV)
        ctx = torch.cuda.stream(stream) if stream is not None else torch.cuda.stream(
            torch.cuda.current_stream())
        torch.cuda.synchronize()
        with ctx:
            o, lse, idx = ssa.ssa_decode_step(data["q"].to(DEV), data["k_new"].to(DEV),
                                              data["v_new"].to(DEV), Kc, Vc, cl, mu, sigma,
                                              block_size=wl.block, top_k=wl.top_k,
                                              window=wl.window, beta=wl.beta, scale=wl.scale,
                                              return_idx=True, workspace=ws)
        torch.cuda.synchronize()
        return o, lse, idx, mu, sigma, Kc, cl

    ref = step()
    p = ssa.make_params(batch=wl.batch, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                        head_dim=wl.head_dim, seq_len=L + 8, block_size=wl.block, top_k=wl.top_k,
                        window=wl.window, beta=wl.beta, scale=wl.scale,
                        in_dtype=data["q"].dtype)
    ws = torch.empty(ssa.ssa_workspace_size(p, 3), dtype=torch.uint8, device=DEV).fill_(0xFF)
    for got, what in ((step(ws), "workspace of ones"), (step(stream=torch.cuda.Stream()), "side stream")):
        for x, y, name in zip(ref, got, ("o", "lse", "idx", "mu", "sigma", "K cache", "cache_len")):
            assert torch.equal(x, y), f"{what}: {name} differs"

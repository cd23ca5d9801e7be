"""The allocation-free decode entry point against the one with a workspace.

ssa_decode_step_noalloc runs the decode step's kernels with their scratch in a
device array inside the library.  Two calls in a row -- the second with a
smaller input, so the scratch still holds the first call's larger contents --
must give exactly what ssa_decode_step gives on identical copies of the
inputs (the same kernels on the same data: bitwise equal outputs, selections,
caches, statistics and cache lengths).  A size beyond the scratch is refused
before anything is enqueued.
"""
from __future__ import annotations

import ctypes
import sys

import pytest
import torch

import content_routed_block_stats_amd as ssa
from content_routed_block_stats_amd import binding as B
from synth_inputs import CONFIGS, make_decode

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _state(data, block):
    Kc, Vc = data["K_cache"].to(DEV), data["V_cache"].to(DEV)
    mu, sigma = ssa.ssa_block_stats(Kc, block)
    cl = torch.full((Kc.shape[0],), data["cache_len"], dtype=torch.int32, device=DEV)
    return [Kc, Vc, cl, mu, sigma]


def _one(wl, cap, seed):
    data = make_decode(wl, seed=seed, capacity=cap)
    q, kn, vn = (data[k].to(DEV) for k in ("q", "k_new", "v_new"))
    ref = _state(data, wl.block)
    new = [t.clone() for t in ref]
    kw = dict(block_size=wl.block, top_k=wl.top_k, window=wl.window, beta=wl.beta,
              scale=wl.scale)
    o_r, l_r, i_r = ssa.ssa_decode_step(q, kn, vn, ref[0], ref[1], ref[2], ref[3], ref[4],
                                        return_idx=True, **kw)
    out = torch.empty_like(o_r)
    lse = torch.empty_like(l_r)
    idx = torch.empty_like(i_r)
    ssa.ssa_decode_step_noalloc(q, kn, vn, new[0], new[1], new[2], new[3], new[4], out=out,
                                lse=lse, idx=idx, **kw)
    torch.cuda.synchronize()
    assert torch.equal(idx, i_r), "selections differ"
    assert torch.equal(out, o_r), "outputs differ"
    assert torch.equal(lse, l_r), "LSE differs"
    for name, a, b in zip(("K_cache", "V_cache", "cache_len", "mu", "sigma"), new, ref):
        assert torch.equal(a, b), f"{name} differs"
    assert torch.isfinite(out.float()).all()
    return int(B.ssa_workspace_size(B.make_params(
        batch=wl.batch, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
        seq_len=cap, block_size=wl.block, top_k=wl.top_k, window=wl.window,
        in_dtype=wl.torch_dtype), B.SSA_OP_DECODE))


def test_noalloc_decode_matches_workspace_entry_point():
    big = CONFIGS["decode_256k"].replace(batch=4, n_q_heads=32, n_kv_heads=8, block=64, top_k=12,
                                         window=64, plants=4, seq_len=8191)
    small = CONFIGS["decode_256k"].replace(batch=2, n_q_heads=4, n_kv_heads=2, block=128,
                                           top_k=5, window=100, plants=2, seq_len=700,
                                           dtype="f32", head_dim=64)
    say("case no-alloc decode: first call b=4 Hq=32 L=8191 (completes a block), bf16 d=128")
    ws_big = _one(big, 8300, seed=11)
    say("case no-alloc decode: second call b=2 Hq=4 L=700, f32 d=64 (smaller)")
    ws_small = _one(small, 900, seed=12)
    assert ws_small < ws_big <= 16 << 20
    say(f"  scratch used: {ws_big} then {ws_small} bytes")


def test_noalloc_decode_rejects_sizes_beyond_scratch():
    # 64 sequences x 64 q-heads x 4096 block slots: 64 MB of scores alone
    p = B.make_params(batch=64, n_q_heads=64, n_kv_heads=8, head_dim=128, seq_len=4096 * 64,
                      block_size=64, top_k=8, window=64)
    assert B.ssa_workspace_size(p, B.SSA_OP_DECODE) > 16 << 20
    got = B.lib().ssa_decode_step_noalloc(ctypes.byref(p), 256, 256, 256, 256, 256, 256, 256, 256, None, 256,
                                          256, None)
    assert got == B.SSA_ERR_UNSUPPORTED, B.status_string(got)
    assert "scratch" in B.lib().ssa_last_error().decode()

"""GPU parity of ssa_sparse_attn_bwd (gradients through the exact attention
over fixed selections) against the oracle's head_backward, evaluated on the
GPU's own selections.

Tolerances (max-abs error over a tensor, relative to that tensor's largest
reference magnitude): float32 inputs 1e-5 (float32 MFMA, float32
accumulation); bfloat16 inputs 2e-3 (K^T, Q^T, dO^T, p and dS enter their
products as float16: 11 significant bits, relative 2^-12 per term).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import content_routed_block_stats_amd as ssa
import oracle as O
from synth_inputs import CONFIGS, make_prefill

pytestmark = pytest.mark.gpu
DEV = "cuda"
REL_TOL = {"f32": 1e-5, "bf16": 2e-3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


_TINY = CONFIGS["tiny_prefill_4k"]
_GQA = CONFIGS["gqa_prefill_128k"]
_P32 = CONFIGS["prefill_32k"]

CASES = {
    "f32_d64_B64": _TINY.replace(seq_len=700, top_k=4, plants=2),
    "bf16_gqa_B256": _GQA.replace(n_q_heads=8, n_kv_heads=2, seq_len=1024 + 96, top_k=3, plants=4),
    "bf16_d64_b2": _P32.replace(batch=2, n_q_heads=4, n_kv_heads=2, seq_len=1500, head_dim=64,
                                block=64, top_k=8, window=64, plants=4),
    "f32_d128_B192_W100": _P32.replace(n_q_heads=4, n_kv_heads=2, seq_len=1000, dtype="f32",
                                       block=192, top_k=2, window=100, plants=2),
    "bf16_B128_W300_ragged": _P32.replace(n_q_heads=2, n_kv_heads=1, seq_len=1000, top_k=4,
                                          window=300, plants=2),
    # 17 key chunks: the last pair of chunks has only its first inside the sequence
    "bf16_gqa_B256_odd_chunks": _GQA.replace(n_q_heads=8, n_kv_heads=2, seq_len=64 * 16 + 30,
                                             top_k=3, plants=4),
    # blocks of 192 keys (not a multiple of 128): one workgroup per 64-key chunk
    "bf16_d128_B192": _P32.replace(n_q_heads=4, n_kv_heads=2, seq_len=900, block=192, top_k=2,
                                   window=100, plants=2),
}


def run(wl, seed=0, top_k=None):
    data = make_prefill(wl, seed=seed)
    Q, K, V = data["Q"].to(DEV), data["K"].to(DEV), data["V"].to(DEV)
    k = wl.top_k if top_k is None else top_k
    mu, sigma = ssa.ssa_block_stats(K, wl.block)
    idx = ssa.ssa_route_topk(Q, mu, sigma, block_size=wl.block, top_k=k, beta=wl.beta)
    Oo, lse = ssa.ssa_sparse_attn_fwd(Q, K, V, idx, block_size=wl.block, window=wl.window,
                                      scale=wl.scale, out_dtype=torch.float32)
    g = torch.Generator(device="cpu").manual_seed(1000 + seed)
    dO = torch.randn(Q.shape, generator=g).to(Q.dtype).to(DEV)
    dQ, dK, dV = ssa.ssa_sparse_attn_bwd(Q, K, V, idx, Oo, lse, dO, block_size=wl.block,
                                         window=wl.window, scale=wl.scale)
    torch.cuda.synchronize()
    return data, idx, dO, dQ, dK, dV


def compare(wl, data, idx, dO, dQ, dK, dV):
    p = O.Params(wl.block, idx.shape[3], wl.window, wl.beta, wl.scale)
    g = wl.group
    idx_h = idx.cpu().numpy()
    worst = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    for b in range(wl.batch):
        for kv in range(wl.n_kv_heads):
            hs = slice(kv * g, (kv + 1) * g)
            rq, rk, rv = O.head_backward(O.as_f64(data["Q"][b, hs]), O.as_f64(data["K"][b, kv]),
                                         O.as_f64(data["V"][b, kv]), idx_h[b, hs], p,
                                         O.as_f64(dO[b, hs].cpu()))
            for name, got, ref in (("dQ", dQ[b, hs], rq), ("dK", dK[b, kv], rk),
                                   ("dV", dV[b, kv], rv)):
                err = np.abs(got.double().cpu().numpy() - ref).max() / max(1e-30, np.abs(ref).max())
                worst[name] = max(worst[name], err)
                assert err <= REL_TOL[wl.dtype], f"{name} relative error {err:.3g} at b={b} kv={kv}"
    say("  relative errors: " + ", ".join(f"{k} {v:.3g}" for k, v in worst.items()))


@pytest.mark.parametrize("name", list(CASES))
def test_backward_parity(name):
    wl = CASES[name]
    say(f"case {name}: b={wl.batch} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} n={wl.seq_len} "
        f"d={wl.head_dim} {wl.dtype} B={wl.block} k={wl.top_k} W={wl.window}")
    compare(wl, *run(wl, seed=3))


def test_backward_window_only():
    """k = 0: gradients of sliding-window attention."""
    wl = CASES["bf16_gqa_B256"]
    say("case backward k=0")
    compare(wl, *run(wl, seed=4, top_k=0))


def test_backward_dense_matches_autograd():
    """k >= nb and W >= B: the gradients of dense causal attention (torch
    autograd on the GPU's own float32 inputs, computed in float64 on the CPU)."""
    wl = CONFIGS["tiny_prefill_4k"].replace(seq_len=300, top_k=8, window=64, plants=2)
    say("case backward dense reduction")
    data, idx, dO, dQ, dK, dV = run(wl, seed=5)
    q = data["Q"][0, 0].double().requires_grad_(True)
    k = data["K"][0, 0].double().requires_grad_(True)
    v = data["V"][0, 0].double().requires_grad_(True)
    s = (q @ k.T) * wl.scale
    s = s.masked_fill(torch.ones_like(s, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.softmax(s, -1) @ v
    (o * dO[0, 0].double().cpu()).sum().backward()
    for name, got, ref in (("dQ", dQ[0, 0], q.grad), ("dK", dK[0, 0], k.grad), ("dV", dV[0, 0], v.grad)):
        err = (got.double().cpu() - ref).abs().max().item() / ref.abs().max().item()
        assert err <= REL_TOL["f32"], f"{name} relative error {err:.3g}"


def test_backward_repeatability():
    """dQ is bitwise repeatable; dK and dV sum a block's rows in dispatch order,
    which follows atomic reservations, so repeated runs agree to rounding."""
    wl = CASES["bf16_gqa_B256"]
    say("case backward repeatability")
    a = run(wl, seed=6)
    b = run(wl, seed=6)
    assert torch.equal(a[3], b[3])
    for x, y in zip(a[4:], b[4:]):
        assert ((x - y).abs().max() / y.abs().max()).item() <= 1e-6

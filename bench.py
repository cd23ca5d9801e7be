#!/usr/bin/env python
"""Throughput of the SSA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --recall-sweep [--workload NAME]

A step is one pass of the prefill hot path over one batch of seeded synthetic
input already resident in HBM: ssa_block_stats -> ssa_route_topk ->
ssa_sparse_attn_fwd.  The default workload is the n = 131072 GQA prefill
(32 q-heads / 8 KV heads, d = 128, bf16, B = 256, k = 16, W = 256, beta = 2).
Prints ONE JSON line: query-tokens/s, per-stage times from HIP events on the
launch stream, the routing kernel against the bf16 MFMA roofline, the gather
against the HBM roofline, the backward through the attention (ssa_sparse_attn_bwd on the step's
selections, against the MFMA roofline), the query-tile-shared variant (ssa_route_tiles +
ssa_tile_attn_fwd on the same workload: its step time, planted recall and the
tile attention against the MFMA roofline), the exact tempered router
(ssa_route_tempered, same workload and beta, outside the step) against the
MFMA roofline, a decode step
on the 32 x 256K-token cache, and the CPU oracle timed on a bounded sample of
the same workload.  --recall-sweep instead prints the planted-target recall of
the centroid, second-cumulant and tempered scores across beta.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0               # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")


def route_flops(wl) -> float:
    """Algorithmic routing flops: (2d^2 + 4d) per (query row, routable block)."""
    n, B, d = wl.seq_len, wl.block, wl.head_dim
    nb = n // B
    # sum over t of min(nb, floor((t+1)/B)), in closed form
    pairs_per_head = B * nb * (nb - 1) // 2 + (n - nb * B + 1) * nb
    return float(wl.batch * wl.n_q_heads * pairs_per_head) * (2 * d * d + 4 * d)


def gather_bytes(wl) -> float:
    """Design HBM bytes of ssa_sparse_attn_fwd with block-major dispatch (the
    bytes this design reads and writes, its own intermediates included).

    Per selected (row, block): the query row (2d bytes, bf16) read by the
    block's task, the fp16 partial written and read back (2 * (2d + 8)), the
    idx entry read twice by the dispatch (8), its sorted entry written and
    read (8) and the partial's position written and read (8).  Per row: the query row for the window pass (2d), the idx row
    (4k), O written (2d) and LSE (4).  Per (sequence, KV head): K and V read
    once for the blocks and once for the windows (4 * n * d * 2).
    """
    n, B, d, k = wl.seq_len, wl.block, wl.head_dim, wl.top_k
    nb = n // B
    sel_per_head = sum(min(k, min(nb, (t + 1) // B)) for t in range(n))
    rows = wl.batch * wl.n_q_heads * n
    sel = wl.batch * wl.n_q_heads * sel_per_head
    per_sel = 2 * d + 2 * (2 * d + 8) + 8 + 8 + 8
    per_row = 2 * d + 4 * k + 2 * d + 4
    kv = wl.batch * wl.n_kv_heads * 4 * n * d * 2
    return float(sel * per_sel + rows * per_row + kv)


def stats_bytes(wl) -> float:
    """Algorithmic HBM bytes of ssa_block_stats: K read once, mu and Sigma written."""
    e = 2 if wl.dtype == "bf16" else 4
    nb = wl.seq_len // wl.block
    heads = wl.batch * wl.n_kv_heads
    return float(heads * (wl.seq_len * wl.head_dim * e + nb * (wl.head_dim + wl.head_dim ** 2) * 4))


def compulsory_gather_bytes(wl) -> float:
    """Bytes ssa_sparse_attn_fwd cannot avoid: Q, K and V read once, idx read
    once, O and LSE written once."""
    e = 2 if wl.dtype == "bf16" else 4
    rows = wl.batch * wl.n_q_heads * wl.seq_len
    return float(rows * wl.head_dim * e * 2 + rows * (4 * wl.top_k + 4)
                 + wl.batch * wl.n_kv_heads * wl.seq_len * wl.head_dim * e * 2)


def kernel_source_digest(*names: str) -> str:
    h = hashlib.sha256()
    for nm in names:
        with open(os.path.join(ROOT, "content_routed_block_stats_amd", "csrc", nm), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counted_traffic(kernel: str, digest: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when the summary is missing, was taken on another workload, or the kernel
    source changed since."""
    path = os.path.join(PROFILES, f"{kernel}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("workload") != workload:
        return None          # counters of another workload's shapes
    if rec.get("source_digest") != digest:
        return None          # the kernel changed since the counters were taken
    return rec.get("hbm_bytes_per_launch")


def counted_mfma_busy(prefix: str, digest: str, workload: str):
    """Share of SIMD cycles with the matrix core busy, from the committed
    rocprofv3 counter summary of the routing kernel (taken on the 128K GQA
    workload), or None for another workload or if the kernel changed."""
    path = os.path.join(PROFILES, "gqa_prefill_128k_mfma_busy.json")
    if workload != "gqa_prefill_128k" or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("route_topk_source_digest") != digest:
        return None
    for name, v in rec.get("kernels", {}).items():
        if name.startswith(prefix):
            return {"busy_frac": round(v["mfma_busy_frac"], 4), "clock_ghz": round(v["clock_ghz"], 3)}
    return None


# -- CPU oracle baseline and dropped mass (worker processes) -------------------

_W: dict = {}


def _cpu_worker_init(folder: str, params: tuple) -> None:
    """Worker start-up: BLAS on one thread, the KV head's arrays memory-mapped
    from the parent's files (shared page cache), the oracle imported."""
    from threadpoolctl import threadpool_limits

    import numpy as np

    import oracle as O

    _W["limits"] = threadpool_limits(limits=1)
    for name in ("K", "V", "mu", "sigma", "q", "t", "sel"):
        _W[name] = np.load(os.path.join(folder, name + ".npy"), mmap_mode="r")
    _W["p"] = O.Params(*params)
    _W["O"] = O


def _cpu_worker_ready(_: int) -> int:
    return int(_W["t"].shape[0])


def _cpu_worker_rows(span: tuple) -> tuple:
    """Rows [i0, i1) of the sample: the oracle's full row (timed), then the
    dropped mass of the GPU's own selection for the row (untimed)."""
    import numpy as np

    O, p = _W["O"], _W["p"]
    K, V, mu, sigma = _W["K"], _W["V"], _W["mu"], _W["sigma"]
    busy, eps = 0.0, []
    for i in range(*span):
        t = int(_W["t"][i])
        q = np.asarray(_W["q"][i])
        t0 = time.perf_counter()
        O.prefill_row(q, K, V, mu, sigma, p, t)
        busy += time.perf_counter() - t0
        S = O.key_set(t, np.asarray(_W["sel"][i]), p.block, p.window)
        eps.append(O.dropped_mass(q, K, S, t, p.scale)[0])
    return busy, eps


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(wl, data, idx, seconds: float, max_workers: int = 16) -> tuple[dict, dict]:
    """The CPU oracle on a bounded sample of the workload, in worker processes
    on the host cores this process may use (at most max_workers), one BLAS
    thread each; also the dropped mass of the GPU's selection on the sampled
    rows.  Returns (cpu_baseline, dropped_mass)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import tempfile

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O

    p = O.Params(wl.block, wl.top_k, wl.window, wl.beta, wl.scale)
    cores = max(1, min(max_workers, len(os.sched_getaffinity(0))))
    rng = np.random.default_rng(0)
    kv, g = 0, wl.group
    Kh = O.as_f64(data["K"][0, kv].cpu())
    Vh = O.as_f64(data["V"][0, kv].cpu())
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        mu, sigma = O.block_stats(Kh, wl.block)
        t_stats = time.perf_counter() - t0
        # one-thread rate on a few rows sizes the sample
        t1 = time.perf_counter()
        probe = 0
        while time.perf_counter() - t1 < 1.0 and probe < 64:
            t = int(rng.integers(0, wl.seq_len))
            O.prefill_row(O.as_f64(data["Q"][0, kv * g, t].cpu()), Kh, Vh, mu, sigma, p, t)
            probe += 1
        per_row_1 = (time.perf_counter() - t1) / probe
    rows = int(min(32768, max(cores * 8, cores * seconds / per_row_1)))
    rows = (rows + cores - 1) // cores * cores
    ts = rng.integers(0, wl.seq_len, size=rows)
    hs = kv * g + rng.integers(0, g, size=rows)
    import torch

    ti = torch.as_tensor(ts, device=data["Q"].device)
    hi = torch.as_tensor(hs, device=data["Q"].device)
    qs = data["Q"][0][hi, ti].double().cpu().numpy()
    sel = idx[0][hi, ti].cpu().numpy()
    with tempfile.TemporaryDirectory(prefix="ssa_bench_") as folder:
        for name, arr in (("K", Kh), ("V", Vh), ("mu", mu), ("sigma", sigma), ("q", qs),
                          ("t", ts), ("sel", sel)):
            np.save(os.path.join(folder, name + ".npy"), np.ascontiguousarray(arr))
        params = (p.block, p.top_k, p.window, p.beta, p.scale)
        # fresh interpreters (spawn): the workers never touch the GPU; a worker
        # that fails breaks the pool (an exception here), it is not restarted
        with cf.ProcessPoolExecutor(cores, mp_context=mp.get_context("spawn"),
                                    initializer=_cpu_worker_init,
                                    initargs=(folder, params)) as pool:
            list(pool.map(_cpu_worker_ready, range(cores)))
            per = rows // cores
            spans = [(i * per, (i + 1) * per) for i in range(cores)]
            t0 = time.perf_counter()
            out = list(pool.map(_cpu_worker_rows, spans))
            wall = time.perf_counter() - t0
    busy = sum(o[0] for o in out)
    eps = np.array([e for o in out for e in o[1]])
    rate_rows = rows / wall                      # rows per second, all workers
    n_rows = wl.batch * wl.n_q_heads * wl.seq_len
    heads = wl.batch * wl.n_kv_heads
    total = math.ceil(heads / cores) * t_stats + n_rows / rate_rows
    total_1 = heads * t_stats + n_rows * (busy / rows)
    base = {
        "value": wl.batch * wl.seq_len / total,
        "unit": "query-tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"block statistics of 1 of {heads} KV heads ({t_stats:.2f} s, one thread) + "
                   f"{rows} query rows of KV head 0 at uniform positions, {cores} worker "
                   f"processes x 1 BLAS thread ({wall:.1f} s wall, {busy / rows * 1e3:.2f} ms "
                   f"per row per worker), NumPy float64; full-job time extrapolated to "
                   f"{total:.0f} s (heads' statistics in parallel rounds of {cores})"),
        "cpu_model": _cpu_model(),
        "host_cpus_available": len(os.sched_getaffinity(0)),
        "value_one_thread": wl.batch * wl.seq_len / total_1,
    }
    dm = {"what": "dropped softmax mass 1 - exp(LSE_S - LSE_full) of the GPU's own selection "
                  "(ssa_route_topk), oracle float64, on the sampled rows",
          "rows": int(eps.size), "mean": float(eps.mean()), "p50": float(np.percentile(eps, 50)),
          "p99": float(np.percentile(eps, 99)), "max": float(eps.max())}
    return base, dm


def bench_decode(steps: int, warmup: int) -> dict:
    """ssa_decode_step on the 32-sequence x 262144-token cache workload."""
    import torch

    import content_routed_block_stats_amd as ssa
    from synth_inputs import CONFIGS, make_decode

    wl = CONFIGS["decode_256k"]
    L = wl.seq_len
    cap = L + 1024
    data = make_decode(wl, seed=0, device="cuda", capacity=cap)
    Kc, Vc = data["K_cache"], data["V_cache"]
    mu, sigma = ssa.ssa_block_stats(Kc, wl.block)
    cache_len = torch.full((wl.batch,), L, dtype=torch.int32, device="cuda")
    q, kn, vn = data["q"], data["k_new"], data["v_new"]
    p = ssa.make_params(batch=wl.batch, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                        head_dim=wl.head_dim, seq_len=cap, block_size=wl.block, top_k=wl.top_k,
                        window=wl.window, beta=wl.beta, scale=wl.scale, in_dtype=q.dtype)
    ws = torch.empty(ssa.ssa_workspace_size(p, 3), dtype=torch.uint8, device="cuda")

    def step():
        ssa.ssa_decode_step(q, kn, vn, Kc, Vc, cache_len, mu, sigma, block_size=wl.block,
                            top_k=wl.top_k, window=wl.window, beta=wl.beta, scale=wl.scale,
                            workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # HBM bytes a step must read: Sigma upper 32x32 tiles (10 of 16 at d=128) and mu of
    # every complete block, plus K and V of the selected blocks and the window
    nbc = (L + 1) // wl.block
    d = wl.head_dim
    tiles = (d // 32) * (d // 32 + 1) // 2
    sig = wl.batch * wl.n_kv_heads * nbc * (tiles * 32 * 32 * 4 + d * 4)
    gat = wl.batch * wl.n_q_heads * (wl.top_k * wl.block + wl.window) * d * 2 * 2
    # exact hierarchical routing of the same queries over the same statistics
    m = 16
    e0.record()
    gs = ssa.ssa_group_stats(mu, sigma, block_size=wl.block, group_blocks=m)
    e1.record()
    torch.cuda.synchronize()
    gs_ms = e0.elapsed_time(e1)
    pos = cache_len.clone()
    hws = torch.empty(ssa.ssa_workspace_size(p, 7), dtype=torch.uint8, device="cuda")
    idx, ev = ssa.ssa_route_hier(q, mu, sigma, *gs, pos, block_size=wl.block, group_blocks=m,
                                 top_k=wl.top_k, beta=wl.beta, want_evaluated=True,
                                 workspace=hws)
    e0.record()
    for _ in range(steps):
        ssa.ssa_route_hier(q, mu, sigma, *gs, pos, block_size=wl.block, group_blocks=m,
                           top_k=wl.top_k, beta=wl.beta, idx=idx, workspace=hws)
    e1.record()
    torch.cuda.synchronize()
    hier_ms = e0.elapsed_time(e1) / steps
    routable = int(((pos.long() + 1) // wl.block).clamp(max=mu.shape[2]).sum()) * wl.n_kv_heads
    scored = int(ev.long().sum())
    del data
    # the same on clustered keys with a topical query (the query leans toward
    # one earlier group; no plants): the case a tree router prunes
    wt = wl.replace(center_std=0.05, noise_std=0.05, group_std=1.0, group_blocks=m, plants=0,
                    query_topic=0.5, topic_span=1024)
    dt_ = make_decode(wt, seed=0, device="cuda", capacity=cap)
    mu_t, sg_t = ssa.ssa_block_stats(dt_["K_cache"], wt.block)
    gs_t = ssa.ssa_group_stats(mu_t, sg_t, block_size=wt.block, group_blocks=m)
    idx_t, ev_t = ssa.ssa_route_hier(dt_["q"], mu_t, sg_t, *gs_t, pos, block_size=wt.block,
                                     group_blocks=m, top_k=wt.top_k, beta=wt.beta,
                                     want_evaluated=True, workspace=hws)
    e0.record()
    for _ in range(steps):
        ssa.ssa_route_hier(dt_["q"], mu_t, sg_t, *gs_t, pos, block_size=wt.block, group_blocks=m,
                           top_k=wt.top_k, beta=wt.beta, idx=idx_t, workspace=hws)
    e1.record()
    torch.cuda.synchronize()
    hier_t_ms = e0.elapsed_time(e1) / steps
    scored_t = int(ev_t.long().sum())
    del dt_, mu_t, sg_t, gs_t
    return {"workload": wl.name, "ms_per_step": round(ms, 4),
            "tokens_per_s": round(wl.batch / (ms * 1e-3), 1),
            "hbm_gbs_algorithmic": round((sig + gat) / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round((sig + gat) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_step": float(sig + gat),
            "traffic": counted_traffic("decode_step", kernel_source_digest("decode.hip",
                                                                           "ssa_common.hpp"),
                                       wl.name),
            "steps": steps,
            "hier_route": {"group_blocks": m, "ms": round(hier_ms, 4),
                           "group_stats_ms_once": round(gs_ms, 3),
                           "blocks_scored_frac": round(scored / max(1, routable), 4),
                           "keys": "standard decode keys (no group structure)",
                           "topical": {"ms": round(hier_t_ms, 4),
                                       "blocks_scored_frac": round(scored_t / max(1, routable), 4),
                                       "keys": "clustered keys, topical query (query_topic 0.5), "
                                               "no plants"}}}


def tempered_flops(wl) -> float:
    """Algorithmic flops of the exact tempered score: 2d per (query row, key of a routable block)."""
    n, B, d = wl.seq_len, wl.block, wl.head_dim
    nb = n // B
    pairs_per_head = B * nb * (nb - 1) // 2 + (n - nb * B + 1) * nb
    return float(wl.batch * wl.n_q_heads * pairs_per_head) * B * 2 * d


def tile_attn_flops(wl, idx_t) -> float:
    """Algorithmic flops of ssa_tile_attn_fwd on its actual selections: 4d per
    (row, key of S(t)), S(t) = the tile's selected blocks + the row's window,
    each key once (window keys inside a selected block counted once)."""
    import torch

    n, B, W, d = wl.seq_len, wl.block, wl.window, wl.head_dim
    dev = idx_t.device
    t = torch.arange(n, device=dev)
    win = torch.clamp(t + 1, max=W).to(torch.float64)            # window keys per row
    total = 0.0
    for b in range(idx_t.shape[0]):
        for h in range(idx_t.shape[1]):
            sel = idx_t[b, h].to(torch.int64)                      # [tiles, k]
            rows_sel = sel[t // B]                                 # [n, k]
            valid = rows_sel >= 0
            lo = torch.maximum(rows_sel * B, (t - W + 1)[:, None])
            hi = torch.minimum(rows_sel * B + B - 1, t[:, None])
            overlap = torch.clamp(hi - lo + 1, min=0) * valid
            keys = valid.sum(-1) * B + win - overlap.sum(-1)
            total += float(keys.sum())
    return 4.0 * d * total


def attn_pairs(wl, idx) -> float:
    """(row, key) pairs of S(t) summed over all rows, on the actual selections:
    the selected blocks' keys plus the window keys outside them."""
    import torch

    n, B, W = wl.seq_len, wl.block, wl.window
    dev = idx.device
    t = torch.arange(n, device=dev)
    win = torch.clamp(t + 1, max=W).to(torch.float64)
    total = 0.0
    for b in range(idx.shape[0]):
        for h in range(idx.shape[1]):
            sel = idx[b, h].to(torch.int64)                       # [n, k]
            valid = sel >= 0
            lo = torch.maximum(sel * B, (t - W + 1)[:, None])
            hi = torch.minimum(sel * B + B - 1, t[:, None])
            overlap = torch.clamp(hi - lo + 1, min=0) * valid
            total += float((valid.sum(-1) * B + win - overlap.sum(-1)).sum())
    return total


def recall_sweep(wl, seed: int, betas: list[float]) -> dict:
    """Planted-target recall of the centroid / second-cumulant / exact tempered
    scores across beta, and how often the cumulant selection agrees with the
    tempered one, on the seeded planted generator (every plant's target row
    asks whether its planted block is selected)."""
    import torch

    import content_routed_block_stats_amd as ssa
    from synth_inputs import make_prefill

    data = make_prefill(wl, seed=seed, device="cuda")
    Q, K = data["Q"], data["K"]
    mu, sigma = ssa.ssa_block_stats(K, wl.block)
    plants = data["plants"]
    pb = torch.tensor([p["b"] for p in plants], device="cuda")
    ph = torch.tensor([p["h"] for p in plants], device="cuda")
    pt = torch.tensor([p["t"] for p in plants], device="cuda")
    pc = torch.tensor([p["block"] for p in plants], device="cuda", dtype=torch.int32)
    # agreement sample: rows with more routable blocks than k
    gen = torch.Generator(device="cpu").manual_seed(seed)
    t_lo = (wl.top_k + 1) * wl.block - 1
    m = 16384
    sb = torch.randint(wl.batch, (m,), generator=gen).cuda()
    sh = torch.randint(wl.n_q_heads, (m,), generator=gen).cuda()
    st = torch.randint(t_lo, wl.seq_len, (m,), generator=gen).cuda()

    def recall(idx):
        return float((idx[pb, ph, pt] == pc[:, None]).any(-1).float().mean())

    rows = []
    for beta in betas:
        idx_c = ssa.ssa_route_topk(Q, mu, sigma, block_size=wl.block, top_k=wl.top_k, beta=beta)
        rec = {"beta": beta, "recall_cumulant": round(recall(idx_c), 4)}
        if beta > 0:
            idx_t = ssa.ssa_route_tempered(Q, K, block_size=wl.block, top_k=wl.top_k, beta=beta)
            a, b_ = idx_c[sb, sh, st], idx_t[sb, sh, st]
            agree = (a[:, :, None] == b_[:, None, :]).any(-1).float().mean()
            rec.update(recall_tempered=round(recall(idx_t), 4),
                       cumulant_vs_tempered_overlap=round(float(agree), 4))
            del idx_t
        del idx_c
        rows.append(rec)
    torch.cuda.synchronize()
    return {"study": "planted recall vs beta", "workload": wl.name, "seed": seed,
            "plants": len(plants), "agreement_rows": m, "centroid_is_beta_0": True,
            "rows": rows}


def hier_prefill_study(wl, m: int, reps: int, seed: int) -> dict:
    """Exact hierarchical routing of the prefill rows (ssa_group_stats +
    ssa_route_hier_prefill, groups of m blocks) beside the flat router
    (ssa_route_topk) on the same inputs, for the standard keys, for
    clustered keys (tight blocks around well separated group centres) and for
    clustered keys with topical queries (each 1024-token segment's queries
    lean toward one earlier group; no planted outliers, whose single far keys
    widen their group's spectral bound for every query): median times, the
    (row, block) scores the visit computed (each listed tile's blocks times
    its 512 rows) over the routable pairs, and whether the selections agree."""
    import statistics

    import torch

    import content_routed_block_stats_amd as ssa
    from synth_inputs import make_prefill

    def timed(fn):
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        return statistics.median(out)

    rows = []
    clustered = wl.replace(center_std=0.05, noise_std=0.05, group_std=1.0, group_blocks=m)
    for keys, w in (("standard", wl), ("clustered", clustered),
                    ("clustered, topical queries",
                     clustered.replace(plants=0, query_topic=0.5, topic_span=1024))):
        data = make_prefill(w, seed=seed, device="cuda")
        Q, K = data["Q"], data["K"]
        del data["V"]
        mu, sigma = ssa.ssa_block_stats(K, w.block)
        b, hq, n, d = Q.shape
        hkv, nb = mu.shape[1], mu.shape[2]
        idx_f = torch.empty((b, hq, n, w.top_k), dtype=torch.int32, device="cuda")
        idx_h = torch.empty_like(idx_f)
        p = ssa.make_params(batch=b, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, seq_len=n,
                            block_size=w.block, top_k=w.top_k, beta=w.beta, in_dtype=Q.dtype)
        ws_f = torch.empty(ssa.ssa_workspace_size(p, 1), dtype=torch.uint8, device="cuda")
        ws_h = torch.empty(ssa.ssa_route_hier_prefill_workspace_size(p, m), dtype=torch.uint8,
                           device="cuda")
        flat = lambda: ssa.ssa_route_topk(Q, mu, sigma, block_size=w.block, top_k=w.top_k,
                                          beta=w.beta, idx=idx_f, workspace=ws_f)
        gs = ssa.ssa_group_stats(mu, sigma, block_size=w.block, group_blocks=m)
        hier = lambda: ssa.ssa_route_hier_prefill(Q, mu, sigma, *gs, block_size=w.block,
                                                  group_blocks=m, top_k=w.top_k, beta=w.beta,
                                                  idx=idx_h, workspace=ws_h)
        flat()
        _, ev = ssa.ssa_route_hier_prefill(Q, mu, sigma, *gs, block_size=w.block, group_blocks=m,
                                           top_k=w.top_k, beta=w.beta, idx=idx_h,
                                           want_evaluated=True, workspace=ws_h)
        torch.cuda.synchronize()
        t_flat = timed(flat)
        t_gs = timed(lambda: ssa.ssa_group_stats(mu, sigma, block_size=w.block, group_blocks=m))
        t_hier = timed(hier)
        g = hq // hkv
        nbk = n // w.block
        # (row, block) pairs routable: sum over positions of min(nb, (t+1)/B), per q-head
        full = max(0, n - nbk * w.block + 1)
        pairs = (w.block * nbk * (nbk - 1) // 2 + full * nbk) * g * b * hkv
        agree = float((idx_f == idx_h).all(-1).float().mean())
        rows.append({"keys": keys, "flat_route_ms": round(t_flat, 3),
                     "group_stats_ms": round(t_gs, 3), "hier_route_ms": round(t_hier, 3),
                     "pairs_scored_frac": round(float(ev.long().sum()) * 512 / max(1, pairs), 4),
                     "rows_equal_to_flat": round(agree, 6)})
        del Q, K, mu, sigma, idx_f, idx_h, ws_f, ws_h, gs, ev, data
        torch.cuda.empty_cache()
    return {"study": "exact hierarchical prefill routing vs the flat router",
            "workload": wl.name, "group_blocks": m, "reps": reps, "rows": rows}


def onbox_peaks() -> dict:
    """The card's own ceilings: the dense bf16 MFMA loop and a streaming read
    of 4 GiB (larger than every cache), medians of 5 timed launches each."""
    import statistics

    import torch

    import content_routed_block_stats_amd as ssa

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        return statistics.median(out)

    wgs, iters = 2048, 5000
    flops = ssa.ssa_probe_mfma_bf16(wgs, 1)[1] * iters
    ms_m = timed(lambda: ssa.ssa_probe_mfma_bf16(wgs, iters))
    buf = torch.ones(1 << 30, dtype=torch.int32, device="cuda")     # 4 GiB
    rwgs = 8192
    out = torch.empty(rwgs * 256, dtype=torch.int32, device="cuda")
    ms_r = timed(lambda: ssa.ssa_probe_hbm_read(buf, rwgs, out))
    nbytes = buf.numel() * 4
    del buf, out
    return {"mfma_bf16_tflops": round(flops / (ms_m * 1e-3) / 1e12, 1),
            "hbm_read_gbs": round(nbytes / (ms_r * 1e-3) / 1e9, 1),
            "how": (f"ssa_probe_mfma_bf16: {wgs} workgroups x 4 waves x {iters} x 16 "
                    "v_mfma_f32_32x32x16_bf16 on 4 chains; ssa_probe_hbm_read: 4 GiB, "
                    f"{rwgs} workgroups x 256 threads x 8 nontemporal 16 B loads in flight; "
                    "medians of 5 launches")}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gqa_prefill_128k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="only the prefill step (no tile-shared, backward or tempered sections)")
    ap.add_argument("--recall-sweep", action="store_true",
                    help="only print the planted-recall-vs-beta study for --workload")
    ap.add_argument("--hier-prefill", action="store_true",
                    help="only the hierarchical-vs-flat prefill routing study for --workload")
    ap.add_argument("--group-blocks", type=int, default=16)
    ap.add_argument("--peaks", action="store_true",
                    help="only measure the on-card bf16 MFMA and HBM read ceilings")
    ap.add_argument("--no-flush", action="store_true",
                    help="do not overwrite a 512 MB buffer (flushing the MALL) before each step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 2 GiB device->device (the reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by independent KV heads and sequences, see the design notes)",
              file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        n = 1 << 31
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n}), flush=True)
        return 0

    if args.peaks:
        print(json.dumps(onbox_peaks()), flush=True)
        return 0

    import statistics

    import content_routed_block_stats_amd as ssa
    from synth_inputs import CONFIGS, make_prefill

    wl = CONFIGS[args.workload]
    if wl.decode:
        print("choose a prefill workload", file=sys.stderr)
        return 2
    if args.hier_prefill:
        print(json.dumps(hier_prefill_study(wl, args.group_blocks, max(3, args.steps // 2),
                                            args.seed)), flush=True)
        return 0
    if args.recall_sweep:
        betas = [0.0, 0.25, 0.5, 1.0, 2.0, 4.0, 8.0, 16.0, 32.0]
        print(json.dumps(recall_sweep(wl, args.seed, betas)), flush=True)
        return 0
    dev = "cuda"
    print(f"[bench] generating {wl.name} on {torch.cuda.get_device_name(0)}", file=sys.stderr,
          flush=True)
    data = make_prefill(wl, seed=args.seed, device=dev)
    Q, K, V = data["Q"], data["K"], data["V"]
    b, hq, n, d = Q.shape
    hkv = K.shape[1]
    nb = n // wl.block
    mu = torch.empty((b, hkv, nb, d), dtype=torch.float32, device=dev)
    sigma = torch.empty((b, hkv, nb, d, d), dtype=torch.float32, device=dev)
    idx = torch.empty((b, hq, n, wl.top_k), dtype=torch.int32, device=dev)
    O = torch.empty((b, hq, n, d), dtype=Q.dtype, device=dev)
    lse = torch.empty((b, hq, n), dtype=torch.float32, device=dev)
    p = ssa.make_params(batch=b, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, seq_len=n,
                        block_size=wl.block, top_k=wl.top_k, window=wl.window, beta=wl.beta,
                        scale=wl.scale, in_dtype=Q.dtype)
    ws_r = torch.empty(ssa.ssa_workspace_size(p, 1), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(ssa.ssa_workspace_size(p, 2), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev:
            ev[0].record()
        ssa.ssa_block_stats(K, wl.block, mu=mu, sigma=sigma)
        if ev:
            ev[1].record()
        ssa.ssa_route_topk(Q, mu, sigma, block_size=wl.block, top_k=wl.top_k, beta=wl.beta,
                           idx=idx, workspace=ws_r)
        if ev:
            ev[2].record()
        ssa.ssa_sparse_attn_fwd(Q, K, V, idx, block_size=wl.block, window=wl.window,
                                scale=wl.scale, out=O, lse=lse, workspace=ws_a)
        if ev:
            ev[3].record()

    # the MALL (256 MB) is flushed before each step by overwriting 512 MB,
    # outside the step's events
    flush_buf = None if args.no_flush else torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def flush():
        if flush_buf is not None:
            flush_buf.fill_(1)

    print("[bench] on-card peaks", file=sys.stderr, flush=True)
    peaks = onbox_peaks()
    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {args.steps} steps", file=sys.stderr, flush=True)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        flush()
        step(evs[i])
    stop.record()
    torch.cuda.synchronize()
    ms_wall = start.elapsed_time(stop) / args.steps
    # medians over the timed steps: the whole step and each stage
    ms = statistics.median(e[0].elapsed_time(e[3]) for e in evs)
    ms_mean = sum(e[0].elapsed_time(e[3]) for e in evs) / args.steps
    st = [statistics.median(e[j].elapsed_time(e[j + 1]) for e in evs) for j in range(3)]
    t_stats, t_route, t_attn = st
    idx_step = idx.clone()     # later stages reuse idx; the dropped mass needs the step's

    rf = route_flops(wl)
    achieved = rf / (t_route * 1e-3) / 1e12
    gb = gather_bytes(wl)
    gbs = gb / (t_attn * 1e-3) / 1e9
    cb = compulsory_gather_bytes(wl)
    pairs = attn_pairs(wl, idx)
    logical = pairs * 2 * wl.head_dim * (2 if wl.dtype == "bf16" else 4)
    route_digest = kernel_source_digest("route_topk.hip", "ssa_common.hpp")
    attn_digest = kernel_source_digest("sparse_attn.hip", "kv_chunks.hpp", "ssa_common.hpp")
    tokens = b * n
    res = {
        "metric": "SSA prefill query-tokens/s at n=128K + % of MFMA/HBM roofline",
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_mean": round(ms_mean, 4),
        "ms_per_step_wall_incl_flush": round(ms_wall, 4),
        "timing": ("medians over the timed steps of HIP events on the launch stream; "
                   + ("a 512 MB buffer overwritten before each step (MALL flush), outside the "
                      "events" if flush_buf is not None else "no cache flush")),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": b, "q_heads": hq, "kv_heads": hkv,
                   "seq_len": n, "head_dim": d, "block": wl.block, "top_k": wl.top_k,
                   "window": wl.window, "beta": wl.beta, "seed": args.seed},
        "stages_ms": {"block_stats": round(t_stats, 4), "route_topk": round(t_route, 4),
                      "sparse_attn_fwd": round(t_attn, 4)},
        "roofline": {"kernel": "route_topk", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "peak_onbox": peaks["mfma_bf16_tflops"],
                     "frac_onbox": round(achieved / peaks["mfma_bf16_tflops"], 4),
                     "traffic": counted_traffic("route_topk", route_digest, wl.name),
                     "mfma_busy_counted": counted_mfma_busy("route_fast_kernel", route_digest, wl.name),
                     "algorithmic_flops_per_launch": rf},
        "roofline_gather": {"kernel": "sparse_attn_fwd", "bound": "hbm", "achieved": round(gbs, 1),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(gbs / HBM_PEAK_GBS, 4),
                            "peak_onbox": peaks["hbm_read_gbs"],
                            "frac_onbox": round(gbs / peaks["hbm_read_gbs"], 4),
                            "traffic": counted_traffic("sparse_attn_fwd", attn_digest, wl.name),
                            "bytes_basis": "design bytes (this design's reads and writes, "
                                           "fp16 partials included)",
                            "design_bytes_per_launch": gb,
                            "compulsory_bytes_per_launch": cb,
                            "compulsory_gbs": round(cb / (t_attn * 1e-3) / 1e9, 1),
                            "effective_gather_gbs": round(logical / (t_attn * 1e-3) / 1e9, 1),
                            "effective_gather_note": ("K and V bytes of every (row, key of S(t)) "
                                                      "pair as a per-row gather would read them, "
                                                      "over the stage time"),
                            # the same stage against the matrix cores: 4d flops
                            # (q.k and p v) per (row, key of S(t)); with large
                            # blocks (the 1M workload) this, not HBM, is the bound
                            "algorithmic_flops_per_launch": pairs * 4 * wl.head_dim,
                            "mfma_tflops": round(pairs * 4 * wl.head_dim / (t_attn * 1e-3) / 1e12, 1),
                            "mfma_frac": round(pairs * 4 * wl.head_dim / (t_attn * 1e-3) / 1e12
                                               / MFMA_BF16_PEAK_TFLOPS, 4)},
        "onbox_peaks": peaks,
        "block_stats": {"kernel": "block_stats", "bound": "alu", "ms": round(t_stats, 4),
                        "algorithmic_bytes_per_launch": stats_bytes(wl),
                        "gbs": round(stats_bytes(wl) / (t_stats * 1e-3) / 1e9, 1),
                        "traffic": counted_traffic("block_stats", kernel_source_digest(
                            "block_stats.hip", "ssa_common.hpp"), wl.name)},
    }
    if not args.step_only:
        # the query-tile-shared variant: one selection per tile of B positions
        tiles = (n + wl.block - 1) // wl.block
        idx_t = torch.empty((b, hq, tiles, wl.top_k), dtype=torch.int32, device=dev)
        ws_rt = torch.empty(ssa.ssa_workspace_size(p, 4), dtype=torch.uint8, device=dev)
        ws_ta = torch.empty(ssa.ssa_workspace_size(p, 5), dtype=torch.uint8, device=dev)

        def tile_step(ev=None):
            if ev:
                ev[0].record()
            ssa.ssa_block_stats(K, wl.block, mu=mu, sigma=sigma)
            if ev:
                ev[1].record()
            ssa.ssa_route_tiles(Q, mu, sigma, block_size=wl.block, top_k=wl.top_k, beta=wl.beta,
                                idx=idx_t, workspace=ws_rt)
            if ev:
                ev[2].record()
            ssa.ssa_tile_attn_fwd(Q, K, V, idx_t, block_size=wl.block, window=wl.window,
                                  scale=wl.scale, out=O, lse=lse, workspace=ws_ta)
            if ev:
                ev[3].record()

        tile_step()
        torch.cuda.synchronize()
        treps = max(3, args.steps // 2)
        tevs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(treps)]
        for i in range(treps):
            tile_step(tevs[i])
        torch.cuda.synchronize()
        tst = [sum(e[j].elapsed_time(e[j + 1]) for e in tevs) / treps for j in range(3)]
        t_tile = sum(tst)
        ta_fl = tile_attn_flops(wl, idx_t)
        ta_tf = ta_fl / (tst[2] * 1e-3) / 1e12
        plants = data["plants"]
        pb = torch.tensor([q["b"] for q in plants], device=dev)
        ph = torch.tensor([q["h"] for q in plants], device=dev)
        pt = torch.tensor([q["t"] for q in plants], device=dev)
        pc = torch.tensor([q["block"] for q in plants], device=dev, dtype=torch.int32)
        rec_tile = float((idx_t[pb, ph, pt // wl.block] == pc[:, None]).any(-1).float().mean())
        rec_row = float((idx[pb, ph, pt] == pc[:, None]).any(-1).float().mean())
        res["tile_routed"] = {
            "what": "one selection per query tile of B positions (summed routing score), same workload",
            "ms_per_step": round(t_tile, 4), "value": round(tokens / (t_tile * 1e-3), 1),
            "unit": "query-tokens/s", "speedup_vs_per_query": round(ms / t_tile, 3),
            "stages_ms": {"block_stats": round(tst[0], 4), "route_tiles": round(tst[1], 4),
                          "tile_attn_fwd": round(tst[2], 4)},
            "planted_recall": round(rec_tile, 4), "planted_recall_per_query": round(rec_row, 4),
            "roofline": {"kernel": "tile_attn", "bound": "mfma", "achieved": round(ta_tf, 1),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ta_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": counted_traffic("tile_attn", kernel_source_digest(
                             "tile_attn.hip", "kv_chunks.hpp", "ssa_common.hpp"), wl.name),
                         "algorithmic_flops_per_launch": ta_fl},
            "steps": treps}
        del ws_rt, ws_ta, idx_t

        # the backward through the attention with the step's selections (training);
        # the tile-shared step above overwrote O and lse, so the forward runs again
        ssa.ssa_sparse_attn_fwd(Q, K, V, idx, block_size=wl.block, window=wl.window, scale=wl.scale,
                                out=O, lse=lse, workspace=ws_a)
        dO = torch.randn(Q.shape, generator=torch.Generator(device=dev).manual_seed(7), device=dev,
                         dtype=torch.float32).to(Q.dtype)
        ws_b = torch.empty(ssa.ssa_workspace_size(p, 6), dtype=torch.uint8, device=dev)
        bwd = lambda: ssa.ssa_sparse_attn_bwd(Q, K, V, idx, O, lse, dO, block_size=wl.block,
                                              window=wl.window, scale=wl.scale, workspace=ws_b)
        bwd()
        torch.cuda.synchronize()
        tb0, tb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        breps = 2
        tb0.record()
        for _ in range(breps):
            bwd()
        tb1.record()
        torch.cuda.synchronize()
        t_bwd = tb0.elapsed_time(tb1) / breps
        bwd_fl = 14.0 * wl.head_dim * pairs
        res["backward"] = {"what": "dQ, dK, dV through the attention over the step's selections",
                           "ms": round(t_bwd, 3), "ms_vs_forward_attention": round(t_bwd / t_attn, 2),
                           "bound": "mfma", "achieved": round(bwd_fl / (t_bwd * 1e-3) / 1e12, 1),
                           "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(bwd_fl / (t_bwd * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                           "algorithmic_flops_per_launch": bwd_fl, "reps": breps,
                           "traffic_dkv_kernel": counted_traffic("attn_bwd_dkv", kernel_source_digest(
                               "attn_bwd.hip", "kv_chunks.hpp", "ssa_common.hpp"), wl.name)}
        del ws_b, dO

        # the exact tempered score (same workload and beta), outside the step
        ssa.ssa_route_tempered(Q, K, block_size=wl.block, top_k=wl.top_k, beta=wl.beta, idx=idx)
        te0, te1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        te0.record()
        for _ in range(reps):
            ssa.ssa_route_tempered(Q, K, block_size=wl.block, top_k=wl.top_k, beta=wl.beta, idx=idx)
        te1.record()
        torch.cuda.synchronize()
        t_temp = te0.elapsed_time(te1) / reps
        tf = tempered_flops(wl) / (t_temp * 1e-3) / 1e12
        res["tempered_route"] = {"kernel": "tempered_route", "ms": round(t_temp, 3), "bound": "mfma",
                                 "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                                 "traffic": counted_traffic("tempered_route", kernel_source_digest(
                                     "tempered_route.hip", "kv_chunks.hpp", "ssa_common.hpp"),
                                     wl.name),
                                 "algorithmic_flops_per_launch": tempered_flops(wl), "reps": reps}
    del O, lse, ws_a, ws_r
    if not args.no_decode:
        print("[bench] decode step", file=sys.stderr, flush=True)
        res["decode"] = bench_decode(steps=max(5, args.steps), warmup=2)
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"], res["dropped_mass"] = cpu_baseline(wl, data, idx_step,
                                                                args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

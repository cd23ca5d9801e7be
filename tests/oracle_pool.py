"""The oracle over many sampled rows of one (sequence, KV head), in worker
processes (fresh interpreters that never touch the GPU), for the full-size
parity tests.

The parent hands each head's keys and values (float64) and the oracle's own
block statistics to the workers through files they memory-map (one copy in
the page cache, shared by every worker); each task is a chunk of rows with the GPU's results for
them.  Per row a worker runs the oracle's prefill row, checks the GPU's
selection under R1, its O and LSE under R2/R3 on the GPU's own selection
(R6), and computes the dropped softmax mass of that selection.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import shutil
import tempfile

import numpy as np

_HEAD: dict = {}


def _init() -> None:
    from threadpoolctl import threadpool_limits

    _HEAD["limits"] = threadpool_limits(limits=1)


def _load(folder: str) -> dict:
    if _HEAD.get("folder") != folder:
        _HEAD["folder"] = folder
        for name in ("K", "V", "mu", "sigma"):
            _HEAD[name] = np.load(os.path.join(folder, name + ".npy"), mmap_mode="r")
    return _HEAD


def _rows(folder: str, params: tuple, rows: list) -> list:
    import oracle as O
    from parity import attn_errors, idx_ok

    h = _load(folder)
    p = O.Params(*params)
    K, V, mu, sigma = h["K"], h["V"], h["mu"], h["sigma"]
    out = []
    for r in rows:
        q = O.as_f64(r["q"])
        row = O.prefill_row(q, K, V, mu, sigma, p, r["t"])
        ok, exact = idx_ok(r["idx"], row)
        res = dict(key=r["key"], t=r["t"], ok=ok, exact=exact, oracle_idx=row["idx"].tolist())
        for name, (Og, lse, bf16_out) in r["outputs"].items():
            eo, el = attn_errors(Og, lse, q, K, V, r["idx"], r["t"], p, bf16_out=bf16_out)
            res["O_err_" + name], res["lse_err_" + name] = eo, el
        S = O.key_set(r["t"], np.asarray(r["idx"]), p.block, p.window)
        res["eps"] = O.dropped_mass(q, K, S, r["t"], p.scale)[0]
        out.append(res)
    return out


class OraclePool:
    """Worker processes (at most `workers`, at most the cores this process may
    use) and a scratch folder; use as a context manager."""

    def __init__(self, params: tuple, workers: int = 16, chunk: int = 32):
        self.params = params
        self.chunk = chunk
        self.workers = max(1, min(workers, len(os.sched_getaffinity(0))))
        self.dir = tempfile.mkdtemp(prefix="ssa_oracle_")
        self.pool = cf.ProcessPoolExecutor(self.workers, mp_context=mp.get_context("spawn"),
                                           initializer=_init)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.pool.shutdown(wait=True, cancel_futures=True)
        shutil.rmtree(self.dir, ignore_errors=True)
        return False

    def run_head(self, name: str, K: np.ndarray, V: np.ndarray, mu: np.ndarray,
                 sigma: np.ndarray, rows: list) -> list:
        """rows: dicts with key, t, q, idx (the GPU's row) and outputs
        {label: (O row, lse, bf16_out)}.  Returns one result dict per row."""
        folder = os.path.join(self.dir, name)
        os.makedirs(folder, exist_ok=True)
        for nm, arr in (("K", K), ("V", V), ("mu", mu), ("sigma", sigma)):
            np.save(os.path.join(folder, nm + ".npy"), np.ascontiguousarray(arr))
        futs = [self.pool.submit(_rows, folder, self.params, rows[i:i + self.chunk])
                for i in range(0, len(rows), self.chunk)]
        out = [r for f in futs for r in f.result()]
        shutil.rmtree(folder, ignore_errors=True)
        return out

"""Acceptance rules for comparing the HIP path with the CPU oracle.

  R1  selected block sets equal per row, except for blocks whose oracle score
      lies within 1e-5 relative of the oracle's k-th score (near ties, where
      more than one selection is correct);
  R2  O max-abs error <= 1e-5 for float32 inputs, <= 2e-3 for bfloat16 inputs
      (float32 accumulation).  A bfloat16 OUTPUT is additionally allowed its
      own rounding, half a bfloat16 ulp of the exact value (2e-3 is below that
      half-ulp once |O| >= 0.5, where no bf16 tensor could meet it);
  R3  LSE max-abs error <= 1e-4;
  R4  block statistics max-abs error <= 1e-5 * max|Sigma| (float32 sums over B
      keys of O(1) values: ~B * 2^-24 relative worst case, 1e-5 covers B <= 1024
      with margin while a wrong term or index is off by O(|Sigma|));
  R6  O and LSE are compared against the oracle evaluated on the GPU's own
      selection, so an allowed tie cannot turn into an output failure.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import attend, key_set

TIE_REL = 1e-5
O_TOL = {"f32": 1e-5, "bf16": 2e-3}
LSE_TOL = 1e-4
STATS_REL = 1e-5


def idx_ok(gpu_row: np.ndarray, orc: dict, tie_rel: float = TIE_REL) -> tuple[bool, bool]:
    """(passes R1, exact match) for one row; orc is an oracle prefill_row result."""
    g = set(int(c) for c in gpu_row if c >= 0)
    o = set(int(c) for c in orc["idx"] if c >= 0)
    # layout: ascending, -1 only as padding at the end
    lst = [int(c) for c in gpu_row]
    valid = [c for c in lst if c >= 0]
    if valid != sorted(valid) or len(valid) != len(set(valid)):
        return False, False
    if any(c >= 0 for c in lst[len(valid):]):
        return False, False
    if len(g) != len(o):
        return False, False
    if g == o:
        return True, True
    r = orc["scores"]
    rk, rk1 = orc["r_k"], orc["r_k1"]
    band = tie_rel * max(abs(rk), abs(rk1) if not math.isnan(rk1) else 0.0)
    for c in g ^ o:
        if c >= len(r) or abs(r[c] - rk) > band:
            return False, False
    return True, False


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bfloat16 ulp at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.ldexp(1.0, np.floor(np.log2(ax)).astype(int) - 8)


def attn_errors(gpu_O: np.ndarray, gpu_lse: float, q, K, V, gpu_idx, t: int, p,
                bf16_out: bool = False) -> tuple[float, float]:
    """O error (beyond a bf16 output's own rounding) and LSE error of one row,
    against the oracle evaluated on the GPU's selection."""
    S = key_set(t, np.asarray(gpu_idx), p.block, p.window)
    O, lse = attend(q, K, V, S, p.scale)
    err = np.abs(np.asarray(gpu_O, np.float64) - O)
    if bf16_out:
        err = np.maximum(err - bf16_half_ulp(O), 0.0)
    return float(err.max()), abs(float(gpu_lse) - lse)


def check_idx_properties(idx: np.ndarray, n: int, B: int, k: int) -> None:
    """Properties every selection has at any size: ascending, distinct, routable,
    exactly min(k, #routable) entries, -1 padding at the end.  idx: [rows, n, k]."""
    t = np.arange(n)
    routable = np.minimum((t + 1) // B, n // B)
    want = np.minimum(k, routable)                               # [n]
    valid = idx >= 0
    cnt = valid.sum(-1)                                          # [rows, n]
    assert np.array_equal(cnt, np.broadcast_to(want, cnt.shape)), "wrong number of selections"
    pos = np.arange(k)
    assert np.all(valid == (pos[None, None, :] < cnt[..., None])), "-1 padding not at the end"
    big = np.where(valid, idx, np.iinfo(np.int32).max)
    assert np.all(np.diff(big, axis=-1)[..., :] >= 0) and np.all(
        (np.diff(big, axis=-1) > 0) | ~valid[..., 1:]), "not ascending / not distinct"
    assert np.all(np.where(valid, idx < routable[None, :, None], True)), "non-routable block selected"


def check_tile_properties(idx: np.ndarray, n: int, B: int, k: int) -> None:
    """Every tile: ascending distinct blocks before the tile, min(k, min(j, nb))
    of them, -1 padding at the end.  idx: [rows, tiles, k]."""
    nb = n // B
    tiles = idx.shape[-2]
    want = np.minimum(k, np.minimum(np.arange(tiles), nb))
    valid = idx >= 0
    assert np.array_equal(valid.sum(-1), np.broadcast_to(want, valid.shape[:-1]))
    assert np.all(valid == (np.arange(k) < want[:, None]))
    big = np.where(valid, idx, np.iinfo(np.int32).max)
    assert np.all((np.diff(big, axis=-1) > 0) | ~valid[..., 1:])
    assert np.all(np.where(valid, idx < np.arange(tiles)[:, None], True))

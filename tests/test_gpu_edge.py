"""GPU edge cases through the C ABI: exact ties and non-finite inputs.

Exact ties.  Blocks whose keys are bitwise copies of one another have
bitwise-equal statistics, so every query scores them equally; the documented
rule is that ties go to the lower block index.  The tie band of rule R1 would
accept either member of such a group, so these tests check the rule itself:
among a group's routable members the selected ones are always the lowest.

Non-finite inputs.  NaN and Inf in Q, K or a decode query must reach the
outputs of the rows whose arithmetic they enter (the oracle, evaluated on the
GPU's own selection, says which rows and which elements), never fault, and
leave every other row as it would be.  A block whose statistics are not finite
scores NaN for every query and is never selected; every selection keeps its
layout (ascending, distinct, routable, -1 padding last).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import content_routed_block_stats_amd as ssa
import oracle as O
from parity import LSE_TOL, O_TOL, bf16_half_ulp, idx_ok
from synth_inputs import CONFIGS, make_decode, make_prefill

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _params(wl):
    return O.Params(wl.block, wl.top_k, wl.window, wl.beta, wl.scale)


def _layout_ok(row: np.ndarray, C: int) -> bool:
    """Ascending distinct routable blocks, then -1 padding."""
    lst = [int(c) for c in row]
    valid = [c for c in lst if c >= 0]
    return (valid == sorted(valid) and len(valid) == len(set(valid))
            and all(c < C for c in valid) and all(c == -1 for c in lst[len(valid):]))


def _lowest_members(sel: set, group: list[int], C: int) -> bool:
    """The selected members of a group of identical blocks are its lowest routable ones."""
    routable = sorted(c for c in group if c < C)
    chosen = sorted(c for c in routable if c in sel)
    return chosen == routable[:len(chosen)]


# ----------------------------------------------------------------- exact ties --

# groups of identical blocks: the source block's keys are scaled so the group
# outscores ordinary blocks for most queries (its variance term is larger)
TIE_GROUPS = [([3, 9, 17, 30], 2.0), ([4, 12, 25], 1.6), ([6, 7], 1.3)]


def _tie_prefill(wl, seed=0):
    data = make_prefill(wl, seed=seed)
    K = data["K"]
    B = wl.block
    for members, gain in TIE_GROUPS:
        src = members[0]
        blk = (K[:, :, src * B:(src + 1) * B].float() * gain).to(K.dtype)
        for c in members:
            K[:, :, c * B:(c + 1) * B] = blk
    return data


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_exact_ties_prefill_route(dtype):
    wl = CONFIGS["gqa_prefill_128k"].replace(n_q_heads=4, n_kv_heads=2, seq_len=2048 + 100,
                                             block=64, top_k=5, window=64, plants=0, dtype=dtype)
    say(f"case exact ties prefill {dtype}: n={wl.seq_len} B={wl.block} k={wl.top_k}")
    data = _tie_prefill(wl)
    Q, K = data["Q"].to(DEV), data["K"].to(DEV)
    mu, sigma = ssa.ssa_block_stats(K, wl.block)
    idx = ssa.ssa_route_topk(Q, mu, sigma, block_size=wl.block, top_k=wl.top_k, beta=wl.beta)
    torch.cuda.synchronize()
    for members, _ in TIE_GROUPS:   # the statistics of a group are bitwise equal
        for c in members[1:]:
            assert torch.equal(mu[:, :, c], mu[:, :, members[0]])
            assert torch.equal(sigma[:, :, c], sigma[:, :, members[0]])
    idx_h = idx.cpu().numpy()
    orc = O.PrefillOracle(data["Q"], data["K"], data["V"], _params(wl))
    n_tied = 0
    for h in range(wl.n_q_heads):
        for t in range(0, wl.seq_len, 3):
            row = orc.row(0, h, t)
            ok, _ = idx_ok(idx_h[0, h, t], row)
            assert ok, f"selection mismatch at {(h, t)}: {idx_h[0, h, t]} vs {row['idx']}"
            sel = set(int(c) for c in idx_h[0, h, t] if c >= 0)
            C = len(row["scores"])
            for members, _ in TIE_GROUPS:
                routable = [c for c in members if c < C]
                picked = [c for c in routable if c in sel]
                n_tied += 0 < len(picked) < len(routable)
                assert _lowest_members(sel, members, C), \
                    f"tie not broken to the lower block at {(h, t)}: {sorted(sel)} group {members}"
            # the oracle's own selection obeys the same rule (a check of the case;
            # only where its float64 arithmetic is exact: for float32 keys the
            # library products round in an order that depends on the slice)
            if dtype == "bf16":
                assert all(_lowest_members(set(row["idx"].tolist()), m, C) for m, _ in TIE_GROUPS)
    say(f"  rows with a group split by the tie rule: {n_tied}")
    assert n_tied > 100, "the case does not exercise ties"


def test_exact_ties_tempered_route():
    wl = CONFIGS["gqa_prefill_128k"].replace(n_q_heads=4, n_kv_heads=2, seq_len=2048 + 100,
                                             block=64, top_k=5, window=64, plants=0)
    say("case exact ties tempered routing")
    data = _tie_prefill(wl, seed=3)
    idx = ssa.ssa_route_tempered(data["Q"].to(DEV), data["K"].to(DEV), block_size=wl.block,
                                 top_k=wl.top_k, beta=1.0)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    n_tied = 0
    for h in range(wl.n_q_heads):
        kv = h // wl.group
        for t in range(0, wl.seq_len, 5):
            row = O.tempered_row(O.as_f64(data["Q"][0, h, t]), O.as_f64(data["K"][0, kv]),
                                 wl.block, wl.top_k, 1.0, t)
            ok, _ = idx_ok(idx_h[0, h, t], row)
            assert ok, f"selection mismatch at {(h, t)}"
            sel = set(int(c) for c in idx_h[0, h, t] if c >= 0)
            C = len(row["scores"])
            for members, _ in TIE_GROUPS:
                routable = [c for c in members if c < C]
                n_tied += 0 < len([c for c in routable if c in sel]) < len(routable)
                assert _lowest_members(sel, members, C), f"tie at {(h, t)}: {sorted(sel)}"
    say(f"  rows with a group split by the tie rule: {n_tied}")
    assert n_tied > 50


# Decode keeps one sorted list per lane over the blocks c = lane, lane + 64,
# ...: a group of identical blocks in one lane (3, 67, 131, 195) with a
# stronger block arriving after them in that lane (259) must keep its order
# when the stronger block pushes through it.
DEC_GROUPS = [([3, 67, 131, 195], 1.6), ([4, 12, 25], 1.4)]
DEC_PUSHER = (259, 2.2)


def test_exact_ties_decode():
    wl = CONFIGS["decode_256k"].replace(batch=2, n_q_heads=8, n_kv_heads=2, block=64, top_k=4,
                                        window=64, plants=0, seq_len=64 * 300 + 20)
    say("case exact ties decode: 300 blocks, a tied group inside one lane's list")
    data = make_decode(wl, seed=4, capacity=64 * 300 + 100)
    Kc = data["K_cache"]
    B = wl.block
    for members, gain in DEC_GROUPS:
        blk = (Kc[:, :, members[0] * B:(members[0] + 1) * B].float() * gain).to(Kc.dtype)
        for c in members:
            Kc[:, :, c * B:(c + 1) * B] = blk
    c, gain = DEC_PUSHER
    Kc[:, :, c * B:(c + 1) * B] = (Kc[:, :, c * B:(c + 1) * B].float() * gain).to(Kc.dtype)
    Kd, Vd = Kc.to(DEV), data["V_cache"].to(DEV)
    mu, sigma = ssa.ssa_block_stats(Kd, B)
    cl = torch.full((wl.batch,), wl.seq_len, dtype=torch.int32, device=DEV)
    o, lse, idx = ssa.ssa_decode_step(data["q"].to(DEV), data["k_new"].to(DEV),
                                      data["v_new"].to(DEV), Kd, Vd, cl, mu, sigma, block_size=B,
                                      top_k=wl.top_k, window=wl.window, beta=wl.beta,
                                      scale=wl.scale, return_idx=True)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    p = _params(wl)
    n_tied = 0
    for b in range(wl.batch):
        for h in range(wl.n_q_heads):
            kv = h // wl.group
            row = O.decode_step(data["q"][b, h], data["k_new"][b, kv], data["v_new"][b, kv],
                                Kc[b, kv], data["V_cache"][b, kv], wl.seq_len, p)
            ok, _ = idx_ok(idx_h[b, h], row)
            assert ok, f"decode selection mismatch at {(b, h)}"
            sel = set(int(c) for c in idx_h[b, h] if c >= 0)
            C = len(row["scores"])
            for members, _ in DEC_GROUPS:
                routable = [c for c in members if c < C]
                n_tied += 0 < len([c for c in routable if c in sel]) < len(routable)
                assert _lowest_members(sel, members, C), f"decode tie at {(b, h)}: {sorted(sel)}"
            assert all(_lowest_members(set(row["idx"].tolist()), m, C) for m, _ in DEC_GROUPS)
    say(f"  rows with a group split by the tie rule: {n_tied}")
    assert n_tied > 0


# ---------------------------------------------------------- non-finite inputs --

def _out_matches(gpu_o: np.ndarray, gpu_lse: float, ref_o: np.ndarray, ref_lse: float,
                 tol: float, bf16_out: bool) -> bool:
    """Non-finite where the oracle is non-finite (NaN for NaN, the same Inf for
    Inf), within tolerance where it is finite."""
    if np.isnan(ref_lse) != np.isnan(gpu_lse):
        return False
    if not np.isnan(ref_lse) and (np.isinf(ref_lse) or np.isinf(gpu_lse)):
        if ref_lse != gpu_lse:
            return False
    elif not np.isnan(ref_lse) and abs(gpu_lse - ref_lse) > LSE_TOL:
        return False
    if not np.array_equal(np.isnan(gpu_o), np.isnan(ref_o)):
        return False
    fin = np.isfinite(ref_o)
    if not np.array_equal(np.isfinite(gpu_o), fin):
        return False
    if not np.array_equal(gpu_o[~fin & ~np.isnan(ref_o)], ref_o[~fin & ~np.isnan(ref_o)]):
        return False
    err = np.abs(gpu_o[fin] - ref_o[fin])
    if bf16_out:
        err = np.maximum(err - bf16_half_ulp(ref_o[fin]), 0.0)
    return err.size == 0 or float(err.max()) <= tol


def test_nonfinite_prefill():
    wl = CONFIGS["gqa_prefill_128k"].replace(n_q_heads=8, n_kv_heads=2, seq_len=2048 + 37,
                                             block=64, top_k=6, window=64, plants=4)
    say(f"case non-finite prefill: n={wl.seq_len} B={wl.block} k={wl.top_k}")
    data = make_prefill(wl, seed=6)
    Qh, Kh = data["Q"], data["K"]
    nan_row = (1, 700)            # (q-head, t): one NaN element
    inf_row = (6, 1500)           # (q-head, t): one +Inf element
    Qh[0, nan_row[0], nan_row[1], 5] = float("nan")
    Qh[0, inf_row[0], inf_row[1], 17] = float("inf")
    inf_key = (1, 1000, 40)       # (KV head, position, element) of a +Inf key
    Kh[0, inf_key[0], inf_key[1], inf_key[2]] = float("inf")
    Q, K, V = Qh.to(DEV), Kh.to(DEV), data["V"].to(DEV)
    mu, sigma = ssa.ssa_block_stats(K, wl.block)
    idx = ssa.ssa_route_topk(Q, mu, sigma, block_size=wl.block, top_k=wl.top_k, beta=wl.beta)
    Oo, lse = ssa.ssa_sparse_attn_fwd(Q, K, V, idx, block_size=wl.block, window=wl.window,
                                      scale=wl.scale)
    torch.cuda.synchronize()
    idx_h, Og, lg = idx.cpu().numpy(), Oo.float().cpu().numpy(), lse.cpu().numpy()
    p = _params(wl)
    orc = O.PrefillOracle(Qh, Kh, data["V"], p)
    bad_block = inf_key[1] // wl.block
    n_nonfinite = n_rows = 0
    for h in range(wl.n_q_heads):
        kv = h // wl.group
        Kf, Vf, _, _ = orc.head(0, kv)
        for t in range(wl.seq_len):
            row = orc.row(0, h, t)
            C = len(row["scores"])
            sel = idx_h[0, h, t]
            assert _layout_ok(sel, C), f"layout at {(h, t)}: {sel}"
            finite = np.isfinite(row["scores"])
            q_finite = (h, t) not in (nan_row, inf_row)
            if q_finite:   # with a finite query only blocks with non-finite statistics score NaN
                assert not any(np.isnan(row["scores"][c]) for c in sel if c >= 0), \
                    f"NaN-scored block chosen at {(h, t)}"
            if finite.all():
                ok, _ = idx_ok(sel, row)
                assert ok, f"selection mismatch at {(h, t)}: {sel} vs {row['idx']}"
            elif (h, t) == nan_row:
                assert np.all(sel == -1), "a NaN query must select no block"
            # outputs: the oracle on the GPU's own selection
            S = O.key_set(t, sel, wl.block, wl.window)
            with np.errstate(invalid="ignore", over="ignore"):
                ref_o, ref_l = O.attend(O.as_f64(Qh[0, h, t]), Kf, Vf, S, wl.scale)
            ok = _out_matches(Og[0, h, t], float(lg[0, h, t]), ref_o, ref_l, O_TOL["bf16"], True)
            assert ok, (f"output at {(h, t)}: gpu lse {lg[0, h, t]} ref {ref_l}, "
                        f"gpu nan {np.isnan(Og[0, h, t]).sum()} ref nan {np.isnan(ref_o).sum()}")
            n_nonfinite += not np.isfinite(ref_l)
            n_rows += 1
            if (h, t) in (nan_row, inf_row):
                assert np.isnan(lg[0, h, t]) and np.isnan(Og[0, h, t]).all()
            if kv == inf_key[0] and C > bad_block:
                assert not np.isfinite(row["scores"][bad_block])
    say(f"  rows {n_rows}, rows with a non-finite result {n_nonfinite}")
    assert n_nonfinite >= 2


def test_nonfinite_decode():
    wl = CONFIGS["decode_256k"].replace(batch=3, n_q_heads=4, n_kv_heads=2, block=64, top_k=6,
                                        window=64, plants=2, seq_len=1023)
    say("case non-finite decode: NaN query, Inf appended key completing a block")
    data = make_decode(wl, seed=8, capacity=1100)
    q, kn = data["q"].clone(), data["k_new"].clone()
    q[0, 1, 3] = float("nan")
    kn[2, 1, 9] = float("inf")    # sequence 2, KV head 1: completes block 15
    Kd, Vd = data["K_cache"].to(DEV), data["V_cache"].to(DEV)
    mu, sigma = ssa.ssa_block_stats(Kd, wl.block)
    cl = torch.full((wl.batch,), wl.seq_len, dtype=torch.int32, device=DEV)
    o, lse, idx = ssa.ssa_decode_step(q.to(DEV), kn.to(DEV), data["v_new"].to(DEV), Kd, Vd, cl,
                                      mu, sigma, block_size=wl.block, top_k=wl.top_k,
                                      window=wl.window, beta=wl.beta, scale=wl.scale,
                                      return_idx=True)
    torch.cuda.synchronize()
    assert cl.cpu().tolist() == [wl.seq_len + 1] * wl.batch
    idx_h, og, lg = idx.cpu().numpy(), o.float().cpu().numpy(), lse.cpu().numpy()
    p = _params(wl)
    L = wl.seq_len
    for b in range(wl.batch):
        for h in range(wl.n_q_heads):
            kv = h // wl.group
            with np.errstate(invalid="ignore", over="ignore"):
                row = O.decode_step(q[b, h], kn[b, kv], data["v_new"][b, kv],
                                    data["K_cache"][b, kv], data["V_cache"][b, kv], L, p)
            C = len(row["scores"])
            sel = idx_h[b, h]
            assert _layout_ok(sel, C), f"decode layout at {(b, h)}: {sel}"
            finite = np.isfinite(row["scores"])
            assert not any(np.isnan(row["scores"][c]) for c in sel if c >= 0)
            if finite.all():
                ok, _ = idx_ok(sel, row)
                assert ok, f"decode selection mismatch at {(b, h)}"
            if (b, h) == (0, 1):
                assert np.all(sel == -1), "a NaN query must select no block (-1 padding)"
                assert np.isnan(lg[b, h]) and np.isnan(og[b, h]).all()
            Kfull = np.concatenate([O.as_f64(data["K_cache"][b, kv, :L]), O.as_f64(kn[b, kv])[None]])
            Vfull = np.concatenate([O.as_f64(data["V_cache"][b, kv, :L]),
                                    O.as_f64(data["v_new"][b, kv])[None]])
            S = O.key_set(L, sel, wl.block, wl.window)
            with np.errstate(invalid="ignore", over="ignore"):
                ref_o, ref_l = O.attend(O.as_f64(q[b, h]), Kfull, Vfull, S, wl.scale)
            assert _out_matches(og[b, h], float(lg[b, h]), ref_o, ref_l, O_TOL["bf16"], True), \
                f"decode output at {(b, h)}: gpu lse {lg[b, h]} ref {ref_l}"
    # the Inf key's block got non-finite statistics, the others stayed finite
    assert not torch.isfinite(sigma[2, 1, 15]).all()
    assert torch.isfinite(sigma[:2]).all() and torch.isfinite(sigma[2, 0]).all()

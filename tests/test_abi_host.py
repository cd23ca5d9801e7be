"""The C ABI on the host (no GPU): the library loads, exports every function
the headers under include/ declare, and rejects invalid arguments before
touching a device."""
import ctypes
import glob
import os
import re

import pytest
import torch

import content_routed_block_stats_amd as ssa
from content_routed_block_stats_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(ssa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = ssa.lib()
    names = _declared_functions()
    assert {"ssa_block_stats", "ssa_route_topk", "ssa_sparse_attn_fwd", "ssa_decode_step",
            "ssa_probe_mfma_bf16", "ssa_probe_hbm_read"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"
    assert lib.ssa_version() >= 100


def test_params_struct_matches_header_layout():
    # int32 x4, int64, int32 x3, float x2, int32 x2 with natural alignment
    assert ctypes.sizeof(B.SSAParams) == 56
    assert B.SSAParams.seq_len.offset == 16 and B.SSAParams.beta.offset == 36


def _p(**kw):
    base = dict(batch=1, n_q_heads=4, n_kv_heads=2, head_dim=128, seq_len=4096, block_size=128,
                top_k=8, window=128, beta=2.0)
    base.update(kw)
    return B.make_params(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), B.SSA_ERR_UNSUPPORTED),
    (dict(n_q_heads=3), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(block_size=48), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(block_size=2048), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(top_k=33), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(top_k=-1), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(window=0), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(seq_len=0), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(batch=0), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(beta=float("nan")), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(scale=0.0), B.SSA_ERR_INVALID_ARGUMENT),
])
def test_invalid_params_rejected_on_host(kw, status):
    p = _p(**kw)
    n = ctypes.c_size_t(0)
    got = ssa.lib().ssa_workspace_size(ctypes.byref(p), B.SSA_OP_ATTN, ctypes.byref(n))
    assert got == status, B.status_string(got)
    assert ssa.lib().ssa_last_error().decode() != ""
    # the compute entry points reject the same parameters before any launch
    got = ssa.lib().ssa_block_stats(ctypes.byref(p), 1 << 20, 1 << 20, 1 << 20, None)
    assert got == status


def test_null_pointers_and_workspace_checked_on_host():
    p = _p()
    L = ssa.lib()
    assert L.ssa_block_stats(None, 1, 1, 1, None) == B.SSA_ERR_INVALID_ARGUMENT
    assert L.ssa_block_stats(ctypes.byref(p), None, 1, 1, None) == B.SSA_ERR_INVALID_ARGUMENT
    need = B.ssa_workspace_size(p, B.SSA_OP_ROUTE)
    assert need > 0
    got = L.ssa_route_topk(ctypes.byref(p), 256, 256, 256, 256, None, 256, need - 1, None)
    assert got == B.SSA_ERR_WORKSPACE_TOO_SMALL
    got = L.ssa_route_topk(ctypes.byref(p), 256, 256, 256, 256, None, 128, need, None)
    assert got == B.SSA_ERR_INVALID_ARGUMENT          # workspace not 256-byte aligned
    need_a = B.ssa_workspace_size(p, B.SSA_OP_ATTN)
    got = L.ssa_sparse_attn_fwd(ctypes.byref(p), 256, 256, 256, None, 256, 256, 256, need_a, None)
    assert got == B.SSA_ERR_INVALID_ARGUMENT          # idx NULL with top_k > 0
    need_d = B.ssa_workspace_size(p, B.SSA_OP_DECODE)
    got = L.ssa_decode_step(ctypes.byref(p), 256, 256, 256, 256, 256, None, 256, 256, None, 256,
                            256, 256, need_d, None)
    assert got == B.SSA_ERR_INVALID_ARGUMENT          # cache_len NULL
    assert L.ssa_workspace_size(ctypes.byref(p), 99, ctypes.byref(ctypes.c_size_t())) == \
        B.SSA_ERR_INVALID_ARGUMENT


def test_workspace_sizes_scale_with_problem():
    small = B.ssa_workspace_size(_p(seq_len=4096), B.SSA_OP_ATTN)
    big = B.ssa_workspace_size(_p(seq_len=8192), B.SSA_OP_ATTN)
    assert big > small > 0
    assert B.ssa_workspace_size(_p(top_k=0), B.SSA_OP_ATTN) < small
    # decode workspace: scores, selections and per-(row, item) partials
    assert B.ssa_workspace_size(_p(), B.SSA_OP_DECODE) > 0


def test_status_strings():
    for code in range(5):
        assert B.status_string(code).startswith("SSA_")


@pytest.mark.parametrize("beta", [0.0, -1.0, float("inf")])
def test_tempered_route_rejects_non_positive_beta(beta):
    p = _p(beta=beta)
    got = ssa.lib().ssa_route_tempered(ctypes.byref(p), 256, 256, 256, None, None)
    assert got == B.SSA_ERR_INVALID_ARGUMENT, B.status_string(got)
    assert "beta" in ssa.lib().ssa_last_error().decode()


def test_tempered_route_checks_pointers_on_host():
    p = _p(beta=2.0)
    L = ssa.lib()
    assert L.ssa_route_tempered(ctypes.byref(p), None, 256, 256, None, None) == \
        B.SSA_ERR_INVALID_ARGUMENT                    # Q NULL
    assert L.ssa_route_tempered(ctypes.byref(p), 256, None, 256, None, None) == \
        B.SSA_ERR_INVALID_ARGUMENT                    # K NULL
    assert L.ssa_route_tempered(ctypes.byref(p), 256, 256, None, None, None) == \
        B.SSA_ERR_INVALID_ARGUMENT                    # idx NULL with top_k > 0
    # nothing requested (k = 0, no kth): returns before any launch
    p0 = _p(beta=2.0, top_k=0)
    assert L.ssa_route_tempered(ctypes.byref(p0), 256, 256, None, None, None) == B.SSA_OK


@pytest.mark.parametrize("m", [0, -3, 65])
def test_group_calls_reject_group_size_out_of_range(m):
    L = ssa.lib()
    p = _p()
    assert L.ssa_group_stats(ctypes.byref(p), 256, 256, m, 256, 256, 256, None) == \
        B.SSA_ERR_INVALID_ARGUMENT
    assert "group_blocks" in L.ssa_last_error().decode()
    assert L.ssa_route_hier(ctypes.byref(p), 256, 256, 256, 256, 256, 256, m, 256, 256, None,
                            256, 1 << 30, None) == B.SSA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("beta", [-0.5, float("nan")])
def test_hier_route_needs_non_negative_beta(beta):
    p = _p()
    p.beta = beta  # make_params validation is the library's job
    got = ssa.lib().ssa_route_hier(ctypes.byref(p), 256, 256, 256, 256, 256, 256, 8, 256, 256,
                                   None, 256, 1 << 30, None)
    assert got == B.SSA_ERR_INVALID_ARGUMENT, B.status_string(got)


def test_hier_route_limits_and_pointers_on_host():
    L = ssa.lib()
    # more than 16 q-heads per KV head
    p = _p(n_q_heads=32, n_kv_heads=1)
    assert L.ssa_route_hier(ctypes.byref(p), 256, 256, 256, 256, 256, 256, 8, 256, 256, None,
                            256, 1 << 30, None) == B.SSA_ERR_UNSUPPORTED
    # G * g beyond the bound table: 2^20 tokens / B 64 = 16384 blocks, m = 1, g = 2
    p = _p(seq_len=1 << 20, block_size=64)
    assert L.ssa_route_hier(ctypes.byref(p), 256, 256, 256, 256, 256, 256, 1, 256, 256, None,
                            256, 1 << 30, None) == B.SSA_ERR_UNSUPPORTED
    p = _p()
    # q, mu, sigma, gmu, gsigma, grl, group_blocks, pos, idx, evaluated, workspace
    need = B.ssa_workspace_size(p, B.SSA_OP_ROUTE_HIER)
    assert need > 0
    good = [256, 256, 256, 256, 256, 256, 8, 256, 256, None, 256]
    for i in (0, 1, 2, 3, 4, 5, 7, 8, 10):
        args = list(good)
        args[i] = None
        got = L.ssa_route_hier(ctypes.byref(p), *args, need, None)
        assert got == B.SSA_ERR_INVALID_ARGUMENT, (i, B.status_string(got))
    got = L.ssa_route_hier(ctypes.byref(p), *good, need - 1, None)
    assert got == B.SSA_ERR_WORKSPACE_TOO_SMALL
    # nothing requested (k = 0, no counts): returns before any launch
    p0 = _p(top_k=0)
    assert L.ssa_route_hier(ctypes.byref(p0), 256, 256, 256, 256, 256, 256, 8, 256, None, None,
                            None, 0, None) == B.SSA_OK
    # group stats: NULL outputs
    assert L.ssa_group_stats(ctypes.byref(p), 256, 256, 8, None, 256, 256, None) == \
        B.SSA_ERR_INVALID_ARGUMENT


def test_decode_noalloc_checked_on_host():
    """The allocation-free decode step refuses, before touching a device, a
    size beyond its scratch and the same invalid arguments as ssa_decode_step."""
    L = ssa.lib()
    big = B.make_params(batch=64, n_q_heads=64, n_kv_heads=8, head_dim=128, seq_len=4096 * 64,
                        block_size=64, top_k=8, window=64)
    assert B.ssa_workspace_size(big, B.SSA_OP_DECODE) > 16 << 20
    got = L.ssa_decode_step_noalloc(ctypes.byref(big), 256, 256, 256, 256, 256, 256, 256, 256,
                                    None, 256, 256, None)
    assert got == B.SSA_ERR_UNSUPPORTED, B.status_string(got)
    assert "scratch" in L.ssa_last_error().decode()
    p = _p()
    got = L.ssa_decode_step_noalloc(ctypes.byref(p), 256, 256, 256, 256, 256, None, 256, 256,
                                    None, 256, 256, None)
    assert got == B.SSA_ERR_INVALID_ARGUMENT          # cache_len NULL
    got = L.ssa_decode_step_noalloc(ctypes.byref(_p(block_size=48)), 256, 256, 256, 256, 256,
                                    256, 256, 256, None, 256, 256, None)
    assert got == B.SSA_ERR_INVALID_ARGUMENT


def test_peak_probes_check_arguments_on_host():
    lib = ssa.lib()
    fl = ctypes.c_double(0.0)
    dummy = ctypes.c_void_p(4096)   # never dereferenced: every call below is rejected first
    assert lib.ssa_probe_mfma_bf16(None, 8, 8, ctypes.byref(fl), None) == B.SSA_ERR_INVALID_ARGUMENT
    assert lib.ssa_probe_mfma_bf16(dummy, 0, 8, ctypes.byref(fl), None) == B.SSA_ERR_INVALID_ARGUMENT
    assert lib.ssa_probe_mfma_bf16(dummy, 8, 0, ctypes.byref(fl), None) == B.SSA_ERR_INVALID_ARGUMENT
    assert lib.ssa_probe_mfma_bf16(dummy, 8, 8, None, None) == B.SSA_ERR_INVALID_ARGUMENT
    assert lib.ssa_probe_hbm_read(None, 1024, dummy, 8, None) == B.SSA_ERR_INVALID_ARGUMENT
    assert lib.ssa_probe_hbm_read(dummy, 1000, dummy, 8, None) == B.SSA_ERR_INVALID_ARGUMENT
    assert lib.ssa_probe_hbm_read(dummy, 0, dummy, 8, None) == B.SSA_ERR_INVALID_ARGUMENT
    assert lib.ssa_probe_hbm_read(dummy, 1024, None, 8, None) == B.SSA_ERR_INVALID_ARGUMENT
    assert lib.ssa_probe_hbm_read(ctypes.c_void_p(4100), 1024, dummy, 8, None) == \
        B.SSA_ERR_INVALID_ARGUMENT
    assert lib.ssa_probe_hbm_read(dummy, 1024, dummy, 0, None) == B.SSA_ERR_INVALID_ARGUMENT


def test_hier_prefill_checked_on_host():
    L = ssa.lib()
    p = _p(in_dtype=torch.bfloat16)
    need = B.ssa_route_hier_prefill_workspace_size(p, 8)
    assert need > B.ssa_route_hier_prefill_workspace_size(p, 64) > 0   # more groups, more bounds
    # Q, mu, sigma, gmu, gsigma, grl, group_blocks, idx, evaluated, workspace
    good = [256, 256, 256, 256, 256, 256, 8, 256, None, 256]
    for i in (0, 1, 2, 3, 4, 5, 7, 9):
        args = list(good)
        args[i] = None
        got = L.ssa_route_hier_prefill(ctypes.byref(p), *args, need, None)
        assert got == B.SSA_ERR_INVALID_ARGUMENT, (i, B.status_string(got))
    assert L.ssa_route_hier_prefill(ctypes.byref(p), *good, need - 1, None) == \
        B.SSA_ERR_WORKSPACE_TOO_SMALL
    for m in (0, 65):
        args = list(good)
        args[6] = m
        assert L.ssa_route_hier_prefill(ctypes.byref(p), *args, need, None) == \
            B.SSA_ERR_INVALID_ARGUMENT
    pb = _p(in_dtype=torch.bfloat16)
    pb.beta = -1.0
    assert L.ssa_route_hier_prefill(ctypes.byref(pb), *good, need, None) == \
        B.SSA_ERR_INVALID_ARGUMENT
    pf = _p(in_dtype=torch.float32)
    assert L.ssa_route_hier_prefill(ctypes.byref(pf), *good, need, None) == B.SSA_ERR_UNSUPPORTED
    # more than 4096 groups: 2^20 tokens / B 64 = 16384 blocks, m = 2
    pg = _p(in_dtype=torch.bfloat16, seq_len=1 << 20, block_size=64)
    n = ctypes.c_size_t(0)
    assert L.ssa_route_hier_prefill_workspace_size(ctypes.byref(pg), 2, ctypes.byref(n)) == \
        B.SSA_ERR_UNSUPPORTED
    # nothing requested (k = 0, no counts): returns before any launch
    p0 = _p(in_dtype=torch.bfloat16, top_k=0)
    assert L.ssa_route_hier_prefill(ctypes.byref(p0), 256, 256, 256, 256, 256, 256, 8, None, None,
                                    None, 0, None) == B.SSA_OK

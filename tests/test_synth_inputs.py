"""The seeded workload generator: shapes, determinism and planted outliers (CPU)."""
import numpy as np
import torch

from synth_inputs import CONFIGS, bf16_round_f32, make_decode, make_prefill


def test_configs_match_workload_table():
    t = CONFIGS["tiny_prefill_4k"]
    assert (t.seq_len, t.head_dim, t.block, t.top_k, t.window, t.dtype) == (4096, 64, 64, 8, 64, "f32")
    g = CONFIGS["gqa_prefill_128k"]
    assert (g.n_q_heads, g.n_kv_heads, g.seq_len, g.block, g.top_k, g.window) == (32, 8, 131072, 256, 16, 256)
    d = CONFIGS["decode_256k"]
    assert d.decode and d.batch == 32 and d.seq_len == 262144 and d.block == 512
    assert CONFIGS["long_prefill_1m"].block == 1024
    assert abs(t.scale - 0.125) == 0 and np.float32(g.scale) == np.float32(1 / np.sqrt(np.float32(128)))


def test_prefill_deterministic_and_planted():
    wl = CONFIGS["tiny_prefill_4k"]
    a = make_prefill(wl, seed=0)
    b = make_prefill(wl, seed=0)
    c = make_prefill(wl, seed=1)
    for key in ("Q", "K", "V"):
        assert torch.equal(a[key], b[key])
        assert not torch.equal(a[key], c[key])
    assert a["Q"].shape == (1, 1, 4096, 64) and a["K"].dtype == torch.float32
    assert len(a["plants"]) == 8 and len({p["block"] for p in a["plants"]}) == 8
    for p in a["plants"]:
        assert p["block"] <= wl.seq_len // wl.block - 2
        assert (p["block"] + 1) * wl.block <= p["t"] < wl.seq_len
        q = a["Q"][0, p["h"], p["t"]]
        np.testing.assert_allclose(a["K"][0, 0, p["pos"]].numpy(), (3 * q / q.norm()).numpy(), rtol=1e-6)


def test_bf16_workload_and_rounding():
    wl = CONFIGS["prefill_32k"].replace(n_q_heads=2, n_kv_heads=1, seq_len=1024, plants=4)
    data = make_prefill(wl, seed=0)
    assert data["Q"].dtype == torch.bfloat16 and data["K"].shape == (1, 1, 1024, 128)
    x = np.random.default_rng(0).normal(size=1000).astype(np.float32)
    np.testing.assert_array_equal(bf16_round_f32(x),
                                  torch.tensor(x).to(torch.bfloat16).float().numpy())
    for p in data["plants"]:
        assert p["h"] in (0, 1)


def test_positions_plant_mode():
    wl = CONFIGS["long_prefill_1m"].replace(seq_len=8192, block=256, plants=40, n_q_heads=2,
                                            n_kv_heads=1)
    data = make_prefill(wl, seed=3)
    pos = [p["pos"] for p in data["plants"]]
    assert len(set(pos)) == 40 and max(pos) < (8192 // 256 - 1) * 256


def test_decode_inputs():
    wl = CONFIGS["decode_256k"].replace(batch=2, n_q_heads=4, n_kv_heads=2, seq_len=1000, block=64,
                                        plants=5)
    data = make_decode(wl, seed=0, capacity=1100)
    assert data["K_cache"].shape == (2, 2, 1100, 128) and data["cache_len"] == 1000
    assert torch.count_nonzero(data["K_cache"][:, :, 1000:]) == 0
    assert data["q"].shape == (2, 4, 128) and data["k_new"].shape == (2, 2, 128)
    for p in data["plants"]:
        assert p["pos"] < 1000 and p["t"] == 1000

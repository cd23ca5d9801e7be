"""Seeded synthetic workloads (see the package docstring for the model)."""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import numpy as np
import torch

_TAG_Q, _TAG_K_CENTRE, _TAG_K_NOISE, _TAG_V, _TAG_PLANT = 11, 13, 17, 19, 23
_TAG_QNEW, _TAG_VNEW, _TAG_K_GROUP, _TAG_Q_TOPIC = 29, 31, 37, 41


def _mix(*parts: int) -> int:
    """Deterministic 63-bit seed from integer parts (FNV-1a over 8-byte words)."""
    h = 0xCBF29CE484222325
    for p in parts:
        for byte in int(p).to_bytes(8, "little", signed=False):
            h ^= byte
            h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h & 0x7FFFFFFFFFFFFFFF


@dataclass(frozen=True)
class Workload:
    """One workload shape.  Field names follow the method's notation."""

    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_len: int          # prefill: n.  decode: L, the tokens already cached
    head_dim: int         # d
    dtype: str            # "f32" or "bf16" for Q, K, V
    block: int            # B
    top_k: int            # k
    window: int           # W
    beta: float           # routing inverse temperature on raw q
    center_std: float     # std of the block centre m_c
    noise_std: float      # std of the within-block noise
    plants: int           # planted outliers per (sequence, KV head)
    plant_mode: str       # "blocks" | "positions" | "decode"
    decode: bool = False
    group_std: float = 0.0    # std of a centre shared by group_blocks consecutive blocks
    group_blocks: int = 16    # (0 std: no group structure, the default)
    query_topic: float = 0.0  # strength of a segment's topic in its queries (needs group_std)
    topic_span: int = 1024    # tokens per topic segment
    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def scale(self) -> float:
        """Softmax scale on raw logits: the float32 value of 1/sqrt(d)."""
        return float(np.float32(1.0) / np.sqrt(np.float32(self.head_dim)))

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


# The five workloads the method's measurements are quoted on.  The first is the
# small case that the oracle finishes in seconds; the third is the n = 128K
# prefill the headline throughput is quoted on.
CONFIGS: dict[str, Workload] = {
    "tiny_prefill_4k": Workload(
        "tiny_prefill_4k", 1, 1, 1, 4096, 64, "f32", 64, 8, 64, 2.0,
        math.sqrt(0.5), 0.5, 8, "blocks"),
    "prefill_32k": Workload(
        "prefill_32k", 1, 8, 8, 32768, 128, "bf16", 128, 16, 128, 2.0,
        math.sqrt(0.5), 0.5, 64, "blocks"),
    "gqa_prefill_128k": Workload(
        "gqa_prefill_128k", 1, 32, 8, 131072, 128, "bf16", 256, 16, 256, 2.0,
        0.7, 0.5, 256, "blocks"),
    "decode_256k": Workload(
        "decode_256k", 32, 32, 8, 262144, 128, "bf16", 512, 16, 512, 2.0,
        0.7, 0.5, 256, "decode", decode=True),
    "long_prefill_1m": Workload(
        "long_prefill_1m", 1, 16, 4, 1048576, 128, "bf16", 1024, 8, 1024, 2.0,
        0.7, 0.5, 1024, "positions"),
}


def bf16_round_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_mix(*parts))
    return g


def _randn(shape, device, *parts) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(device, *parts), device=device,
                       dtype=torch.float32)


def _plan_plants(wl: Workload, seed: int, b: int, kv: int, n_keys: int,
                 q_len: int) -> list[dict]:
    """Choose planted-outlier positions, target queries and heads.

    Uses a CPU generator so the ledger does not depend on the device.
    "blocks": distinct blocks from 0..nb-2, position uniform in the block,
    target t uniform in [(c+1)B, q_len-1].  "positions": positions uniform
    without replacement from [0, (nb-1)B).  "decode": distinct blocks among
    those fully inside the cache; the target is the decode query.
    """
    B, g = wl.block, wl.group
    gen = _gen("cpu", seed, _TAG_PLANT, b, kv)
    nb = n_keys // B
    plants = []
    if wl.plant_mode in ("blocks", "decode"):
        n_cand = nb - 1 if wl.plant_mode == "blocks" else n_keys // B
        count = min(wl.plants, max(n_cand, 0))
        blocks = torch.randperm(n_cand, generator=gen)[:count].tolist()
        for c in blocks:
            pos = c * B + int(torch.randint(B, (1,), generator=gen))
            if wl.plant_mode == "blocks":
                lo = (c + 1) * B
                t = lo + int(torch.randint(q_len - lo, (1,), generator=gen))
            else:
                t = q_len - 1
            h = kv * g + int(torch.randint(g, (1,), generator=gen))
            plants.append(dict(b=b, kv=kv, h=h, t=t, pos=pos, block=c))
    elif wl.plant_mode == "positions":
        span = (nb - 1) * B
        count = min(wl.plants, max(span, 0))
        positions = torch.randperm(span, generator=gen)[:count].tolist()
        for pos in positions:
            c = pos // B
            lo = (c + 1) * B
            t = lo + int(torch.randint(q_len - lo, (1,), generator=gen))
            h = kv * g + int(torch.randint(g, (1,), generator=gen))
            plants.append(dict(b=b, kv=kv, h=h, t=t, pos=pos, block=c))
    else:
        raise ValueError(f"unknown plant mode {wl.plant_mode!r}")
    return plants


def _keys(wl: Workload, seed: int, b: int, kv: int, n_keys: int, device) -> torch.Tensor:
    """Clustered-Gaussian keys (float32) for one (sequence, KV head)."""
    B, d = wl.block, wl.head_dim
    nbp = -(-n_keys // B)
    centre = _randn((nbp, d), device, seed, _TAG_K_CENTRE, b, kv) * wl.center_std
    if wl.group_std > 0:
        # routable geometry: block centres scattered around shared group centres
        grp = _group_centres(wl, seed, b, kv, n_keys, device)
        centre = centre + grp.repeat_interleave(wl.group_blocks, dim=0)[:nbp]
    noise = _randn((n_keys, d), device, seed, _TAG_K_NOISE, b, kv) * wl.noise_std
    return noise.add_(centre.repeat_interleave(B, dim=0)[:n_keys])


def _group_centres(wl: Workload, seed: int, b: int, kv: int, n_keys: int, device) -> torch.Tensor:
    nbp = -(-n_keys // wl.block)
    ngp = -(-nbp // wl.group_blocks)
    return _randn((ngp, wl.head_dim), device, seed, _TAG_K_GROUP, b, kv) * wl.group_std


def _topics(wl: Workload, seed: int, b: int, kv: int, n: int) -> list[int]:
    """Topic group of every topic_span-token segment of one (sequence, KV head):
    uniform over the groups whose blocks are all complete before the segment
    starts, -1 while there is none.  A CPU generator keeps it device-independent."""
    gen = _gen("cpu", seed, _TAG_Q_TOPIC, b, kv)
    out = []
    for t0 in range(0, n, wl.topic_span):
        top = t0 // wl.block // wl.group_blocks - 1
        out.append(int(torch.randint(top + 1, (1,), generator=gen)) if top >= 0 else -1)
    return out


def _add_topics(Qf: torch.Tensor, wl: Workload, seed: int, b: int, kv: int, device) -> None:
    """Queries of a segment lean toward their topic group's key centre:
    q += query_topic * sqrt(d) * (unit group centre), the same for every
    q-head of the KV head."""
    n, d = Qf.shape[-2], Qf.shape[-1]
    grp = _group_centres(wl, seed, b, kv, n, device)
    unit = grp / torch.linalg.vector_norm(grp, dim=-1, keepdim=True)
    for s, gi in enumerate(_topics(wl, seed, b, kv, n)):
        if gi >= 0:
            t0 = s * wl.topic_span
            Qf[:, t0:t0 + wl.topic_span] += wl.query_topic * math.sqrt(d) * unit[gi]


def _plant(K: torch.Tensor, plants: list[dict], qrow) -> None:
    for p in plants:
        q = qrow(p).to(torch.float32)
        K[p["pos"]] = 3.0 * q / torch.linalg.vector_norm(q)


def make_prefill(wl: Workload, seed: int = 0, device="cpu") -> dict:
    """Q [b,Hq,n,d], K and V [b,Hkv,n,d] in the workload dtype, plus the plant ledger."""
    if wl.decode:
        raise ValueError("make_prefill needs a prefill workload")
    b_, hq, hkv, n, d = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.seq_len, wl.head_dim
    dt = wl.torch_dtype
    Q = torch.empty((b_, hq, n, d), dtype=dt, device=device)
    K = torch.empty((b_, hkv, n, d), dtype=dt, device=device)
    V = torch.empty((b_, hkv, n, d), dtype=dt, device=device)
    ledger: list[dict] = []
    if wl.query_topic > 0 and wl.group_std <= 0:
        raise ValueError("query topics lean toward key group centres: set group_std > 0")
    g = wl.group
    for b in range(b_):
        for kv in range(hkv):
            Qf = torch.stack([_randn((n, d), device, seed, _TAG_Q, b, h)
                              for h in range(kv * g, (kv + 1) * g)])
            if wl.query_topic > 0:
                _add_topics(Qf, wl, seed, b, kv, device)
            Q[b, kv * g:(kv + 1) * g] = Qf.to(dt)
        for kv in range(hkv):
            V[b, kv] = _randn((n, d), device, seed, _TAG_V, b, kv).to(dt)
            plants = _plan_plants(wl, seed, b, kv, n, n)
            Kf = _keys(wl, seed, b, kv, n, device)
            _plant(Kf, plants, lambda p: Q[p["b"], p["h"], p["t"]])
            K[b, kv] = Kf.to(dt)
            ledger.extend(plants)
    return dict(Q=Q, K=K, V=V, plants=ledger, workload=wl, seed=seed)


def make_decode(wl: Workload, seed: int = 0, device="cpu", capacity: int | None = None) -> dict:
    """One decode step's inputs.

    The cache holds L = wl.seq_len keys per (sequence, KV head); the step appends
    k_new/v_new at position L and queries at t = L.  Returns q [b,Hq,d],
    k_new/v_new [b,Hkv,d], K_cache/V_cache [b,Hkv,capacity,d] (positions >= L
    are zero), cache_len = L and the plant ledger.
    """
    if not wl.decode:
        raise ValueError("make_decode needs a decode workload")
    b_, hq, hkv, L, d = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.seq_len, wl.head_dim
    cap = capacity if capacity is not None else L + 1
    if cap < L + 1:
        raise ValueError("capacity must hold the appended key")
    dt = wl.torch_dtype
    q = torch.empty((b_, hq, d), dtype=dt, device=device)
    k_new = torch.empty((b_, hkv, d), dtype=dt, device=device)
    v_new = torch.empty((b_, hkv, d), dtype=dt, device=device)
    K = torch.zeros((b_, hkv, cap, d), dtype=dt, device=device)
    V = torch.zeros((b_, hkv, cap, d), dtype=dt, device=device)
    ledger: list[dict] = []
    if wl.query_topic > 0 and wl.group_std <= 0:
        raise ValueError("query topics lean toward key group centres: set group_std > 0")
    g = wl.group
    for b in range(b_):
        for kv in range(hkv):
            qf = torch.stack([_randn((d,), device, seed, _TAG_QNEW, b, h)
                              for h in range(kv * g, (kv + 1) * g)])
            if wl.query_topic > 0:
                # the query at t = L takes the topic of the segment holding L
                gi = _topics(wl, seed, b, kv, L + 1)[L // wl.topic_span]
                if gi >= 0:
                    grp = _group_centres(wl, seed, b, kv, L + 1, device)[gi]
                    qf += wl.query_topic * math.sqrt(d) * grp / torch.linalg.vector_norm(grp)
            q[b, kv * g:(kv + 1) * g] = qf.to(dt)
        for kv in range(hkv):
            vals = _randn((L + 1, d), device, seed, _TAG_V, b, kv).to(dt)
            V[b, kv, :L] = vals[:L]
            v_new[b, kv] = vals[L]
            plants = _plan_plants(wl, seed, b, kv, L, L + 1)
            Kf = _keys(wl, seed, b, kv, L + 1, device)
            _plant(Kf, plants, lambda p: q[p["b"], p["h"]])
            Kd = Kf.to(dt)
            K[b, kv, :L] = Kd[:L]
            k_new[b, kv] = Kd[L]
            ledger.extend(plants)
    return dict(q=q, k_new=k_new, v_new=v_new, K_cache=K, V_cache=V, cache_len=L,
                plants=ledger, workload=wl, seed=seed)

"""Seeded synthetic inputs for content-routed sparse attention workloads.

This module is the only code that both the CPU oracle's tests and the HIP path's
tests, smoke check and benchmark share.  It draws inputs; it holds none of the
method's arithmetic (no statistics, scores, selection or attention).

Workload model (from the five workload descriptions that accompany the method
write-up "Subquadratic Sparse Attention (SSA)", section "The idea in one
screen"): Q and V are iid N(0, 1).  K is built per block: a block centre
m_c ~ N(0, center_std^2 I) plus per-key noise N(0, noise_std^2 I).  A number of
"planted outliers" replace single keys by 3 * q_t / ||q_t|| for a query t that
lies after the key's block, so that the block is routable for that query.
These plants play the role of single-needle targets.  With group_std > 0 each
run of group_blocks consecutive block centres also shares a group centre
N(0, group_std^2 I), a geometry in which whole groups of blocks can be ruled out
for a query (the hierarchical router's test case); group_std = 0, the default,
leaves every existing stream unchanged.  query_topic > 0 (with group_std > 0)
also gives the queries topics: the sequence is cut into segments of
topic_span tokens, each segment picks one earlier key group (uniformly among
those whose blocks all end before it) and every query of the segment, in all
q-heads of the KV head, gets query_topic * sqrt(d) times that group centre's
unit vector added -- neighbouring queries then want the same groups, the
structure a tree router prunes on; query_topic = 0, the default, leaves Q
unchanged.

Everything is drawn with torch generators seeded per tensor, so a workload is a
pure function of (config, seed, device).  CPU and GPU generators give different
streams; a caller that needs one data set on both sides draws it once and copies.
"""
from .generate import (
    Workload,
    CONFIGS,
    make_prefill,
    make_decode,
    bf16_round_f32,
)

__all__ = ["Workload", "CONFIGS", "make_prefill", "make_decode", "bf16_round_f32"]

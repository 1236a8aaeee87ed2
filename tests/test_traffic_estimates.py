"""The host-side traffic arithmetic against the numbers page
"张量、流水线与数据并行" prints (tests/golden/p3_traffic_estimates.json)."""

import json
import os

from megatron_sharded_linears_amd import traffic as T

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "p3_traffic_estimates.json")))
MODEL = G["model"]
H, L, V = MODEL["hidden"], MODEL["layers"], MODEL["vocab"]


def test_counts_and_payloads():
    assert T.all_reduces_per_forward(L) == G["all_reduce_per_forward"]
    assert T.payload_per_token(H) == G["payload_per_token_per_all_reduce_bytes"]
    assert T.payload_per_token_per_forward(H, L) == G["payload_per_token_per_forward_KiB"] * T.KIB


def test_ring_and_logits():
    for row in G["ring"]:
        assert T.ring_factor(row["t"]) == row["factor"]
        assert T.ring_sent_per_rank_per_token(H, L, row["t"]) == row["sent_per_rank_per_token_KiB"] * T.KIB
    for row in G["logits_all_gather_received_per_rank_per_sampled_token_KiB"]:
        assert round(T.logits_gather_received_per_token(V, row["t"]) / T.KIB) == row["KiB_rounded"]


def test_per_step():
    for row in G["per_step"]:
        one, total = T.per_step(row["tokens"], H, L)
        assert one == row["per_all_reduce_KiB"] * T.KIB
        assert round(total / T.MIB, row["printed_MiB_decimals"]) == row["per_forward_MiB"]

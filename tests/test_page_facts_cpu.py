"""The workloads and the oracle's routing statistics against the numbers the
pages fix (tests/golden/page_facts.json, each with its citation).

The pages print no worked example of the layer's arithmetic, so these pins
cover what they do fix: the model's geometry, the share of experts a token
uses, the prefill chunk, the number of drafted tokens, and the hit rates of
a hot-expert cache.  The hit rates are computed with the oracle's own top-k
on the synthetic router logits.
"""
import json
import os

import numpy as np
import pytest

import synth
from oracle import moe_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
FACTS = {f["id"]: f for f in json.load(open(os.path.join(HERE, "golden", "page_facts.json")))["facts"]}
FULL = ["decode_t1", "mtp_verify_t4_48l", "prefill_8192", "slot_q3s_t1_48l", "decode_q2s_t1",
        "prefill_q3s_8192", "prefill_slot_q3s_8192", "slot_host_q3s_t1_8l", "slot_policy_q3s_t1_8l"]


def _v(name):
    return FACTS[name]["value"]


def test_every_fact_has_a_citation():
    for f in FACTS.values():
        assert f["cite"].startswith("[") and f["fact"], f["id"]


def test_model_geometry():
    for name in FULL:
        w = synth.WORKLOADS[name]
        assert w["n_experts"] == _v("experts_per_layer"), name
        assert w["top_k"] == _v("routed_per_token"), name
        assert (w["d_ff_shared"] > 0) == (_v("shared_per_token") == 1), name
    for name in ("mtp_verify_t4_48l", "slot_q3s_t1_48l"):
        assert synth.WORKLOADS[name]["layers"] == _v("layers")
    assert _v("layers") * _v("experts_per_layer") == _v("experts_total")


def test_share_of_experts_a_token_uses():
    f = FACTS["share_of_experts_used"]
    w = synth.WORKLOADS["decode_t1"]
    assert abs(w["top_k"] / w["n_experts"] - f["value"]) <= f["tolerance"]


def test_prefill_chunk_and_drafted_tokens():
    for name in ("prefill_8192", "prefill_q3s_8192", "prefill_slot_q3s_8192"):
        assert synth.WORKLOADS[name]["tokens"] == _v("prefill_chunk_max_tokens")
    assert synth.WORKLOADS["mtp_verify_t4_48l"]["tokens"] == 1 + _v("mtp_draft_tokens")


def _hit_rate(logits, ranks, k, n_res):
    idx, _ = O.route(logits, k)
    return float(np.mean(ranks[idx] <= n_res))


def test_hot_cache_hit_rate_of_the_slot_workload():
    """The slot workload keeps the 128 most popular experts resident; the
    oracle's routing of its logits hits them about as often as the pages'
    cache hits its experts."""
    f = FACTS["hot_cache_hit_rate"]
    w = synth.WORKLOADS["slot_q3s_t1_48l"]
    rates = [_hit_rate(synth.router_logits(0, l, 1024, w["n_experts"], zipf_s=w["zipf_s"],
                                           alpha=w["alpha"]),
                       synth.expert_ranks(0, l, w["n_experts"]), w["top_k"], w["n_slots"])
             for l in range(4)]
    assert abs(np.mean(rates) - f["value"]) <= f["tolerance"], rates


def test_frequency_only_hit_rate_on_the_drifting_stream():
    """On the drifting stream of the slot-policy workload, the set fixed from
    the overall popularity ranking (the frequency curve alone) hits about as
    often as the pages report for that choice."""
    f = FACTS["frequency_only_hit_rate"]
    w = synth.WORKLOADS["slot_policy_q3s_t1_8l"]
    rates = [_hit_rate(synth.router_logits_drifting(0, l, w["stream_tokens"], w["n_experts"],
                                                    w["zipf_s"], w["alpha"], w["alpha_context"],
                                                    w["segment"]),
                       synth.expert_ranks(0, l, w["n_experts"]), w["top_k"], w["n_slots"])
             for l in range(2)]
    assert abs(np.mean(rates) - f["value"]) <= f["tolerance"], rates

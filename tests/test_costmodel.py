"""Cost model against the pages' worked numbers (no GPU)."""

import json
import os

import pytest

import synth
from unified_transformer_recommender_amd import costmodel as cm

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def test_pyramid_worked_problem():
    g = GOLD["pyramid_7_5_3"]
    fr = g["query_fractions"]
    assert sum(fr) == pytest.approx(g["sum_in_units_of_L2"])
    assert round(sum(fr), 2) == g["printed_sum_approx"]
    assert round(cm.pyramid_attention_ratio(fr), 2) == g["printed_ratio_approx"]


def test_kv_cache_worked_problem():
    g = GOLD["kv_cache_7_5_4"]
    plain, cached, ratio = cm.kv_cache_saving(g["n_cand"], g["l_s"], g["l_ns"])
    assert plain == g["printed_plain"] and cached == g["printed_cached"]
    assert round(ratio) == g["printed_ratio_approx"]


def test_pyramid_schedule_endpoints():
    g = GOLD["pyramid_endpoints"]
    q = synth.workload("onetrans_s").s_queries
    assert q[0] == g["first"] and q[-1] == g["last"]
    assert list(q) == sorted(q, reverse=True)
    assert q == (1190, 955, 719, 484, 248, 12)
    assert synth.workload("onetrans_l").s_queries == (2048, 1760, 1472, 1184, 896, 608, 320, 32)


def test_visible_pairs_brute_force():
    for p0 in (0, 3, 17):
        for r in (1, 5, 30):
            assert cm.visible_pairs(p0, r) == sum(p0 + i + 1 for i in range(r))


def test_complexity_orders():
    # attention O(L^2 d) -> O(L L' d); FFN O(L d^2) -> O(L' d^2): halving queries halves FFN work
    full = cm.block_work(256, 1024, 1000, 1000, 0)
    half = cm.block_work(256, 1024, 1000, 500, 500)
    ffn_full = 2 * 2 * 256 * 1024 * 1000
    assert full.gemm - half.gemm == pytest.approx(ffn_full / 2 + 2 * 256 * 256 * 2 * 500)
    # serving: O(C L_S) -> O(L_S + C L_NS); append: O(L_S) -> O(dL)
    w = synth.workload("onetrans_s")
    m = w.model
    pre = cm.prefill_work(m.d_model, m.d_ff, w.l_s, w.s_queries)
    sc = cm.score_work(m.d_model, m.d_ff, m.l_ns, w.l_s, w.s_queries)
    fw = cm.forward_work(m.d_model, m.d_ff, m.l_ns, w.l_s, w.s_queries)
    assert pre.total + sc.total == pytest.approx(fw.total, rel=1e-12)
    app = cm.append_work(m.d_model, m.d_ff, m.n_blocks, 1158, 32)
    full_pre = cm.prefill_work(m.d_model, m.d_ff, 1190, (1190,) * 6)
    assert full_pre.gemm / app.gemm == pytest.approx(1190 / 32)
    assert full_pre.attn / app.attn == pytest.approx(cm.visible_pairs(0, 1190) / cm.visible_pairs(1158, 32))


def test_onetrans_s_flops():
    w = synth.workload("onetrans_s")
    m = w.model
    fw = cm.forward_work(m.d_model, m.d_ff, m.l_ns, w.l_s, w.s_queries)
    assert fw.total == pytest.approx(8.407e9, rel=1e-3)
    assert fw.attn == pytest.approx(2.272e9, rel=1e-3)


def test_mixed_parameter_count_order():
    # O(L_NS d^2 + d^2): linear in the number of NS tokens, not in the sequence length
    a = cm.mixed_param_count(256, 1024, 16)
    b = cm.mixed_param_count(256, 1024, 32)
    assert b / a == pytest.approx(33 / 17)


def test_kernel_classes_sum_to_forward_work():
    w = synth.workload("onetrans_s")
    m = w.model
    c = cm.forward_classes(m.d_model, m.d_ff, m.l_ns, w.l_s, w.s_queries, 2)
    fw = cm.forward_work(m.d_model, m.d_ff, m.l_ns, w.l_s, w.s_queries)
    assert c["qkv"] + c["post"] == pytest.approx(fw.gemm)
    assert c["attn"] == pytest.approx(fw.attn)

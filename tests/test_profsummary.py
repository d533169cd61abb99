"""Host tests of the profile-summary helpers that feed bench.py's roofline traffic figure."""

import os

from unified_transformer_recommender_amd import profsummary


def test_traffic_record_roundtrip(tmp_path):
    path = os.path.join(tmp_path, "traffic_post_onetrans_s.txt")
    profsummary.write_traffic(path, "post", "onetrans_s", fetch_kib=100.0, write_kib=50.0,
                              f_fetch=2.0, f_write=1.0, command="cmd")
    rec = profsummary.read_traffic(path)
    assert rec is not None
    assert float(rec["traffic_bytes_per_launch"]) == 1024.0 * (100.0 * 2.0 + 50.0 * 1.0)


def test_traffic_record_ignored_after_kernel_change(tmp_path):
    path = os.path.join(tmp_path, "traffic_qkv_onetrans_s.txt")
    profsummary.write_traffic(path, "qkv", "onetrans_s", 1.0, 1.0, 1.0, 1.0, "cmd")
    text = open(path).read().replace(profsummary.source_sha256("qkv"), "0" * 64)
    open(path, "w").write(text)
    assert profsummary.read_traffic(path) is None
    assert profsummary.read_traffic(os.path.join(tmp_path, "missing.txt")) is None


def test_kernel_classes_match_source_files():
    for k, (syms, srcs) in profsummary.KERNELS.items():
        texts = []
        for src in srcs:
            assert os.path.exists(os.path.join(profsummary.CSRC, src))
            texts.append(open(os.path.join(profsummary.CSRC, src)).read())
        for sym in syms:
            assert profsummary.classify("void ot::(anonymous namespace)::" + sym + "<bf16>") == k
            assert any(sym in t for t in texts), (k, sym)
    assert profsummary.classify("__amd_rocclr_copyBuffer") is None


def test_mfma_summary_weights_by_duration(tmp_path):
    """Duration-weighted MfmaUtil / VALUBusy and executed flops from a counters table laid out as
    rocprofv3 writes it (one row per dispatch and counter)."""
    import sqlite3
    db = os.path.join(tmp_path, "run_results.db")
    c = sqlite3.connect(db)
    c.execute("create table counters_collection (dispatch_id int, kernel_name text, counter_name text, "
              "value real, duration real)")
    rows = [(1, "attn_kernel<bf16>", "MfmaUtil", 10.0, 100.0), (1, "attn_kernel<bf16>", "VALUBusy", 50.0, 100.0),
            (1, "attn_kernel<bf16>", "SQ_INSTS_VALU_MFMA_MOPS_BF16", 2.0, 100.0),
            (2, "attn_split_kernel<bf16>", "MfmaUtil", 40.0, 300.0), (2, "attn_split_kernel<bf16>", "VALUBusy", 10.0, 300.0),
            (2, "attn_split_kernel<bf16>", "SQ_INSTS_VALU_MFMA_MOPS_BF16", 4.0, 300.0),
            (3, "qkv_kernel<bf16>", "MfmaUtil", 99.0, 1.0)]
    c.executemany("insert into counters_collection values (?,?,?,?,?)", rows)
    c.commit()
    m = profsummary.mfma_summary(db, "attn")
    assert m["dispatches"] == 2
    assert abs(m["MfmaUtil"] - (10 * 100 + 40 * 300) / 400) < 1e-9
    assert abs(m["VALUBusy"] - (50 * 100 + 10 * 300) / 400) < 1e-9
    assert m["mfma_flops_per_dispatch"] == 512.0 * 3.0
    assert profsummary.mfma_summary(db, "post") is None

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
    for k, (sym, src) in profsummary.KERNELS.items():
        assert os.path.exists(os.path.join(profsummary.CSRC, src))
        assert profsummary.classify("void ot::(anonymous namespace)::" + sym + "<bf16>") == k

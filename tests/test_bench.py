"""CPU checks of bench.py's arithmetic and contract: the algorithmic flop and byte counts behind
every reported fraction (against brute-force pair counts and closed forms), the traffic
summary reader (its source-hash guard), and the refusal of more than one GPU before any GPU
work."""
import numpy as np
import pytest

import bench
from synth import WORKLOADS, context_lens


def _pairs_brute(S, causal, window):
    n = 0
    for i in range(S):
        for j in range(S):
            if causal and j > i:
                continue
            if window > 0 and i - j >= window:
                continue
            n += 1
    return n


@pytest.mark.parametrize("S", [1, 5, 37, 64])
@pytest.mark.parametrize("window", [0, 1, 3, 16, 100])
def test_prefill_pairs_match_a_brute_force_count(S, window):
    assert bench.prefill_pairs(S, True, window) == _pairs_brute(S, True, window)


def test_prefill_flops_of_the_workloads():
    # 4*D flops per visible (query, key) pair: QK^T and PV, 2*D each
    c4p = WORKLOADS["prefill_swa_s16384"]
    per_head = 4096 * 4097 // 2 + (16384 - 4096) * 4096
    assert bench.prefill_flops(c4p) == 4.0 * 128 * 32 * 2 * per_head == 1924212457472.0
    c2 = WORKLOADS["prefill_llama1b_s4096"]
    assert bench.prefill_flops(c2) == 4.0 * 64 * 32 * 1 * (4096 * 4097 // 2)
    # chunked: 4 sequences, 1024 rows after 3072-token prefixes, 32 heads, D = 64
    assert bench.chunked_flops() == 4.0 * 64 * 32 * 4 * (1024 * 3072 + 1024 * 1025 // 2)


def test_decode_bytes_of_the_workloads():
    c5 = WORKLOADS["decode_int8_70b_b16"]
    # every token's int8 K and V rows of 8 heads x 128 plus their fp16 scales; Q read, O written
    want = 16 * 32768 * (2 * 8 * 128 + 2 * 8 * 2) + 2 * 16 * 64 * 128 * 2
    assert bench.decode_bytes(c5, context_lens(c5)) == want == 1091043328
    c4d = WORKLOADS["decode_swa_b32"]
    # the window bounds the visible keys: 4096 of each 16384-token context
    assert bench.decode_bytes(c4d, context_lens(c4d)) == 32 * 4096 * 2 * 8 * 128 * 2 + 2 * 32 * 32 * 128 * 2
    c3 = WORKLOADS["decode_llama1b_b64"]
    ctx = context_lens(c3)
    assert bench.decode_bytes(c3, ctx) == float(ctx.sum()) * 2 * 8 * 64 * 2 + 2 * 64 * 32 * 64 * 2


def test_traffic_reader_guards_on_the_source_hash(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "k.hip").write_text("kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "unit", "k.hip")
    h = bench.source_hash("unit")
    (tmp_path / "profiles" / "traffic_unit_w.txt").write_text(
        f"# header\n\nsource_sha256_16 = {h}\nhbm_bytes_per_launch = 12345\n")
    assert bench.measured_traffic("unit", "w") == 12345.0
    (tmp_path / "k.hip").write_text("kernel v2\n")  # the source changed since the counters
    assert bench.measured_traffic("unit", "w") is None
    assert bench.measured_traffic("unit", "missing") is None


def test_more_than_one_gpu_is_refused_before_any_gpu_work(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err

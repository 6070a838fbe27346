"""Host-side trace analysis (persistent_decode_megakernel_amd.trace) on
synthetic 8-word records: spans, idle fraction and per-stage phases."""
import numpy as np
import pytest

from persistent_decode_megakernel_amd import trace as T


def _records():
    # 2 stages x 2 workgroups; ticks of 10 ns (100 MHz)
    plan = [{"type": "qkv", "layer": 0, "weight_bytes": 1000}, {"type": "attn", "layer": 0, "weight_bytes": 0}]
    tr = np.zeros((2, 2, 8), dtype=np.int64)
    #            enter ready done  epoch staged consumed epi  entry
    tr[0, 0] = [100, 200, 1100, 1, 300, 900, 1000, 60]
    tr[0, 1] = [100, 300, 1300, 1, 400, 1100, 1200, 80]
    tr[1, 0] = [1200, 1400, 2000, 1, 1500, 1800, 1900, 1150]
    tr[1, 1] = [1400, 1500, 2100, 1, 0, 0, 0, 1350]  # a workgroup without marks
    return tr, plan


def test_summary_spans_and_idle():
    tr, plan = _records()
    s = T.summarize(tr, plan)
    assert s["total_us"] == pytest.approx((2100 - 100) / 100)
    assert [r["span_us"] for r in s["stages"]] == pytest.approx([12.0, 8.0])
    busy = ((1100 - 200) + (1300 - 300) + (2000 - 1400) + (2100 - 1500)) / 100
    assert s["idle_frac"] == pytest.approx(1 - busy / (20.0 * 2))
    agg = T.by_type(s)
    assert agg["qkv"]["GBps"] == pytest.approx(1000 / 12.0 / 1e3)


def test_phases():
    tr, plan = _records()
    ph = T.phases(tr, plan)
    assert ph[0]["setup"] == pytest.approx((0.3, 0.4))
    assert ph[0]["wait"] == pytest.approx((1.5, 2.0))
    assert ph[0]["stage_in"] == pytest.approx((1.0, 1.0))
    assert ph[0]["stream"] == pytest.approx((6.5, 7.0))
    assert ph[0]["epi"] == pytest.approx((1.0, 1.0))
    assert ph[0]["ack"] == pytest.approx((1.0, 1.0))
    assert ph[0]["gap"] == pytest.approx((0.5, 0.5))  # signalled -> next stage entered
    # stage 1: only workgroup 0 carries marks
    assert ph[1]["stream"] == pytest.approx((3.0, 3.0))
    assert ph[1]["gap"] is None
    text = T.format_phases(ph)
    assert "qkv" in text and "attn" in text

"""The calibration driver's host-side rules (no GPU): the draw limit of the
8-bit votes, and the schedule variants of the sensitivity sweep."""

import pytest
import torch

from calibrated_block_sparse_amd import calibrate as cal_mod


def test_more_than_255_draws_are_rejected():
    # votes saturate at 255, so 256 or more draws would binarise wrongly;
    # every entry point refuses before doing any device work
    v = torch.zeros(1, 2, 2, dtype=torch.uint8)
    cal = cal_mod.Calibration(1, 256, 300, {0: v}, None, {0: 1})
    with pytest.raises(ValueError, match="255"):
        cal_mod.finalize(cal)
    with pytest.raises(ValueError, match="255"):
        cal_mod.densities(cal, [0.5])
    with pytest.raises(ValueError, match="255"):
        cal_mod.vote_stats(v, 256)
    with pytest.raises(ValueError, match="255"):
        cal_mod.main(["--draws", "256"])


def test_accumulate_stops_at_the_256th_draw(monkeypatch):
    """accumulate() counts draws and refuses the 256th before enqueueing its
    work (the library calls are replaced by counters here, so the test runs
    without a GPU)."""
    calls = {"energy": 0, "select": 0}
    monkeypatch.setattr(cal_mod, "calibatt_block_energy",
                        lambda *a, **k: calls.__setitem__("energy", calls["energy"] + 1))
    monkeypatch.setattr(cal_mod, "calibatt_build_mask",
                        lambda *a, **k: calls.__setitem__("select", calls["select"] + 1))
    monkeypatch.setattr(cal_mod, "calibatt_block_energy_workspace", lambda h, n: 8)
    q = torch.zeros(1, 256, 128, dtype=torch.bfloat16)
    cal = cal_mod.accumulate(((q, q) for _ in range(255)), 0.1, {"a": 7, "b": 7, "c": 9})
    assert cal.n_draws == 255 and calls == {"energy": 255, "select": 2 * 255}
    assert cal.votes["a"] is cal.votes["b"] and cal.votes["a"] is not cal.votes["c"]
    with pytest.raises(ValueError, match="255"):
        cal_mod.accumulate(((q, q) for _ in range(256)), 0.1, {"a": 7})
    assert calls["energy"] == 255 + 255


def test_accumulate_rejects_a_draw_of_another_shape(monkeypatch):
    calls = []
    monkeypatch.setattr(cal_mod, "calibatt_block_energy", lambda *a, **k: calls.append("e"))
    monkeypatch.setattr(cal_mod, "calibatt_build_mask", lambda *a, **k: calls.append("s"))
    monkeypatch.setattr(cal_mod, "calibatt_block_energy_workspace", lambda h, n: 8)
    a = torch.zeros(2, 256, 128, dtype=torch.bfloat16)
    b = torch.zeros(2, 384, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="draw 1"):
        cal_mod.accumulate(iter([(a, a), (b, b)]), 0.1, {0: 7})
    assert calls == ["e", "s"]   # nothing of the second draw was enqueued


def test_schedule_variants_one_parameter_at_a_time():
    v = cal_mod.schedule_variants(50, [0, 25], [0.84, 0.8], [0.99, 0.97, 0.95], [5.0, 3.0])
    assert [(s.A, s.C, s.k) for s in v] == [(0.84, 0.99, 5.0), (0.8, 0.99, 5.0), (0.84, 0.97, 5.0),
                                            (0.84, 0.95, 5.0), (0.84, 0.99, 3.0)]
    assert all(s.T == 50 and s.steps == (0, 25) for s in v)
    assert v[0].label == "T=50 A=0.84 C=0.99 k=5"
    assert len({s for s in v}) == len(v)          # hashable and distinct: usable as keys

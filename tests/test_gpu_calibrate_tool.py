"""GPU: the offline calibration driver (calibrated_block_sparse_amd.calibrate)
on the small synthetic recipe. Votes equal those of direct library calls bit
for bit; the kept density is non-increasing in rho and, within a schedule,
in the step (eps decreases, and a larger eps selects a superset of blocks
per draw, so votes and masks are monotone exactly); the vote histogram
counts every block; the bank it writes returns the finalised lists."""

import json

import numpy as np
import pytest
import torch

from calibrated_block_sparse_amd import calibrate as cal_mod
from calibrated_block_sparse_amd.bank import MaskBank
from synth import CALIB_WORKLOADS, calib_basis, calib_draw, n_blocks
from tests._util import say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def draws(w, n):
    basis = calib_basis(w, DEV)
    return [calib_draw(w, p, basis, DEV) for p in range(n)]


def test_driver_votes_monotone_density_and_bank(gpu, tmp_path):
    w = CALIB_WORKLOADS["calibration_small"]
    R = n_blocks(w.n_tokens)
    grid = (w.grid.frames, w.grid.rows, w.grid.cols, 5)
    say(f"case calibrate driver H={w.heads} N={w.n_tokens}")
    sched = cal_mod.Schedule(50, w.eps_floor, w.eps_start, w.eps_rate, (0, 25, 49))
    ds = draws(w, 6)
    cal = cal_mod.accumulate(ds, w.scale, sched.eps_fx(), grid)
    assert cal.n_draws == 6 and cal.similarity.shape == (w.heads,)
    # votes equal direct calls
    for t, e in sched.eps_fx().items():
        v = torch.zeros(w.heads, R, R, dtype=torch.uint8, device=DEV)
        for q, k in ds:
            gpu.calibatt_build_mask(gpu.block_energy(q, k, w.scale), e, v)
        assert torch.equal(v, cal.votes[t]), t
    rhos = [0.3, 0.4, 0.5, 0.6, 0.7]
    rep = cal_mod.sensitivity(cal, rhos)
    for t in (0, 25, 49):
        d = [rep[str(t)]["density"][str(r)] for r in rhos]
        assert all(a >= b for a, b in zip(d, d[1:])), d
        assert sum(rep[str(t)]["votes"]["histogram"]) == w.heads * R * R
        assert 0.0 <= rep[str(t)]["votes"]["outer_tenths"] <= 1.0
    for r in rhos:
        d = [rep[str(t)]["density"][str(r)] for t in (0, 25, 49)]
        assert all(a >= b for a, b in zip(d, d[1:])), (r, d)
    # the finalised masks are the rho rule, plus one column in rows it leaves empty
    fin = cal_mod.finalize(cal, 0.5)
    for t, (mask, off, idx) in fin.items():
        rule = (cal.votes[t].long() * 2 >= cal.n_draws).cpu().numpy()
        m = mask.cpu().numpy().astype(bool)
        empty = ~rule.any(axis=-1)
        assert np.array_equal(m[~empty], rule[~empty])
        assert (m[empty].sum(axis=-1) == 1).all()
        assert abs(rule.mean() - rep[str(t)]["density"]["0.5"]) < 1e-4
    path = str(tmp_path / "cal.cbsm")
    cal_mod.write_calibration_bank(path, cal, 0.5, grid)
    bank = MaskBank(path)
    for i, t in enumerate(sorted(fin)):
        _, off, idx, flags = bank.lookup_host(i, 0)
        assert np.array_equal(off, fin[t][1].cpu().numpy())
        assert np.array_equal(idx, fin[t][2].cpu().numpy())
    say(f"  density at rho 0.5: {[rep[str(t)]['density']['0.5'] for t in (0, 25, 49)]}")


def test_driver_few_step_schedule_and_cli(gpu, capsys):
    w = CALIB_WORKLOADS["calibration_small"]
    say("case calibrate CLI, T=50 and T=4")
    cal_mod.main(["--workload", "calibration_small", "--draws", "4", "--rho", "0.4", "0.5", "0.6",
                  "--schedule", "50:0,25,49", "4:0,1,2,3"])
    rep = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert set(rep["schedules"]) == {"T=50", "T=4"}
    few = rep["schedules"]["T=4"]
    eps = [few[f"t={t}"]["eps"] for t in range(4)]
    assert all(a > b for a, b in zip(eps, eps[1:]))            # eps(t) decays over 4 steps
    for r in ("0.4", "0.5", "0.6"):
        d = [few[f"t={t}"]["density"][r] for t in range(4)]
        assert all(a >= b for a, b in zip(d, d[1:])), (r, d)
    assert len(rep["similarity"]) == w.heads

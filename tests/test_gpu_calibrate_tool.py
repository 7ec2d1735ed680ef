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
        d = [rep[t]["density"][str(r)] for r in rhos]
        assert all(a >= b for a, b in zip(d, d[1:])), d
        assert sum(rep[t]["votes"]["histogram"]) == w.heads * R * R
        assert 0.0 <= rep[t]["votes"]["outer_tenths"] <= 1.0
    for r in rhos:
        d = [rep[t]["density"][str(r)] for t in (0, 25, 49)]
        assert all(a >= b for a, b in zip(d, d[1:])), (r, d)
    # the finalised masks are the rho rule, plus one column in rows it leaves empty
    fin = cal_mod.finalize(cal, 0.5)
    for t, (mask, off, idx) in fin.items():
        rule = (cal.votes[t].long() * 2 >= cal.n_draws).cpu().numpy()
        m = mask.cpu().numpy().astype(bool)
        empty = ~rule.any(axis=-1)
        assert np.array_equal(m[~empty], rule[~empty])
        assert (m[empty].sum(axis=-1) == 1).all()
        assert abs(m.mean() - rep[t]["density"]["0.5"]) < 1e-6
    path = str(tmp_path / "cal.cbsm")
    cal_mod.write_calibration_bank(path, cal, 0.5, grid)
    bank = MaskBank(path)
    for i, t in enumerate(sorted(fin)):
        _, off, idx, flags = bank.lookup_host(i, 0)
        assert np.array_equal(off, fin[t][1].cpu().numpy())
        assert np.array_equal(idx, fin[t][2].cpu().numpy())
    say(f"  density at rho 0.5: {[rep[t]['density']['0.5'] for t in (0, 25, 49)]}")


def test_driver_few_step_schedule_and_cli(gpu, capsys):
    w = CALIB_WORKLOADS["calibration_small"]
    say("case calibrate CLI, T=50 and T=4")
    cal_mod.main(["--workload", "calibration_small", "--draws", "4", "--rho", "0.4", "0.5", "0.6",
                  "--schedule", "50:0,25,49", "4:0,1,2,3"])
    rep = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert set(rep["schedules"]) == {"T=50 A=0.84 C=0.99 k=5", "T=4 A=0.84 C=0.99 k=5"}
    few = rep["schedules"]["T=4 A=0.84 C=0.99 k=5"]
    eps = [few[f"t={t}"]["eps"] for t in range(4)]
    assert all(a > b for a, b in zip(eps, eps[1:]))            # eps(t) decays over 4 steps
    for r in ("0.4", "0.5", "0.6"):
        d = [few[f"t={t}"]["density"][r] for t in range(4)]
        assert all(a >= b for a, b in zip(d, d[1:])), (r, d)
    assert len(rep["similarity"]) == w.heads


def test_driver_sweeps_schedule_parameters(gpu, capsys):
    """A, C and k varied one at a time from the base schedule: every
    variant is reported, and at each step t > 0 the kept density is monotone
    in each parameter exactly as eps is (a larger eps selects a superset of
    blocks per draw): non-decreasing in A and in C, non-increasing in k.
    At t = 0 eps = C whatever A and k are, so those variants share votes."""
    say("case calibrate CLI, A / C / k sweep")
    cal_mod.main(["--workload", "calibration_small", "--draws", "3", "--rho", "0.5",
                  "--schedule", "50:0,25,49", "--A", "0.84", "0.80", "0.88",
                  "--C", "0.99", "0.97", "--k", "5", "3", "8"])
    rep = json.loads(capsys.readouterr().out.strip().splitlines()[-1])["schedules"]
    lab = lambda A=0.84, C=0.99, k=5: f"T=50 A={A:g} C={C:g} k={k:g}"
    assert set(rep) == {lab(), lab(A=0.80), lab(A=0.88), lab(C=0.97), lab(k=3), lab(k=8)}
    dens = lambda l, t: rep[l][f"t={t}"]["density"]["0.5"]
    eps = lambda l, t: rep[l][f"t={t}"]["eps"]
    for t in (25, 49):
        for lo, hi in ((lab(A=0.80), lab()), (lab(), lab(A=0.88)), (lab(C=0.97), lab()),
                       (lab(k=8), lab()), (lab(), lab(k=3))):
            assert eps(lo, t) < eps(hi, t), (t, lo, hi)
            assert dens(lo, t) <= dens(hi, t), (t, lo, hi, dens(lo, t), dens(hi, t))
    for l in (lab(A=0.80), lab(A=0.88), lab(k=3), lab(k=8)):
        assert dens(l, 0) == dens(lab(), 0) and eps(l, 0) == eps(lab(), 0)
    say("  density at t=49: " + ", ".join(f"{l}: {dens(l, 49):.4f}" for l in sorted(rep)))


def test_sensitivity_masks_match_oracle(gpu):
    """The sweep's compiled masks and densities at every rho equal
    oracle.binarize over oracle votes, where the oracle's greedy selection
    runs on the same fp32 energies the library computed (the energy pass is
    bitwise reproducible, so a separate call gives the energies the driver
    used); the votes themselves are compared first."""
    import oracle
    w = CALIB_WORKLOADS["calibration_small"]
    R = n_blocks(w.n_tokens)
    say(f"case sensitivity vs oracle H={w.heads} N={w.n_tokens}")
    ds = draws(w, 5)
    sched = cal_mod.Schedule(50, w.eps_floor, w.eps_start, w.eps_rate, (0, 25, 49))
    efx = sched.eps_fx()
    cal = cal_mod.accumulate(ds, w.scale, efx)
    energies = [gpu.block_energy(q, k, w.scale).cpu().numpy() for q, k in ds]
    rhos = [0.3, 0.5, 0.7, 1.0]
    dens, masks = cal_mod.densities(cal, rhos, keep_masks=True)
    for t, e in efx.items():
        votes_o = oracle.accumulate_votes([oracle.greedy_select(E, e)[0] for E in energies])
        assert np.array_equal(cal.votes[t].cpu().numpy(), votes_o), t
        for rho in rhos:
            num, den = cal_mod.rho_fraction(rho)
            want = oracle.binarize(votes_o, len(ds), num, den)
            assert np.array_equal(masks[t][rho].cpu().numpy(), want), (t, rho)
            assert dens[t][rho] == want.sum() / (w.heads * R * R), (t, rho)
        say(f"  t={t}: densities {[round(dens[t][r], 4) for r in rhos]}")

"""Offline calibration driver (zhichai.net article on CalibAtt, §三 offline
calibration): for one (layer) over prompt draws, block energies and the
spatial similarity score per draw, greedy selections at eps(t) for every
calibrated step accumulated as votes, then binarisation at rho, statistics
of the vote histogram, repeat flags at gamma, and a mask bank.

Every step runs in the library's kernels (calibatt_block_energy,
calibatt_spatial_similarity, calibatt_build_mask, calibatt_finalize_mask);
this module orchestrates them. `python -m calibrated_block_sparse_amd.calibrate`
runs it on the synthetic calibration recipe and prints a sensitivity report
(kept density and vote-histogram bimodality against rho and the eps
schedule, including a few-step schedule).
"""

from __future__ import annotations

import argparse
import json
from dataclasses import dataclass, field
from fractions import Fraction
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import (calibatt_block_energy, calibatt_block_energy_workspace, calibatt_build_mask,
               calibatt_eps_fx, calibatt_finalize_mask, calibatt_spatial_similarity, n_blocks)

GAMMA = 0.87


@dataclass
class Schedule:
    """eps(t) = A + (C - A) exp(-k t / T) evaluated at the calibrated steps."""
    T: int
    A: float = 0.84
    C: float = 0.99
    k: float = 5.0
    steps: Tuple[int, ...] = ()

    def calibrated_steps(self) -> Tuple[int, ...]:
        return self.steps or tuple(range(self.T))

    def eps_fx(self) -> Dict[int, int]:
        return {t: calibatt_eps_fx(t, self.T, self.A, self.C, self.k) for t in self.calibrated_steps()}


@dataclass
class Calibration:
    """Votes per calibrated step (uint8 CUDA [H][R][R]) after n_draws, and
    the prompt-averaged similarity score per head (None without a grid)."""
    heads: int
    n_tokens: int
    n_draws: int
    votes: Dict[int, torch.Tensor]
    similarity: Optional[np.ndarray] = None
    eps_fx: Dict[int, int] = field(default_factory=dict)


def accumulate(draws: Iterable[Tuple[torch.Tensor, torch.Tensor]], scale: float,
               eps_fx: Dict[int, int], grid: Optional[Sequence[int]] = None) -> Calibration:
    """Run every draw (q, k: [H][N][128] bf16 CUDA) through the energy pass,
    the similarity score (when grid = (frames, rows, cols, anchors)) and the
    greedy selection at each eps; votes saturate at 255 draws."""
    votes = None
    sim_sum = None
    n = 0
    for q, k in draws:
        H, N, _ = q.shape
        R = n_blocks(N)
        if votes is None:
            votes = {t: torch.zeros(H, R, R, dtype=torch.uint8, device=q.device) for t in eps_fx}
            energy = torch.empty(H, R, R, dtype=torch.float32, device=q.device)
            ws = torch.empty(max(calibatt_block_energy_workspace(H, N), 8), dtype=torch.uint8,
                             device=q.device)
            if grid is not None:
                prof = torch.empty(H, grid[0] * grid[1], R, dtype=torch.float32, device=q.device)
                sim = torch.empty(H, dtype=torch.float32, device=q.device)
                sim_sum = torch.zeros(H, dtype=torch.float64, device=q.device)
        calibatt_block_energy(q, k, energy, scale, ws)
        if grid is not None:
            calibatt_spatial_similarity(ws, H, N, grid, prof, sim)
            sim_sum += sim.double()
        for t, e in eps_fx.items():
            calibatt_build_mask(energy, e, votes[t])
        n += 1
    if n == 0:
        raise ValueError("no draws")
    s = None if sim_sum is None else (sim_sum / n).cpu().numpy()
    return Calibration(H, N, n, votes, s, dict(eps_fx))


def rho_fraction(rho: float) -> Tuple[int, int]:
    f = Fraction(rho).limit_denominator(1000)
    return f.numerator, f.denominator


def finalize(cal: Calibration, rho: float = 0.5) -> Dict[int, Tuple[torch.Tensor, torch.Tensor, torch.Tensor]]:
    """Per calibrated step: (mask [H][R][R], kv_offsets, kv_indices[:nnz])."""
    num, den = rho_fraction(rho)
    out = {}
    for t, v in cal.votes.items():
        H, R, _ = v.shape
        mask = torch.empty_like(v)
        off = torch.empty(H * R + 1, dtype=torch.int32, device=v.device)
        idx = torch.empty(max(H * R * R, 1), dtype=torch.int32, device=v.device)
        nnz = calibatt_finalize_mask(v, min(cal.n_draws, 255), num, den, mask, off, idx)
        out[t] = (mask, off, idx[:nnz])
    return out


def vote_stats(votes: torch.Tensor, n_draws: int, bins: int = 10) -> dict:
    """Histogram of per-block vote fractions (the keep-rate histogram the
    pages describe as bimodal, [CalibAtt blog] §二 observation 3), the share
    of blocks in the outer tenths (<= 0.1 or >= 0.9) and Sarle's bimodality
    coefficient (skew^2 + 1) / kurtosis of the fractions."""
    frac = votes.double().flatten() / min(n_draws, 255)
    hist = torch.histc(frac, bins=bins, min=0.0, max=1.0).cpu().numpy()
    outer = float(((frac <= 0.1) | (frac >= 0.9)).double().mean())
    m = float(frac.mean())
    d = frac - m
    var = float((d ** 2).mean())
    if var == 0.0:
        coeff = float("nan")
    else:
        skew = float((d ** 3).mean()) / var ** 1.5
        kurt = float((d ** 4).mean()) / var ** 2
        coeff = (skew ** 2 + 1) / kurt
    return {"histogram": [int(x) for x in hist], "outer_tenths": round(outer, 4),
            "bimodality_coefficient": round(coeff, 4)}


def sensitivity(cal: Calibration, rhos: Sequence[float]) -> dict:
    """Kept density per calibrated step and rho, and the vote statistics."""
    H = cal.heads
    R = n_blocks(cal.n_tokens)
    report = {}
    for t, v in cal.votes.items():
        row = {"eps": cal.eps_fx[t] / 2.0 ** 40, "votes": vote_stats(v, cal.n_draws), "density": {}}
        for rho in rhos:
            num, den = rho_fraction(rho)
            kept = (v.long() * den >= num * min(cal.n_draws, 255)).sum().item()
            row["density"][str(rho)] = round(kept / (H * R * R), 4)
        report[str(t)] = row
    return report


def repeat_flags(cal: Calibration, gamma: float = GAMMA) -> Optional[np.ndarray]:
    """Heads whose prompt-averaged similarity exceeds gamma (uint8 [H])."""
    if cal.similarity is None:
        return None
    return (cal.similarity > gamma).astype(np.uint8)


def write_calibration_bank(path: str, cal: Calibration, rho: float = 0.5,
                           grid: Optional[Sequence[int]] = None, gamma: float = GAMMA) -> None:
    """A one-layer bank with one entry per calibrated step (in ascending step
    order), the repeat flags at gamma in every entry."""
    from .bank import write_bank
    fin = finalize(cal, rho)
    steps = sorted(fin)
    flags = repeat_flags(cal, gamma)
    if flags is not None and not flags.any():
        flags = None
    entries = [(fin[t][1], fin[t][2], flags) for t in steps]
    write_bank(path, len(steps), 1, cal.heads, cal.n_tokens, [[i] for i in range(len(steps))], entries,
               None if grid is None else tuple(grid))


def _synthetic_draws(name: str, n: int, device: str):
    from synth import CALIB_WORKLOADS, calib_basis, calib_draw
    w = CALIB_WORKLOADS[name]
    basis = calib_basis(w, device)
    for p in range(n):
        yield calib_draw(w, p, basis, device)


def main(argv: Optional[List[str]] = None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="calibration_480p")
    ap.add_argument("--draws", type=int, default=16)
    ap.add_argument("--rho", type=float, nargs="+", default=[0.3, 0.4, 0.5, 0.6, 0.7])
    ap.add_argument("--schedule", nargs="+", default=["50:0,25,49", "4:0,1,2,3"],
                    help="T:steps (comma-separated calibrated steps)")
    ap.add_argument("--A", type=float, default=0.84)
    ap.add_argument("--C", type=float, default=0.99)
    ap.add_argument("--k", type=float, default=5.0)
    ap.add_argument("--bank", default=None, help="write a bank of the first schedule at rho 0.5")
    args = ap.parse_args(argv)
    from synth import CALIB_WORKLOADS
    w = CALIB_WORKLOADS[args.workload]
    grid = (w.grid.frames, w.grid.rows, w.grid.cols, 5)
    eps = {}
    scheds = []
    for s in args.schedule:
        T, steps = s.split(":")
        sc = Schedule(int(T), args.A, args.C, args.k, tuple(int(x) for x in steps.split(",")))
        scheds.append(sc)
        for t, e in sc.eps_fx().items():
            eps[(sc.T, t)] = e
    # one pass over the draws serves every schedule (keys are (T, t))
    flat = {i: e for i, e in enumerate(eps.values())}
    keys = list(eps)
    cal = accumulate(_synthetic_draws(args.workload, args.draws, "cuda"), w.scale, flat, grid)
    report = {"workload": args.workload, "draws": args.draws, "rho": args.rho, "schedules": {}}
    sens = sensitivity(cal, args.rho)
    for i, (T, t) in enumerate(keys):
        report["schedules"].setdefault(f"T={T}", {})[f"t={t}"] = sens[str(i)]
    if cal.similarity is not None:
        report["similarity"] = [round(float(x), 4) for x in cal.similarity]
        report["repeat_heads"] = int((cal.similarity > GAMMA).sum())
    if args.bank:
        first = scheds[0]
        sub = Calibration(cal.heads, cal.n_tokens, cal.n_draws,
                          {t: cal.votes[keys.index((first.T, t))] for t in first.calibrated_steps()},
                          cal.similarity, first.eps_fx())
        write_calibration_bank(args.bank, sub, 0.5, grid)
    print(json.dumps(report))


if __name__ == "__main__":
    main()

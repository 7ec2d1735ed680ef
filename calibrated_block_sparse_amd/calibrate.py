"""Offline calibration driver (zhichai.net article on CalibAtt, §三 offline
calibration): for one (layer) over prompt draws, block energies and the
spatial similarity score per draw, greedy selections at eps(t) for every
calibrated step accumulated as votes, then binarisation at rho, statistics
of the vote histogram, repeat flags at gamma, and a mask bank.

Every step runs in the library's kernels (calibatt_block_energy,
calibatt_spatial_similarity, calibatt_build_mask, calibatt_finalize_mask);
this module orchestrates them. `python -m calibrated_block_sparse_amd.calibrate`
runs it on the synthetic calibration recipe and prints a sensitivity report
(kept density of the compiled masks and vote-histogram bimodality against
rho, the number of steps T, and the schedule's floor A, first-step value C
and decay rate k, one parameter varied at a time).
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
MAX_DRAWS = 255   # votes are uint8 counts


@dataclass(frozen=True)
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

    @property
    def label(self) -> str:
        return f"T={self.T} A={self.A:g} C={self.C:g} k={self.k:g}"


def schedule_variants(T: int, steps: Sequence[int], A: Sequence[float], C: Sequence[float],
                      k: Sequence[float]) -> List[Schedule]:
    """The base schedule (the first value of each parameter) and one variant
    per further value of A, C or k, the other two held at their base values
    ([CalibAtt blog] §五: insensitive to large changes of the schedule's
    parameters)."""
    base = Schedule(T, A[0], C[0], k[0], tuple(steps))
    out = [base]
    out += [Schedule(T, a, C[0], k[0], tuple(steps)) for a in A[1:]]
    out += [Schedule(T, A[0], c, k[0], tuple(steps)) for c in C[1:]]
    out += [Schedule(T, A[0], C[0], kk, tuple(steps)) for kk in k[1:]]
    return out


@dataclass
class Calibration:
    """Votes per calibration key (uint8 CUDA [H][R][R]) after n_draws, and
    the prompt-averaged similarity score per head (None without a grid).
    Keys with the same threshold share one votes tensor."""
    heads: int
    n_tokens: int
    n_draws: int
    votes: Dict[object, torch.Tensor]
    similarity: Optional[np.ndarray] = None
    eps_fx: Dict[object, int] = field(default_factory=dict)


def _check_draws(n: int) -> None:
    if not 1 <= n <= MAX_DRAWS:
        raise ValueError(f"{n} draws: votes are 8-bit counts, so 1 to {MAX_DRAWS} draws are supported")


def accumulate(draws: Iterable[Tuple[torch.Tensor, torch.Tensor]], scale: float,
               eps_fx: Dict[object, int], grid: Optional[Sequence[int]] = None) -> Calibration:
    """Run every draw (q, k: [H][N][128] bf16 CUDA) through the energy pass,
    the similarity score (when grid = (frames, rows, cols, anchors)) and the
    greedy selection at each distinct eps. Every draw has the first one's
    shape and device. At most MAX_DRAWS draws (the 255th is the last one
    counted; a 256th raises ValueError before its work is enqueued)."""
    by_eps = {}
    sim_sum = None
    n = 0
    for q, k in draws:
        if n == MAX_DRAWS:
            raise ValueError(f"more than {MAX_DRAWS} draws: votes are 8-bit counts")
        if n > 0 and (tuple(q.shape[:2]) != (H, N) or q.device != energy.device):
            raise ValueError(f"draw {n}: q is {tuple(q.shape)} on {q.device}, the first draw "
                             f"was [{H}, {N}, 128] on {energy.device}")
        H, N, _ = q.shape
        R = n_blocks(N)
        if n == 0:
            by_eps = {e: torch.zeros(H, R, R, dtype=torch.uint8, device=q.device)
                      for e in sorted(set(eps_fx.values()))}
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
        for e, v in by_eps.items():
            calibatt_build_mask(energy, e, v)
        n += 1
    if n == 0:
        raise ValueError("no draws")
    s = None if sim_sum is None else (sim_sum / n).cpu().numpy()
    votes = {key: by_eps[e] for key, e in eps_fx.items()}
    return Calibration(H, N, n, votes, s, dict(eps_fx))


def rho_fraction(rho: float) -> Tuple[int, int]:
    f = Fraction(rho).limit_denominator(1000)
    return f.numerator, f.denominator


def _finalize_votes(v: torch.Tensor, n_draws: int, rho: float):
    """calibatt_finalize_mask of one votes tensor: (mask, kv_offsets,
    kv_indices[:nnz], nnz)."""
    num, den = rho_fraction(rho)
    H, R, _ = v.shape
    mask = torch.empty_like(v)
    off = torch.empty(H * R + 1, dtype=torch.int32, device=v.device)
    idx = torch.empty(max(H * R * R, 1), dtype=torch.int32, device=v.device)
    nnz = calibatt_finalize_mask(v, n_draws, num, den, mask, off, idx)
    return mask, off, idx[:nnz], nnz


def finalize(cal: Calibration, rho: float = 0.5) -> Dict[object, Tuple[torch.Tensor, torch.Tensor, torch.Tensor]]:
    """Per calibration key: (mask [H][R][R], kv_offsets, kv_indices[:nnz])."""
    _check_draws(cal.n_draws)
    out = {}
    for key, v in cal.votes.items():
        mask, off, idx, _ = _finalize_votes(v, cal.n_draws, rho)
        out[key] = (mask, off, idx)
    return out


def vote_stats(votes: torch.Tensor, n_draws: int, bins: int = 10) -> dict:
    """Histogram of per-block vote fractions (the keep-rate histogram the
    pages describe as bimodal, [CalibAtt blog] §二 observation 3), the share
    of blocks in the outer tenths (<= 0.1 or >= 0.9) and Sarle's bimodality
    coefficient (skew^2 + 1) / kurtosis of the fractions."""
    _check_draws(n_draws)
    frac = votes.double().flatten() / n_draws
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


def densities(cal: Calibration, rhos: Sequence[float], keep_masks: bool = False) -> dict:
    """Kept density of the compiled mask (calibatt_finalize_mask: the rho
    rule plus the empty-row column) for every key and rho:
    {key: {rho: density}}, and with keep_masks also {key: {rho: mask}}
    (uint8 CUDA [H][R][R]). Keys sharing a votes tensor are finalised
    once."""
    _check_draws(cal.n_draws)
    H = cal.heads
    R = n_blocks(cal.n_tokens)
    done = {}
    dens, masks = {}, {}
    for key, v in cal.votes.items():
        hit = done.get(id(v))
        if hit is None:
            hit = ({}, {})
            for rho in rhos:
                mask, _, _, nnz = _finalize_votes(v, cal.n_draws, rho)
                hit[0][rho] = nnz / (H * R * R)
                if keep_masks:
                    hit[1][rho] = mask
            done[id(v)] = hit
        dens[key] = dict(hit[0])
        if keep_masks:
            masks[key] = dict(hit[1])
    return (dens, masks) if keep_masks else dens


def sensitivity(cal: Calibration, rhos: Sequence[float]) -> dict:
    """Per key: eps, the compiled-mask density per rho and the vote
    statistics."""
    dens = densities(cal, rhos)
    stats = {}
    report = {}
    for key, v in cal.votes.items():
        st = stats.get(id(v))
        if st is None:
            st = stats[id(v)] = vote_stats(v, cal.n_draws)
        report[key] = {"eps": cal.eps_fx[key] / 2.0 ** 40, "votes": st,
                       "density": {str(r): round(d, 6) for r, d in dens[key].items()}}
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
    ap.add_argument("--A", type=float, nargs="+", default=[0.84],
                    help="floor A; the first value is the base, others are variants")
    ap.add_argument("--C", type=float, nargs="+", default=[0.99], help="first-step value C (as --A)")
    ap.add_argument("--k", type=float, nargs="+", default=[5.0], help="decay rate k (as --A)")
    ap.add_argument("--bank", default=None, help="write a bank of the base schedule of the first T at rho 0.5")
    args = ap.parse_args(argv)
    _check_draws(args.draws)
    from synth import CALIB_WORKLOADS
    w = CALIB_WORKLOADS[args.workload]
    grid = (w.grid.frames, w.grid.rows, w.grid.cols, 5)
    scheds = []
    for sp in args.schedule:
        T, steps = sp.split(":")
        scheds += schedule_variants(int(T), [int(x) for x in steps.split(",")], args.A, args.C, args.k)
    # one pass over the draws serves every schedule; keys are (schedule, t)
    eps = {(sc, t): e for sc in scheds for t, e in sc.eps_fx().items()}
    cal = accumulate(_synthetic_draws(args.workload, args.draws, "cuda"), w.scale, eps, grid)
    report = {"workload": args.workload, "draws": args.draws, "rho": args.rho, "schedules": {}}
    for (sc, t), row in sensitivity(cal, args.rho).items():
        report["schedules"].setdefault(sc.label, {})[f"t={t}"] = row
    if cal.similarity is not None:
        report["similarity"] = [round(float(x), 4) for x in cal.similarity]
        report["repeat_heads"] = int((cal.similarity > GAMMA).sum())
    if args.bank:
        first = scheds[0]
        sub = Calibration(cal.heads, cal.n_tokens, cal.n_draws,
                          {t: cal.votes[(first, t)] for t in first.calibrated_steps()},
                          cal.similarity, first.eps_fx())
        write_calibration_bank(args.bank, sub, 0.5, grid)
    print(json.dumps(report))


if __name__ == "__main__":
    main()

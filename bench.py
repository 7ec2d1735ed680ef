#!/usr/bin/env python3
"""Benchmark of calibrated block-sparse attention on one MI355X.

A step is one block-sparse attention forward (calibatt_sparse_attn_fwd) over
a Wan 2.1 14B-shaped 720p self-attention layer: 40 heads, N = 75600 tokens
(21 frames x 45 x 80), D = 128, bf16, per-head seeded block masks at 62.5%
block sparsity (frame band + random blocks, diagonal kept). Inputs are
resident in HBM before timing starts.

Prints one JSON line. `value` is the effective TFLOP/s over kept blocks:
4 * 128 * 128 * 128 FLOP per kept (query block, key block) pair divided by
the measured time. Also reported: the speedup against the same kernel run
with every block kept, the roofline of the kernel (bf16 MFMA peak), the
other layer shapes and the calibration pass, and the fp64 CPU oracle timed
on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--no-extras] [--no-cpu]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6     # 256 CU x 4 SIMD x 1024 FLOP/clk x 2.4 GHz (AMD spec: 2.5 PFLOP/s)
HBM_PEAK_GBS = 8000.0
PAIR_FLOP = 4.0 * 128 * 128 * 128  # QK^T and PV of one 128x128 block, D = 128
METRIC = "effective TFLOP/s on kept blocks + speedup vs dense mask, Wan-720p shape, 1 GPU"
KERNEL_SOURCES = ("calibrated_block_sparse_amd/csrc/attn_fwd.hip",
                  "calibrated_block_sparse_amd/csrc/device_common.h",
                  "calibrated_block_sparse_amd/csrc/kernels.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    """Hash of what the attention kernel's code is made from: its sources
    and the compiler flags of the library build (paths left out, so that the
    hash does not depend on where the tree sits)."""
    from calibrated_block_sparse_amd.build import HIP_FLAGS
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    h.update(" ".join(f for f in HIP_FLAGS if not os.path.isabs(f)).encode())
    return h.hexdigest()[:16]


def time_launches(fns, steps: int, warmup: int):
    """Runs the launch sequence `fns` (callables enqueueing on torch's current
    stream, the stream the library launches on) `steps` times after `warmup`
    untimed runs. Returns per-step durations (ms) of each callable, from HIP
    events recorded around it on that stream, and the bracketed wall time of
    all steps."""
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
    outer0, outer1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    outer0.record()
    for i in range(steps):
        for j, f in enumerate(fns):
            ev[i][j].record()
            f()
        ev[i][-1].record()
    outer1.record()
    torch.cuda.synchronize()
    per = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(len(fns))] for i in range(steps)])
    return per, outer0.elapsed_time(outer1)


def attn_case(cbs, name: str, steps: int, warmup: int, dense: bool = False, mask=None,
              tensors=None, repeat_value: int = 1):
    from synth import ATTN_WORKLOADS, block_mask, qkv, repeat_flags
    w = ATTN_WORKLOADS[name]
    q, k, v = tensors if tensors is not None else qkv(w, device="cuda")
    o = torch.empty_like(q)
    if mask is None:
        mask = np.ones((w.heads, w.n_blocks, w.n_blocks), np.uint8) if dense else block_mask(w)
    off, idx = cbs.compile_skiplist(torch.from_numpy(mask).cuda())
    flags = repeat_flags(w) * repeat_value
    grid = None
    if flags.any():
        grid = (w.grid.frames, w.grid.rows, w.grid.cols, w.anchors)
    else:
        flags = None
    pairs = int(idx.numel()) if flags is None else int(
        mask[flags == 0].sum() + int((flags != 0).sum()) * -(-(w.grid.frames * w.anchors * w.grid.cols) // 128) * w.n_blocks)

    ws = torch.empty(cbs.calibatt_sparse_attn_fwd_workspace(w.heads, w.n_tokens), dtype=torch.uint8,
                     device="cuda")

    # One step = calibatt_sparse_attn_fwd, issued as its two halves so that
    # the attention kernel's own launches are timed apart from the V^T
    # pre-pass (the full call runs exactly these two launches).
    def prepare():
        cbs.calibatt_prepare_vt(v, ws)

    def attend():
        cbs.calibatt_sparse_attn_fwd_vt(q, k, ws, o, off, idx, w.scale, flags, grid)

    per, total = time_launches([prepare, attend], steps, warmup)
    return dict(workload=w, pairs=pairs, per_ms=per.sum(axis=1), attn_ms=per[:, 1],
                prep_ms=per[:, 0], total_ms=total, mask=mask, tensors=(q, k, v))


def bank_case(cbs, case, steps: int = 50, layers: int = 40, reps: int = 20):
    """Mask bank at the layer's shape: a steps x layers bank whose (t, l)
    share three entries (the layer's mask and two reshuffles of its heads),
    written, opened and uploaded; then the host cost of a lookup and of a
    CalibAttention call against the direct call with the same lists."""
    import tempfile
    from calibrated_block_sparse_amd.bank import CalibAttention, MaskBank, write_bank
    w = case["workload"]
    mask = case["mask"]
    q, k, v = case["tensors"]
    entries = []
    for e in range(3):
        m = mask if e == 0 else mask[np.random.default_rng(e).permutation(w.heads)]
        off, idx = cbs.compile_skiplist(torch.from_numpy(np.ascontiguousarray(m)).cuda())
        entries.append((off.cpu().numpy(), idx.cpu().numpy(), None))
    entry_of = [[(t * layers + l) % 3 for l in range(layers)] for t in range(steps)]
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "bank.cbsm")
        t0 = time.perf_counter()
        write_bank(path, steps, layers, w.heads, w.n_tokens, entry_of, entries)
        t_write = time.perf_counter() - t0
        size = os.path.getsize(path)
        t0 = time.perf_counter()
        bank = MaskBank(path, device="cuda")
        torch.cuda.synchronize()
        t_open = time.perf_counter() - t0
    n = 20000
    t0 = time.perf_counter()
    for i in range(n):
        bank.lookup(i % steps, (i // steps) % layers)
    t_lookup = (time.perf_counter() - t0) / n
    attn = CalibAttention(bank, w.scale)
    lk = bank.lookup(0, 0)
    o = torch.empty_like(q)
    ws = torch.empty(cbs.calibatt_sparse_attn_fwd_workspace(w.heads, w.n_tokens), dtype=torch.uint8,
                     device="cuda")

    def via_bank():
        return attn(q, k, v, 0, 0)

    def direct():
        cbs.calibatt_sparse_attn_fwd(q, k, v, o, lk.kv_offsets, lk.kv_indices, w.scale, workspace=ws)

    ms = {}
    for name, fn in (("bank", via_bank), ("direct", direct)):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        ms[name] = (time.perf_counter() - t0) * 1e3 / reps
    out_bank = via_bank()
    direct()
    torch.cuda.synchronize()
    bank.close()
    return {"steps_x_layers": [steps, layers], "entries": 3, "file_mb": round(size / 2 ** 20, 2),
            "write_s": round(t_write, 3), "open_upload_s": round(t_open, 3),
            "lookup_us": round(t_lookup * 1e6, 2),
            "attention_ms_via_bank": round(ms["bank"], 3), "attention_ms_direct": round(ms["direct"], 3),
            "bitwise_equal": bool(torch.equal(out_bank, o))}


def noalloc_case(cbs, case, reps: int = 10):
    """calibatt_sparse_attn_fwd_noalloc on the same layer and lists: its V^T
    tiles go to the library's 256 MiB scratch, heads in chunks that fit
    (pre-pass and attention per chunk); per-call time against the
    workspace call (both including the V^T pre-pass), outputs compared."""
    w = case["workload"]
    q, k, v = case["tensors"]
    off, idx = cbs.compile_skiplist(torch.from_numpy(case["mask"]).cuda())
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(cbs.calibatt_sparse_attn_fwd_workspace(w.heads, w.n_tokens), dtype=torch.uint8,
                     device="cuda")
    fns = {"workspace": lambda: cbs.calibatt_sparse_attn_fwd(q, k, v, o1, off, idx, w.scale, workspace=ws),
           "noalloc": lambda: cbs.calibatt_sparse_attn_fwd_noalloc(q, k, v, o2, off, idx, w.scale)}
    ms = {}
    for name, fn in fns.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms[name] = e0.elapsed_time(e1) / reps
    R = w.n_blocks
    per = -(-w.heads // -(-w.heads // (8192 // R)))
    return {"workload": w.name, "head_chunks": -(-w.heads // per), "heads_per_chunk": per,
            "ms": round(ms["noalloc"], 3), "workspace_call_ms": round(ms["workspace"], 3),
            "bitwise_equal": bool(torch.equal(o1, o2))}


SWEEP_FRACTIONS = (1.0, 0.75, 0.5, 0.375, 0.25, 0.125)


def sweep_case(cbs, name: str, tensors, steps: int = 5, warmup: int = 2):
    """Kept-fraction sweep at one shape: band + random masks at each kept
    fraction, median step time of the attention kernel, and a least-squares
    line of time against kept pairs (slope, intercept, R^2)."""
    from synth import ATTN_WORKLOADS, mask_for_fraction
    w = ATTN_WORKLOADS[name]
    rows = []
    for f in SWEEP_FRACTIONS:
        mask = mask_for_fraction(w, f)
        c = attn_case(cbs, name, steps, warmup, mask=mask, tensors=tensors)
        ms = float(np.median(c["attn_ms"]))
        rows.append((f, c["pairs"], ms))
        del c
    x = np.array([r[1] for r in rows], dtype=np.float64)
    y = np.array([r[2] for r in rows], dtype=np.float64)
    slope, icpt = np.polyfit(x, y, 1)
    r2 = 1.0 - float(np.sum((y - (slope * x + icpt)) ** 2)) / float(np.sum((y - y.mean()) ** 2))
    return {
        "workload": name,
        "kept_fraction": [r[0] for r in rows],
        "pairs": [r[1] for r in rows],
        "attn_ms": [round(r[2], 3) for r in rows],
        "tflops": [round(r[1] * PAIR_FLOP / (r[2] * 1e-3) / 1e12, 1) for r in rows],
        "fit_ms_per_million_pairs": round(slope * 1e6, 4),
        "fit_intercept_ms": round(icpt, 4),
        "fit_r2": round(r2, 6),
    }


def mfma_probe_case(cbs, iters: int = 20000, workgroups: int = 2048, reps: int = 3):
    """Sustained matrix-core rate on this device (register-operand MFMA
    loop), TFLOP/s: the median of `reps` timed launches after one warm-up."""
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    cbs.calibatt_mfma_rate_probe(sink, iters, workgroups)
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        flop = cbs.calibatt_mfma_rate_probe(sink, iters, workgroups)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    return flop / (ms * 1e-3) / 1e12, ms


# Issue cost of one 128 x 128 energy tile in SIMD cycles. VALU: 16384
# scores, each an fma, an exp2 and an add (256 wave64 instructions of each);
# fma and add at the published fp32 vector rate (157.3 TFLOP/s = 1024 SIMDs
# x 2.4 GHz x 32 lanes x 2 FLOP: a wave64 instruction every 2 cycles),
# v_exp_f32 at a quarter of it (8 cycles; a register-only probe with two
# waves per SIMD measures 8.2 for v_exp_f32 and 2.7 for v_fma_f32). MFMA:
# 2 * 128^3 FLOP at 1024 FLOP per cycle.
ENERGY_TILE_VALU_CYCLES = 256 * (2 + 8 + 2)
ENERGY_TILE_MFMA_CYCLES = 2 * 128 ** 3 // 1024
SIMDS = 256 * 4
NOMINAL_CLOCK_HZ = 2.4e9


def calibration_case(cbs, draws: int):
    """The calibration pass as configured: 40 heads, N = 32760, `draws`
    prompt draws; per draw the energy pass, the spatial-similarity score and
    the greedy selection at eps(t) for t in {0, 25, 49} into votes; then for
    each t binarisation at rho = 1/2 and kept-list compilation. Per-stage
    device times from HIP events on the launch stream (the synthetic draws
    are generated between the timed stages and not counted), the kept
    fractions, and the keep-rate (vote fraction) histograms."""
    from calibrated_block_sparse_amd.calibrate import vote_stats
    from synth import CALIB_WORKLOADS, calib_basis, calib_draw, n_blocks
    w = CALIB_WORKLOADS["calibration_480p"]
    R = n_blocks(w.n_tokens)
    basis = calib_basis(w, "cuda")
    energy = torch.empty(w.heads, R, R, dtype=torch.float32, device="cuda")
    ws = torch.empty(cbs.calibatt_block_energy_workspace(w.heads, w.n_tokens), dtype=torch.uint8,
                     device="cuda")
    votes = {t: torch.zeros(w.heads, R, R, dtype=torch.uint8, device="cuda") for t in w.steps}
    efx = {t: cbs.calibatt_eps_fx(t, w.total_steps, w.eps_floor, w.eps_start, w.eps_rate)
           for t in w.steps}
    grid = (w.grid.frames, w.grid.rows, w.grid.cols, 5)
    prof = torch.empty(w.heads, w.grid.frames * w.grid.rows, R, dtype=torch.float32, device="cuda")
    sim = torch.empty(w.heads, dtype=torch.float32, device="cuda")
    sim_sum = torch.zeros(w.heads, dtype=torch.float64, device="cuda")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(draws)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for p in range(draws):
        q, k = calib_draw(w, p, basis, "cuda")
        ev[p][0].record()
        cbs.calibatt_block_energy(q, k, energy, w.scale, ws)
        ev[p][1].record()
        cbs.calibatt_spatial_similarity(ws, w.heads, w.n_tokens, grid, prof, sim)
        ev[p][2].record()
        for t in w.steps:
            cbs.calibatt_build_mask(energy, efx[t], votes[t])
        ev[p][3].record()
        sim_sum += sim.double()
    torch.cuda.synchronize()
    t_energy = sum(e[0].elapsed_time(e[1]) for e in ev)
    t_sim = sum(e[1].elapsed_time(e[2]) for e in ev)
    t_select = sum(e[2].elapsed_time(e[3]) for e in ev)
    s_mean = (sim_sum / draws).cpu().numpy()
    mask = torch.empty(w.heads, R, R, dtype=torch.uint8, device="cuda")
    off = torch.empty(w.heads * R + 1, dtype=torch.int32, device="cuda")
    idx = torch.empty(w.heads * R * R, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    kept = {}
    t_fin = 0.0
    for t in w.steps:
        e0.record()
        nnz = cbs.calibatt_finalize_mask(votes[t], draws, *w.rho, mask, off, idx)
        e1.record()
        torch.cuda.synchronize()
        t_fin += e0.elapsed_time(e1)
        kept[t] = nnz / (w.heads * R * R)
    t_wall = time.perf_counter() - t_wall
    tiles = w.heads * R * R
    flop_energy = 2.0 * tiles * 128 ** 3      # one Q K^T pass over every pair
    e_ms = t_energy / draws
    valu_bound_ms = tiles * ENERGY_TILE_VALU_CYCLES / (SIMDS * NOMINAL_CLOCK_HZ) * 1e3
    mfma_bound_ms = tiles * ENERGY_TILE_MFMA_CYCLES / (SIMDS * NOMINAL_CLOCK_HZ) * 1e3
    return {
        "workload": "calibration_480p", "heads": w.heads, "n_tokens": w.n_tokens, "draws": draws,
        "steps": list(w.steps), "rho": list(w.rho),
        "device_ms_total": round(t_energy + t_sim + t_select + t_fin, 2),
        "wall_s_incl_synthetic_draws": round(t_wall, 2),
        "energy_ms_per_draw": round(e_ms, 3),
        "energy_tflops": round(flop_energy / (e_ms * 1e-3) / 1e12, 1),
        "energy_mfma_frac": round(flop_energy / (e_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "energy_mfma_bound_ms": round(mfma_bound_ms, 3),
        "energy_valu_bound_ms": round(valu_bound_ms, 3),
        "energy_valu_frac": round(valu_bound_ms / e_ms, 4),
        # the time with no overlap of matrix-core and vector issue
        "energy_mfma_plus_valu_bound_ms": round(mfma_bound_ms + valu_bound_ms, 3),
        "energy_mfma_plus_valu_frac": round((mfma_bound_ms + valu_bound_ms) / e_ms, 4),
        "select_votes_ms_per_draw_3eps": round(t_select / draws, 3),
        "similarity_ms_per_draw": round(t_sim / draws, 3),
        "finalize_compile_ms_3steps": round(t_fin, 3),
        "similarity_mean_min_max": [round(float(s_mean.mean()), 4), round(float(s_mean.min()), 4),
                                    round(float(s_mean.max()), 4)],
        "repeat_heads_at_gamma_0_87": int((s_mean > 0.87).sum()),
        "kept_fraction_by_step": {str(t): round(v, 4) for t, v in kept.items()},
        "keep_rate_histogram_by_step": {str(t): vote_stats(votes[t], draws)["histogram"]
                                        for t in w.steps},
        "_energy_last_draw": energy,
    }


def cpu_calibration_baseline(energy_gpu, seconds: float = 10.0):
    """The fp64 oracle on one calibration draw: block energies of draw 0,
    head 0, block-row by block-row for about `seconds`, extrapolated to all
    heads and rows of the draw, plus the oracle's greedy selection at the
    three eps(t) and binarisation over every head's rows (run in full, on the
    library's energies of the last draw)."""
    import oracle
    from synth import CALIB_WORKLOADS, bf16_bits, calib_basis, calib_draw, n_blocks
    w = CALIB_WORKLOADS["calibration_480p"]
    R = n_blocks(w.n_tokens)
    q, k = calib_draw(w, 0, calib_basis(w, "cpu"), "cpu", heads=1)
    qb, kb = oracle.as_f64(bf16_bits(q[0])), oracle.as_f64(bf16_bits(k[0]))
    t0 = time.perf_counter()
    rows = 0
    while time.perf_counter() - t0 < seconds and rows < R:
        oracle.block_energy_row(qb, kb, w.scale, rows)
        rows += 1
    t_rows = time.perf_counter() - t0
    E = energy_gpu.cpu().numpy().astype(np.float64)
    t0 = time.perf_counter()
    for t in w.steps:
        eps = oracle.eps_fx(oracle.eps_schedule(t, w.total_steps, w.eps_floor, w.eps_start, w.eps_rate))
        sel, _ = oracle.greedy_select(E, eps)
        oracle.binarize(sel, 1, *w.rho)
    t_sel = time.perf_counter() - t0
    per_draw_s = t_rows / rows * R * w.heads + t_sel
    return {"value": round(per_draw_s, 2), "unit": "s per calibration draw (40 heads, 3 eps)",
            "cores": _blas_threads(), "kind": "oracle",
            "sample": f"energy of head 0 block-rows 0..{rows - 1} of draw 0 ({t_rows:.1f} s, "
                      f"extrapolated to {R} rows x {w.heads} heads); greedy selection at 3 eps and "
                      f"binarisation of all 40 heads run in full ({t_sel:.1f} s)"}


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return int(os.cpu_count() or 1)


def cpu_baseline(case, seconds: float = 15.0):
    """The fp64 oracle on host cores over whole query blocks of head 0 of the
    same workload, until about `seconds` of work; scaled to TFLOP/s over the
    kept pairs it covered."""
    import oracle
    from synth import bf16_bits
    cores = _blas_threads()
    w = case["workload"]
    mask = case["mask"]
    q, k, v = case["tensors"]
    qb, kb, vb = (oracle.as_f64(bf16_bits(t[0])) for t in (q, k, v))
    pairs = 0
    blocks = 0
    t0 = time.perf_counter()
    r = 0
    while time.perf_counter() - t0 < seconds and r < w.n_blocks:
        cols = np.flatnonzero(mask[0, r])
        oracle.block_sparse_attention_block(qb, kb, vb, w.scale, cols, r)
        pairs += cols.size
        blocks += 1
        r += 1
    dt = time.perf_counter() - t0
    return {"value": round(pairs * PAIR_FLOP / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "host_cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "sample": f"{w.name} head 0, query blocks 0..{blocks - 1} ({pairs} kept pairs, fp64 numpy), {dt:.1f} s"}


def traffic_record():
    """HBM bytes per launch from committed rocprofv3 counter runs, valid only
    while the kernel sources are unchanged."""
    p = os.path.join(ROOT, "profiles", "attn_fwd_wan21_720p_counters.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("kernel_hash") != kernel_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan21_720p_layer")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calib-draws", type=int, default=64)
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-mask run")
    ap.add_argument("--no-sweep", action="store_true", help="skip the kept-fraction sweep")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (counter reference)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(heads would shard across GPUs without communication)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    import calibrated_block_sparse_amd as cbs
    cbs.load_library()

    if args.copy_ref_mib:
        n = args.copy_ref_mib * 2 ** 20 // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] reference copy of {args.copy_ref_mib} MiB done")
        del src, dst
    log(f"[bench] {args.workload}: sparse mask, {args.steps} steps after {args.warmup} warmup")
    sp = attn_case(cbs, args.workload, args.steps, args.warmup)
    w = sp["workload"]
    ms = float(np.median(sp["per_ms"]))
    ms_step = sp["total_ms"] / args.steps
    flop = sp["pairs"] * PAIR_FLOP
    eff = flop / (ms_step * 1e-3) / 1e12
    log(f"[bench] sparse: {ms_step:.3f} ms/step, {eff:.1f} TFLOP/s effective")

    dense_ms = dense_tflops = None
    if not args.no_dense:
        log("[bench] dense mask (every block kept)")
        dn = attn_case(cbs, args.workload, max(3, args.steps // 4), 2, dense=True)
        dense_ms = float(np.median(dn["per_ms"]))
        dense_tflops = dn["pairs"] * PAIR_FLOP / (dense_ms * 1e-3) / 1e12
        del dn

    # roofline of the dominant kernel: its own launches (the V^T pre-pass,
    # under 1% of a step, is reported beside it)
    per_launch_ms = float(np.mean(sp["attn_ms"]))
    achieved = flop / (per_launch_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(eff, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "heads": w.heads, "n_tokens": w.n_tokens,
                   "head_dim": w.head_dim, "block": 128, "block_sparsity": w.sparsity,
                   "kept_pairs": sp["pairs"], "frames_x_rows_x_cols": [w.grid.frames, w.grid.rows, w.grid.cols]},
        "speedup_vs_dense_mask": round(dense_ms / ms, 3) if dense_ms else None,
        "dense_mask": {"ms": round(dense_ms, 3), "tflops": round(dense_tflops, 1)} if dense_ms else None,
        "sparse_ms_p10_p50_p90": [round(float(x), 4) for x in np.percentile(sp["per_ms"], [10, 50, 90])],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_record(), "kernel": "calibatt::attn_fwd_kernel",
                     "kernel_ms_mean": round(per_launch_ms, 4), "kernel_hash": kernel_hash()},
        "v_transpose_ms_mean": round(float(np.mean(sp["prep_ms"])), 4),
    }
    if out["roofline"]["traffic"]:
        out["roofline"]["achieved_hbm_gbs"] = round(out["roofline"]["traffic"] / (per_launch_ms * 1e-3) / 1e9, 1)
    # the pages' own end-to-end numbers (video generation, hardware and precision
    # not stated): context only, not comparable with a kernel rate
    out["pages_context_end_to_end"] = {
        "wan21_14b_720p": {"dense_s": 1244, "calibatt_s": 785, "speedup": 1.58, "block_sparsity": 0.625},
        "wan21_14b_480p": {"dense_s": 363, "calibatt_s": 250, "speedup": 1.45, "block_sparsity": 0.681},
        "mochi1_480p": {"dense_s": 188, "calibatt_s": 161, "speedup": 1.16, "block_sparsity": 0.691},
    }
    log("[bench] matrix-core rate probe")
    onbox, probe_ms = mfma_probe_case(cbs)
    out["roofline"]["onbox_mfma_loop_tflops"] = round(onbox, 1)
    out["roofline"]["frac_of_onbox_mfma_loop"] = round(achieved / onbox, 4)
    if not args.no_sweep:
        log("[bench] kept-fraction sweep")
        out["sweep"] = sweep_case(cbs, args.workload, sp["tensors"])
    if not args.no_extras:
        extras = {}
        for name in ("wan21_480p_layer", "mochi1_480p_layer"):
            if name == args.workload:
                continue
            log(f"[bench] extra: {name}")
            c = attn_case(cbs, name, 10, 3)
            m = float(np.median(c["per_ms"]))
            extras[name] = {"ms": round(m, 3), "pairs": c["pairs"],
                            "effective_tflops": round(c["pairs"] * PAIR_FLOP / (m * 1e-3) / 1e12, 1)}
            del c
        log("[bench] extra: masked repeat heads (Mochi 480p)")
        c = attn_case(cbs, "mochi1_480p_layer", 10, 3, repeat_value=2)
        extras["mochi1_480p_layer_masked_repeat"] = {
            "ms": round(float(np.median(c["per_ms"])), 3),
            "plain_repeat_ms": extras.get("mochi1_480p_layer", {}).get("ms")}
        del c
        log("[bench] extra: mask bank")
        extras["mask_bank"] = bank_case(cbs, sp)
        log("[bench] extra: attention without workspace (calibatt_sparse_attn_fwd_noalloc)")
        extras["noalloc"] = noalloc_case(cbs, sp)
        log(f"[bench] extra: calibration, {args.calib_draws} draws")
        cal = calibration_case(cbs, args.calib_draws)
        e_last = cal.pop("_energy_last_draw")
        extras["calibration"] = cal
        out["extras"] = extras
    if not args.no_cpu:
        log("[bench] cpu baseline (fp64 oracle)")
        out["cpu_baseline"] = cpu_baseline(sp)
        if not args.no_extras:
            log("[bench] cpu baseline of one calibration draw (fp64 oracle)")
            cb = cpu_calibration_baseline(e_last)
            cb["gpu_s_per_draw"] = round(out["extras"]["calibration"]["device_ms_total"]
                                         / args.calib_draws / 1e3, 4)
            out["extras"]["calibration"]["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

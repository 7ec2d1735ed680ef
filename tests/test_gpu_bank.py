"""GPU: attention through the mask bank. The uploaded lists equal the host
copies bit for bit; calibatt::sparse_attn / CalibAttention for (t, l) give
exactly the output of calibatt_sparse_attn_fwd called with that entry's
lists and flags, and match the oracle (max-abs <= 2e-2, rel-Frobenius <=
1e-2); a bank written from a calibration run returns the finalised lists."""

import numpy as np
import pytest
import torch

import oracle
from calibrated_block_sparse_amd.bank import CalibAttention, MaskBank, write_bank
from synth import CALIB_WORKLOADS, bernoulli_mask, bf16_bits, calib_basis, calib_draw, gaussian_bf16, n_blocks
from tests._util import assert_attn_close, f64, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_bank_attention_matches_direct_call_and_oracle(gpu, tmp_path):
    H, N = 3, 1000
    grid = (2, 20, 25, 5)
    R = n_blocks(N)
    scale = 128 ** -0.5
    say(f"case bank attention H={H} N={N}")
    entries = []
    for i, (seed, flags) in enumerate([(81, [0, 0, 0]), (82, [0, 1, 0]), (83, [1, 0, 1])]):
        mask = bernoulli_mask(seed, H, R, 0.35, True)
        off, idx = oracle.compile_skiplist(mask)
        entries.append((off.astype(np.int32), idx.astype(np.int32), np.array(flags, np.uint8), mask))
    entry_of = [[0, 1], [2, 0]]
    path = str(tmp_path / "bank.cbsm")
    write_bank(path, 2, 2, H, N, entry_of, [e[:3] for e in entries], grid)
    bank = MaskBank(path, device=DEV)
    attn = CalibAttention(bank, scale)
    q = gaussian_bf16(91, (H, N, 128)).to(DEV)
    k = gaussian_bf16(92, (H, N, 128)).to(DEV)
    v = gaussian_bf16(93, (H, N, 128)).to(DEV)
    qb, kb, vb = ([bf16_bits(t[h]) for h in range(H)] for t in (q, k, v))
    for t in range(2):
        for l in range(2):
            e = entry_of[t][l]
            off, idx, flags, mask = entries[e]
            lk = bank.lookup(t, l)
            assert lk.entry == e
            assert np.array_equal(lk.kv_offsets.cpu().numpy(), off)
            assert np.array_equal(lk.kv_indices.cpu().numpy(), idx)
            assert np.array_equal(lk.repeat_flags, flags)
            o_bank = attn(q, k, v, t, l)
            o_dir = torch.empty_like(q)
            gpu.calibatt_sparse_attn_fwd(q, k, v, o_dir, torch.from_numpy(off).to(DEV),
                                         torch.from_numpy(idx).to(DEV), scale,
                                         flags if flags.any() else None,
                                         grid if flags.any() else None)
            torch.cuda.synchronize()
            assert torch.equal(o_bank, o_dir), f"(t, l) = ({t}, {l})"
            for h in range(H):
                if flags[h]:
                    want = oracle.repeat_head_attention(qb[h], kb[h], vb[h], scale, *grid)
                else:
                    want = oracle.block_sparse_attention(qb[h], kb[h], vb[h], scale, mask[h])
                e_ = assert_attn_close(f64(o_bank[h]), want, f"(t, l) = ({t}, {l}) head {h}")
            say(f"  (t, l) = ({t}, {l}) entry {e}: last head max-abs {e_[0]:.2e}")
    # one V^T workspace serves every call of the module
    ws = attn._workspace(q)
    assert ws.numel() == gpu.calibatt_sparse_attn_fwd_workspace(H, N)
    ptr = ws.data_ptr()
    o1 = attn(q, k, v, 1, 0)
    assert attn._workspace(q).data_ptr() == ptr
    # a caller-owned workspace gives the same output
    own = torch.empty(gpu.calibatt_sparse_attn_fwd_workspace(H, N), dtype=torch.uint8, device=DEV)
    o2 = CalibAttention(bank, scale, workspace=own)(q, k, v, 1, 0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    bank.close()


def test_calibration_run_to_bank(gpu, tmp_path):
    """Calibration (GPU energies, selections at the three eps(t), votes,
    binarisation) written as a bank with one entry per calibrated step; the
    bank returns exactly the finalised lists and attention through it equals
    the direct call."""
    w = CALIB_WORKLOADS["calibration_small"]
    R = n_blocks(w.n_tokens)
    say(f"case calibration -> bank H={w.heads} N={w.n_tokens} draws={w.draws}")
    basis = calib_basis(w, DEV)
    votes = {t: torch.zeros(w.heads, R, R, dtype=torch.uint8, device=DEV) for t in w.steps}
    for p in range(w.draws):
        q, k = calib_draw(w, p, basis, DEV)
        e = gpu.block_energy(q, k, w.scale)
        for t in w.steps:
            gpu.calibatt_build_mask(e, gpu.calibatt_eps_fx(t, w.total_steps, w.eps_floor,
                                                           w.eps_start, w.eps_rate), votes[t])
    lists = []
    for t in w.steps:
        mask = torch.empty(w.heads, R, R, dtype=torch.uint8, device=DEV)
        off = torch.empty(w.heads * R + 1, dtype=torch.int32, device=DEV)
        idx = torch.empty(w.heads * R * R, dtype=torch.int32, device=DEV)
        nnz = gpu.calibatt_finalize_mask(votes[t], w.draws, *w.rho, mask, off, idx)
        lists.append((off.cpu().numpy(), idx[:nnz].cpu().numpy(), None))
    path = str(tmp_path / "calib.cbsm")
    write_bank(path, len(w.steps), 1, w.heads, w.n_tokens, [[i] for i in range(len(w.steps))], lists)
    bank = MaskBank(path, device=DEV)
    attn = CalibAttention(bank, w.scale)
    q = gaussian_bf16(95, (w.heads, w.n_tokens, 128)).to(DEV)
    k = gaussian_bf16(96, (w.heads, w.n_tokens, 128)).to(DEV)
    v = gaussian_bf16(97, (w.heads, w.n_tokens, 128)).to(DEV)
    for i, t in enumerate(w.steps):
        lk = bank.lookup(i, 0)
        assert np.array_equal(lk.kv_offsets.cpu().numpy(), lists[i][0])
        assert np.array_equal(lk.kv_indices.cpu().numpy(), lists[i][1])
        o_bank = attn(q, k, v, i, 0)
        o_dir = gpu.sparse_attention(q, k, v, torch.from_numpy(lists[i][0]).to(DEV),
                                     torch.from_numpy(lists[i][1]).to(DEV), w.scale)
        torch.cuda.synchronize()
        assert torch.equal(o_bank, o_dir)
        say(f"  step {t}: {lists[i][1].size} kept blocks")
    bank.close()

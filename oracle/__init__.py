"""fp64 CPU oracle for calibrated block-sparse attention (CalibAtt).

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. The library under
calibrated_block_sparse_amd/ never imports it and shares no code with it.

It is a plain, slow, obviously correct numpy implementation of what the
method computes, written from the pages:

* "让视频生成快 1.58 倍，却不改一行模型代码：CalibAtt 的"注意力考古学"" (zhichai.net),
  cited below as [CalibAtt blog] with its section numbers;
* "Accelerating Text-to-Video Generation with Calibrated Sparse Attention"
  (the paper's abstract, as reposted), cited as [abstract].

Floating point is fp64 throughout; bf16 inputs are decoded exactly.

Pins (what ties each function to something other than itself) live in
tests/test_oracle_*.py. One function is not pinned to anything independent:
the selection on energies that come from attention rather than from a given
array is only as good as its two pinned halves (energy, selection). The
spatial similarity score is PARITY UNPINNED as to its formula (the pages
give none; calibration.py states the reading taken), and pinned to that
reading by closed forms.
"""

from .attention import (  # noqa: F401
    BLOCK, as_f64, dense_attention, kept_keys, block_sparse_attention_block,
    block_sparse_attention, check_anchor_geometry, anchor_rows, anchor_of_row, repeat_source_token,
    repeat_head_attention, repeat_head_attention_masked,
)
from .calibration import (  # noqa: F401
    FX_BITS, block_energy_row, block_energy, quantize_energy, eps_schedule,
    eps_fx, greedy_select_row, greedy_select, accumulate_votes, binarize,
    compile_skiplist, skiplist_to_mask,
    GAMMA, row_profiles, spatial_similarity, classify_repeat,
)

"""Seeded verify batches for greedy MTP verify/accept.

The verify batch of "Support Step3.5/3.7 flash mtp3" (Overview, data-flow
trace of one MTP step) is the last accepted token plus up to three drafts;
the target returns logits for every row and its hidden state per row.  The
pages give no vocabulary size: the workload below takes 131072 columns (a
128k-class vocabulary) and the Step-5 hidden size 4096 ("Step-5 Preview
GGUF", Model background, configuration table) for the hidden-state rows.

Logits are N(0, 1) in float32.  To steer how many drafts a batch accepts,
row j gets one planted column set to ``spike`` (far above the N(0, 1)
maximum of a row), and the drafts copy the planted columns of the first
``n_plan`` rows, then differ at row ``n_plan``.  Nothing here takes an
argmax or applies the accept rule: what the batch accepts is for the oracle
and the kernel to work out.
"""

from __future__ import annotations

import dataclasses

import numpy as np

_MASTER_SEED = 20261202
_T_VERIFY = 9

# Verify/accept workload timed by the bench: four verify rows (the last
# accepted token and three drafts), 131072-column logits, hidden size 4096.
ACCEPT_WORKLOADS = {
    "accept_m4": dict(rows=4, vocab=131072, h_dim=4096),
}


@dataclasses.dataclass
class VerifyBatch:
    logits: np.ndarray    # [M][V] float32
    drafts: np.ndarray    # [M-1] int32
    verify_h: np.ndarray  # [M][h_dim] float32 (h_dim may be 0)
    planted: np.ndarray   # [M] int32, the planted column of each row


def draw_verify_batch(rows: int, vocab: int, h_dim: int, n_plan: int, seed: int = 0,
                      spike: float = 8.0) -> VerifyBatch:
    """Seeded verify batch of `rows` rows; 0 <= n_plan <= rows - 1."""
    if not 0 <= n_plan <= max(rows - 1, 0):
        raise ValueError("n_plan must lie in [0, rows - 1]")
    rng = np.random.default_rng(np.random.SeedSequence([_MASTER_SEED, _T_VERIFY, seed, rows, vocab]))
    logits = rng.standard_normal((rows, vocab), dtype=np.float32)
    planted = rng.integers(0, vocab, rows).astype(np.int32)
    logits[np.arange(rows), planted] = np.float32(spike)
    drafts = rng.integers(0, vocab, max(rows - 1, 0)).astype(np.int32)
    drafts[:n_plan] = planted[:n_plan]
    if n_plan < rows - 1 and vocab > 1:
        # A draft that differs from the planted column of row n_plan.
        drafts[n_plan] = (planted[n_plan] + 1 + rng.integers(0, vocab - 1)) % vocab
    verify_h = rng.standard_normal((rows, h_dim), dtype=np.float32)
    return VerifyBatch(logits, drafts, verify_h, planted)

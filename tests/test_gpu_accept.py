"""GPU parity of greedy MTP verify/accept (include/moe_accept.h) against the
CPU oracle (oracle/accept_oracle.py), every call through the C ABI.

Tokens, n_accepted and the accepted list are integers: bit-exact.  pending_h
is a copy of one verify row: bit-exact.  Comparisons on both sides are exact
on the same fp32 values, so ties are decided by the same rule (lower index).

Cases: the pages' worked trace; seeded batches over rows 1..64 and
vocabularies from 1 column to several workgroups with ragged tails, with
every planned acceptance count; equal maxima inside and across workgroups;
signed zeros and infinities; NaN (the library's documented rule); rows that
are not 16-byte aligned; a vocabulary that takes several passes per
workgroup; repeated calls on one workspace; the bench workload at full size.
"""

import os

import numpy as np
import pytest
import torch

import speculative_verify_router_amd as svr
import synth
from gpu_common import dev, log
from oracle import accept_oracle as ao

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "accept_trace.txt")


def gpu_accept(logits: np.ndarray, drafts, verify_h=None, ws=None, misalign=False):
    """Run moe_verify_accept; returns (tokens, accepted, n, pending or None)."""
    L = np.ascontiguousarray(logits, dtype=np.float32)
    M, V = L.shape
    if misalign:
        # Rows start 4 bytes past a 16-byte boundary: the scalar-load path.
        buf = torch.empty(M * V + 1, dtype=torch.float32, device="cuda")
        buf[1:].copy_(torch.from_numpy(L.reshape(-1)).to("cuda"))
        ld = buf[1:].view(M, V)
        assert ld.data_ptr() % 16 == 4
    else:
        ld = dev(L)
    dr = dev(np.asarray(drafts, dtype=np.int32)) if M > 1 else None
    vh = None if verify_h is None else dev(np.asarray(verify_h, dtype=np.float32))
    tok = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    acc = torch.full((M,), -7, dtype=torch.int32, device="cuda")
    n = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pend = None if vh is None else torch.full((vh.shape[1],), np.nan, dtype=torch.float32,
                                             device="cuda")
    svr.moe_verify_accept(ld, dr, tok, acc, n, vh, pend, ws=ws)
    torch.cuda.synchronize()
    return (tok.cpu().numpy(), acc.cpu().numpy(), int(n.cpu().item()),
            None if pend is None else pend.cpu().numpy())


def check(logits, drafts, verify_h=None, **kw):
    ref = ao.verify_accept(logits, drafts, verify_h)
    tok, acc, n, pend = gpu_accept(logits, drafts, verify_h, **kw)
    M = np.atleast_2d(logits).shape[0]
    assert tok.tolist() == ref["tokens"]
    assert n == ref["n_accepted"]
    want = ref["accepted"] + [-1] * (M - len(ref["accepted"]))
    assert acc.tolist() == want
    if verify_h is not None:
        assert np.array_equal(pend, ref["pending_h"])  # bit-exact copy
    return ref


def test_worked_trace_of_the_pages():
    kv = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if line:
                kv[line[0]] = [int(t) for t in line[1:]]
    V = kv["vocab"][0]
    L = np.zeros((4, V), dtype=np.float32)
    for j, t in enumerate(kv["row_argmax"]):
        L[j, t] = 1.0
    H = np.arange(4 * 8, dtype=np.float32).reshape(4, 8)
    tok, acc, n, pend = gpu_accept(L, kv["drafts"], H)
    assert n == kv["expect_n_accepted"][0]
    assert acc.tolist()[:n + 1] == kv["expect_accepted"]
    assert np.array_equal(pend, H[kv["expect_pending_row"][0]])


@pytest.mark.parametrize("M,V,h", [
    (1, 1, 0), (1, 7, 3), (2, 1023, 8), (3, 1024, 16), (4, 1025, 4096), (4, 5000, 33),
    (5, 4096, 1), (8, 131072, 64), (16, 77777, 0), (64, 3001, 128), (64, 131072, 4096),
])
def test_seeded_batches_every_acceptance_count(M, V, h):
    log(f"accept sweep M={M} V={V} h={h}")
    for n_plan in range(M) if M <= 8 else (0, 1, M // 2, M - 1):
        b = synth.draw_verify_batch(M, V, h, n_plan, seed=n_plan)
        ref = check(b.logits, b.drafts, b.verify_h if h else None)
        if V > 1:
            assert ref["n_accepted"] == n_plan  # the planted spikes decide the batch


def test_equal_maxima_go_to_the_lower_index():
    V = 5000  # five workgroups of 1024 columns, ragged last one
    L = np.random.default_rng(1).standard_normal((6, V)).astype(np.float32)
    L[0, [4999, 5, 2500]] = 9.0           # across workgroups
    L[1, [1024, 1023]] = 9.0              # on a workgroup boundary
    L[2, [77, 76]] = 9.0                  # inside one 4-column load
    L[3, :] = 0.5                         # every column equal
    L[4, [3000, 4096, 4998]] = 9.0        # ragged tail workgroup
    L[5, [1, 4999]] = 9.0
    ref = check(L, [5, 1023, 76, 0, 3000], np.ones((6, 4), np.float32))
    assert ref["tokens"] == [5, 1023, 76, 0, 3000, 1]


def test_signed_zeros_and_infinities():
    V = 3000
    L = np.full((4, V), -1.0, dtype=np.float32)
    L[0, 10] = -0.0
    L[0, 3] = 0.0                         # -0 == +0: the lower index
    L[1, [2999, 777]] = np.inf            # equal infinities
    L[2, :] = -np.inf                     # all -inf: column 0
    L[3, 2048] = np.float32(3.4e38)
    L[3, 2049] = np.inf
    ref = check(L, [3, 777, 0])
    assert ref["tokens"] == [3, 777, 0, 2049]


def test_nan_counts_as_lowest():
    # The library's documented rule for bad input: NaN ranks below -inf.
    V = 2000
    L = np.random.default_rng(2).standard_normal((3, V)).astype(np.float32)
    L[0, [5, 900]] = np.nan
    L[1, :] = np.nan
    L[1, 1500] = -np.inf
    L[2, :] = np.nan
    tok, _, _, _ = gpu_accept(L, [0, 0])
    clean = np.where(np.isnan(L), -np.inf, L)
    want0 = int(np.argmax(clean[0]))
    assert tok.tolist() == [want0, 0, 0]  # rows 1 and 2: every key is -inf's, column 0 wins


@pytest.mark.parametrize("M,V", [(4, 131072), (3, 1027), (64, 999)])
def test_rows_not_16_byte_aligned(M, V):
    b = synth.draw_verify_batch(M, V, 16, min(2, M - 1), seed=5)
    check(b.logits, b.drafts, b.verify_h, misalign=True)


@pytest.mark.parametrize("V", [(1 << 22) + 3, 1 << 22])
def test_several_passes_per_workgroup(V):
    # Above 2^20 columns each workgroup covers several 1024-column passes.
    M = 4
    b = synth.draw_verify_batch(M, V, 64, 1, seed=9)
    b.logits[2, V - 1] = 9.0   # the last column of the last pass
    b.logits[3, 1 << 21] = 9.0
    check(b.logits, b.drafts, b.verify_h)


def test_repeated_calls_on_one_workspace():
    M, V = 4, 131072
    ws = svr.accept_workspace(M, V)
    for i in range(5):
        b = synth.draw_verify_batch(M, V, 4096, i % M, seed=100 + i)
        check(b.logits, b.drafts, b.verify_h, ws=ws)
        assert int(ws[:256].count_nonzero().item()) == 0  # the counter line is back to zero
    # A smaller batch on the same workspace.
    b = synth.draw_verify_batch(2, 4000, 8, 1, seed=7)
    check(b.logits, b.drafts, b.verify_h, ws=ws)


def test_empty_batch_is_a_no_op():
    L = torch.empty((0, 100), dtype=torch.float32, device="cuda")
    tok = torch.empty(0, dtype=torch.int32, device="cuda")
    n = torch.full((1,), -3, dtype=torch.int32, device="cuda")
    svr.moe_verify_accept(L, None, tok, tok, n, ws=svr.accept_workspace(1, 100))
    torch.cuda.synchronize()
    assert int(n.item()) == -3


def test_bench_workload_full_size():
    w = synth.ACCEPT_WORKLOADS["accept_m4"]
    for n_plan in range(w["rows"]):
        b = synth.draw_verify_batch(w["rows"], w["vocab"], w["h_dim"], n_plan, seed=1000 + n_plan)
        ref = check(b.logits, b.drafts, b.verify_h)
        assert ref["n_accepted"] == n_plan

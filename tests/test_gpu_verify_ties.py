"""Ties in the verifier's total order (larger value first, lower token id on
equal values): a row whose maximum is reached by -0.0 and +0.0 at two ids
(equal values, so the lower id wins whichever zero it holds), a row of -inf
and NaN entries only (NaN reads as -inf, so token 0), greedy and top-1
sampling, fp32 logits, against the oracle and the expected ids."""
import numpy as np
import pytest
import torch

from oracle.verifier import verify_greedy, verify_sample

from gpu_util import DEV
from test_gpu_parity import _run_verify
from attention_dna_lms_amd import evs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("V", [37, 512])
def test_verify_signed_zero_and_neg_inf_ties(V):
    B, gamma = 4, 2
    rng = np.random.default_rng(V)
    lf = (-1.0 - np.abs(rng.normal(0, 2.0, (B, gamma + 1, V)))).astype(np.float32)
    want = {}
    # (id holding -0.0, id holding +0.0): the lower id wins either way
    for b, (neg, pos) in enumerate([(3, 9), (11, 4), (V - 1, V - 2)]):
        lf[b, :, neg] = -0.0
        lf[b, :, pos] = 0.0
        want[b] = min(neg, pos)
    lf[3] = -np.inf
    lf[3, :, ::3] = np.nan
    want[3] = 0
    # drafts propose the other zero (or token 1), so position 0 rejects and
    # the emitted token is the row's top entry
    drafts = np.array([[9, 0], [11, 0], [V - 1, 0], [1, 0]], np.int32)
    q = np.zeros((B, gamma, V), np.float32)
    for b in range(B):
        q[b, np.arange(gamma), drafts[b]] = 1.0
    u = np.full((B, gamma + 1), 0.5, np.float32)
    logits = torch.from_numpy(lf).to(DEV)
    a, n = _run_verify(B, gamma, V, logits, evs.EVS_TARGET_LOGITS_F32, None, drafts, None, greedy=1)
    for b in range(B):
        assert (a[b], n[b]) == verify_greedy(lf[b], drafts[b]) == (0, want[b]), b
    a, n = _run_verify(B, gamma, V, logits, evs.EVS_TARGET_LOGITS_F32, q, drafts, u, 1.0, 1)
    for b in range(3):
        assert (a[b], n[b]) == verify_sample(lf[b], q[b], drafts[b], u[b], 1.0, 1) == (0, want[b]), b


@pytest.mark.parametrize("V", [37, 512])
def test_verify_greedy_probability_targets_nan_reads_as_zero(V):
    """Greedy over probability targets: a NaN probability reads as 0, as in
    sampling mode. Rows: [NaN, 0, 0, ...] (all zero after the rule: token 0,
    the lowest id); NaN at the largest id of a row whose maximum sits lower;
    a NaN beside an entry equal to the maximum at a higher id."""
    B, gamma = 3, 2
    rng = np.random.default_rng(V + 1)
    p = rng.dirichlet(np.ones(V), size=(B, gamma + 1)).astype(np.float32)
    p[0] = 0.0
    p[0, :, 0] = np.nan
    top = 5
    p[1, :, top] = 1.0
    p[1, :, V - 1] = np.nan
    p[2, :, 2] = 0.75
    p[2, :, 7] = 0.75
    p[2, :, 1] = np.nan
    want = {0: 0, 1: top, 2: 2}
    drafts = np.array([[want[0], 3], [top, top], [7, 0]], np.int32)
    pt = torch.from_numpy(p).to(DEV)
    a, n = _run_verify(B, gamma, V, pt, evs.EVS_TARGET_PROBS_F32, None, drafts, None, greedy=1)
    for b in range(B):
        ref = verify_greedy(p[b], drafts[b], target_is_probs=True)
        assert (a[b], n[b]) == ref, (b, (a[b], n[b]), ref)
    # the expected decisions: sequence 0 accepts token 0 and rejects 3 (the
    # argmax of an all-zero row is token 0); sequence 1 accepts both drafts and
    # emits the bonus argmax; sequence 2 rejects 7 in favour of the lower id 2
    assert [(a[b], n[b]) for b in range(B)] == [(1, 0), (2, top), (0, 2)]

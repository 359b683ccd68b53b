"""Pins of the CPU oracle against facts that do not come from the oracle itself.

The pages print no worked example and no formula, so the oracle (plain C, fp64)
is pinned by:
  * closed forms of special cases (tests/golden/closed_forms.json),
  * reductions to library routines (torch CPU float64: kl_div, cross_entropy,
    and a whole second implementation through autograd),
  * invariances and sum rules that the definition implies,
  * central finite differences of the oracle's own loss for its gradients.
Each is chosen so that a plausible slip in the oracle (a dropped term, a wrong
sign, a wrong index, a transposed operand, a missing temperature factor) breaks
at least one of them; tests/test_oracle_mutations.py plants such slips and
checks that they are caught.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def rand_problem(seed, N=7, H=12, V=50, K=6, T=1.3, w_sigma=0.3, tl_sigma=2.0):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((N, H))
    W = w_sigma * rng.standard_normal((V, H))
    idx = np.stack([rng.permutation(V)[:K] for _ in range(N)]).astype(np.int32)
    tl = tl_sigma * rng.standard_normal((N, K))
    return h, W, idx, tl, T


def torch_reference(h, W, idx, tl, T, grad_scale=1.0):
    """Independent implementation through torch autograd (CPU, float64)."""
    ht = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    it = torch.tensor(idx, dtype=torch.int64)
    tt = torch.tensor(tl, dtype=torch.float64)
    logq_full = torch.log_softmax((ht @ Wt.t()) / T, dim=1)
    logq = torch.gather(logq_full, 1, it)
    logp = torch.log_softmax(tt / T, dim=1)
    per_tok = (T * T) * (logp.exp() * (logp - logq)).sum(dim=1)
    mean = per_tok.mean()
    (grad_scale * mean).backward()
    return per_tok.detach().numpy(), mean.item(), ht.grad.numpy(), Wt.grad.numpy()


# ---------------------------------------------------------------- P11: a second implementation

@pytest.mark.parametrize("seed,T,gs", [(0, 1.0, 1.0), (1, 2.0, 0.5), (2, 4.0, -3.0), (3, 0.7, 1.0)])
def test_matches_torch_autograd(seed, T, gs):
    h, W, idx, tl, _ = rand_problem(seed, T=T)
    ref_loss, ref_mean, ref_dH, ref_dW = torch_reference(h, W, idx, tl, T, gs)
    loss, lse = oracle.forward(h, W, idx, tl, T)
    dH, dW = oracle.backward(h, W, idx, tl, T, grad_scale=gs)
    np.testing.assert_allclose(loss, ref_loss, rtol=1e-12, atol=1e-13)
    assert abs(oracle.loss_mean(h, W, idx, tl, T) - ref_mean) < 1e-12 * max(1.0, abs(ref_mean))
    np.testing.assert_allclose(dH, ref_dH, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(dW, ref_dW, rtol=1e-10, atol=1e-14)
    ref_lse = torch.logsumexp(torch.tensor(h @ W.T) / T, dim=1).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13)


# ---------------------------------------------------------------- P1: sign and Gibbs bound

def test_loss_nonnegative_and_gibbs_bound():
    for seed in range(6):
        h, W, idx, tl, T = rand_problem(100 + seed, V=80, K=9, T=0.5 + seed * 0.5, w_sigma=1.0)
        loss, _ = oracle.forward(h, W, idx, tl, T)
        assert (loss >= 0).all()
        # loss_i >= -T^2 log(sum_k q[idx_k]) with q the student softmax (library routine)
        q = torch.softmax(torch.tensor(h @ W.T) / T, dim=1).numpy()
        qk = np.take_along_axis(q, idx.astype(np.int64), axis=1).sum(axis=1)
        assert (loss >= -T * T * np.log(qk) - 1e-12).all()


# ---------------------------------------------------------------- P2, P3: the full-vocabulary teacher

def test_full_vocab_teacher_equal_to_student_gives_zero():
    rng = np.random.default_rng(7)
    N, H, V, T = 5, 9, 31, 1.7
    h = rng.standard_normal((N, H))
    W = 0.5 * rng.standard_normal((V, H))
    z = h @ W.T
    idx = np.stack([rng.permutation(V) for _ in range(N)]).astype(np.int32)
    tl = np.take_along_axis(z, idx.astype(np.int64), axis=1)          # teacher = the student
    loss, _ = oracle.forward(h, W, idx, tl, T)
    dH, dW = oracle.backward(h, W, idx, tl, T)
    assert np.abs(loss).max() < 1e-12
    assert np.abs(dH).max() < 1e-13 and np.abs(dW).max() < 1e-13


@pytest.mark.parametrize("T", [1.0, 2.5])
def test_full_vocab_teacher_is_dense_kl(T):
    rng = np.random.default_rng(8)
    N, H, V = 6, 10, 37
    h = rng.standard_normal((N, H))
    W = 0.7 * rng.standard_normal((V, H))
    idx = np.stack([rng.permutation(V) for _ in range(N)]).astype(np.int32)
    tl = 2.0 * rng.standard_normal((N, V))
    full = np.empty((N, V))
    np.put_along_axis(full, idx.astype(np.int64), tl, axis=1)     # teacher logits in vocab order
    dense = torch.nn.functional.kl_div(torch.log_softmax(torch.tensor(h @ W.T) / T, 1),
                                       torch.log_softmax(torch.tensor(full) / T, 1),
                                       reduction="none", log_target=True).sum(1).numpy() * T * T
    loss, _ = oracle.forward(h, W, idx, tl, T)
    np.testing.assert_allclose(loss, dense, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- P4: one cached entry = cross-entropy

@pytest.mark.parametrize("T", [1.0, 3.0])
def test_single_entry_is_cross_entropy(T):
    rng = np.random.default_rng(9)
    N, H, V = 8, 16, 64
    h = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H))
    idx = rng.integers(0, V, (N, 1)).astype(np.int32)
    tl = rng.standard_normal((N, 1))
    ce = torch.nn.functional.cross_entropy(torch.tensor(h @ W.T) / T, torch.tensor(idx[:, 0], dtype=torch.int64),
                                           reduction="none").numpy() * T * T
    loss, lse = oracle.forward(h, W, idx, tl, T)
    np.testing.assert_allclose(loss, ce, rtol=1e-12)


# ---------------------------------------------------------------- P5: closed forms

def test_golden_uniform_teacher_zero_head():
    cases = json.load(open(GOLDEN))["uniform_teacher_zero_head"]
    for c in cases:
        V, K, T = c["V"], c["K"], c["T"]
        N, H = 4, 8
        rng = np.random.default_rng(10)
        h = rng.standard_normal((N, H))
        W = np.zeros((V, H))
        idx = np.stack([rng.permutation(V)[:K] for _ in range(N)]).astype(np.int32)
        tl = np.full((N, K), 0.37)
        loss, lse = oracle.forward(h, W, idx, tl, T)
        np.testing.assert_allclose(loss, c["loss"], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse, math.log(V), rtol=1e-14)


def test_zero_head_closed_form_gradients():
    """W = 0: z = 0, q = 1/V; dH = 0 and dW = g^T h with g = (T/N)(1/V - scatter p)."""
    rng = np.random.default_rng(11)
    N, H, V, K, T = 6, 7, 23, 4, 1.9
    h = rng.standard_normal((N, H))
    W = np.zeros((V, H))
    idx = np.stack([rng.permutation(V)[:K] for _ in range(N)]).astype(np.int32)
    tl = rng.standard_normal((N, K)) * 1.5
    p = np.exp(tl / T) / np.exp(tl / T).sum(1, keepdims=True)
    loss, _ = oracle.forward(h, W, idx, tl, T)
    entropy = -(p * np.log(p)).sum(1)
    np.testing.assert_allclose(loss, T * T * (math.log(V) - entropy), rtol=1e-12)
    g = np.full((N, V), 1.0 / V)
    for i in range(N):
        for k in range(K):
            g[i, idx[i, k]] -= p[i, k]
    g *= T / N
    dH, dW = oracle.backward(h, W, idx, tl, T)
    assert np.abs(dH).max() == 0.0
    np.testing.assert_allclose(dW, g.T @ h, rtol=1e-12, atol=1e-15)


def test_zero_hidden_closed_form_gradients():
    """h = 0: dW = 0 and dH_i = (T/N)(mean_v W_v - sum_k p_k W_{idx_k})."""
    rng = np.random.default_rng(12)
    N, H, V, K, T = 5, 6, 19, 3, 0.8
    h = np.zeros((N, H))
    W = rng.standard_normal((V, H))
    idx = np.stack([rng.permutation(V)[:K] for _ in range(N)]).astype(np.int32)
    tl = rng.standard_normal((N, K))
    p = np.exp(tl / T) / np.exp(tl / T).sum(1, keepdims=True)
    dH, dW = oracle.backward(h, W, idx, tl, T)
    assert np.abs(dW).max() == 0.0
    expect = np.stack([(T / N) * (W.mean(0) - (p[i][:, None] * W[idx[i]]).sum(0)) for i in range(N)])
    np.testing.assert_allclose(dH, expect, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- P6: invariances

def test_invariances():
    h, W, idx, tl, T = rand_problem(13, N=6, H=8, V=40, K=5, T=1.4)
    loss0, lse0 = oracle.forward(h, W, idx, tl, T)
    dH0, dW0 = oracle.backward(h, W, idx, tl, T)
    rng = np.random.default_rng(14)
    # per-token shift of the cached teacher logits
    shift = rng.standard_normal((h.shape[0], 1)) * 5
    loss1, _ = oracle.forward(h, W, idx, tl + shift, T)
    np.testing.assert_allclose(loss1, loss0, rtol=1e-11, atol=1e-13)
    # the same vector added to every head row: z shifts uniformly per token, sum_v g = 0
    u = rng.standard_normal(h.shape[1])
    loss2, _ = oracle.forward(h, W + u, idx, tl, T)
    dH2, dW2 = oracle.backward(h, W + u, idx, tl, T)
    np.testing.assert_allclose(loss2, loss0, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dH2, dH0, rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(dW2, dW0, rtol=1e-9, atol=1e-13)
    # permuting the K (index, logit) pairs
    perm = rng.permutation(idx.shape[1])
    loss3, _ = oracle.forward(h, W, idx[:, perm], tl[:, perm], T)
    dH3, dW3 = oracle.backward(h, W, idx[:, perm], tl[:, perm], T)
    np.testing.assert_allclose(loss3, loss0, rtol=1e-13)
    np.testing.assert_allclose(dH3, dH0, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dW3, dW0, rtol=1e-12, atol=1e-15)
    # permuting tokens permutes per-token outputs and leaves dW alone
    tp = rng.permutation(h.shape[0])
    loss4, lse4 = oracle.forward(h[tp], W, idx[tp], tl[tp], T)
    dH4, dW4 = oracle.backward(h[tp], W, idx[tp], tl[tp], T)
    np.testing.assert_allclose(loss4, loss0[tp], rtol=1e-13)
    np.testing.assert_allclose(dH4, dH0[tp], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dW4, dW0, rtol=1e-12, atol=1e-15)
    # relabelling the vocabulary: W rows permuted, indices mapped
    vp = rng.permutation(W.shape[0])            # new row r holds old row vp[r]
    inv = np.argsort(vp)
    loss5, lse5 = oracle.forward(h, W[vp], inv[idx].astype(np.int32), tl, T)
    dH5, dW5 = oracle.backward(h, W[vp], inv[idx].astype(np.int32), tl, T)
    np.testing.assert_allclose(loss5, loss0, rtol=1e-12)
    np.testing.assert_allclose(lse5, lse0, rtol=1e-13)
    np.testing.assert_allclose(dH5, dH0, rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(dW5, dW0[vp], rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- P7: sum rule

def test_dW_rows_sum_to_zero():
    h, W, idx, tl, T = rand_problem(15, N=9, H=11, V=60, K=7, T=2.2)
    _, dW = oracle.backward(h, W, idx, tl, T)
    assert np.abs(dW.sum(0)).max() < 1e-13 * np.abs(dW).sum(0).max()


# ---------------------------------------------------------------- P8: temperature scaling

@pytest.mark.parametrize("c", [2.0, 0.25, 4.0])
def test_temperature_scaling(c):
    h, W, idx, tl, T = rand_problem(16, T=1.1)
    l0, _ = oracle.forward(h, W, idx, tl, T)
    l1, _ = oracle.forward(h, c * W, idx, c * tl, c * T)
    np.testing.assert_allclose(l1, c * c * l0, rtol=1e-12)


# ---------------------------------------------------------------- P9: finite differences

@pytest.mark.parametrize("seed,T,gs", [(17, 1.0, 1.0), (18, 2.5, 0.75)])
def test_gradients_match_central_differences(seed, T, gs):
    h, W, idx, tl, _ = rand_problem(seed, N=5, H=6, V=20, K=4, T=T, w_sigma=0.8)
    dH, dW = oracle.backward(h, W, idx, tl, T, grad_scale=gs)

    def f(hh, WW):
        return gs * oracle.loss_mean(hh, WW, idx, tl, T)

    rng = np.random.default_rng(seed + 100)
    eps = 1e-5
    for _ in range(40):
        i, j = rng.integers(0, h.shape[0]), rng.integers(0, h.shape[1])
        hp, hm = h.copy(), h.copy()
        hp[i, j] += eps
        hm[i, j] -= eps
        fd = (f(hp, W) - f(hm, W)) / (2 * eps)
        assert abs(fd - dH[i, j]) <= 1e-7 * max(1e-3, np.abs(dH).max())
        v, j = rng.integers(0, W.shape[0]), rng.integers(0, W.shape[1])
        Wp, Wm = W.copy(), W.copy()
        Wp[v, j] += eps
        Wm[v, j] -= eps
        fd = (f(h, Wp) - f(h, Wm)) / (2 * eps)
        assert abs(fd - dW[v, j]) <= 1e-7 * max(1e-3, np.abs(dW).max())


# ---------------------------------------------------------------- row selection and n_norm

def test_row_selection_and_token_additivity():
    h, W, idx, tl, T = rand_problem(19, N=10, H=8, V=30, K=5)
    loss, lse = oracle.forward(h, W, idx, tl, T)
    rows = np.array([7, 2, 9])
    l_r, s_r = oracle.forward(h, W, idx, tl, T, rows=rows)
    np.testing.assert_array_equal(l_r, loss[rows])
    np.testing.assert_array_equal(s_r, lse[rows])
    dH, dW = oracle.backward(h, W, idx, tl, T)
    dHa, dWa = oracle.backward(h, W, idx, tl, T, rows=np.arange(0, 4), n_norm=10)
    dHb, dWb = oracle.backward(h, W, idx, tl, T, rows=np.arange(4, 10), n_norm=10)
    np.testing.assert_allclose(np.concatenate([dHa, dHb]), dH, rtol=1e-14, atol=1e-17)
    np.testing.assert_allclose(dWa + dWb, dW, rtol=1e-12, atol=1e-16)


# ---------------------------------------------------------------- rejected arguments

def test_rejects_bad_arguments():
    h, W, idx, tl, T = rand_problem(20)
    bad = idx.copy()
    bad[0, 0] = W.shape[0]
    with pytest.raises(oracle.OracleError, match="index"):
        oracle.forward(h, W, bad, tl, T)
    bad[0, 0] = -1
    with pytest.raises(oracle.OracleError, match="index"):
        oracle.backward(h, W, bad, tl, T)
    for badT in (0.0, -1.0, float("nan")):
        with pytest.raises(oracle.OracleError):
            oracle.forward(h, W, idx, tl, badT)
    with pytest.raises(oracle.OracleError):
        oracle.forward(h, W, idx, tl, T, rows=[h.shape[0]])


# ---------------------------------------------------------------- token weights and masks
#
# The weighted reduction: mean_w = sum_i w_i loss_i / sum_i w_i; a masked token has w = 0.

def torch_weighted_reference(h, W, idx, tl, T, w, grad_scale=1.0):
    """The weighted mean and its gradients through torch autograd (CPU, float64)."""
    ht = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    logq = torch.gather(torch.log_softmax((ht @ Wt.t()) / T, dim=1), 1, torch.tensor(idx, dtype=torch.int64))
    logp = torch.log_softmax(torch.tensor(tl, dtype=torch.float64) / T, dim=1)
    per_tok = (T * T) * (logp.exp() * (logp - logq)).sum(dim=1)
    wt = torch.tensor(w, dtype=torch.float64)
    mean = (wt * per_tok).sum() / wt.sum()
    (grad_scale * mean).backward()
    return mean.item(), ht.grad.numpy(), Wt.grad.numpy()


@pytest.mark.parametrize("seed,T,gs", [(30, 1.0, 1.0), (31, 2.0, -0.5)])
def test_weighted_matches_torch_autograd(seed, T, gs):
    h, W, idx, tl, _ = rand_problem(seed, N=9, T=T)
    w = np.random.default_rng(seed + 1).uniform(0.0, 2.0, size=h.shape[0])
    w[3] = 0.0
    ref_mean, ref_dH, ref_dW = torch_weighted_reference(h, W, idx, tl, T, w, gs)
    mean = oracle.weighted_mean(h, W, idx, tl, T, w)
    dH, dW = oracle.weighted_backward(h, W, idx, tl, T, w, grad_scale=gs)
    assert abs(mean - ref_mean) <= 1e-12 * abs(ref_mean)
    np.testing.assert_allclose(dH, ref_dH, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(dW, ref_dW, rtol=1e-10, atol=1e-14)


def test_unit_weights_are_the_plain_mean():
    h, W, idx, tl, T = rand_problem(32)
    w = np.ones(h.shape[0])
    assert abs(oracle.weighted_mean(h, W, idx, tl, T, w) - oracle.loss_mean(h, W, idx, tl, T)) <= 1e-14
    dH, dW = oracle.weighted_backward(h, W, idx, tl, T, w, grad_scale=1.7)
    dH0, dW0 = oracle.backward(h, W, idx, tl, T, grad_scale=1.7)
    np.testing.assert_allclose(dH, dH0, rtol=1e-13, atol=1e-17)
    np.testing.assert_allclose(dW, dW0, rtol=1e-13, atol=1e-17)


def test_mask_is_the_plain_mean_of_the_kept_tokens():
    """A 0/1 mask gives the unweighted loss of the kept tokens alone; masked rows get no gradient."""
    h, W, idx, tl, T = rand_problem(33, N=10)
    keep = np.array([1, 0, 1, 1, 0, 0, 1, 1, 0, 1], dtype=bool)
    w = keep.astype(np.float64)
    mean = oracle.weighted_mean(h, W, idx, tl, T, w)
    assert abs(mean - oracle.loss_mean(h[keep], W, idx[keep], tl[keep], T)) <= 1e-13 * abs(mean)
    dH, dW = oracle.weighted_backward(h, W, idx, tl, T, w)
    dHs, dWs = oracle.backward(h[keep], W, idx[keep], tl[keep], T)
    np.testing.assert_allclose(dH[keep], dHs, rtol=1e-12, atol=1e-17)
    assert np.abs(dH[~keep]).max() == 0.0
    np.testing.assert_allclose(dW, dWs, rtol=1e-12, atol=1e-17)


def test_integer_weights_are_repeated_tokens():
    """Weight m on a token equals that token appearing m times in a plain mean."""
    h, W, idx, tl, T = rand_problem(34, N=6)
    m = np.array([2, 1, 3, 0, 1, 4])
    rep = np.repeat(np.arange(h.shape[0]), m)
    mean = oracle.weighted_mean(h, W, idx, tl, T, m.astype(np.float64))
    assert abs(mean - oracle.loss_mean(h[rep], W, idx[rep], tl[rep], T)) <= 1e-13 * abs(mean)
    dH, dW = oracle.weighted_backward(h, W, idx, tl, T, m.astype(np.float64), grad_scale=0.6)
    dHr, dWr = oracle.backward(h[rep], W, idx[rep], tl[rep], T, grad_scale=0.6)
    np.testing.assert_allclose(dW, dWr, rtol=1e-12, atol=1e-17)
    # each copy of token i carries the same gradient; the weighted row is their sum
    summed = np.zeros_like(dH)
    np.add.at(summed, rep, dHr)
    np.testing.assert_allclose(dH, summed, rtol=1e-12, atol=1e-17)


def test_weight_scale_invariance_and_all_masked():
    h, W, idx, tl, T = rand_problem(35)
    w = np.random.default_rng(36).uniform(0.1, 1.0, size=h.shape[0])
    a = oracle.weighted_mean(h, W, idx, tl, T, w)
    b = oracle.weighted_mean(h, W, idx, tl, T, 8.0 * w)
    assert abs(a - b) <= 1e-13 * abs(a)
    dHa, dWa = oracle.weighted_backward(h, W, idx, tl, T, w)
    dHb, dWb = oracle.weighted_backward(h, W, idx, tl, T, 8.0 * w)
    np.testing.assert_allclose(dHa, dHb, rtol=1e-12, atol=1e-17)
    np.testing.assert_allclose(dWa, dWb, rtol=1e-12, atol=1e-17)
    z = np.zeros(h.shape[0])
    assert oracle.weighted_mean(h, W, idx, tl, T, z) == 0.0
    dH0, dW0 = oracle.weighted_backward(h, W, idx, tl, T, z)
    assert np.abs(dH0).max() == 0.0 and np.abs(dW0).max() == 0.0
    bad = w.copy()
    bad[2] = -1.0
    with pytest.raises(oracle.OracleError):
        oracle.weighted_mean(h, W, idx, tl, T, bad)
    bad[2] = float("nan")
    with pytest.raises(oracle.OracleError):
        oracle.weighted_backward(h, W, idx, tl, T, bad)


# ---------------------------------------------------------------- teacher top-K extraction

def brute_topk(h, W, K):
    """numpy: full logits, then a lexicographic sort (value descending, index ascending)."""
    z = np.asarray(h, np.float64) @ np.asarray(W, np.float64).T
    idx = np.empty((z.shape[0], K), np.int64)
    for i in range(z.shape[0]):
        order = np.lexsort((np.arange(z.shape[1]), -z[i]))
        idx[i] = order[:K]
    return idx, np.take_along_axis(z, idx, axis=1)


@pytest.mark.parametrize("seed,K", [(60, 1), (61, 7), (62, 50)])
def test_topk_matches_a_full_sort(seed, K):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((9, 16))
    W = rng.standard_normal((120, 16))
    idx, val = oracle.topk(h, W, K)
    ref_idx, ref_val = brute_topk(h, W, K)
    np.testing.assert_array_equal(idx, ref_idx)
    np.testing.assert_allclose(val, ref_val, rtol=1e-12, atol=1e-12)


def test_topk_ties_go_to_the_smaller_index_and_full_sort():
    rng = np.random.default_rng(63)
    h = rng.standard_normal((4, 8))
    W = rng.standard_normal((30, 8))
    W[17] = W[4]            # equal logits for 4 and 17 in every token
    W[25] = W[4]
    idx, _ = oracle.topk(h, W, 30)
    for i in range(4):
        order = list(idx[i])
        assert order.index(4) < order.index(17) < order.index(25)
        assert sorted(order) == list(range(30))          # K = V is a permutation
    idx0, val0 = oracle.topk(h, np.zeros_like(W), 5)     # all logits equal
    assert (idx0 == np.arange(5)).all() and (val0 == 0).all()


def test_topk_invariances():
    rng = np.random.default_rng(64)
    h = rng.standard_normal((6, 10))
    W = rng.standard_normal((80, 10))
    idx, val = oracle.topk(h, W, 12)
    perm = rng.permutation(80)                             # W_perm[r] = W[perm[r]]
    idx_p, val_p = oracle.topk(h, W[perm], 12)
    np.testing.assert_array_equal(perm[idx_p], idx)
    np.testing.assert_allclose(val_p, val, rtol=1e-13)
    idx_s, val_s = oracle.topk(3.0 * h, W, 12)             # positive scaling keeps the order
    np.testing.assert_array_equal(idx_s, idx)
    np.testing.assert_allclose(val_s, 3.0 * val, rtol=1e-13)
    for badK in (0, 81):
        with pytest.raises(oracle.OracleError):
            oracle.topk(h, W, badK)


# ---------------------------------------------------------------- online full-vocabulary teacher

def full_problem(seed, N=6, Hs=10, Ht=14, V=40, T=1.5):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, Hs)), 0.4 * rng.standard_normal((V, Hs)),
            rng.standard_normal((N, Ht)), 0.4 * rng.standard_normal((V, Ht)), T)


@pytest.mark.parametrize("seed,gs", [(80, 1.0), (81, -2.0)])
def test_full_teacher_is_the_cached_teacher_with_K_equal_V(seed, gs):
    """The cached-teacher oracle with K = V, the teacher's own logits as the cache and
    every vocabulary index, is the same loss: a second implementation."""
    hs, Ws, ht, Wt, T = full_problem(seed)
    N, V = hs.shape[0], Ws.shape[0]
    zt = ht @ Wt.T
    idx = np.tile(np.arange(V, dtype=np.int32), (N, 1))
    loss, lse, mean, dH, dW = oracle.full(hs, Ws, ht, Wt, T, grad_scale=gs)
    ref_loss, ref_lse = oracle.forward(hs, Ws, idx, zt, T)
    ref_dH, ref_dW = oracle.backward(hs, Ws, idx, zt, T, grad_scale=gs)
    np.testing.assert_allclose(loss, ref_loss, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13)
    assert abs(mean - ref_loss.mean()) <= 1e-10 * abs(mean)
    np.testing.assert_allclose(dH, ref_dH, rtol=1e-9, atol=1e-14)
    np.testing.assert_allclose(dW, ref_dW, rtol=1e-9, atol=1e-14)


def test_full_teacher_against_torch_and_identities():
    hs, Ws, ht, Wt, T = full_problem(82)
    w = np.random.default_rng(83).uniform(0.0, 2.0, size=hs.shape[0])
    hst = torch.tensor(hs, requires_grad=True)
    Wst = torch.tensor(Ws, requires_grad=True)
    logp = torch.log_softmax(torch.tensor(ht @ Wt.T) / T, dim=1)
    logq = torch.log_softmax(hst @ Wst.t() / T, dim=1)
    per_tok = (T * T) * torch.nn.functional.kl_div(logq, logp, reduction="none", log_target=True).sum(1)
    wt = torch.tensor(w)
    mean_t = (wt * per_tok).sum() / wt.sum()
    (0.7 * mean_t).backward()
    loss, _, mean, dH, dW = oracle.full(hs, Ws, ht, Wt, T, w=w, grad_scale=0.7)
    np.testing.assert_allclose(loss, per_tok.detach().numpy(), rtol=1e-10, atol=1e-13)
    assert abs(mean - mean_t.item()) <= 1e-10 * abs(mean)
    np.testing.assert_allclose(dH, hst.grad.numpy(), rtol=1e-9, atol=1e-14)
    np.testing.assert_allclose(dW, Wst.grad.numpy(), rtol=1e-9, atol=1e-14)
    # a teacher equal to the student: zero loss and zero gradient
    l0, _, m0, dH0, dW0 = oracle.full(hs, Ws, hs, Ws, T)
    assert np.abs(l0).max() <= 1e-13 and abs(m0) <= 1e-13
    assert np.abs(dH0).max() <= 1e-14 and np.abs(dW0).max() <= 1e-14

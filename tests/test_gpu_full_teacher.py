"""GPU parity of the online full-vocabulary teacher variant (fckl_full_forward_backward)
against the CPU oracle (oracle.full, pinned in test_oracle_pins.py).

Tolerances as in tests/gpu_util.py: per-token loss 1e-3 relative, lse 1e-3 absolute,
dH and dW within 2e-2 of max|oracle|.  The student's exponentials are kept in bf16 as
in the single-call top-K path, so g carries a bf16 rounding of its own size.
"""
import numpy as np
import pytest
import torch

import chunked_top_kl_chunk_amd as fckl
import oracle
import synth
from gpu_util import LSE_ATOL, check_grad, check_loss, device, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def models(seed, N, Hs, Ht, V, z_sigma=2.0, related=0.0):
    """Student (h, W) and teacher (h_t, W_t), bf16-exact.  With related > 0 and Ht == Hs
    the teacher is the student plus noise of that relative size (a small KL)."""
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((N, Hs)).astype(np.float32)
    W = (rng.standard_normal((V, Hs)) * (z_sigma / np.sqrt(Hs))).astype(np.float32)
    if related > 0:
        assert Ht == Hs
        ht = h + related * rng.standard_normal((N, Ht)).astype(np.float32)
        Wt = W + related * (rng.standard_normal((V, Ht)) * (z_sigma / np.sqrt(Ht))).astype(np.float32)
    else:
        ht = rng.standard_normal((N, Ht)).astype(np.float32)
        Wt = (rng.standard_normal((V, Ht)) * (z_sigma / np.sqrt(Ht))).astype(np.float32)
    return tuple(synth.round_bf16(x) for x in (h, W, ht, Wt))


def to_dev(*xs):
    return tuple(torch.from_numpy(synth.bf16_bits(x).view(np.int16)).to(device()).view(torch.bfloat16) for x in xs)


def weights_for(seed, N, zero_frac=0.2):
    rng = np.random.default_rng(seed)
    w = rng.uniform(0.25, 2.0, size=N).astype(np.float32)
    w[rng.permutation(N)[:int(round(zero_frac * N))]] = 0.0
    return w


CASES = [
    # seed, N, Hs, Ht, V, T, chunk, weighted, related
    (80, 300, 256, 384, 4100, 1.0, 0, False, 0.0),     # ragged vocabulary tail, one chunk
    (81, 517, 136, 200, 1000, 2.0, 256, True, 0.0),    # three chunks, ragged, Ht != Hs
    (82, 130, 2880, 2880, 777, 0.7, 0, False, 0.3),    # the 20B model's hidden size, a close teacher
    (83, 600, 512, 512, 5000, 1.5, 512, True, 0.5),    # two chunks, weighted, close teacher
    (87, 1, 8, 16, 100, 1.0, 0, False, 0.0),           # one token, the smallest hidden sizes, V < one tile
    (88, 257, 64, 64, 257, 3.0, 0, True, 0.2),         # one row into the second vocabulary tile
    (89, 64, 96, 40, 600, 0.25, 0, False, 0.0),        # low temperature: sharp distributions
]
IDS = ["ragged-V", "chunks-Ht", "H2880-close", "weighted-close", "N1-H8", "V257", "T0.25"]


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_full_teacher_matches_oracle(case):
    seed, N, Hs, Ht, V, T, chunk, weighted, related = case
    say("case: full teacher", case)
    h, W, ht, Wt = models(seed, N, Hs, Ht, V, related=related)
    w = weights_for(seed + 100, N) if weighted else None
    wt = None if w is None else torch.from_numpy(w).to(device())
    dh, dW_, dht, dWt = to_dev(h, W, ht, Wt)
    out = fckl.full_forward_backward(dh, dW_, dht, dWt, T=T, grad_scale=-1.25, weights=wt, chunk=chunk)
    again = fckl.full_forward_backward(dh, dW_, dht, dWt, T=T, grad_scale=-1.25, weights=wt, chunk=chunk)
    torch.cuda.synchronize()
    for x, y in zip(out, again):
        assert torch.equal(x, y), "not deterministic"
    loss, lse, mean, dH, dWg = (x.cpu().numpy() for x in out)
    r_loss, r_lse, r_mean, r_dH, r_dW = oracle.full(h, W, ht, Wt, T, w=w, grad_scale=-1.25)
    e_loss = check_loss(loss, r_loss, "full%d" % seed)
    e_lse = float(np.abs(lse - r_lse).max())
    assert e_lse <= LSE_ATOL, "lse abs err %.3e" % e_lse
    e_mean = abs(float(mean[0]) - r_mean) / abs(r_mean)
    assert e_mean <= 1e-3, "mean rel err %.3e" % e_mean
    e_dH = check_grad(dH, r_dH, "full%d dH" % seed)
    e_dW = check_grad(dWg, r_dW, "full%d dW" % seed)
    if w is not None:
        assert np.abs(dH[w == 0.0]).max() == 0.0, "masked tokens got a gradient"
    say("full%d: loss %.2e (mean KL %.3f) lse %.2e mean %.2e dH %.2e dW %.2e"
        % (seed, e_loss, r_mean, e_lse, e_mean, e_dH, e_dW))


def test_teacher_equal_to_student_gives_zero():
    """p = q: every per-token loss is 0 up to rounding (both products form bitwise equal logits), and the
    gradient is only the bf16 rounding of the kept exponentials."""
    N, H, V, T = 300, 256, 3000, 1.0
    h, W, _, _ = models(84, N, H, H, V)
    dh, dW_ = to_dev(h, W)
    loss, lse, mean, dH, dWg = fckl.full_forward_backward(dh, dW_, dh, dW_, T=T)
    _, _, _, dH_o, _ = fckl.full_forward_backward(dh, dW_, *to_dev(*models(85, N, H, H, V)[2:]), T=T)
    torch.cuda.synchronize()
    # a few ulps of the base-2 logsumexp (about 12 here): the two products round L alike
    # only up to the contraction of their epilogues
    assert float(loss.abs().max()) <= 1e-5 and abs(float(mean[0])) <= 1e-5
    r_lse = oracle.full(h, W, h, W, T, want_grads=False)[1]
    assert float(np.abs(lse.cpu().numpy() - r_lse).max()) <= LSE_ATOL
    ratio = float(dH.abs().max()) / float(dH_o.abs().max())
    say("teacher = student: max|loss| %.1e, max|dH| / max|dH of another teacher| %.1e"
        % (float(loss.abs().max()), ratio))
    assert ratio <= 1e-2


def test_accumulate_and_the_full_plan():
    N, Hs, Ht, V = 400, 128, 192, 2000
    h, W, ht, Wt = models(86, N, Hs, Ht, V)
    t = to_dev(h, W, ht, Wt)
    # the scheduler: one chunk of 512 tokens by default, two of 256 in the workspace of 256
    c_one, ws_one = fckl.full_plan(fckl.make_desc(N, Hs, V, 1, 1.0), Ht)
    _, ws_256 = fckl.full_plan(fckl.make_desc(N, Hs, V, 1, 1.0, 256), Ht)
    c_two, _ = fckl.full_plan(fckl.make_desc(N, Hs, V, 1, 1.0), Ht, budget_bytes=ws_256)
    assert (c_one, c_two) == (512, 256) and ws_256 < ws_one
    a = fckl.full_forward_backward(*t, T=1.0, budget_bytes=ws_256)
    b = fckl.full_forward_backward(*t, T=1.0)
    dW2 = a[4].clone()
    fckl.full_forward_backward(*t, T=1.0, chunk=256, dW=dW2, accumulate=True)
    torch.cuda.synchronize()
    assert float((dW2 - 2 * a[4]).abs().max()) <= 1e-6 * float(a[4].abs().max())
    # per-token results do not depend on the chunking
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    r = oracle.full(h, W, ht, Wt, 1.0)
    for x, what in ((a, "two chunks"), (b, "one chunk")):
        check_grad(x[3].cpu().numpy(), r[3], what + " dH")
        check_grad(x[4].cpu().numpy(), r[4], what + " dW")


def test_full_teacher_module():
    """FullTeacherKLLoss through autograd, with a padding mask and an upstream scale,
    against the oracle; the teacher gets no gradient."""
    from chunked_top_kl_chunk_amd.loss import FullTeacherKLLoss
    N, Hs, Ht, V, T = 2 * 200, 128, 192, 2500, 1.5
    h, W, ht, Wt = models(96, N, Hs, Ht, V)
    dh, dW_, dht, dWt = to_dev(h, W, ht, Wt)
    keep = np.ones(N, dtype=bool)
    keep[180:200] = False
    hb = dh.clone().reshape(2, 200, Hs).requires_grad_(True)
    Wb = dW_.clone().requires_grad_(True)
    htb = dht.reshape(2, 200, Ht)
    mask = torch.from_numpy(keep).to(device()).reshape(2, 200)
    loss = FullTeacherKLLoss(temperature=T, chunk=256)(hb, Wb, htb, dWt, mask=mask)
    (-2.0 * loss).backward()
    torch.cuda.synchronize()
    w = keep.astype(np.float64)
    _, _, r_mean, r_dH, r_dW = oracle.full(h, W, ht, Wt, T, w=w, grad_scale=-2.0)
    assert abs(float(loss.detach()) - r_mean) <= 1e-3 * abs(r_mean)
    check_grad(hb.grad.float().reshape(N, Hs).cpu().numpy(), r_dH, "full module dH")
    check_grad(Wb.grad.float().cpu().numpy(), r_dW, "full module dW")
    assert float(hb.grad.reshape(N, Hs)[~torch.from_numpy(keep)].abs().max()) == 0.0
    with torch.no_grad():
        l2 = FullTeacherKLLoss(temperature=T, chunk=256)(hb, Wb, htb, dWt, mask=mask)
    assert float(l2) == float(loss.detach())


def test_full_teacher_in_vocabulary_slabs():
    """g, dH and dW one vocabulary slab at a time (slabs of 2 tiles over V = 4100, the
    last slab of 3 tiles ending in a 4-row tile), weighted, two chunks: the oracle's
    results, and bit for bit those of one slab except for the order of the dH sum."""
    N, Hs, Ht, V, T = 600, 256, 384, 4100, 1.2
    say("case: full teacher, vocabulary slabs")
    h, W, ht, Wt = models(90, N, Hs, Ht, V)
    w = weights_for(190, N)
    wt = torch.from_numpy(w).to(device())
    t = to_dev(h, W, ht, Wt)
    a = fckl.full_forward_backward(*t, T=T, grad_scale=0.8, weights=wt, chunk=512, vocab_slab=512)
    b = fckl.full_forward_backward(*t, T=T, grad_scale=0.8, weights=wt, chunk=512,
                                   vocab_slab=(V + 255) // 256 * 256)
    torch.cuda.synchronize()
    for k, x, y in zip(("loss", "lse", "mean", "dH", "dW"), a, b):
        if k == "dH":
            d = (x - y).abs().max().item() / y.abs().max().item()
            assert d < 1e-5, d
        else:
            assert torch.equal(x, y), k
    loss, lse, mean, dH, dWg = (x.cpu().numpy() for x in a)
    r_loss, r_lse, r_mean, r_dH, r_dW = oracle.full(h, W, ht, Wt, T, w=w, grad_scale=0.8)
    check_loss(loss, r_loss, "full-slab")
    assert float(np.abs(lse - r_lse).max()) <= LSE_ATOL
    check_grad(dH, r_dH, "full-slab dH")
    check_grad(dWg, r_dW, "full-slab dW")

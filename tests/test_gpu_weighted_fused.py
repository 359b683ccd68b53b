"""GPU parity of the weighted reduction (token masks, per-token weights), the single-call
forward + backward and the torch autograd module, against the CPU oracle.

Tolerances as in tests/gpu_util.py: loss 1e-3 relative, lse 1e-3 absolute, dH and dW
within 2e-2 of max|oracle|.  The single-call path keeps 2^(z/T log2 e - m) in bf16 and
forms g from it, so its dH and dW differ from the two-call path by roundings of the
size of g's own bf16 rounding; its per-token loss and lse come from the same forward
arithmetic and must match the two-call path exactly.
"""
import numpy as np
import pytest
import torch

import chunked_top_kl_chunk_amd as fckl
import oracle
from chunked_top_kl_chunk_amd.loss import FusedChunkedKLLoss
from gpu_util import LSE_ATOL, arrays, check_grad, check_loss, device, rel_max, say, synthetic

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def weights_for(seed, N, zero_frac=0.2):
    rng = np.random.default_rng(seed)
    w = rng.uniform(0.25, 2.0, size=N).astype(np.float32)
    w[rng.permutation(N)[:int(round(zero_frac * N))]] = 0.0
    return w


def check_weighted(g, h, W, idx, tl, T, w, grad_scale, what):
    ref_loss, ref_lse = oracle.forward(h, W, idx, tl, T)
    check_loss(g["loss"], ref_loss, what)
    e_lse = float(np.abs(g["lse"] - ref_lse).max())
    assert e_lse <= LSE_ATOL, "%s lse abs err %.3e" % (what, e_lse)
    ref_mean = oracle.weighted_mean(h, W, idx, tl, T, w)
    e_mean = abs(float(g["mean"][0]) - ref_mean) / abs(ref_mean)
    assert e_mean <= 1e-3, "%s weighted mean rel err %.3e" % (what, e_mean)
    ref_dH, ref_dW = oracle.weighted_backward(h, W, idx, tl, T, w, grad_scale=grad_scale)
    e_dH = check_grad(g["dH"], ref_dH, what + " dH")
    e_dW = check_grad(g["dW"], ref_dW, what + " dW")
    masked = w == 0.0
    if masked.any():
        assert np.abs(g["dH"][masked]).max() == 0.0, what + ": masked tokens got a gradient"
    say("%s: mean %.2e dH %.2e dW %.2e" % (what, e_mean, e_dH, e_dW))


CASES = [
    # seed, N, H, V, K, T, chunk
    (41, 1000, 200, 4100, 7, 1.7, 384),
    (42, 257, 136, 1000, 128, 0.5, 256),
    (43, 700, 1024, 5000, 100, 1.0, 512),
    (44, 130, 2880, 777, 20, 2.0, 0),
]
IDS = ["ragged", "K128", "K100", "H2880"]


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_weighted_two_call(case):
    seed, N, H, V, K, T, chunk = case
    say("case: weighted two-call", case)
    h, W, idx, tl = synthetic(seed, N, H, V, K, T)
    w = weights_for(seed, N)
    dh, dW_, di, dt = arrays(h, W, idx, tl)
    wt = torch.from_numpy(w).to(device())
    loss, lse, mean = fckl.forward(dh, dW_, di, dt, T=T, chunk=chunk, weights=wt)
    dH, dWg = fckl.backward(dh, dW_, di, dt, lse, T=T, grad_scale=-1.5, chunk=chunk, weights=wt)
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in dict(loss=loss, lse=lse, mean=mean, dH=dH, dW=dWg).items()}
    check_weighted(g, h, W, idx, tl, T, w, -1.5, "weighted%d" % seed)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_single_call_matches_oracle_and_two_call(case):
    seed, N, H, V, K, T, chunk = case
    say("case: single call", case)
    h, W, idx, tl = synthetic(seed, N, H, V, K, T)
    t = arrays(h, W, idx, tl)
    lt, ls, mn, dH, dWg = fckl.forward_backward(*t, T=T, grad_scale=0.75, chunk=chunk)
    l2, s2, m2 = fckl.forward(*t, T=T, chunk=chunk)
    dH2, dW2 = fckl.backward(*t, s2, T=T, grad_scale=0.75, chunk=chunk)
    torch.cuda.synchronize()
    # the forward outputs come from the same arithmetic
    assert torch.equal(lt, l2) and torch.equal(ls, s2) and torch.equal(mn, m2)
    ref_loss, ref_lse = oracle.forward(h, W, idx, tl, T)
    check_loss(lt.cpu().numpy(), ref_loss, "single%d" % seed)
    ref_dH, ref_dW = oracle.backward(h, W, idx, tl, T, grad_scale=0.75)
    e_dH = check_grad(dH.cpu().numpy(), ref_dH, "single%d dH" % seed)
    e_dW = check_grad(dWg.cpu().numpy(), ref_dW, "single%d dW" % seed)
    d_dH = rel_max(dH.cpu().numpy(), dH2.cpu().numpy())
    d_dW = rel_max(dWg.cpu().numpy(), dW2.cpu().numpy())
    say("single%d: dH %.2e dW %.2e vs oracle; %.2e %.2e vs two-call" % (seed, e_dH, e_dW, d_dH, d_dW))
    assert d_dH <= 2e-2 and d_dW <= 2e-2


def test_single_call_weighted_accumulate_and_deterministic():
    h, W, idx, tl = synthetic(45, 600, 256, 3000, 10, 1.3)
    w = weights_for(46, 600, zero_frac=0.3)
    t = arrays(h, W, idx, tl)
    wt = torch.from_numpy(w).to(device())
    a = fckl.forward_backward(*t, T=1.3, grad_scale=2.0, weights=wt, chunk=256)
    b = fckl.forward_backward(*t, T=1.3, grad_scale=2.0, weights=wt, chunk=256)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    g = {k: v.cpu().numpy() for k, v in zip(("loss", "lse", "mean", "dH", "dW"), a)}
    check_weighted(g, h, W, idx, tl, 1.3, w, 2.0, "single weighted")
    dW2 = a[4].clone()
    fckl.forward_backward(*t, T=1.3, grad_scale=2.0, weights=wt, chunk=256, dW=dW2, accumulate=True)
    torch.cuda.synchronize()
    assert rel_max(dW2.cpu().numpy(), 2 * a[4].cpu().numpy()) <= 1e-6


def test_all_masked_gives_zero():
    h, W, idx, tl = synthetic(47, 300, 128, 1500, 12, 1.0)
    t = arrays(h, W, idx, tl)
    wt = torch.zeros(300, dtype=torch.float32, device=device())
    loss, lse, mean, dH, dWg = fckl.forward_backward(*t, T=1.0, weights=wt)
    _, lse2, mean2 = fckl.forward(*t, T=1.0, weights=wt)
    dH2, dW2 = fckl.backward(*t, lse2, T=1.0, weights=wt)
    torch.cuda.synchronize()
    for x in (mean, mean2):
        assert float(x[0]) == 0.0
    for x in (dH, dWg, dH2, dW2):
        assert float(x.abs().max()) == 0.0


def test_autograd_module_with_mask_and_upstream_scale():
    """loss = 3 * FusedChunkedKLLoss(...) with a padding mask, through torch autograd."""
    N, H, V, K, T = 2 * 300, 256, 3000, 16, 2.0
    h, W, idx, tl = synthetic(48, N, H, V, K, T)
    t = arrays(h, W, idx, tl)
    keep = np.ones(N, dtype=bool)
    keep[250:300] = False           # padding at the end of the first sequence
    keep[590:] = False
    hb = t[0].clone().reshape(2, 300, H).requires_grad_(True)
    Wb = t[1].clone().requires_grad_(True)
    mod = FusedChunkedKLLoss(temperature=T, chunk=256)
    mask = torch.from_numpy(keep).to(device()).reshape(2, 300)
    loss = mod(hb, Wb, t[2].reshape(2, 300, K), t[3].reshape(2, 300, K), mask=mask)
    (3.0 * loss).backward()
    torch.cuda.synchronize()
    w = keep.astype(np.float64)
    ref_mean = oracle.weighted_mean(h, W, idx, tl, T, w)
    assert abs(float(loss.detach()) - ref_mean) <= 1e-3 * abs(ref_mean)
    ref_dH, ref_dW = oracle.weighted_backward(h, W, idx, tl, T, w, grad_scale=3.0)
    # autograd hands the float32 gradients to the bf16 leaves in their dtype
    check_grad(hb.grad.float().reshape(N, H).cpu().numpy(), ref_dH, "module dH")
    check_grad(Wb.grad.float().cpu().numpy(), ref_dW, "module dW")
    assert float(hb.grad.reshape(N, H)[~torch.from_numpy(keep)].abs().max()) == 0.0


def test_autograd_module_ignore_index():
    N, H, V, K, T = 400, 128, 2000, 8, 1.0
    h, W, idx, tl = synthetic(49, N, H, V, K, T)
    ignored = np.zeros(N, dtype=bool)
    ignored[np.random.default_rng(50).permutation(N)[:60]] = True
    idx_in = idx.copy()
    idx_in[ignored] = -100
    t = arrays(h, W, idx_in, tl)
    hb = t[0].clone().requires_grad_(True)
    Wb = t[1].clone().requires_grad_(True)
    loss = FusedChunkedKLLoss(temperature=T, ignore_index=-100)(hb, Wb, t[2], t[3])
    loss.backward()
    torch.cuda.synchronize()
    keep = ~ignored
    ref = oracle.loss_mean(h[keep], W, idx[keep], tl[keep], T)
    assert abs(float(loss.detach()) - ref) <= 1e-3 * abs(ref)
    ref_dH, ref_dW = oracle.backward(h[keep], W, idx[keep], tl[keep], T)
    check_grad(hb.grad.float().cpu().numpy()[keep], ref_dH, "ignore_index dH")
    check_grad(Wb.grad.float().cpu().numpy(), ref_dW, "ignore_index dW")


def test_scale_in_place():
    dev = device()
    for n in (1, 3, 1003, 1 << 20):
        x = torch.randn(n, device=dev)
        s = torch.tensor([-2.5], device=dev)
        ref = x * -2.5
        fckl.scale_(x, s)
        torch.cuda.synchronize()
        assert torch.equal(x, ref), n


def test_autograd_module_single_call():
    """FusedChunkedKLLoss(single_call=True): both passes in the forward call, the backward
    only scales by the upstream gradient; loss equal to the two-pass module, gradients
    within the bf16 rounding of the kept exponentials, both against the oracle."""
    N, H, V, K, T = 2 * 300, 256, 3000, 16, 2.0
    h, W, idx, tl = synthetic(51, N, H, V, K, T)
    t = arrays(h, W, idx, tl)
    keep = np.ones(N, dtype=bool)
    keep[280:300] = False
    mask = torch.from_numpy(keep).to(device()).reshape(2, 300)
    grads = {}
    for single in (False, True):
        hb = t[0].clone().reshape(2, 300, H).requires_grad_(True)
        Wb = t[1].clone().requires_grad_(True)
        mod = FusedChunkedKLLoss(temperature=T, chunk=256, single_call=single)
        loss = mod(hb, Wb, t[2].reshape(2, 300, K), t[3].reshape(2, 300, K), mask=mask)
        (3.0 * loss).backward()
        torch.cuda.synchronize()
        grads[single] = (float(loss.detach()), hb.grad.float().reshape(N, H).cpu().numpy(),
                         Wb.grad.float().cpu().numpy())
    assert grads[True][0] == grads[False][0]
    w = keep.astype(np.float64)
    ref_dH, ref_dW = oracle.weighted_backward(h, W, idx, tl, T, w, grad_scale=3.0)
    check_grad(grads[True][1], ref_dH, "single-call module dH")
    check_grad(grads[True][2], ref_dW, "single-call module dW")
    assert rel_max(grads[True][1], grads[False][1]) <= 2e-2 and rel_max(grads[True][2], grads[False][2]) <= 2e-2
    # no gradient wanted: the module takes the forward-only path
    with torch.no_grad():
        l2 = FusedChunkedKLLoss(temperature=T, chunk=256, single_call=True)(
            t[0].reshape(2, 300, H), t[1], t[2].reshape(2, 300, K), t[3].reshape(2, 300, K), mask=mask)
    assert float(l2) == grads[True][0]


def test_single_call_validate():
    """FCKL_FLAG_VALIDATE on the single call: valid indices give the unvalidated results
    bit for bit; an index out of range or repeated within a token is reported."""
    h, W, idx, tl = synthetic(52, 400, 128, 1200, 8, 1.0)
    t = arrays(h, W, idx, tl)
    a = fckl.forward_backward(*t, T=1.0, validate=True)
    b = fckl.forward_backward(*t, T=1.0)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    for bad_value in (1200, -5, None):
        bad = t[2].clone()
        if bad_value is None:
            bad[9, 4] = bad[9, 0]
        else:
            bad[3, 6] = bad_value
        with pytest.raises(fckl.FCKLError) as e:
            fckl.forward_backward(t[0], t[1], bad, t[3], T=1.0, validate=True)
        assert e.value.status == fckl.ERR_INDEX


def test_masked_rows_with_non_finite_cached_logits():
    """Padding rows often carry -inf or NaN as cached logits.  With weight 0 such a row
    reaches neither the weighted mean nor any gradient: the two calls, the single call
    and the autograd module give the oracle's results for the same batch with those
    rows' logits finite (their weight is 0 either way); the kept rows' loss and every
    lse match it too."""
    N, H, V, K, T = 600, 160, 3000, 12, 1.2
    say("case: masked rows with non-finite cached logits", N, H, V, K, T)
    h, W, idx, tl = synthetic(51, N, H, V, K, T)
    w = weights_for(52, N, zero_frac=0.0)
    bad = np.random.default_rng(53).permutation(N)[:60]
    w[bad] = 0.0
    tl_bad = tl.copy()
    tl_bad[bad[:20]] = -np.inf
    tl_bad[bad[20:35]] = np.nan
    tl_bad[bad[35:50], : K // 2] = np.nan
    tl_bad[bad[50:]] = np.inf
    dh, dW_, di, dt = arrays(h, W, idx, tl_bad)
    wt = torch.from_numpy(w).to(device())
    kept = w != 0.0
    ref_loss, ref_lse = oracle.forward(h, W, idx, tl, T)
    ref_mean = oracle.weighted_mean(h, W, idx, tl, T, w)
    ref_dH, ref_dW = oracle.weighted_backward(h, W, idx, tl, T, w, grad_scale=1.0)

    def check(loss, lse, mean, dH, dWg, what):
        torch.cuda.synchronize()
        loss, lse, mean, dH, dWg = (v.detach().cpu().numpy() for v in (loss, lse, mean, dH, dWg))
        check_loss(loss[kept], ref_loss[kept], what)
        assert float(np.abs(lse - ref_lse).max()) <= LSE_ATOL, what + " lse"
        assert np.isfinite(mean).all(), what + " mean not finite"
        e_mean = abs(float(mean.reshape(-1)[0]) - ref_mean) / abs(ref_mean)
        assert e_mean <= 1e-3, "%s weighted mean rel err %.3e" % (what, e_mean)
        check_grad(dH, ref_dH, what + " dH")
        check_grad(dWg, ref_dW, what + " dW")
        assert np.abs(dH[~kept]).max() == 0.0, what + ": masked tokens got a gradient"

    loss, lse, mean = fckl.forward(dh, dW_, di, dt, T=T, chunk=256, weights=wt)
    dH, dWg = fckl.backward(dh, dW_, di, dt, lse, T=T, chunk=256, weights=wt)
    check(loss, lse, mean, dH, dWg, "two calls")
    check(*fckl.forward_backward(dh, dW_, di, dt, T=T, weights=wt, chunk=256), "single call")
    for single in (False, True):
        hl = dh.float().requires_grad_(True)
        Wl = dW_.float().requires_grad_(True)
        mod = FusedChunkedKLLoss(temperature=T, chunk=256, single_call=single)
        out = mod(hl.to(torch.bfloat16), Wl.to(torch.bfloat16), di, dt, weights=wt)
        out.backward()
        check(loss, lse, out.detach().reshape(1), hl.grad, Wl.grad, "module single_call=%s" % single)


@pytest.mark.parametrize("slab", [512, 256])
def test_single_call_in_vocabulary_slabs(slab):
    """The single call forms g, dH and dW one vocabulary slab at a time (V = 3000: slabs
    of 2 tiles or 1 tile, the last holding the 184-row tail), with weights, over three
    chunks: the oracle's results, and bit for bit those of one slab except for the order
    of the dH sum."""
    N, H, V, K, T = 700, 264, 3000, 12, 1.3
    say("case: single call, vocabulary slab", slab)
    h, W, idx, tl = synthetic(151, N, H, V, K, T)
    w = weights_for(152, N)
    t = arrays(h, W, idx, tl)
    wt = torch.from_numpy(w).to(device())
    a = fckl.forward_backward(*t, T=T, grad_scale=0.5, weights=wt, chunk=256, vocab_slab=slab)
    b = fckl.forward_backward(*t, T=T, grad_scale=0.5, weights=wt, chunk=256, vocab_slab=(V + 255) // 256 * 256)
    torch.cuda.synchronize()
    for k, x, y in zip(("loss", "lse", "mean"), a[:3], b[:3]):
        assert torch.equal(x, y), k
    assert torch.equal(a[4], b[4]), "dW"
    assert rel_max(a[3].cpu().numpy(), b[3].cpu().numpy()) < 1e-5
    g = {k: v.cpu().numpy() for k, v in zip(("loss", "lse", "mean", "dH", "dW"), a)}
    check_weighted(g, h, W, idx, tl, T, w, 0.5, "single-slab%d" % slab)

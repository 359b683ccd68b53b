"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element.

Sizes are ones the oracle finishes in seconds while still spanning several vocabulary
and token tiles, ragged tails in every dimension, several chunks and the edge cases
(one token, one cached entry, the largest K, high temperature, rows with large
norms).  Tolerances: see tests/gpu_util.py.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import chunked_top_kl_chunk_amd as fckl
import oracle
import synth
from gpu_util import (GRAD_TOL, LOSS_RTOL, LSE_ATOL, arrays, check_grad, check_loss, device, rel_max, run, say,
                      synthetic, upload)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def compare_all(g, h, W, idx, tl, T, grad_scale=1.0, what=""):
    ref_loss, ref_lse = oracle.forward(h, W, idx, tl, T)
    ref_dH, ref_dW = oracle.backward(h, W, idx, tl, T, grad_scale=grad_scale)
    e_loss = check_loss(g["loss"], ref_loss, what)
    e_lse = float(np.abs(g["lse"] - ref_lse).max())
    assert e_lse <= LSE_ATOL, "%s lse abs err %.3e" % (what, e_lse)
    e_mean = abs(float(g["mean"][0]) - ref_loss.mean()) / abs(ref_loss.mean())
    assert e_mean <= LOSS_RTOL, "%s mean loss rel err %.3e" % (what, e_mean)
    e_dH = check_grad(g["dH"], ref_dH, what + " dH")
    e_dW = check_grad(g["dW"], ref_dW, what + " dW")
    say("%s: loss %.2e lse %.2e mean %.2e dH %.2e dW %.2e" % (what, e_loss, e_lse, e_mean, e_dH, e_dW))


def test_tiny_workload_full_parity():
    """The tiny CPU-checkable workload: N=512, H=256, V=4096, K=10, T=1, 4 chunks of 128."""
    wl = synth.WORKLOADS["c1"]
    x = synth.make_inputs(wl)
    say("case: tiny workload", wl)
    g = run(*upload(x, device()), T=wl.T, chunk=wl.chunk)
    compare_all(g, x.h, x.W, x.idx, x.tl, wl.T, what="tiny")
    # for information: the same GPU result against the oracle on the unrounded fp32 draws
    ref_loss, _ = oracle.forward(x.h_raw, x.W_raw, x.idx, x.tl_raw, wl.T)
    say("tiny vs unrounded fp32 inputs: max per-token loss rel err %.3e"
        % float((np.abs(g["loss"] - ref_loss) / ref_loss).max()))


CASES = [
    # seed, N, H, V, K, T, chunk, extra
    (1, 1000, 200, 4100, 7, 1.7, 384, {}),
    (2, 1, 64, 300, 3, 1.0, 0, {}),
    (3, 257, 136, 1000, 128, 0.5, 256, {}),
    (4, 600, 256, 2048, 1, 3.0, 0, {}),
    (5, 300, 2880, 777, 20, 2.0, 100, {}),
    (6, 512, 512, 3000, 10, 4.0, 0, {"scaled_frac": 0.01, "tl_sigma": 1.0}),
    (7, 700, 1024, 5000, 100, 1.0, 512, {"z_sigma": 4.0}),
    (8, 130, 3072, 513, 16, 1.0, 0, {}),
    (9, 200, 64, 100, 100, 1.0, 0, {}),                                   # K = V, V < one tile
    (10, 300, 128, 2000, 10, 0.25, 0, {"z_sigma": 20.0, "tl_sigma": 10.0}),  # z/T spread ~80: sharp softmaxes
    (12, 300, 8, 600, 5, 1.0, 256, {}),                                    # smallest H: one partial k-step
    (13, 333, 264, 1500, 12, 1.0, 0, {}),                                  # a hidden tail of 8 columns
    (14, 400, 256, 3000, 20, 50.0, 0, {"z_sigma": 8.0, "tl_sigma": 8.0}),  # high T: near-uniform p and q
]


@pytest.mark.parametrize("case", CASES, ids=["ragged", "one-token", "K128", "K1", "H2880", "scaled-rows",
                                             "K100", "H3072", "K-equals-V", "sharp", "H8", "H264", "T50"])
def test_parity_shapes(case):
    seed, N, H, V, K, T, chunk, extra = case
    say("case:", case)
    h, W, idx, tl = synthetic(seed, N, H, V, K, T, **extra)
    g = run(*arrays(h, W, idx, tl), T=T, chunk=chunk, grad_scale=1.0)
    compare_all(g, h, W, idx, tl, T, what="shape%d" % seed)


def test_grad_scale_and_f32_logits():
    h, W, idx, tl = synthetic(11, 300, 128, 1500, 12, 1.3)
    dh, dW_, di, dt = arrays(h, W, idx, tl)
    g = run(dh, dW_, di, dt, T=1.3, grad_scale=-2.5)
    compare_all(g, h, W, idx, tl, 1.3, grad_scale=-2.5, what="grad_scale")
    # the same logits given as float32 give the same results
    g32 = run(dh, dW_, di, dt.float().contiguous(), T=1.3, grad_scale=-2.5)
    for k in g:
        np.testing.assert_array_equal(g[k], g32[k])


def test_deterministic_and_chunk_invariant():
    h, W, idx, tl = synthetic(12, 1100, 256, 3000, 10, 1.0)
    t = arrays(h, W, idx, tl)
    a = run(*t, T=1.0, chunk=256)
    b = run(*t, T=1.0, chunk=256)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    for chunk in (128, 512, 1100, 0):
        c = run(*t, T=1.0, chunk=chunk)
        # per-token results do not depend on how tokens are grouped into chunks
        np.testing.assert_array_equal(c["loss"], a["loss"])
        np.testing.assert_array_equal(c["lse"], a["lse"])
        assert rel_max(c["dH"], a["dH"]) < 1e-5
        assert rel_max(c["dW"], a["dW"]) < 1e-5


SLAB_CASES = [
    # seed, N, H, V, K, T, chunk, vocab_slab: 6 slabs of 2 tiles, the last with a ragged
    # tile of 184 rows, 3 chunks; 2 slabs, the last of 3 tiles; a 1-tile slab per tile
    (31, 1100, 264, 3000, 12, 1.3, 512, 512),
    (32, 700, 2880, 1400, 20, 1.0, 0, 512),
    (33, 300, 128, 1800, 7, 0.7, 256, 256),
]


@pytest.mark.parametrize("case", SLAB_CASES, ids=["slab512-ragged", "slab512-H2880", "slab256"])
def test_vocabulary_slabs(case):
    """The backward taken one vocabulary slab at a time (the slab set by the caller):
    against the oracle, and against one slab for the whole vocabulary.  The slabs only
    regroup the dH sum: loss, lse and dW are bit for bit those of one slab."""
    seed, N, H, V, K, T, chunk, slab = case
    say("case: vocabulary slabs", case)
    h, W, idx, tl = synthetic(seed, N, H, V, K, T)
    t = arrays(h, W, idx, tl)
    g = run(*t, T=T, chunk=chunk, vocab_slab=slab)
    compare_all(g, h, W, idx, tl, T, what="slabs%d" % seed)
    whole = run(*t, T=T, chunk=chunk, vocab_slab=(V + 255) // 256 * 256)
    for k in ("loss", "lse", "mean", "dW"):
        np.testing.assert_array_equal(g[k], whole[k], err_msg=k)
    assert rel_max(g["dH"], whole["dH"]) < 1e-5
    # deterministic
    again = run(*t, T=T, chunk=chunk, vocab_slab=slab)
    for k in g:
        np.testing.assert_array_equal(g[k], again[k], err_msg=k)


# Shapes whose dH launch takes the XCD block order (blocks of 4 hidden x 8 token tiles,
# whole rounds of one block per XCD): one chunk of 8 token tiles, V = 2048 (8 vocabulary
# tiles, so the planner's split count may reach 8), and H with 4 hidden tiles (1024) or 12
# with a quarter-full last tile (2880).  For both, 8 splits are the first count that fills
# whole waves of 256 work-groups (32 x 8 and 96 x 8 work-groups), each split 256 rows.
XBLOCK_CASES = [
    (41, 2000, 1024, 2048, 16, 1.0),
    (42, 1900, 2880, 2048, 16, 1.5),
]


@pytest.mark.parametrize("case", XBLOCK_CASES, ids=["H1024", "H2880-tail"])
def test_dh_xcd_block_order(case):
    """dH with its work-groups dealt to the XCDs in blocks of tiles, against the oracle;
    bitwise repeatable."""
    seed, N, H, V, K, T = case
    say("case: dH XCD block order", case)
    h, W, idx, tl = synthetic(seed, N, H, V, K, T)
    t = arrays(h, W, idx, tl)
    g = run(*t, T=T)
    compare_all(g, h, W, idx, tl, T, what="xblock%d" % seed)
    again = run(*t, T=T)
    np.testing.assert_array_equal(g["dH"], again["dH"])


def test_loss_nonnegative():
    h, W, idx, tl = synthetic(13, 800, 256, 2000, 50, 2.0, z_sigma=6.0)
    g = run(*arrays(h, W, idx, tl), T=2.0, backward=False)
    assert (g["loss"] >= -1e-5 * np.abs(g["loss"]).max()).all()


def test_zero_head_closed_form_on_gpu():
    """W = 0 and equal teacher logits: loss = T^2 log(V/K) per token (closed form)."""
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))
    for c in cases["uniform_teacher_zero_head"]:
        V, K, T = c["V"], c["K"], c["T"]
        N, H = 300, 64
        rng = np.random.default_rng(14)
        h = rng.standard_normal((N, H)).astype(np.float32)
        idx = synth.distinct_indices(15, N, K, V)
        g = run(*arrays(h, np.zeros((V, H), np.float32), idx, np.full((N, K), 0.5, np.float32)), T=T)
        np.testing.assert_allclose(g["loss"], c["loss"], rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(g["lse"], math.log(V), rtol=1e-6)
        assert np.abs(g["dH"]).max() == 0.0


def test_dw_accumulate_and_validate():
    h, W, idx, tl = synthetic(16, 400, 128, 1200, 8, 1.0)
    dh, dW_, di, dt = arrays(h, W, idx, tl)
    loss, lse, _ = fckl.forward(dh, dW_, di, dt, T=1.0, validate=True)
    _, dW1 = fckl.backward(dh, dW_, di, dt, lse, T=1.0)
    dW2 = dW1.clone()
    fckl.backward(dh, dW_, di, dt, lse, T=1.0, dW=dW2, accumulate=True)
    torch.cuda.synchronize()
    a, b = dW2.cpu().numpy(), dW1.cpu().numpy()
    assert np.abs(a - 2 * b).max() <= 1e-6 * np.abs(b).max()
    for bad_value in (1200, -1, None):
        bad = di.clone()
        if bad_value is None:
            bad[5, 3] = bad[5, 1]          # a repeated index within one token
        else:
            bad[7, 2] = bad_value
        for fn in ("forward", "backward"):
            with pytest.raises(fckl.FCKLError) as e:
                if fn == "forward":
                    fckl.forward(dh, dW_, bad, dt, T=1.0, validate=True)
                else:
                    fckl.backward(dh, dW_, bad, dt, lse, T=1.0, validate=True)
            assert e.value.status == fckl.ERR_INDEX


def test_nan_in_one_row_stays_in_that_token():
    """No scrubbing: a NaN in one hidden row gives that token a NaN loss, lse and dH row
    and makes the mean and dW NaN; every other token's loss, lse and dH row equal the
    clean run's bit for bit (each column of the logit tiles is its own token)."""
    N, H, V, K, T = 300, 128, 1500, 8, 1.0
    h, W, idx, tl = synthetic(95, N, H, V, K, T)
    clean = arrays(h, W, idx, tl)
    hn = h.copy()
    hn[137, 5] = np.nan
    dirty = arrays(hn, W, idx, tl)
    outs = []
    for t in (clean, dirty):
        loss, lse, mean = fckl.forward(*t, T=T, chunk=256)
        dH, dW = fckl.backward(*t, lse, T=T, chunk=256)
        single = fckl.forward_backward(*t, T=T, chunk=256)
        outs.append((loss, lse, mean, dH, dW) + tuple(single))
    torch.cuda.synchronize()
    c, d = [[x.cpu().numpy() for x in o] for o in outs]
    keep = np.arange(N) != 137
    for base in (0, 5):     # the two passes, then the single call
        loss_c, lse_c, mean_c, dH_c, dW_c = c[base:base + 5]
        loss_d, lse_d, mean_d, dH_d, dW_d = d[base:base + 5]
        assert np.isnan(loss_d[137]) and np.isnan(lse_d[137]) and np.isnan(dH_d[137]).all()
        assert np.isnan(mean_d[0]) and np.isnan(dW_d).all()
        assert np.array_equal(loss_d[keep], loss_c[keep]) and np.array_equal(lse_d[keep], lse_c[keep])
        assert np.array_equal(dH_d[keep], dH_c[keep])
        assert np.isfinite(mean_c[0]) and np.isfinite(dW_c).all()


def test_empty_inputs_are_refused():
    """N = 0 (an empty batch) and K = 0 (no cached entry) are argument errors, reported
    before any kernel is launched; the autograd module passes the error on."""
    from chunked_top_kl_chunk_amd.loss import FusedChunkedKLLoss
    dev = device()
    W = torch.zeros(300, 64, dtype=torch.bfloat16, device=dev)
    for N, K in ((0, 5), (4, 0)):
        h = torch.zeros(N, 64, dtype=torch.bfloat16, device=dev)
        idx = torch.zeros(N, K, dtype=torch.int32, device=dev)
        tl = torch.zeros(N, K, dtype=torch.bfloat16, device=dev)
        with pytest.raises(fckl.FCKLError) as e:
            fckl.forward(h, W, idx, tl)
        assert e.value.status == fckl.ERR_INVALID_ARG, (N, K)
        with pytest.raises(fckl.FCKLError) as e:
            fckl.forward_backward(h, W, idx, tl)
        assert e.value.status == fckl.ERR_INVALID_ARG, (N, K)
        with pytest.raises(fckl.FCKLError):
            FusedChunkedKLLoss()(h.requires_grad_(True), W, idx, tl)
    torch.cuda.synchronize()
    say("empty batch and empty cache rows: refused with ERR_INVALID_ARG")


def test_single_vocabulary_entry_gives_zero():
    """V = K = 1: teacher and student both put all their mass on the one entry, so every
    loss is 0 and so are dH and dW, up to the rounding of lse (stored in natural-log
    units and converted back to base 2 by the backward pass)."""
    N, H, T = 300, 64, 1.3
    h, W, idx, tl = synthetic(130, N, H, 1, 1, T)
    g = run(*arrays(h, W, idx, tl), T=T, chunk=256)
    z = h.astype(np.float64) @ W.astype(np.float64).T          # [N, 1]
    assert np.abs(g["lse"] - z[:, 0] / T).max() <= LSE_ATOL
    assert float(np.abs(g["loss"]).max()) <= 1e-5 and abs(float(g["mean"][0])) <= 1e-5
    # against the gradient scale T/N of one entry of probability 1
    assert float(np.abs(g["dH"]).max()) <= 1e-5 * (T / N) * float(np.abs(W).max())
    assert float(np.abs(g["dW"]).max()) <= 1e-5 * (T / N) * float(np.abs(h).sum(axis=0).max())
    say("V = K = 1: max|loss| %.1e, max|dH| %.1e, max|dW| %.1e"
        % (float(np.abs(g["loss"]).max()), float(np.abs(g["dH"]).max()), float(np.abs(g["dW"]).max())))


@pytest.mark.parametrize("case", [
    # seed, N, H, V, K, T, chunk: the largest hidden size; the largest vocabulary (its g
    # and W^T pitch of 2^24 takes the products' 32-bit operand offsets to their limit);
    # 2M tokens in 256 chunks of the scheduler's 8192 (dW accumulated across all of them,
    # the mean a fixed-order sum over 2M tokens)
    (140, 40, 65536, 300, 8, 1.0, 256),
    (141, 8, 8, 2 ** 24, 128, 1.0, 256),
    (142, 2 ** 21, 8, 300, 4, 1.0, 0),
], ids=["H65536", "V2^24", "N2^21"])
def test_largest_supported_shapes(case):
    seed, N, H, V, K, T, chunk = case
    say("case: largest shapes", case)
    h, W, idx, tl = synthetic(seed, N, H, V, K, T)
    t = arrays(h, W, idx, tl)
    dev = device()
    desc = fckl.desc_for(*t, T, chunk)
    chunk = chunk or fckl.plan(desc)[0]
    ws = torch.empty(fckl.workspace_size(desc, chunk), dtype=torch.uint8, device=dev)
    loss, lse, mean = fckl.forward(*t, T=T, chunk=chunk, ws=ws)
    dH, dW = fckl.backward(*t, lse, T=T, chunk=chunk, ws=ws)
    torch.cuda.synchronize()
    g = {"loss": loss.cpu().numpy(), "lse": lse.cpu().numpy(), "mean": mean.cpu().numpy(),
         "dH": dH.cpu().numpy(), "dW": dW.cpu().numpy()}
    del ws, dH, dW
    torch.cuda.empty_cache()
    compare_all(g, h, W, idx, tl, T, what="largest%d" % seed)

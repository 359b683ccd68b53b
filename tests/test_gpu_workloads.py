"""GPU parity at the full workload sizes, in the launch configuration the benchmark uses
(the library's own chunk choice for its default workspace budget).

At these sizes the oracle cannot run every token, so:
  * per-token outputs (loss, lse and dH rows) are compared with the oracle on a seeded
    sample of 512 tokens (the oracle computes each token on its own, normalising dH by
    the full N); the sample includes 64 of the stress workload's large-norm rows;
  * dW is compared element by element, over the full vocabulary and hidden size, on a
    separate run of the same shapes restricted to a sampled subset of 512 tokens, run in
    four chunks of 128 so that the fp32 accumulation of dW across chunks is checked
    against the oracle;
  * at full size, properties that hold at any size are checked: every per-token loss
    is >= 0, the mean equals the average of the per-token losses, the rows of dW sum
    to zero (the softmax part of the gradient sums to the teacher mass it removes),
    and <dW, W> = <dH, h> (both equal sum_i <g_i, z_i>);
  * the 256K-token workload runs at chunks of 1024, 2048, 4096 and 8192 tokens: the
    per-token loss and lse do not depend on the chunk, bit for bit, and dH and dW agree
    to fp32 reordering (32 to 256 chunks of accumulation).
An oracle check of dW rows over all N tokens would need every token's lse, 2 N V H
flop in fp64 on the host (about 9 minutes at 32K tokens, over an hour at 256K), so
the multi-chunk accumulation is pinned by the subset run and the chunk sweep, and every
output at full size (all tokens, all of dH and dW) is compared with the same definition
computed densely in float32 by torch's own GEMMs on the GPU, a route pinned against the
oracle on the CPU (tests/test_dense_reference.py).
"""
import functools

import numpy as np
import pytest
import torch

import chunked_top_kl_chunk_amd as fckl
import oracle
import synth
from gpu_util import GRAD_TOL, LOSS_RTOL, LSE_ATOL, check_grad, check_loss, device, say, upload

pytestmark = [pytest.mark.gpu, pytest.mark.slow,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

SAMPLE_ROWS = 512
SCALED_ROWS = 64        # of the stress workload's x20 rows, always in the sample
DW_TOKENS = 512
DW_CHUNK = 128          # the subset's dW accumulates over four chunks


@functools.lru_cache(maxsize=2)
def inputs(key):
    """The workload's seeded inputs, drawn once per session (the 256K-token ones take
    seconds to draw)."""
    return synth.make_inputs(synth.WORKLOADS[key], device=device())


def _run_full(wl, x):
    dev = device()
    h, W, idx, tl = upload(x, dev)
    desc = fckl.desc_for(h, W, idx, tl, wl.T)
    chunk, ws_bytes = fckl.plan(desc)
    say("workload %s N=%d H=%d V=%d K=%d T=%g: chunk %d, workspace %.2f GiB"
        % (wl.name, wl.N, wl.H, wl.V, wl.K, wl.T, chunk, ws_bytes / 2 ** 30))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    loss, lse, mean = fckl.forward(h, W, idx, tl, T=wl.T, chunk=chunk, ws=ws)
    dH, dW = fckl.backward(h, W, idx, tl, lse, T=wl.T, chunk=chunk, ws=ws)
    torch.cuda.synchronize()
    # size-independent identities, evaluated on the GPU in float64
    sum_rows = dW.double().sum(0).abs().max().item()
    scale_rows = dW.double().abs().sum(0).max().item()
    ip_w = (dW.double() * W.double()).sum().item()
    ip_h = (dH.double() * h.double()).sum().item()
    out = dict(loss=loss.cpu().numpy(), lse=lse.cpu().numpy(), mean=float(mean.item()), chunk=chunk,
               sum_rows=sum_rows, scale_rows=scale_rows, ip_w=ip_w, ip_h=ip_h)
    rows = synth.sample_rows(wl, SAMPLE_ROWS, must_include=synth.scaled_rows(wl)[:SCALED_ROWS])
    out["rows"] = rows
    out["dH_rows"] = dH[torch.from_numpy(rows).to(dev)].cpu().numpy()
    del dH, dW, ws, h, W, idx, tl, loss, lse
    torch.cuda.empty_cache()
    return out


def _check_workload(key):
    wl = synth.WORKLOADS[key]
    say("case: full workload", key, wl.name)
    x = inputs(key)
    g = _run_full(wl, x)
    # properties at full size
    assert np.isfinite(g["loss"]).all()
    assert (g["loss"] >= -1e-5 * np.abs(g["loss"]).max()).all()
    assert abs(g["mean"] - g["loss"].astype(np.float64).mean()) <= 1e-5 * abs(g["mean"])
    assert g["sum_rows"] <= 1e-3 * g["scale_rows"], (g["sum_rows"], g["scale_rows"])
    assert abs(g["ip_w"] - g["ip_h"]) <= 2e-2 * max(abs(g["ip_w"]), abs(g["ip_h"]), 1e-30), (g["ip_w"], g["ip_h"])
    # sampled tokens against the oracle
    rows = g["rows"]
    hs, idxs, tls = x.h[rows], x.idx[rows], x.tl[rows]
    W64 = x.W.astype(np.float64)
    ref_loss, ref_lse = oracle.forward(hs, W64, idxs, tls, wl.T)
    e_loss = check_loss(g["loss"][rows], ref_loss, key)
    e_lse = float(np.abs(g["lse"][rows] - ref_lse).max())
    assert e_lse <= LSE_ATOL, "%s lse abs err %.3e" % (key, e_lse)
    ref_dH, _ = oracle.backward(hs, W64, idxs, tls, wl.T, n_norm=wl.N, want_dW=False)
    e_dH = check_grad(g["dH_rows"], ref_dH, key + " dH rows")
    say("%s: chunk %d, sampled %d rows: loss %.2e lse %.2e dH %.2e; sum_v dW %.1e of %.1e; <dW,W> %.6e <dH,h> %.6e"
        % (key, g["chunk"], rows.size, e_loss, e_lse, e_dH, g["sum_rows"], g["scale_rows"], g["ip_w"], g["ip_h"]))
    # dW over the full vocabulary x hidden size, on a token subset run in several chunks
    sub = synth.sample_rows(wl, DW_TOKENS)
    dev = device()
    hb = torch.from_numpy(x.h_bits[sub].view(np.int16)).to(dev).view(torch.bfloat16)
    Wb = torch.from_numpy(x.W_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    ib = torch.from_numpy(np.ascontiguousarray(x.idx[sub])).to(dev)
    tb = torch.from_numpy(x.tl_bits[sub].view(np.int16)).to(dev).view(torch.bfloat16)
    _, lse_s, _ = fckl.forward(hb, Wb, ib, tb, T=wl.T, chunk=DW_CHUNK)
    dH_s, dW_s = fckl.backward(hb, Wb, ib, tb, lse_s, T=wl.T, chunk=DW_CHUNK)
    torch.cuda.synchronize()
    ref_dHs, ref_dWs = oracle.backward(x.h[sub], W64, x.idx[sub], x.tl[sub], wl.T)
    e_dHs = check_grad(dH_s.cpu().numpy(), ref_dHs, key + " subset dH")
    e_dWs = check_grad(dW_s.cpu().numpy(), ref_dWs, key + " subset dW")
    say("%s: %d-token subset in chunks of %d, full V x H: dH %.2e dW %.2e" % (key, sub.size, DW_CHUNK, e_dHs, e_dWs))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", ["c2", "c3", "c4", "c5"])
def test_full_workload(key):
    _check_workload(key)


def _dense_fp32(h, W, idx, tl, T, block=4096):
    """The definition written out densely in torch float32 on the GPU (its own GEMMs, not
    this library), a block of tokens at a time: teacher softmax over the K cached
    entries, z = h W^T, lse over the vocabulary, the per-token KL, g, dH = g W and
    dW = g^T h accumulated over the blocks in float32.  The bf16 inputs are upcast
    exactly.  Returns (loss, lse, dH, dW) as float32 tensors on the GPU."""
    N, H = h.shape
    V = W.shape[0]
    Wf = W.float()
    loss = torch.empty(N, dtype=torch.float32, device=h.device)
    lse = torch.empty(N, dtype=torch.float32, device=h.device)
    dH = torch.empty(N, H, dtype=torch.float32, device=h.device)
    dW = torch.zeros(V, H, dtype=torch.float32, device=h.device)
    for c0 in range(0, N, block):
        c1 = min(N, c0 + block)
        hc = h[c0:c1].float()
        ic = idx[c0:c1].long()
        a = tl[c0:c1].float() / T
        lp = a - torch.logsumexp(a, dim=1, keepdim=True)
        p = lp.exp()
        s = torch.mm(hc, Wf.t()) / T
        l = torch.logsumexp(s, dim=1)
        zk = s.gather(1, ic)
        loss[c0:c1] = T * T * (p * (lp - zk + l[:, None])).sum(1)
        lse[c0:c1] = l
        g = (s - l[:, None]).exp_()
        g *= p.sum(1, keepdim=True)
        g.scatter_add_(1, ic, -p)
        g *= T / N
        dH[c0:c1] = torch.mm(g, Wf)
        dW += torch.mm(g.t().contiguous(), hc)
        del s, g, zk
    return loss, lse, dH, dW


@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", ["c2", "c3", "c4", "c5"])
def test_dense_fp32_reference_at_full_size(key):
    """Every output at full size (all tokens' loss and lse, all of dH and dW after the
    fp32 accumulation over every chunk and vocabulary slab) against the plain dense
    definition computed in float32 by torch on the GPU: a second, independent route at
    the sizes the oracle cannot run whole.  Tolerances as for the oracle."""
    wl = synth.WORKLOADS[key]
    say("case: dense float32 reference", key, wl.name)
    x = inputs(key)
    dev = device()
    h, W, idx, tl = upload(x, dev)
    desc = fckl.desc_for(h, W, idx, tl, wl.T)
    chunk, ws_bytes = fckl.plan(desc)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    loss, lse, mean = fckl.forward(h, W, idx, tl, T=wl.T, chunk=chunk, ws=ws)
    dH, dW = fckl.backward(h, W, idx, tl, lse, T=wl.T, chunk=chunk, ws=ws)
    torch.cuda.synchronize()
    del ws
    r_loss, r_lse, r_dH, r_dW = _dense_fp32(h, W, idx, tl, wl.T)
    torch.cuda.synchronize()
    e_loss = ((loss.double() - r_loss.double()).abs() / r_loss.double().abs().clamp_min(1e-30)).max().item()
    e_lse = (lse - r_lse).abs().max().item()
    e_mean = abs(float(mean.item()) - r_loss.double().mean().item()) / abs(r_loss.double().mean().item())
    e_dH = ((dH - r_dH).abs().max() / r_dH.abs().max()).item()
    e_dW = ((dW - r_dW).abs().max() / r_dW.abs().max()).item()
    say("%s vs dense float32 (chunk %d, %d chunks): loss %.2e lse %.2e mean %.2e dH %.2e dW %.2e"
        % (key, chunk, -(-wl.N // chunk), e_loss, e_lse, e_mean, e_dH, e_dW))
    assert e_loss <= LOSS_RTOL and e_mean <= LOSS_RTOL
    assert e_lse <= LSE_ATOL
    assert e_dH <= GRAD_TOL and e_dW <= GRAD_TOL
    del h, W, idx, tl, loss, lse, dH, dW, r_loss, r_lse, r_dH, r_dW
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_long_context_chunk_sweep():
    """The 256K-token workload (T = 2) at every chunk size the long-context configuration
    sweeps: per-token loss and lse bit for bit equal across chunks (each token's logits
    come from the same tiles whatever chunk holds it), dH and dW equal to fp32 reordering
    (the dH vocabulary splits and the number of dW accumulation steps depend on the chunk)."""
    key = "c4"
    wl = synth.WORKLOADS[key]
    x = inputs(key)
    dev = device()
    h, W, idx, tl = upload(x, dev)
    ref = None
    for chunk in (8192, 4096, 2048, 1024):
        say("case: chunk sweep", key, "chunk", chunk)
        loss, lse, mean = fckl.forward(h, W, idx, tl, T=wl.T, chunk=chunk)
        dH, dW = fckl.backward(h, W, idx, tl, lse, T=wl.T, chunk=chunk)
        torch.cuda.synchronize()
        if ref is None:
            ref = (loss, lse, mean, dH, dW)
            continue
        assert torch.equal(loss, ref[0]) and torch.equal(lse, ref[1]), "chunk %d: per-token outputs differ" % chunk
        e_mean = abs(float(mean.item()) - float(ref[2].item())) / abs(float(ref[2].item()))
        e_dH = float((dH - ref[3]).abs().max() / ref[3].abs().max())
        e_dW = float((dW - ref[4]).abs().max() / ref[4].abs().max())
        say("chunk %d against 8192: mean %.1e dH %.1e dW %.1e" % (chunk, e_mean, e_dH, e_dW))
        assert e_mean <= 1e-6 and e_dH <= 1e-5 and e_dW <= 1e-5
        del loss, lse, mean, dH, dW


@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", ["c3", "c4"])
def test_single_call_at_full_size(key):
    """fckl_forward_backward on the 32K- and 256K-token workloads: the forward outputs
    equal the two-call path's bit for bit, the gradients agree with it to the gradient
    tolerance, and the size-independent identities hold."""
    wl = synth.WORKLOADS[key]
    say("case: single call, full workload", wl.name)
    x = inputs(key)
    h, W, idx, tl = upload(x, device())
    desc = fckl.desc_for(h, W, idx, tl, wl.T)
    chunk, _ = fckl.plan(desc)
    desc.chunk = chunk
    ws = torch.empty(fckl.single_plan(desc)[1], dtype=torch.uint8, device=device())
    loss1, lse1, mean1, dH1, dW1 = fckl.forward_backward(h, W, idx, tl, T=wl.T, chunk=chunk, ws=ws)
    loss2, lse2, mean2 = fckl.forward(h, W, idx, tl, T=wl.T, chunk=chunk, ws=ws)
    assert torch.equal(loss1, loss2) and torch.equal(lse1, lse2) and torch.equal(mean1, mean2)
    dH2, dW2 = fckl.backward(h, W, idx, tl, lse2, T=wl.T, chunk=chunk, ws=ws)
    torch.cuda.synchronize()
    e_dH = float((dH1 - dH2).abs().max() / dH2.abs().max())
    e_dW = float((dW1 - dW2).abs().max() / dW2.abs().max())
    sum_rows = dW1.double().sum(0).abs().max().item()
    scale_rows = dW1.double().abs().sum(0).max().item()
    ip_w = (dW1.double() * W.double()).sum().item()
    ip_h = (dH1.double() * h.double()).sum().item()
    say("single call vs two-call at full size: dH %.2e dW %.2e; sum_v dW %.1e of %.1e; <dW,W> %.6e <dH,h> %.6e"
        % (e_dH, e_dW, sum_rows, scale_rows, ip_w, ip_h))
    assert e_dH <= GRAD_TOL and e_dW <= GRAD_TOL
    assert sum_rows <= 1e-3 * scale_rows
    assert abs(ip_w - ip_h) <= 2e-2 * max(abs(ip_w), abs(ip_h))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", ["c3", "c4"])
def test_full_teacher_at_full_size(key):
    """fckl_full_forward_backward on the 32K- and 256K-token shapes, teacher of the same
    shape (a perturbed copy of the student), in the launch configuration the benchmark
    uses: size-independent identities at full size, sampled tokens against the oracle,
    and dW over the full vocabulary x hidden size on a token subset."""
    wl = synth.WORKLOADS[key]
    say("case: full teacher, full workload", wl.name)
    x = inputs(key)
    tch = synth.full_teacher(wl, x)
    dev = device()

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
    h, W, ht, Wt = bf(x.h_bits), bf(x.W_bits), bf(tch.h_bits), bf(tch.W_bits)
    chunk, ws_bytes = fckl.full_plan(fckl.make_desc(wl.N, wl.H, wl.V, 1, wl.T), wl.H)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    loss, lse, mean, dH, dW = fckl.full_forward_backward(h, W, ht, Wt, T=wl.T, chunk=chunk, ws=ws)
    torch.cuda.synchronize()
    sum_rows = dW.double().sum(0).abs().max().item()
    scale_rows = dW.double().abs().sum(0).max().item()
    ip_w = (dW.double() * W.double()).sum().item()
    ip_h = (dH.double() * h.double()).sum().item()
    loss_n, lse_n = loss.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(loss_n).all()
    assert (loss_n >= -1e-5 * np.abs(loss_n).max()).all()
    assert abs(float(mean.item()) - loss_n.astype(np.float64).mean()) <= 1e-5 * abs(float(mean.item()))
    assert sum_rows <= 1e-3 * scale_rows, (sum_rows, scale_rows)
    assert abs(ip_w - ip_h) <= 2e-2 * max(abs(ip_w), abs(ip_h)), (ip_w, ip_h)
    rows = synth.sample_rows(wl, 32)
    rt = torch.from_numpy(rows).to(dev)
    dH_rows = dH[rt].cpu().numpy()
    del dH, dW, ws
    torch.cuda.empty_cache()
    # the oracle on the sampled tokens alone (its gradient is normalised by their count)
    r_loss, r_lse, _, r_dH, r_dW = oracle.full(x.h[rows], x.W, tch.h[rows], tch.W, wl.T)
    e_loss = check_loss(loss_n[rows], r_loss, "full teacher")
    e_lse = float(np.abs(lse_n[rows] - r_lse).max())
    assert e_lse <= LSE_ATOL, "lse abs err %.3e" % e_lse
    e_dH = check_grad(dH_rows, r_dH * (rows.size / wl.N), "full teacher dH rows")
    # the same tokens as their own batch: dW over the full V x H
    _, _, _, dH_s, dW_s = fckl.full_forward_backward(h[rt].contiguous(), W, ht[rt].contiguous(), Wt, T=wl.T,
                                                     chunk=chunk)
    torch.cuda.synchronize()
    e_dHs = check_grad(dH_s.cpu().numpy(), r_dH, "full teacher subset dH")
    e_dWs = check_grad(dW_s.cpu().numpy(), r_dW, "full teacher subset dW")
    say("full teacher at full size: chunk %d, mean KL %.4f; sampled %d rows: loss %.2e lse %.2e dH %.2e; "
        "subset dH %.2e dW %.2e; sum_v dW %.1e of %.1e; <dW,W> %.6e <dH,h> %.6e"
        % (chunk, float(mean.item()), rows.size, e_loss, e_lse, e_dH, e_dHs, e_dWs, sum_rows, scale_rows,
           ip_w, ip_h))


def test_peak_memory_has_no_tokens_times_vocab_term():
    """Peak device memory of fwd+bwd at the 32K shape's H, V, K for growing N up to 256K
    tokens, fixed chunk: linear in N with the per-token cost of the inputs and outputs
    only."""
    dev = device()
    H, V, K, chunk = 2880, 201088, 100, 4096
    gen = torch.Generator(device=dev)
    gen.manual_seed(31)
    W = (torch.randn(V, H, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    peaks = []
    Ns = (4096, 16384, 32768, 65536, 131072, 262144)
    for N in Ns:
        say("case: peak memory N=%d" % N)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        h = torch.randn(N, H, device=dev, dtype=torch.bfloat16, generator=gen)
        # K distinct indices per token: a random offset plus k (V // K), modulo V
        off = torch.randint(0, V, (N, 1), device=dev, generator=gen)
        idx = ((off + torch.arange(K, device=dev) * (V // K)) % V).to(torch.int32)
        tl = torch.randn(N, K, device=dev, dtype=torch.bfloat16, generator=gen)
        loss, lse, _ = fckl.forward(h, W, idx, tl, T=1.0, chunk=chunk)
        dH, dW = fckl.backward(h, W, idx, tl, lse, T=1.0, chunk=chunk)
        torch.cuda.synchronize()
        peaks.append(torch.cuda.max_memory_allocated() - base)
        del h, off, idx, tl, loss, lse, dH, dW
    per_token = [(peaks[i + 1] - peaks[i]) / (Ns[i + 1] - Ns[i]) for i in range(len(Ns) - 1)]
    expect = 2 * H + 4 * H + K * (4 + 2) + 4 + 4          # h, dH, idx, logits, loss, lse
    say("peak bytes %s, per-token slope %s (expected %d, an N x V term would add %d)"
        % (peaks, per_token, expect, 4 * V))
    for s in per_token:
        assert 0.9 * expect <= s <= 1.1 * expect

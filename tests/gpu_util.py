"""Shared plumbing of the GPU tests: upload synthetic inputs, run the library, compare.

Tolerances (written in the tests that use them): per-token loss and the mean loss
within 1e-3 relative; lse within 1e-3 absolute (it enters the loss additively, so
the loss bound covers it); dH and dW with max|gpu - oracle| <= 2e-2 * max|oracle|.
The GPU path takes bf16 inputs, accumulates in fp32 and rounds the chunk gradient g
to bf16 before the dH / dW products; the oracle sees the same bf16 values in fp64.
"""
import math
import sys

import numpy as np
import torch

import chunked_top_kl_chunk_amd as fckl
import synth

LOSS_RTOL = 1e-3
LSE_ATOL = 1e-3
GRAD_TOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device():
    return torch.device("cuda:0")


def upload(x: synth.Inputs, dev, logits_f32: bool = False):
    h = torch.from_numpy(x.h_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    W = torch.from_numpy(x.W_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    idx = torch.from_numpy(np.ascontiguousarray(x.idx)).to(dev)
    if logits_f32:
        tl = torch.from_numpy(np.ascontiguousarray(x.tl)).to(dev)
    else:
        tl = torch.from_numpy(x.tl_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    return h, W, idx, tl


def arrays(h, W, idx, tl):
    """Upload plain arrays (values already bf16-representable) the same way."""
    hb, Wb, tb = synth.bf16_bits(h.astype(np.float32)), synth.bf16_bits(W.astype(np.float32)), synth.bf16_bits(
        tl.astype(np.float32))
    dev = device()
    return (torch.from_numpy(hb.view(np.int16)).to(dev).view(torch.bfloat16),
            torch.from_numpy(Wb.view(np.int16)).to(dev).view(torch.bfloat16),
            torch.from_numpy(np.ascontiguousarray(idx.astype(np.int32))).to(dev),
            torch.from_numpy(tb.view(np.int16)).to(dev).view(torch.bfloat16))


def run(h, W, idx, tl, T, chunk=0, grad_scale=1.0, backward=True, vocab_slab=0):
    loss, lse, mean = fckl.forward(h, W, idx, tl, T=T, chunk=chunk, vocab_slab=vocab_slab)
    out = {"loss": loss, "lse": lse, "mean": mean}
    if backward:
        dH, dW = fckl.backward(h, W, idx, tl, lse, T=T, grad_scale=grad_scale, chunk=chunk, vocab_slab=vocab_slab)
        out.update(dH=dH, dW=dW)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def rel_max(a, b):
    """max|a - b| / max|b|"""
    b = np.asarray(b, np.float64)
    return float(np.abs(np.asarray(a, np.float64) - b).max() / max(np.abs(b).max(), 1e-300))


def check_loss(gpu_loss, ref_loss, what=""):
    err = np.abs(gpu_loss - ref_loss) / np.maximum(np.abs(ref_loss), 1e-30)
    assert np.isfinite(gpu_loss).all(), what + " loss not finite"
    assert err.max() <= LOSS_RTOL, "%s per-token loss rel err %.3e at %d" % (what, err.max(), int(err.argmax()))
    return float(err.max())


def check_grad(gpu, ref, what):
    assert np.isfinite(gpu).all(), what + " not finite"
    e = rel_max(gpu, ref)
    assert e <= GRAD_TOL, "%s max-abs error %.3e of max|oracle|" % (what, e)
    return e


def synthetic(seed, N, H, V, K, T, tl_sigma=2.0, z_sigma=2.0, scaled_frac=0.0):
    """h ~ N(0,1), W ~ N(0, (z_sigma^2)/H) so that logits spread over a few units, teacher
    logits N(0, tl_sigma^2) sorted descending on K distinct random indices; bf16 values."""
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((N, H)).astype(np.float32)
    if scaled_frac > 0:
        pick = rng.permutation(N)[:max(1, int(round(scaled_frac * N)))]
        h[pick] *= 20.0
    W = (rng.standard_normal((V, H)) * (z_sigma / math.sqrt(H))).astype(np.float32)
    idx = synth.distinct_indices(seed + 1, N, K, V)
    tl = -np.sort(-rng.standard_normal((N, K)).astype(np.float32) * tl_sigma, axis=1)
    return synth.round_bf16(h), synth.round_bf16(W), idx, synth.round_bf16(tl)

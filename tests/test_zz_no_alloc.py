"""fckl_forward_noalloc, the forward pass for callers that cannot allocate: its chunk
buffers live in the library's own device array.  Called through the C ABI and checked
against fckl_forward_ex (the entry point it is a variant of) on the same seeded inputs:
bit for bit at the same chunk, and within the oracle tolerances (per-token and mean loss
1e-3 relative, lse 1e-3 absolute).  Two calls in a row, the second on a smaller problem;
the second call takes no device memory; a chunk whose buffers exceed the array is refused.
"""
import ctypes

import numpy as np
import pytest
import torch

import chunked_top_kl_chunk_amd as fckl
from gpu_util import LOSS_RTOL, LSE_ATOL, arrays, device, say, synthetic

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]


def noalloc(h, W, idx, tl, T, chunk, weights=None):
    """fckl_forward_noalloc through ctypes; the outputs are allocated here, before the call."""
    lib = fckl.load()
    N, dev = h.shape[0], h.device
    loss = torch.full((N,), float("nan"), device=dev)
    lse = torch.full((N,), float("nan"), device=dev)
    mean = torch.full((1,), float("nan"), device=dev)
    desc = fckl.desc_for(h, W, idx, tl, T, chunk)
    torch.cuda.synchronize()
    st = lib.fckl_forward_noalloc(ctypes.byref(desc), h.data_ptr(), W.data_ptr(), idx.data_ptr(), tl.data_ptr(),
                                  None if weights is None else weights.data_ptr(), loss.data_ptr(), lse.data_ptr(),
                                  mean.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return st, loss, lse, mean


def existing(h, W, idx, tl, T, chunk, weights=None):
    return fckl.forward(h, W, idx, tl, T=T, chunk=chunk, weights=weights)


def compare(a, b, what):
    """Bit-identical outputs, and within the oracle tolerances (which bit-identity implies)."""
    for name, x, y in zip(("loss", "lse", "mean"), a, b):
        xs, ys = x.cpu().numpy(), y.cpu().numpy()
        assert np.isfinite(xs).all(), "%s %s not finite" % (what, name)
        assert np.array_equal(xs.view(np.uint32), ys.view(np.uint32)), "%s %s differs" % (what, name)
    rel = (a[0] - b[0]).abs() / b[0].abs().clamp_min(1e-30)
    assert float(rel.max()) <= LOSS_RTOL
    assert float((a[1] - b[1]).abs().max()) <= LSE_ATOL


def test_noalloc_matches_forward_ex_twice_second_smaller():
    dev = device()
    # call 1: three chunks of 1024 tokens, a ragged vocabulary tail, weights with zeros
    N, H, V, K, T = 3000, 264, 5000, 20, 1.3
    say("case: noalloc call 1 N=%d H=%d V=%d K=%d chunk=1024" % (N, H, V, K))
    h, W, idx, tl = arrays(*synthetic(701, N, H, V, K, T))
    w = torch.from_numpy(np.random.default_rng(702).uniform(0.0, 2.0, N).astype(np.float32)).to(dev)
    w[::7] = 0.0
    for weights in (None, w):
        st, *out = noalloc(h, W, idx, tl, T, 1024, weights)
        assert st == fckl.OK, fckl.status_string(st)
        compare(out, existing(h, W, idx, tl, T, 1024, weights), "call 1 (weights %s)" % (weights is not None))
    # call 2: a smaller problem right after; the library's array keeps call 1's contents
    N2, H2, V2, K2, T2 = 700, 128, 3000, 7, 0.7
    say("case: noalloc call 2 N=%d H=%d V=%d K=%d chunk=0" % (N2, H2, V2, K2))
    h2, W2, idx2, tl2 = arrays(*synthetic(703, N2, H2, V2, K2, T2))
    lib = fckl.load()
    outs = [torch.full((N2,), float("nan"), device=dev), torch.full((N2,), float("nan"), device=dev),
            torch.full((1,), float("nan"), device=dev)]
    torch.cuda.synchronize()
    free_mid, _ = torch.cuda.mem_get_info()
    alloc_mid = torch.cuda.memory_allocated()
    desc = fckl.desc_for(h2, W2, idx2, tl2, T2, 0)
    st = lib.fckl_forward_noalloc(ctypes.byref(desc), h2.data_ptr(), W2.data_ptr(), idx2.data_ptr(), tl2.data_ptr(),
                                  None, outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    free_after, _ = torch.cuda.mem_get_info()
    assert st == fckl.OK, fckl.status_string(st)
    assert free_after == free_mid, "the call changed free device memory by %d bytes" % (free_mid - free_after)
    assert torch.cuda.memory_allocated() == alloc_mid
    say("free device memory before/after the call: %d / %d" % (free_mid, free_after))
    # the per-token results do not depend on the chunk, so fckl_forward_ex's own chunk serves
    compare(outs, existing(h2, W2, idx2, tl2, T2, 0), "call 2")


def test_noalloc_large_vocabulary():
    """A 201088-entry vocabulary at 4096 tokens per chunk (about 29 MB of forward buffers in
    the array).  The refusal of a chunk whose buffers exceed the array is a host-side check
    made before any HIP call; tests/test_library_host.py covers it with fake addresses, so
    that no kernel ever runs on buffers that do not match the descriptor."""
    N, H, V, K = 300, 64, 201088, 4
    say("case: noalloc N=%d H=%d V=%d K=%d chunk=4096" % (N, H, V, K))
    h3, W3, idx3, tl3 = arrays(*synthetic(712, N, H, V, K, 1.0))
    st, *out = noalloc(h3, W3, idx3, tl3, 1.0, 4096)
    assert st == fckl.OK, fckl.status_string(st)
    compare(out, existing(h3, W3, idx3, tl3, 1.0, 4096), "large vocabulary")

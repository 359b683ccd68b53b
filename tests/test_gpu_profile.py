"""The per-kernel timing hook of the C ABI (fckl_desc.profile, struct fckl_profile).

bench.py derives its live per-kernel times and the roofline from it, so it is checked
here on its own: every selected launch is bracketed, in launch order, with the token
count and the vocabulary rows it processed; unselected kernels and launches past the
capacity are left out; and profiling changes no result.
"""
import ctypes

import pytest
import torch

import chunked_top_kl_chunk_amd as fckl
from gpu_util import arrays, say, synthetic

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

ID = {name: i for i, name in enumerate(fckl.KERNELS)}


class Events:
    """n hipEvent_t handles from the HIP runtime, for the library to record."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.arr[i] = e.value

    def ms(self, i):
        out = ctypes.c_float(0)
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), self.arr[2 * i], self.arr[2 * i + 1]) == 0
        return float(out.value)

    def close(self):
        for e in self.arr:
            self.hip.hipEventDestroy(e)


def profile(mask, capacity, vocab_rows=None):
    ev = Events(2 * capacity)
    kid = (ctypes.c_int32 * capacity)()
    work = (ctypes.c_int32 * capacity)()
    if vocab_rows is None:
        return fckl.Profile(mask, capacity, 0, ev.arr, kid, work), ev, kid, work
    return fckl.Profile(mask, capacity, 0, ev.arr, kid, work, vocab_rows), ev, kid, work


def problem():
    N, H, V, K, T, C = 600, 256, 3000, 10, 1.0, 256      # chunks of 256, 256 and 88 tokens
    return arrays(*synthetic(120, N, H, V, K, T)), T, C, [256, 256, 88]


def test_profile_brackets_every_selected_launch():
    t, T, C, rows = problem()
    N = t[0].shape[0]
    prof, ev, kid, work = profile((1 << len(fckl.KERNELS)) - 1, 64)
    loss, lse, mean = fckl.forward(*t, T=T, chunk=C, profile=prof)
    dH, dW = fckl.backward(*t, lse, T=T, chunk=C, profile=prof)
    torch.cuda.synchronize()
    got = [(fckl.KERNELS[kid[i]], work[i]) for i in range(prof.count)]
    want = []
    for r in rows:
        want += [("prepare", r), ("fwd_logits", r), ("combine", r)]
    want += [("mean", N), ("transpose", 0)]                  # W^T once per backward call
    for r in rows:
        want += [("prepare", r), ("transpose", r), ("bwd_logits", r), ("dh", r), ("dw", r), ("dh_reduce", r)]
    assert got == want
    times = [ev.ms(i) for i in range(prof.count)]
    assert all(x >= 0.0 for x in times)
    assert all(x > 0.0 for (name, _), x in zip(got, times) if name in ("fwd_logits", "bwd_logits", "dh", "dw"))
    ev.close()
    # profiling records events only: the results equal those of an unprofiled run, bit for bit
    loss2, lse2, mean2 = fckl.forward(*t, T=T, chunk=C)
    dH2, dW2 = fckl.backward(*t, lse2, T=T, chunk=C)
    torch.cuda.synchronize()
    for a, b in ((loss, loss2), (lse, lse2), (mean, mean2), (dH, dH2), (dW, dW2)):
        assert torch.equal(a, b)
    say("profile: %d launches bracketed in order, GEMM times %s ms"
        % (len(got), ", ".join("%.3f" % x for (n, _), x in zip(got, times) if n == "dw")))


def test_profile_mask_and_capacity():
    t, T, C, rows = problem()
    mask = (1 << ID["fwd_logits"]) | (1 << ID["dw"])
    # room for all six selected launches: only those are recorded
    prof, ev, kid, work = profile(mask, 8)
    _, lse, _ = fckl.forward(*t, T=T, chunk=C, profile=prof)
    fckl.backward(*t, lse, T=T, chunk=C, profile=prof)
    torch.cuda.synchronize()
    assert [(fckl.KERNELS[kid[i]], work[i]) for i in range(prof.count)] == \
        [("fwd_logits", r) for r in rows] + [("dw", r) for r in rows]
    ev.close()
    # room for four: the first four are recorded, the rest run untimed
    prof, ev, kid, work = profile(mask, 4)
    _, lse, _ = fckl.forward(*t, T=T, chunk=C, profile=prof)
    fckl.backward(*t, lse, T=T, chunk=C, profile=prof)
    torch.cuda.synchronize()
    assert prof.count == 4
    assert [fckl.KERNELS[kid[i]] for i in range(4)] == ["fwd_logits"] * 3 + ["dw"]
    assert all(ev.ms(i) > 0.0 for i in range(4))
    ev.close()
    # an empty mask records nothing
    prof, ev, kid, work = profile(0, 4)
    fckl.forward(*t, T=T, chunk=C, profile=prof)
    torch.cuda.synchronize()
    assert prof.count == 0
    ev.close()


def test_profile_reports_vocabulary_rows_per_slab():
    """With slabs of 512 vocabulary rows (V = 3000: 6 slabs, the last of 440 rows) the
    backward's logit, dH and dW launches run once per slab and report the slab's rows;
    the other launches report V or, without a vocabulary dimension, 0."""
    t, T, C, rows = problem()
    V = t[1].shape[0]
    slabs = [512] * 5 + [V - 5 * 512]
    cap = 128
    vr = (ctypes.c_int32 * cap)()
    prof, ev, kid, work = profile((1 << len(fckl.KERNELS)) - 1, cap, vr)
    loss, lse, mean = fckl.forward(*t, T=T, chunk=C, profile=prof, vocab_slab=512)
    fckl.backward(*t, lse, T=T, chunk=C, profile=prof, vocab_slab=512)
    torch.cuda.synchronize()
    got = [(fckl.KERNELS[kid[i]], work[i], vr[i]) for i in range(prof.count)]
    N = t[0].shape[0]
    want = []
    for r in rows:
        want += [("prepare", r, 0), ("fwd_logits", r, V), ("combine", r, V)]
    want += [("mean", N, 0), ("transpose", 0, 0)]
    for r in rows:
        want += [("prepare", r, 0), ("transpose", r, 0)]
        for v in slabs:
            want += [("bwd_logits", r, v), ("dh", r, v), ("dw", r, v)]
        want += [("dh_reduce", r, 0)]
    assert got == want
    ev.close()

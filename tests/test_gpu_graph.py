"""The loss calls inside a captured HIP graph, and on concurrent streams.

The library allocates nothing, records no memset and (without FCKL_FLAG_VALIDATE) never
synchronises, so a training or serving loop can capture a whole step -- the two passes,
the single call, or the full-teacher call -- and replay it.  Each graph is replayed
several times with eager work and host synchronisations between the replays (the
outputs are overwritten with garbage first), and every replay must give the eager
results bit for bit: the kernels are deterministic.
"""
import numpy as np
import pytest
import torch

import chunked_top_kl_chunk_amd as fckl
import synth
from gpu_util import arrays, device, say, synthetic

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

REPLAYS = 3


def check_replays(graph, outs, ref, what):
    for rep in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), "%s: replay %d, output %d differs from the eager call" % (what, rep, i)
    say("%s: %d replays equal the eager call" % (what, REPLAYS))


@pytest.mark.parametrize("slab", [0, 512], ids=["planner-slab", "slabs-of-512"])
def test_two_passes_in_a_graph(slab):
    """With slabs of 512 vocabulary rows the backward launches its three kernels six
    times per chunk: the graph holds all of them."""
    N, H, V, K, T = 600, 256, 3000, 10, 1.5
    h, W, idx, tl = synthetic(90, N, H, V, K, T)
    dh, dW_, di, dt = arrays(h, W, idx, tl)
    dev = device()
    desc = fckl.desc_for(dh, dW_, di, dt, T, 256, vocab_slab=slab)
    ws = torch.empty(fckl.workspace_size(desc, 256), dtype=torch.uint8, device=dev)
    outs = [torch.empty(N, device=dev), torch.empty(N, device=dev), torch.empty(1, device=dev),
            torch.empty(N, H, device=dev), torch.empty(V, H, device=dev)]
    loss, lse, mean, dH, dW = outs

    def step():
        fckl.forward(dh, dW_, di, dt, T=T, chunk=256, ws=ws, loss_tok=loss, lse=lse, loss_mean=mean, vocab_slab=slab)
        fckl.backward(dh, dW_, di, dt, lse, T=T, grad_scale=0.5, chunk=256, ws=ws, dH=dH, dW=dW, vocab_slab=slab)

    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                         # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    check_replays(g, outs, ref, "forward + backward")


def test_single_call_and_full_teacher_in_graphs():
    N, H, V, K, T = 520, 128, 2100, 8, 1.0
    h, W, idx, tl = synthetic(91, N, H, V, K, T)
    dh, dW_, di, dt = arrays(h, W, idx, tl)
    dev = device()
    w = torch.from_numpy(np.random.default_rng(92).uniform(0.0, 2.0, N).astype(np.float32)).to(dev)
    desc = fckl.desc_for(dh, dW_, di, dt, T, 256)
    ws = torch.empty(fckl.single_plan(desc)[1], dtype=torch.uint8, device=dev)
    outs = [torch.empty(N, device=dev), torch.empty(N, device=dev), torch.empty(1, device=dev),
            torch.empty(N, H, device=dev), torch.empty(V, H, device=dev)]

    def single():
        fckl.forward_backward(dh, dW_, di, dt, T=T, grad_scale=2.0, weights=w, chunk=256, ws=ws, loss_tok=outs[0],
                              lse=outs[1], loss_mean=outs[2], dH=outs[3], dW=outs[4])

    # the teacher of the full-vocabulary variant: a perturbed copy of the student
    rng = np.random.default_rng(93)
    ht = synth.round_bf16(h + 0.3 * rng.standard_normal(h.shape).astype(np.float32))
    Wt = synth.round_bf16(W + 0.01 * rng.standard_normal(W.shape).astype(np.float32))
    dht, dWt, _, _ = arrays(ht, Wt, idx, tl)
    fchunk, fneed = fckl.full_plan(fckl.make_desc(N, H, V, 1, T, 256), H)
    fws = torch.empty(fneed, dtype=torch.uint8, device=dev)
    fouts = [torch.empty_like(o) for o in outs]

    def full():
        fckl.full_forward_backward(dh, dW_, dht, dWt, T=T, weights=w, chunk=fchunk, ws=fws, loss_tok=fouts[0],
                                   lse=fouts[1], loss_mean=fouts[2], dH=fouts[3], dW=fouts[4])

    for fn, o, what in ((single, outs, "single call"), (full, fouts, "full teacher")):
        fn()
        torch.cuda.synchronize()
        ref = [x.clone() for x in o]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        check_replays(g, o, ref, what)


def test_two_streams_at_once_give_the_sequential_results():
    """No global state: two problems on two streams, each with its own workspace, run
    concurrently and give exactly what they give alone."""
    dev = device()
    probs = []
    for seed, (N, H, V, K, T) in ((97, (700, 256, 4100, 10, 1.0)), (98, (500, 128, 3000, 20, 2.0))):
        t = arrays(*synthetic(seed, N, H, V, K, T))
        desc = fckl.desc_for(*t, T, 256)
        ws = torch.empty(fckl.workspace_size(desc, 256), dtype=torch.uint8, device=dev)
        probs.append((t, T, ws))

    def run_one(p, stream):
        t, T, ws = p
        loss, lse, mean = fckl.forward(*t, T=T, chunk=256, ws=ws, stream=stream)
        dH, dW = fckl.backward(*t, lse, T=T, chunk=256, ws=ws, stream=stream)
        return [loss, lse, mean, dH, dW]

    alone = []
    for p in probs:
        alone.append(run_one(p, None))
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    together = []
    for p, s in zip(probs, streams):
        with torch.cuda.stream(s):
            together.append(run_one(p, s))
    torch.cuda.synchronize()
    for a, b in zip(alone, together):
        for x, y in zip(a, b):
            assert torch.equal(x, y)
    say("two streams at once: outputs equal the sequential ones")

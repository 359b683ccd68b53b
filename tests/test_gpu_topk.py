"""GPU parity of the teacher-side top-K extraction (fckl_topk) against the CPU oracle.

The GPU accumulates z in fp32 from bf16 inputs; the oracle forms z in fp64 from the
same bf16 values.  Where two logits of a token lie closer than that rounding, either
order is correct, so the comparison is:
  * the returned z equal the oracle's z at the returned indices within EPS;
  * the list is ordered by the returned z (descending, equal values by index);
  * every index the oracle ranks above the K-th value by more than 2 EPS is returned,
    and every returned index has an oracle z above the K-th value minus 2 EPS;
  * at every position whose oracle value is more than 2 EPS from both neighbours in the
    oracle's order, the returned index is the oracle's.
Exact ties (duplicated head rows give bitwise equal z on both sides) must go to the
smaller index.
"""
import numpy as np
import pytest
import torch

import chunked_top_kl_chunk_amd as fckl
import oracle
import synth
from gpu_util import arrays, device, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

EPS = 2e-4


def check_topk(h, W, K, gi, gz, what):
    """h, W: the bf16-exact values (numpy); gi, gz: GPU indices and z (numpy)."""
    N = h.shape[0]
    oi, oz = oracle.topk(h, W, K + 1 if K < W.shape[0] else K)
    z_at = np.einsum("nh,nkh->nk", h.astype(np.float64), W.astype(np.float64)[gi])
    assert np.abs(gz - z_at).max() <= EPS * max(1.0, np.abs(z_at).max()), what + ": values"
    exact = 0
    for i in range(N):
        # ordered by the returned values, equal values by index
        key = [(-gz[i, k], gi[i, k]) for k in range(K)]
        assert key == sorted(key), "%s token %d not ordered" % (what, i)
        assert len(set(gi[i].tolist())) == K, "%s token %d repeats an index" % (what, i)
        kth = oz[i, K - 1]
        must = set(oi[i, :K][oz[i, :K] > kth + 2 * EPS].tolist())
        assert must <= set(gi[i].tolist()), "%s token %d misses a clear top-K entry" % (what, i)
        assert (z_at[i] >= kth - 2 * EPS).all(), "%s token %d returned a non-top entry" % (what, i)
        # positions whose oracle value is separated from both neighbours are unique
        for k in range(K):
            lo = k == 0 or oz[i, k - 1] - oz[i, k] > 2 * EPS
            hi = (k + 1 >= oz.shape[1]) or oz[i, k] - oz[i, k + 1] > 2 * EPS
            if lo and hi:
                assert gi[i, k] == oi[i, k], "%s token %d position %d: %d vs %d" % (what, i, k, gi[i, k], oi[i, k])
                exact += 1
    say("%s: %d tokens, %d of %d positions unique and equal" % (what, N, exact, N * K))


CASES = [
    # seed, N, H, V, K, chunk
    (70, 300, 256, 4100, 100, 0),
    (71, 517, 136, 1000, 10, 256),
    (72, 130, 2880, 777, 128, 0),
    (73, 64, 512, 300, 100, 0),          # fewer 16-row slices than K: every logit is a candidate
    (74, 200, 256, 3000, 100, 0),        # fewer 32-row slices than K, 2048 < V: 16-row slices
    (75, 96, 128, 3840, 128, 0),         # the same at the largest K
]


@pytest.mark.parametrize("case", CASES, ids=["K100", "K10-ragged", "K128-H2880", "small-V", "V3000-16-row-slices",
                                           "V3840-K128"])
def test_topk_matches_oracle(case):
    seed, N, H, V, K, chunk = case
    say("case: top-K", case)
    rng = np.random.default_rng(seed)
    h = synth.round_bf16(rng.standard_normal((N, H)).astype(np.float32))
    W = synth.round_bf16((rng.standard_normal((V, H)) * (2.0 / np.sqrt(H))).astype(np.float32))
    th, tW, _, _ = arrays(h, W, np.zeros((N, 1), np.int32), np.zeros((N, 1), np.float32))
    gi, gz = fckl.topk(th, tW, K, chunk=chunk, logits_f32=True)
    gi2, gz2 = fckl.topk(th, tW, K, chunk=chunk, logits_f32=True)
    gib, gzb = fckl.topk(th, tW, K, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(gi, gi2) and torch.equal(gz, gz2), "not deterministic"
    assert torch.equal(gib, gi), "bf16 output changed the order"
    assert torch.equal(gzb, gz.to(torch.bfloat16)), "bf16 values are not the rounded fp32 values"
    check_topk(h, W, K, gi.cpu().numpy(), gz.cpu().numpy().astype(np.float64), "topk%d" % seed)


def test_topk_exact_ties_go_to_the_smaller_index():
    rng = np.random.default_rng(74)
    N, H, V, K = 200, 128, 2000, 20
    h = synth.round_bf16(rng.standard_normal((N, H)).astype(np.float32))
    W = synth.round_bf16((rng.standard_normal((V, H)) * 0.2).astype(np.float32))
    # make rows 1500 and 37 copies of row 900, for every token a three-way exact tie
    W[1500] = W[900]
    W[37] = W[900]
    # and make row 900 large for the first tokens so the tie is inside the top-K
    W[900] = W[37] = W[1500] = synth.round_bf16((h[:10].mean(0) * 3.0).astype(np.float32))
    th, tW, _, _ = arrays(h, W, np.zeros((N, 1), np.int32), np.zeros((N, 1), np.float32))
    gi, gz = fckl.topk(th, tW, K, logits_f32=True)
    torch.cuda.synchronize()
    gi = gi.cpu().numpy()
    seen = 0
    for i in range(N):
        row = list(gi[i])
        present = [v for v in (37, 900, 1500) if v in row]
        if len(present) == 3:
            seen += 1
            assert row.index(37) < row.index(900) < row.index(1500)
            assert row.index(900) == row.index(37) + 1 and row.index(1500) == row.index(900) + 1
    assert seen >= 5
    check_topk(h, W, K, gi, gz.cpu().numpy().astype(np.float64), "ties")


def test_topk_zero_head():
    """All logits equal: small V returns the first K indices; a large V is reported."""
    N, H = 64, 64
    h = np.ones((N, H), np.float32)
    th = torch.from_numpy(synth.bf16_bits(h).view(np.int16)).to(device()).view(torch.bfloat16)
    W = torch.zeros(1000, H, dtype=torch.bfloat16, device=device())
    gi, gz = fckl.topk(th, W, 16, logits_f32=True)
    torch.cuda.synchronize()
    assert (gi.cpu().numpy() == np.arange(16)).all() and float(gz.abs().max()) == 0.0
    Wbig = torch.zeros(5000, H, dtype=torch.bfloat16, device=device())
    with pytest.raises(fckl.FCKLError) as e:
        fckl.topk(th, Wbig, 16)
    assert e.value.status == fckl.ERR_UNSUPPORTED


@pytest.mark.slow
def test_topk_at_the_32k_shape_against_torch():
    """The 32K-token GPT-OSS-20B shape (V = 201088, H = 2880, K = 100): the library's
    top-K against torch.topk of the same fp32 product on sampled tokens, and against
    the oracle on a few of them."""
    wl = synth.WORKLOADS["c3"]
    x = synth.make_inputs(wl.with_tokens(4096), device=device())
    dev = device()
    h = torch.from_numpy(x.h_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    W = torch.from_numpy(x.W_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    gi, gz = fckl.topk(h, W, wl.K, logits_f32=True)
    rows = np.random.default_rng(75).permutation(4096)[:256]
    rt = torch.from_numpy(rows).to(dev)
    z = h[rt].float() @ W.float().t()
    tz, ti = torch.topk(z, wl.K, dim=1)
    torch.cuda.synchronize()
    g_sets = gi[rt].cpu().numpy()
    t_sets = ti.cpu().numpy()
    same = np.mean([set(a) == set(b) for a, b in zip(g_sets, t_sets)])
    vz = torch.gather(z, 1, gi[rt].long())
    say("32K shape: %.3f of sampled tokens give torch.topk's set; max |z diff| %.2e"
        % (same, float((vz - gz[rt]).abs().max())))
    assert float((vz - gz[rt]).abs().max()) <= 1e-3
    assert same >= 0.97
    few = rows[:16]
    check_topk(x.h[few], x.W, wl.K, gi.cpu().numpy()[few], gz.cpu().numpy()[few].astype(np.float64), "32K shape")


PARTIAL_CASES = [
    # seed, N, H, V, K: shapes where the first pass covers every 4th tile
    (76, 300, 128, 20000, 10),
    (77, 257, 64, 120000, 100),
]


@pytest.mark.parametrize("case", PARTIAL_CASES, ids=["K10-V20000", "K100-V120000"])
def test_partial_first_pass_matches_full_and_oracle(case):
    """The first pass over a quarter of the vocabulary and the one over all of it give
    the same result, the oracle's."""
    seed, N, H, V, K = case
    say("case: partial first pass", case)
    rng = np.random.default_rng(seed)
    h = synth.round_bf16(rng.standard_normal((N, H)).astype(np.float32))
    W = synth.round_bf16((rng.standard_normal((V, H)) * (2.0 / np.sqrt(H))).astype(np.float32))
    th, tW, _, _ = arrays(h, W, np.zeros((N, 1), np.int32), np.zeros((N, 1), np.float32))
    gi, gz = fckl.topk(th, tW, K, logits_f32=True)
    fi, fz = fckl.topk(th, tW, K, logits_f32=True, full_first_pass=True)
    torch.cuda.synchronize()
    assert torch.equal(gi, fi) and torch.equal(gz, fz)
    check_topk(h, W, K, gi.cpu().numpy(), gz.cpu().numpy().astype(np.float64), "partial%d" % seed)


def test_partial_first_pass_falls_back_when_candidates_overflow():
    """2400 large logits per token, all in tiles the partial first pass skips: its
    threshold comes from ordinary logits and leaves more than 2048 candidates, so every
    chunk is redone with a first pass over every tile -- with the oracle's result."""
    N, H, V, K = 64, 64, 150000, 100
    rng = np.random.default_rng(78)
    h = rng.standard_normal((N, H)).astype(np.float32)
    h[:, 0] = 3.0
    W = (rng.standard_normal((V, H)) * 0.02).astype(np.float32)
    W[:, 0] = 0.0
    tiles = np.arange((V + 255) // 256)
    skipped = np.concatenate([np.arange(t * 256, min(V, t * 256 + 256)) for t in tiles if t % 4 != 0])
    high = rng.choice(skipped, size=2400, replace=False)
    W[high, 0] = (5.0 + 0.5 * rng.standard_normal(high.size)) / 3.0
    h, W = synth.round_bf16(h), synth.round_bf16(W)
    # the precondition, in fp64: the partial first pass overflows, the full one does not
    z = h.astype(np.float64) @ W.astype(np.float64).T
    visited = np.concatenate([np.arange(t * 256, min(V, t * 256 + 256)) for t in tiles if t % 4 == 0])
    zs = z[:, visited]
    pad = (-zs.shape[1]) % 64
    zs = np.concatenate([zs, np.full((N, pad), -np.inf)], axis=1)
    tau_part = -np.sort(-zs.reshape(N, -1, 64).max(axis=2), axis=1)[:, K - 1]
    n_part = (z >= tau_part[:, None]).sum(axis=1)
    zt = np.concatenate([z, np.full((N, (-V) % 256), -np.inf)], axis=1)
    tau_full = -np.sort(-zt.reshape(N, -1, 256).max(axis=2), axis=1)[:, K - 1]
    n_full = (z >= tau_full[:, None]).sum(axis=1)
    say("candidates per token: partial first pass %d..%d, full first pass %d..%d"
        % (n_part.min(), n_part.max(), n_full.min(), n_full.max()))
    assert n_part.min() > 2048 + 100 and n_full.max() < 2048 - 100
    th, tW, _, _ = arrays(h, W, np.zeros((N, 1), np.int32), np.zeros((N, 1), np.float32))
    gi, gz = fckl.topk(th, tW, K, logits_f32=True)
    fi, fz = fckl.topk(th, tW, K, logits_f32=True, full_first_pass=True)
    torch.cuda.synchronize()
    assert torch.equal(gi, fi) and torch.equal(gz, fz)
    check_topk(h, W, K, gi.cpu().numpy(), gz.cpu().numpy().astype(np.float64), "fallback")


def test_topk_async_in_a_graph_and_its_status():
    """fckl_topk_async: the same result as fckl_topk with its status on the device, no
    host synchronisation, so a captured graph can replay it; a zero head over a large
    vocabulary reports FCKL_ERR_UNSUPPORTED through the status word."""
    rng = np.random.default_rng(79)
    N, H, V, K = 300, 128, 20000, 10
    h = synth.round_bf16(rng.standard_normal((N, H)).astype(np.float32))
    W = synth.round_bf16((rng.standard_normal((V, H)) * 0.2).astype(np.float32))
    th, tW, _, _ = arrays(h, W, np.zeros((N, 1), np.int32), np.zeros((N, 1), np.float32))
    dev = device()
    ri, rz = fckl.topk(th, tW, K, logits_f32=True)
    desc = fckl.make_desc(N, H, V, K, 1.0, 0, fckl.DTYPE_F32)
    ws = torch.empty(fckl.topk_workspace_size(desc), dtype=torch.uint8, device=dev)
    gi = torch.empty(N, K, dtype=torch.int32, device=dev)
    gz = torch.empty(N, K, dtype=torch.float32, device=dev)
    status = torch.full((1,), -1, dtype=torch.int32, device=dev)
    fckl.topk(th, tW, K, logits_f32=True, ws=ws, topk_idx=gi, topk_logit=gz, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == fckl.OK and torch.equal(gi, ri) and torch.equal(gz, rz)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fckl.topk(th, tW, K, logits_f32=True, ws=ws, topk_idx=gi, topk_logit=gz, status=status)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fckl.topk(th, tW, K, logits_f32=True, ws=ws, topk_idx=gi, topk_logit=gz, status=status)
    for _ in range(3):
        gi.fill_(-7)
        gz.fill_(float("nan"))
        status.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == fckl.OK and torch.equal(gi, ri) and torch.equal(gz, rz)
    zero = torch.zeros(5000, H, dtype=torch.bfloat16, device=dev)
    fckl.topk(th, zero, 16, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == fckl.ERR_UNSUPPORTED
    say("topk_async: equal to fckl_topk, 3 graph replays equal, overflow reported as status %d" % int(status.item()))

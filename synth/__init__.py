"""Seeded synthetic inputs for the fused chunked top-K KL loss.

This module only draws random numbers and rounds them to bf16; it holds none of
the loss's arithmetic, so both the CPU oracle's tests and the GPU path's tests
and benchmark draw their inputs from here.

There is no trained model and no teacher cache to load: the workloads the pages
describe (a Llama-3.2-3B-shaped student, a GPT-OSS-20B-shaped student at 32K and
256K tokens, with the teacher's top-100 or top-10 logits cached per token) are
stood in for by tensors of the same shapes and value distributions:

* h ~ N(0, 1) of shape [N, H] (student final hidden states), W ~ N(0, 0.02^2) of
  shape [V, H] (LM head, no bias);
* teacher cache, either "exact top-K of a perturbed head" (W' = W + N(0, 0.01^2),
  logits h @ W'^T with fp32 accumulation, top-K by value, descending), or random
  logits N(0, sigma^2) sorted descending paired with K distinct uniform indices;
* values are drawn in float32 and rounded to bf16 (round to nearest even) where the
  workload is bf16, so the oracle and the GPU path see bit-identical inputs.

For the online variant against the teacher's whole distribution, the teacher's final
hidden states and LM head are perturbed copies of the student's (a related model of
the same shape): h_t = h + N(0, 0.3^2), W_t = W + N(0, (0.3 * 0.02)^2), rounded to bf16.

Seeds: ``seed = 1000 * config_number + stream`` with stream h:0, W:1, W'-noise:2,
idx:3, teacher logits:4, scaled-row pick:5, parity row sample:6, teacher h noise:7,
teacher W noise:8.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np

S_H, S_W, S_WNOISE, S_IDX, S_TL, S_ROWS, S_SAMPLE, S_HT, S_WT = 0, 1, 2, 3, 4, 5, 6, 7, 8
TEACHER_NOISE = 0.3


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, temperature, chunk and generator recipe."""
    name: str
    number: int
    N: int
    H: int
    V: int
    K: int
    T: float
    chunk: int                      # 0 = let the planner choose
    dtype: str                      # "fp32" (GPU sees bf16 copies) or "bf16"
    teacher: str                    # "random" or "topk_perturbed"
    tl_sigma: float = 1.0           # for teacher == "random"
    scaled_row_frac: float = 0.0    # fraction of h rows multiplied by scaled_row_mult
    scaled_row_mult: float = 1.0
    batch: int = 1
    seq: int = 0
    chunk_sweep: Tuple[int, ...] = field(default_factory=tuple)

    def with_tokens(self, N: int) -> "Workload":
        return replace(self, N=int(N), seq=int(N) // max(self.batch, 1))

    def seed(self, stream: int) -> int:
        return 1000 * self.number + stream


WORKLOADS = {
    # tiny CPU-checkable case: 4 chunks of 128 tokens
    "c1": Workload("tiny-512x256x4096-K10", 1, N=512, H=256, V=4096, K=10, T=1.0, chunk=128,
                   dtype="fp32", teacher="random", tl_sigma=2.0, batch=1, seq=512),
    # Llama-3.2-3B-shaped student, batch 4 x 8192
    "c2": Workload("llama3.2-3b-shaped-32k", 2, N=32768, H=3072, V=128256, K=100, T=1.0, chunk=0,
                   dtype="bf16", teacher="topk_perturbed", batch=4, seq=8192),
    # GPT-OSS-20B-shaped student at 32K tokens (the benchmark workload)
    "c3": Workload("gpt-oss-20b-shaped-32k", 3, N=32768, H=2880, V=201088, K=100, T=1.0, chunk=0,
                   dtype="bf16", teacher="topk_perturbed", batch=1, seq=32768),
    # long context: 256K tokens, T = 2
    "c4": Workload("gpt-oss-20b-shaped-256k", 4, N=262144, H=2880, V=201088, K=100, T=2.0, chunk=0,
                   dtype="bf16", teacher="random", tl_sigma=3.0, batch=1, seq=262144,
                   chunk_sweep=(1024, 2048, 4096, 8192)),
    # small K, high temperature, 1% of rows x20
    "c5": Workload("k10-T4-stress-256k", 5, N=262144, H=4096, V=151936, K=10, T=4.0, chunk=0,
                   dtype="bf16", teacher="random", tl_sigma=1.0, scaled_row_frac=0.01,
                   scaled_row_mult=20.0, batch=4, seq=65536),
}


# ---------------------------------------------------------------- bf16 rounding

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = np.isnan(x)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = r.astype(np.uint16)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value, returned as float32."""
    return bf16_to_f32(bf16_bits(x))


# ---------------------------------------------------------------- generators

def normal(seed: int, shape, sigma: float = 1.0, chunk_rows: int = 1 << 14) -> np.ndarray:
    """float32 N(0, sigma^2) from PCG64(seed), drawn row-block by row-block (same stream)."""
    rng = np.random.default_rng(seed)
    out = np.empty(shape, np.float32)
    flat = out.reshape(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        rng.standard_normal(out=flat[r0:r1], dtype=np.float32)
    if sigma != 1.0:
        out *= np.float32(sigma)
    return out


def distinct_indices(seed: int, N: int, K: int, V: int) -> np.ndarray:
    """[N, K] int32: per row K distinct uniform draws from [0, V), in draw order.

    Rows that come out with a repeated value are redrawn whole until none remain
    (when K^2 > V, rows are instead the first K entries of a random permutation).
    """
    if K > V:
        raise ValueError("K > V")
    rng = np.random.default_rng(seed)
    if K * K > V:
        # dense case (K comparable to V): the first K of a random permutation per row
        out = np.empty((N, K), np.int32)
        for r0 in range(0, N, 256):
            r1 = min(N, r0 + 256)
            out[r0:r1] = np.argsort(rng.random((r1 - r0, V)), axis=1)[:, :K]
        return out
    idx = rng.integers(0, V, size=(N, K), dtype=np.int64)
    while True:
        s = np.sort(idx, axis=1)
        bad = np.nonzero((s[:, 1:] == s[:, :-1]).any(axis=1))[0] if K > 1 else np.zeros(0, np.int64)
        if bad.size == 0:
            break
        idx[bad] = rng.integers(0, V, size=(bad.size, K), dtype=np.int64)
    return idx.astype(np.int32)


def sorted_desc_logits(seed: int, N: int, K: int, sigma: float) -> np.ndarray:
    """[N, K] float32 N(0, sigma^2), each row sorted descending."""
    x = normal(seed, (N, K), sigma)
    return -np.sort(-x, axis=1)


def topk_of_perturbed_head(h: np.ndarray, W: np.ndarray, K: int, seed: int, device=None,
                           rows_per_block: int = 4096):
    """Teacher cache as the exact top-K of h @ W'^T, W' = bf16(W + N(0, 0.01^2)).

    h and W hold bf16 values (float32 arrays).  Logits are accumulated in fp32 and
    the K largest are returned descending (indices int32, values float32, not yet
    rounded).  With a torch device the products run there in blocks of rows;
    otherwise numpy does them on the host.
    """
    V, H = W.shape
    Wp = round_bf16(W + normal(seed, W.shape, 0.01))
    N = h.shape[0]
    idx = np.empty((N, K), np.int32)
    val = np.empty((N, K), np.float32)
    if device is None:
        WpT = np.ascontiguousarray(Wp.T)
        for r0 in range(0, N, rows_per_block):
            r1 = min(N, r0 + rows_per_block)
            z = h[r0:r1] @ WpT
            part = np.argpartition(-z, K - 1, axis=1)[:, :K]
            pv = np.take_along_axis(z, part, axis=1)
            order = np.lexsort((part, -pv), axis=1)      # by value descending, then index
            idx[r0:r1] = np.take_along_axis(part, order, axis=1)
            val[r0:r1] = np.take_along_axis(pv, order, axis=1)
        return idx, val
    import torch
    WpT = torch.from_numpy(Wp).to(device).t().contiguous()          # [H, V] fp32
    for r0 in range(0, N, rows_per_block):
        r1 = min(N, r0 + rows_per_block)
        hb = torch.from_numpy(h[r0:r1]).to(device)
        z = torch.mm(hb, WpT)
        v, i = torch.topk(z, K, dim=1, largest=True, sorted=True)
        idx[r0:r1] = i.to(torch.int32).cpu().numpy()
        val[r0:r1] = v.cpu().numpy()
        del z, v, i, hb
    del WpT
    return idx, val


@dataclass
class Inputs:
    """Host copies of one workload's inputs.

    h, W, tl are float32 arrays whose values are the ones the GPU sees (bf16
    values when ``bf16`` is set).  h_bits, W_bits, tl_bits are their bf16 bit
    patterns for upload.  ``h_raw``/``W_raw``/``tl_raw`` keep the unrounded fp32
    draws of an fp32 workload (None otherwise).
    """
    wl: Workload
    h: np.ndarray
    W: np.ndarray
    idx: np.ndarray
    tl: np.ndarray
    h_bits: np.ndarray
    W_bits: np.ndarray
    tl_bits: np.ndarray
    h_raw: Optional[np.ndarray] = None
    W_raw: Optional[np.ndarray] = None
    tl_raw: Optional[np.ndarray] = None


def make_inputs(wl: Workload, device=None) -> Inputs:
    """Draw the inputs of a workload (N may have been overridden with ``with_tokens``)."""
    N, H, V, K = wl.N, wl.H, wl.V, wl.K
    h = normal(wl.seed(S_H), (N, H), 1.0)
    if wl.scaled_row_frac > 0.0:
        nscale = int(round(wl.scaled_row_frac * N))
        pick = np.random.default_rng(wl.seed(S_ROWS)).permutation(N)[:nscale]
        h[pick] *= np.float32(wl.scaled_row_mult)
    W = normal(wl.seed(S_W), (V, H), 0.02)
    h_bits, W_bits = bf16_bits(h), bf16_bits(W)
    hb, Wb = bf16_to_f32(h_bits), bf16_to_f32(W_bits)
    if wl.teacher == "topk_perturbed":
        idx, tl = topk_of_perturbed_head(hb, Wb, K, wl.seed(S_WNOISE), device=device)
    elif wl.teacher == "random":
        idx = distinct_indices(wl.seed(S_IDX), N, K, V)
        tl = sorted_desc_logits(wl.seed(S_TL), N, K, wl.tl_sigma)
    else:
        raise ValueError(wl.teacher)
    tl_bits = bf16_bits(tl)
    tlb = bf16_to_f32(tl_bits)
    if wl.dtype == "fp32":
        return Inputs(wl, hb, Wb, idx, tlb, h_bits, W_bits, tl_bits, h_raw=h, W_raw=W, tl_raw=tl)
    return Inputs(wl, hb, Wb, idx, tlb, h_bits, W_bits, tl_bits)


@dataclass
class Teacher:
    """A full teacher model's final hidden states [N, H] and LM head [V, H]: bf16 values
    as float32 and their bit patterns."""
    h: np.ndarray
    W: np.ndarray
    h_bits: np.ndarray
    W_bits: np.ndarray


def full_teacher(wl: Workload, x: Inputs) -> Teacher:
    """The teacher of the online variant: the student's bf16 h and W plus seeded noise."""
    ht = x.h + normal(wl.seed(S_HT), x.h.shape, TEACHER_NOISE)
    Wt = x.W + normal(wl.seed(S_WT), x.W.shape, TEACHER_NOISE * 0.02)
    hb, Wb = bf16_bits(ht), bf16_bits(Wt)
    del ht, Wt
    return Teacher(bf16_to_f32(hb), bf16_to_f32(Wb), hb, Wb)


def sample_rows(wl: Workload, n: int, must_include=None) -> np.ndarray:
    """Seeded sorted sample of n distinct token rows (plus any rows in must_include)."""
    rng = np.random.default_rng(wl.seed(S_SAMPLE))
    n = min(n, wl.N)
    rows = rng.choice(wl.N, size=n, replace=False)
    if must_include is not None:
        rows = np.union1d(rows, np.asarray(must_include, dtype=np.int64))
    return np.sort(rows).astype(np.int64)


def scaled_rows(wl: Workload) -> np.ndarray:
    """The rows a workload multiplies by scaled_row_mult (empty if none)."""
    if wl.scaled_row_frac <= 0.0:
        return np.zeros(0, np.int64)
    nscale = int(round(wl.scaled_row_frac * wl.N))
    return np.sort(np.random.default_rng(wl.seed(S_ROWS)).permutation(wl.N)[:nscale]).astype(np.int64)

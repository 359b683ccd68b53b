"""The dense float32 torch route that the full-size GPU test compares the library with
(tests/test_gpu_workloads.py::test_dense_fp32_reference_at_full_size), pinned on the CPU
against the oracle: same definition, so agreement to float32 rounding, over several
token blocks and with a temperature other than 1."""
import numpy as np
import torch

import oracle
from gpu_util import synthetic
from test_gpu_workloads import _dense_fp32


def test_dense_fp32_route_matches_the_oracle():
    T = 1.7
    h, W, idx, tl = synthetic(41, 600, 64, 1000, 12, T)
    as_t = lambda a: torch.from_numpy(np.ascontiguousarray(np.asarray(a, np.float32)))
    loss, lse, dH, dW = _dense_fp32(as_t(h), as_t(W), torch.from_numpy(np.ascontiguousarray(idx.astype(np.int32))),
                                    as_t(tl), T, block=256)
    ref_loss, ref_lse = oracle.forward(h, W, idx, tl, T)
    ref_dH, ref_dW = oracle.backward(h, W, idx, tl, T)
    rel = lambda a, b: float(np.abs(a - b).max() / np.abs(b).max())
    assert rel(loss.numpy(), ref_loss) < 1e-5
    assert float(np.abs(lse.numpy() - ref_lse).max()) < 1e-5
    assert rel(dH.numpy(), ref_dH) < 1e-5
    assert rel(dW.numpy(), ref_dW) < 1e-5

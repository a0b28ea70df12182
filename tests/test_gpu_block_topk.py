"""GPU parity of fp4idx_block_topk (top-k blocks along Ktiles of block scores).

The selection is integer work on the scores: on the same scores the chosen blocks and
their counts must equal the oracle's exactly.
"""
import numpy as np
import pytest
import torch

import sparse_attention_fp4_amd as fp4
from oracle import oracle as orc
from sparse_attention_fp4_amd import workloads as wl

from .gpu_helpers import dev, gpu_block_scores, say

pytestmark = pytest.mark.gpu


def _same(scores, k):
    say(f"[gpu] block_topk shape={scores.shape} k={k}")
    idx, cnt = fp4.block_topk(dev(scores.astype(np.float32)), k)
    torch.cuda.synchronize()
    oi, oc = orc.block_topk(scores, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), oi)
    np.testing.assert_array_equal(cnt.cpu().numpy(), oc)


@pytest.mark.parametrize("Hq,Kt,Tq,k", [(3, 40, 300, 16), (2, 80, 257, 1), (2, 80, 65, 64),
                                        (1, 200, 129, 33), (2, 1, 70, 4), (1, 0, 10, 8),
                                        (4, 12, 5, 16), (2, 700, 64, 8)])
def test_same_scores_exact(Hq, Kt, Tq, k):
    rng = np.random.default_rng(Hq * 1000 + Kt * 10 + Tq + k)
    s = (rng.integers(-12, 12, (Hq, Kt, Tq)) / 4).astype(np.float32)   # many ties
    s[rng.random(s.shape) < 0.3] = -np.inf
    if Kt:
        s[0, :, 0] = -np.inf                           # a query with no candidate block
        s[0, rng.integers(0, Kt, 3), 1 % Tq] = np.nan
        s[-1, :, -1] = -0.0                            # -0 ties with +0
        s[-1, 0, -1] = 0.0
    _same(s, k)


def test_distinct_scores_large_tq():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((8, 80, 4099)).astype(np.float32)
    _same(s, 16)


def test_on_block_scores_of_a_prefill_batch():
    """Top-16 blocks of the block scores of a small causal NVFP4 batch (rows whose
    causal window covers fewer than 16 blocks keep them all)."""
    case = wl.make_block("block_topk_small", fmt=wl.NVFP4, q_lens=[300, 1000], k_lens=[2300, 1200],
                         Hq=8, Hkv=2, seed=77)
    got = gpu_block_scores(case)
    _same(got, 16)

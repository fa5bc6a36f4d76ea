"""moe_align on the GPU vs the oracle: every output bit-exact (counts, sorted ids with
fillers, expert per block, padded total, inverse positions) at the block heights the GEMMs
use, with ragged sizes, zero-token experts and skewed loads.  Up to 4096 pairs one
workgroup aligns the batch; up to 65536 one workgroup per 2048-pair chunk, each counting
the whole batch; beyond that (no scratch here) the one workgroup again."""
import numpy as np
import pytest
import torch

import oracle
from moe_layer_02_amd import abi
from tests.gpu_util import needs_gpu, say

pytestmark = [pytest.mark.gpu, needs_gpu]


def gpu_align(ids, T, k, E, BM):
    cap = abi.moe_align_capacity(T, k, E, BM)
    dev = torch.from_numpy(ids.reshape(-1)).cuda()
    out = dict(sorted_token_ids=torch.full((cap,), -5, dtype=torch.int32, device="cuda"),
               expert_ids=torch.full((cap // BM,), -5, dtype=torch.int32, device="cuda"),
               num_tokens_post_padded=torch.full((1,), -5, dtype=torch.int32, device="cuda"),
               expert_counts=torch.full((E,), -5, dtype=torch.int32, device="cuda"),
               inv_pos=torch.full((T * k,), -5, dtype=torch.int32, device="cuda"))
    abi.moe_align(T, k, E, BM, dev, out["sorted_token_ids"], out["expert_ids"], out["num_tokens_post_padded"],
                  out["expert_counts"], out["inv_pos"])
    torch.cuda.synchronize()
    return {k_: v.cpu().numpy() for k_, v in out.items()}


def check(ids, T, k, E, BM):
    say("align T=%d k=%d E=%d BM=%d" % (T, k, E, BM))
    got = gpu_align(ids, T, k, E, BM)
    ref = oracle.align(ids, T, k, E, BM)
    for name in ref:
        assert (got[name] == ref[name]).all(), name


def distinct_ids(rng, T, k, E):
    return np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)


@pytest.mark.parametrize("BM", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("T,k,E", [(1, 1, 8), (1, 8, 256), (3, 2, 8), (37, 2, 8), (100, 8, 64), (512, 8, 256),
                                   (4096, 8, 64), (8192, 1, 16), (4096, 2, 8), (2000, 6, 128), (4097, 1, 8),
                                   (1531, 7, 64)])
def test_align_matches_oracle(T, k, E, BM):
    rng = np.random.default_rng(T * 131 + k * 7 + E + BM)
    check(distinct_ids(rng, T, k, E), T, k, E, BM)


def test_align_skewed_and_empty_experts():
    rng = np.random.default_rng(3)
    T, k, E = 3000, 1, 16
    p = np.array([0.5, 0.3, 0.2] + [0.0] * 13)
    ids = rng.choice(E, size=(T, k), p=p).astype(np.int32)
    for BM in (16, 64, 128):
        check(ids, T, k, E, BM)
    check(np.full((50, 1), 7, np.int32), 50, 1, 16, 16)          # a single expert takes everything


def test_align_largest_pairs_and_block():
    rng = np.random.default_rng(4)
    check(distinct_ids(rng, 8192, 8, 256), 8192, 8, 256, 16)    # 65536 pairs: the largest one-launch batch
    check(distinct_ids(rng, 8193, 8, 256), 8193, 8, 256, 16)    # one workgroup takes every pair beyond it
    check(distinct_ids(rng, 300, 4, 64), 300, 4, 64, 1024)        # largest block height
    check(distinct_ids(rng, 300, 4, 64), 300, 4, 64, 1)


def test_align_is_deterministic():
    rng = np.random.default_rng(5)
    ids = distinct_ids(rng, 4096, 8, 64)
    a = gpu_align(ids, 4096, 8, 64, 64)
    b = gpu_align(ids, 4096, 8, 64, 64)
    for name in a:
        assert (a[name] == b[name]).all()

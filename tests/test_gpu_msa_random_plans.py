"""Block-sparse MSA on the GPU against the oracle over seeded random plans.

Each plan draws its block size (32, 64 or 128 tokens), blocks kept (4, 8 or 16), query and KV
heads (grouped 8:1, 4:1 or 1:1), head width (64 or 128), cache and query format (bf16 or fp32),
index key format (bf16 or fp8), page size (16, 32, 48 or 64 tokens), and one to five requests
that are decode rows (position 0 included, and contexts that end inside or at the edge of a
block) or short prefill chunks, with nonzero page starts. The checks are those of the named MSA
workloads: token scores, the block selection bit-exact on the GPU's scores and in band against
the oracle's block scores, and the attention against the oracle on both selections and on an
edited selection.
"""
import numpy as np
import pytest
import torch

from synth import make_msa_workload
from synth.msa_workloads import MsaSpec
from sparse_attention_dsa_amd import dsa
from tests.gpu_helpers import note
from tests.test_gpu_msa import _check

pytestmark = pytest.mark.gpu

SEEDS = list(range(16))


def random_msa_spec(seed: int) -> MsaSpec:
    rng = np.random.default_rng(9000 + seed)
    block = int(rng.choice([32, 64, 128]))
    heads, kv = [(32, 4), (16, 4), (8, 8)][int(rng.integers(0, 3))]
    reqs = []
    for _ in range(int(rng.integers(1, 6))):
        if rng.random() < 0.6:
            pick = rng.random()
            pos = 0 if pick < 0.15 else (block * int(rng.integers(1, 20)) - 1 if pick < 0.3
                                         else int(rng.integers(1, 9000)))
            reqs.append((1, pos))
        else:
            reqs.append((int(rng.integers(2, 80)), int(rng.integers(0, 1500))))
    page_size = int(rng.choice([16, 32, 48, 64]))
    return MsaSpec(name=f"msa_random_plan_{seed}", seed=9000 + seed, requests=reqs,
                   page_starts=[int(rng.integers(0, 2 * page_size)) for _ in reqs],
                   block=block, topk_blocks=int(rng.choice([4, 8, 16])), n_heads=heads,
                   n_kv_heads=kv, head_dim=int(rng.choice([64, 128])), page_size=page_size,
                   spare_pages=int(rng.integers(0, 3)), q_fmt=str(rng.choice(["bf16", "f32"])),
                   index_key_fmt=str(rng.choice(["bf16", "fp8"])))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dsa.load()


@pytest.mark.parametrize("seed", SEEDS)
def test_msa_random_plan_all_rows(seed):
    s = random_msa_spec(seed)
    note(f"[msa random plan {seed}] blocks of {s.block}, top {s.topk_blocks}, heads {s.n_heads}/"
         f"{s.n_kv_heads} x {s.head_dim} {s.q_fmt}, keys {s.index_key_fmt}, pages of {s.page_size}, "
         f"requests {s.requests}")
    wl = make_msa_workload(s)
    worst = _check(wl, list(range(wl.n_rows)))
    note(f"[msa random plan {seed}] worst attention error {worst:.3g}")

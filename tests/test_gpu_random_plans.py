"""GPU parity on seeded random plans: the whole path through the C ABI against the CPU oracle.

Two families: plans on the matrix-core shapes (below) and plans on small shapes that the generic
kernels take (random_generic_spec).

Each plan draws its own index key and latent formats (bf16 or packed fp8), page size (16, 32, 48
or 64 tokens; 48, not a power of two, goes to the generic kernels), top-k (values that are not a
multiple of the 32-key tile, and above the shortest contexts so that -1 tails appear), one to five
requests that are decode rows (up to 9,000 keys, so over several 4,096-key score blocks; position
0 included: a row that sees only itself) or short prefill chunks, nonzero page starts and, for
half of the plans, an attention sink per head.
The checks are those of the named workloads: store_keys bytes, scores within tolerance, the
fused index_topk equal to its two halves, the selection bit-exact on the GPU's scores and in
band against the oracle's, and the attention against the oracle on both selections.
"""
import numpy as np
import pytest
import torch

from synth import make_workload
from synth.workloads import Spec, _big_dims
from sparse_attention_dsa_amd import dsa
from tests.gpu_helpers import full_parity, note

pytestmark = pytest.mark.gpu

SEEDS = list(range(24))


def random_spec(seed: int) -> Spec:
    rng = np.random.default_rng(7000 + seed)
    key_fmt = str(rng.choice(["bf16", "fp8"]))
    latent_fmt = str(rng.choice(["bf16", "fp8"]))
    page_size = int(rng.choice([16, 32, 48, 64]))
    topk = int(rng.choice([33, 100, 256, 513]))
    reqs = []
    for _ in range(int(rng.integers(1, 6))):
        if rng.random() < 0.6:
            reqs.append((1, 0 if rng.random() < 0.2 else int(rng.integers(1, 9000))))
        else:
            reqs.append((int(rng.integers(2, 100)), int(rng.integers(0, 1500))))
    page_starts = [int(rng.integers(0, 2 * page_size)) for _ in reqs]
    return Spec(name=f"random_plan_{seed}", seed=7000 + seed, requests=reqs, page_starts=page_starts,
                sink=bool(rng.random() < 0.5), spare_pages=int(rng.integers(0, 4)),
                **_big_dims(index_key_fmt=key_fmt, latent_fmt=latent_fmt, topk=topk,
                            page_size=page_size))


def random_generic_spec(seed: int) -> Spec:
    """Small shapes off the matrix-core kernels' 64 x 128 indexer and 128-head 512 + 64 MLA, so the
    generic score and attention kernels run: 4..16 index heads of 32 or 64 dims, fp32 or bf16
    queries and keys, 8 or 16 MLA heads over 64 or 128 latent dims plus 16 or 32 rope dims, fp32
    or bf16 latents and queries."""
    rng = np.random.default_rng(8000 + seed)
    fp = lambda: str(rng.choice(["f32", "bf16"]))
    reqs = []
    for _ in range(int(rng.integers(1, 5))):
        if rng.random() < 0.6:
            reqs.append((1, 0 if rng.random() < 0.2 else int(rng.integers(1, 3000))))
        else:
            reqs.append((int(rng.integers(2, 60)), int(rng.integers(0, 800))))
    page_size = int(rng.choice([16, 32, 48, 64]))
    rank, rope = int(rng.choice([64, 128])), int(rng.choice([16, 32]))
    return Spec(name=f"random_generic_{seed}", seed=8000 + seed, n_index_heads=int(rng.choice([4, 8, 16])),
                index_dim=int(rng.choice([32, 64])), index_q_fmt=fp(), index_key_fmt=fp(),
                topk=int(rng.choice([16, 33, 100])), w_scale=1.0, n_heads=int(rng.choice([8, 16])),
                kv_lora_rank=rank, rope_dim=rope, q_fmt=fp(), latent_fmt=fp(), page_size=page_size,
                sm_scale=1.0 / float(np.sqrt(rank + rope)), requests=reqs,
                page_starts=[int(rng.integers(0, 2 * page_size)) for _ in reqs],
                sink=bool(rng.random() < 0.5))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dsa.load()


@pytest.mark.parametrize("seed", SEEDS)
def test_random_plan_all_rows(seed):
    spec = random_spec(seed)
    note(f"[random plan {seed}] keys {spec.index_key_fmt}, latents {spec.latent_fmt}, "
         f"pages of {spec.page_size}, topk {spec.topk}, sink {spec.sink}, requests {spec.requests}")
    r = full_parity(make_workload(spec))
    note(f"[random plan {seed}] worst score err {r['worst_score']:.3g}x tol, attend {r['worst_attend']:.3g}")


@pytest.mark.parametrize("seed", list(range(12)))
def test_random_generic_plan_all_rows(seed):
    spec = random_generic_spec(seed)
    note(f"[random generic plan {seed}] index {spec.n_index_heads}x{spec.index_dim} "
         f"{spec.index_q_fmt}/{spec.index_key_fmt}, MLA {spec.n_heads} heads {spec.kv_lora_rank}+"
         f"{spec.rope_dim} {spec.q_fmt}/{spec.latent_fmt}, pages of {spec.page_size}, topk {spec.topk}, "
         f"sink {spec.sink}, requests {spec.requests}")
    r = full_parity(make_workload(spec))
    note(f"[random generic plan {seed}] worst score err {r['worst_score']:.3g}x tol, attend {r['worst_attend']:.3g}")

"""Seeded random shapes against the oracle: kv head counts 1..16 (head
groups of 8, 4, 2 and 1, token slices included), 1..16 query heads per kv
head, bf16 / FP8 / FP4 caches, NHD and HND blocks, NeoX or interleaved RoPE
and per-head or per-tensor FP8 scales (cases 24 on), mixes of empty, short
and long contexts, and the library's own plan choice (partition_size 0) or
an explicit partition size.  Every output element of every sequence is
compared, after the append of the step's token, at the parity tolerance.
The shapes come from one fixed generator seed, so a failure names a case
that runs again the same way."""
import numpy as np
import pytest

import workloads as W
from test_gpu_parity import _run_and_check

pytestmark = pytest.mark.gpu

N_CASES = 40


def _case(i):
    rng = np.random.default_rng(9000 + i)
    hkv = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16]))
    G = int(rng.integers(1, 17))
    cache = str(rng.choice(["bf16", "fp8", "fp4"]))
    ps = int(rng.choice([0, 0, 0, 256, 512]))
    max_ctx = int(rng.choice([64, 700, 2048, 8192]))
    budget = 3_000_000 // hkv  # token-heads the oracle walks, a few seconds of fp64 NumPy
    B = int(rng.integers(1, max(2, min(400, budget // max(1, max_ctx // 2)))))
    ctx = rng.integers(0, max_ctx + 1, size=B)
    ctx[rng.random(B) < 0.1] = 0
    ctx[rng.random(B) < 0.1] = max_ctx
    layout = "hnd" if rng.random() < 0.25 else "nhd"
    rope = "interleaved" if i >= 24 and rng.random() < 0.5 else "neox"
    per_tensor = bool(i >= 24 and cache == "fp8" and rng.random() < 0.5)
    return W.Config(f"rand{i}_{cache}_H{hkv}_G{G}_B{B}_ps{ps}_{layout}_{rope}{'_pt' if per_tensor else ''}",
                    seed=9100 + i, num_seqs=B, num_q_heads=hkv * G, num_kv_heads=hkv, head_dim=128, block_size=16,
                    act="bf16", cache=cache, ctx=0, rope_theta=1e4, partition_size=ps, append=True,
                    ctx_list=tuple(int(c) for c in ctx), cache_layout=layout, rope_style=rope,
                    scale_per_tensor=per_tensor)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_matches_oracle(i):
    _run_and_check(_case(i))

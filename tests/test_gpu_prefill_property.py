"""Randomized chunked-prefill parity: seeded cases of random shapes against the oracle.

Each case draws the number of sequences, query / kv heads, head_dim (64 or 128),
the 16-bit dtype, every sequence's chunk and prior-context length (including
empty chunks, chunks longer than one query tile, priors on and off block and step
boundaries) and the logit scale (up to 0.3, a very peaked softmax at d = 128),
writes the chunk through reshape_and_cache into blocks the host block manager
places after a shuffled free list, poisons free blocks and tail slots with NaN,
and compares every output element of pkv_paged_prefill_attention with the fp64
oracle (prefill_ref).  The first failing case stops the sweep and names its draw.

Tolerance.  The prefill's weights enter the PV product rounded to the input type
(unit roundoff u = 2^-9 for bf16, 2^-12 for f16).  With r_j = p_j (1 + e_j),
|e_j| <= u, the normalised output o' = sum r_j v_j / sum r_j differs from
o = sum p_j v_j / sum p_j by exactly sum p_j e_j (v_j - o) / sum r_j, so
|o' - o| <= u / (1 - u) * sum_j w_j |v_j - o| (w the exact softmax weights).
Each element is held to the decode tolerance plus twice that term, computed
here in fp64 from the gathered keys and values.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import TOL, as_f64, check_close, prefill_weight_spread
from tests.test_gpu_prefill import DEV, PrefillCase, _w

pytestmark = pytest.mark.gpu

N_CASES = 60
HEADS = [(4, 4), (8, 2), (16, 2), (6, 3), (8, 1), (2, 2)]


def _len(rng, hi, specials):
    return int(rng.choice(specials)) if rng.random() < 0.35 else int(rng.integers(0, hi + 1))


def draw(rng):
    S = int(rng.integers(1, 5))
    H, KVH = HEADS[int(rng.integers(len(HEADS)))]
    d = int(rng.choice([64, 128]))
    dt = str(rng.choice(["f16", "bf16"]))
    chunk = tuple(_len(rng, 300, [0, 1, 15, 16, 17, 64, 127, 128, 129, 256]) for _ in range(S))
    prior = tuple(_len(rng, 700, [0, 1, 16, 63, 64, 65, 512]) for _ in range(S))
    if sum(chunk) == 0:
        chunk = (1,) + chunk[1:]
    scale = float(rng.choice([1.0 / np.sqrt(d), 0.3, -0.05]))
    return dict(S=S, H=H, KVH=KVH, d=d, dt=dt, chunk=chunk, prior=prior, scale=scale, seed=int(rng.integers(1 << 30)))


def _weight_spread(case, scale, ref):
    """sum_j w_j |v_j - o| per output element (see prefill_weight_spread)."""
    return prefill_weight_spread(as_f64(case.inp.q), as_f64(case.k_cache), as_f64(case.v_cache), case.tables,
                                 case.ctx, case.qsl, scale, case.w.block_size, ref)


@pytest.mark.timeout(600)
def test_random_prefill_shapes_match_oracle():
    from paged_kv_cache_259_amd import ops
    rng = np.random.default_rng(2591)
    seen = set()
    for i in range(N_CASES):
        c = draw(rng)
        what = f"case {i}: {c}"
        print(what, flush=True)
        case = PrefillCase(_w(c["H"], c["KVH"], c["d"], c["dt"], c["S"], seed=c["seed"]), DEV, chunk=c["chunk"],
                           prior=c["prior"])
        out = torch.full_like(case.inp.q, float("nan"))
        mq = max(1, int(case.inp.chunk_lens.max()))
        ops.paged_prefill_attention(out, case.inp.q, case.k_cache, case.v_cache,
                                    torch.from_numpy(case.tables).to(DEV), torch.from_numpy(case.ctx).to(DEV),
                                    torch.from_numpy(case.qsl).to(DEV), c["scale"], mq, int(case.ctx.max()))
        torch.cuda.synchronize()
        ref = oracle.prefill_ref(as_f64(case.inp.q), as_f64(case.k_cache), as_f64(case.v_cache), case.tables,
                                 case.ctx, case.qsl, c["scale"], 16)
        T = int(case.qsl[-1])
        assert torch.isfinite(out[:T]).all(), what
        spread = _weight_spread(case, c["scale"], ref)
        u = 2.0 ** -9 if c["dt"] == "bf16" else 2.0 ** -12
        atol, rtol = TOL[c["dt"]]
        got = as_f64(out[:T])
        bound = atol + rtol * np.abs(ref[:T]) + 2 * u * spread[:T]
        bad = ~(np.abs(got - ref[:T]) <= bound)
        assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance; first {np.argwhere(bad)[:5].tolist()}"
        seen.add((c["d"], c["dt"], c["H"] // c["KVH"] > 1))
    # the sweep covered both head sizes, both dtypes, grouped and ungrouped heads
    assert {d for d, _, _ in seen} == {64, 128} and {t for _, t, _ in seen} == {"f16", "bf16"}
    assert {g for _, _, g in seen} == {True, False}

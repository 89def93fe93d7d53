"""pkv_paged_attention_decode_noalloc against pkv_paged_attention_decode, through the C ABI.

The no-allocation decode keeps its split-context summaries in the library's
static per-GPU scratch instead of a caller workspace.  Each scenario makes two
calls in a row on one stream, the second with a smaller input, so the second
call runs over whatever the first left in the scratch.  Every output is
compared bit for bit with the workspace call of the same arguments, and with
the oracle within the workload tolerance (2e-3 + 1e-2 |ref| for 16-bit caches,
1e-5 + 1e-5 |ref| for fp32).
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_259_amd import synth
from tests.helpers import TOL, DecodeCase, as_f64, check_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def ops():
    from paged_kv_cache_259_amd import ops as _ops
    return _ops


def W(seed, S, H, KVH, d, dt, lens, bs=16):
    return synth.DecodeWorkload(name=f"noalloc-{seed}", seed=seed, num_seqs=S, num_heads=H, num_kv_heads=KVH,
                                head_dim=d, block_size=bs, q_dtype=dt, kv_dtype=dt, lengths=("fixed", tuple(lens)),
                                max_blocks_per_seq=-(-max(lens) // bs))


def _both(ops, case, partition):
    """(workspace call, no-allocation call) outputs of one decode, same arguments, same stream."""
    dev = case.device
    q = case.q.to(dev)
    kc, vc = case.k_cache.to(dev), case.v_cache.to(dev)
    tables = torch.from_numpy(case.tables).to(dev)
    ctx = torch.from_numpy(case.ctx).to(dev)
    args = (q, kc, vc, tables, ctx, case.w.softmax_scale, int(case.ctx.max()))
    out_ws = torch.full_like(q, float("nan"))
    out_na = torch.full_like(q, float("nan"))
    ops.paged_attention_decode(out_ws, *args, partition_size=partition)
    ops.paged_attention_decode_noalloc(out_na, *args, partition_size=partition)
    torch.cuda.synchronize()
    return out_ws.cpu(), out_na.cpu()


# scenario -> two calls (workload, partition size, expected plan mode), the second smaller
SCENARIOS = {
    "mfma fixed partitions": [
        (W(71, 5, 16, 4, 128, "bf16", (3000, 17, 4500, 1030, 2600)), 512, "partitions"),
        (W(72, 3, 8, 2, 128, "f16", (700, 1300, 40)), 256, "partitions"),
    ],
    "mfma balanced slices": [
        (W(73, 2, 16, 2, 128, "bf16", (6000, 2500)), 0, "slices"),
        (W(74, 1, 8, 1, 128, "bf16", (3000,)), 0, "slices"),
    ],
    "vector fixed partitions": [
        (W(75, 3, 4, 4, 64, "f16", (900, 2000, 33)), 128, "partitions"),
        (W(76, 2, 2, 2, 64, "f32", (300, 1000)), 64, "partitions"),
    ],
}


@pytest.mark.parametrize("name", list(SCENARIOS))
def test_noalloc_matches_workspace_decode_two_calls(ops, name):
    for i, (w, part, mode) in enumerate(SCENARIOS[name]):
        qd, kvd = ops.dtype_code(synth.DTYPES[w.q_dtype]), ops.dtype_code(synth.DTYPES[w.kv_dtype])
        plan = ops.attention_plan(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                  max(w.lengths[1]), part, qd, kvd)
        assert (plan[1] == 0) == (mode == "slices") and plan[2] > 1, (name, i, plan)
        case = DecodeCase(w, DEV)
        out_ws, out_na = _both(ops, case, part)
        assert torch.equal(out_na.view(torch.uint8), out_ws.view(torch.uint8)), f"{name} call {i}: bits differ"
        check_close(as_f64(out_na), case.reference(), TOL[w.kv_dtype], f"{name} call {i}")


def test_noalloc_near_the_scratch_limit_then_small(ops):
    """A plan that fills most of the scratch (16-token partitions of 8192-token contexts: 81,920 summary
    rows, about 42.6 MB), then a small call: both bit-identical to the workspace call."""
    w = W(77, 4, 40, 40, 128, "f16", (8192, 8000, 5000, 7777))
    need = ops.attention_workspace_bytes(4, 40, 40, 128, 16, 8192, 16, ops.F16, ops.F16)
    assert 32 << 20 < need <= ops.STATIC_SCRATCH_BYTES
    inp = synth.make_decode_inputs(w, device=DEV)
    from paged_kv_cache_259_amd.block_manager import BlockManager
    bm = BlockManager(inp.num_blocks, 16, inp.free_list)
    for s in range(4):
        bm.add_sequence(s, int(inp.context_lens[s]))
    tables = torch.from_numpy(bm.block_table_array(list(range(4)), w.max_blocks_per_seq)).to(DEV)
    ctx = torch.from_numpy(bm.context_lens_array(list(range(4)))).to(DEV)
    outs = []
    for fn in (ops.paged_attention_decode, ops.paged_attention_decode_noalloc):
        o = torch.full_like(inp.q, float("nan"))
        fn(o, inp.q, inp.k_cache, inp.v_cache, tables, ctx, w.softmax_scale, 8192, partition_size=16)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert not torch.isnan(outs[1]).any()
    # then a small call over the same (now partly stale) scratch
    small = W(78, 2, 8, 2, 128, "bf16", (1500, 600))
    case = DecodeCase(small, DEV)
    out_ws, out_na = _both(ops, case, 128)
    assert torch.equal(out_na.view(torch.uint8), out_ws.view(torch.uint8))
    check_close(as_f64(out_na), case.reference(), TOL["bf16"], "small call after the near-limit one")


def test_noalloc_refuses_plans_beyond_the_scratch(ops):
    """A plan needing more than the static scratch returns PKV_ERR_SCRATCH_LIMIT and launches nothing;
    the next call still works."""
    w = W(79, 2, 8, 2, 128, "bf16", (900, 40))
    case = DecodeCase(w, DEV)
    q = case.q.to(DEV)
    out = torch.zeros_like(q)
    big_ctx = 2_000_000   # 16-token partitions of 2M tokens: far beyond 48 MiB of summaries
    assert ops.attention_workspace_bytes(2, 8, 2, 128, 16, big_ctx, 16, ops.BF16, ops.BF16) > ops.STATIC_SCRATCH_BYTES
    with pytest.raises(ops.PkvError) as e:
        ops.paged_attention_decode_noalloc(out, q, case.k_cache.to(DEV), case.v_cache.to(DEV),
                                           torch.from_numpy(case.tables).to(DEV), torch.from_numpy(case.ctx).to(DEV),
                                           w.softmax_scale, big_ctx, partition_size=16)
    assert e.value.status == -10
    torch.cuda.synchronize()
    assert not out.any()
    out_ws, out_na = _both(ops, case, 256)
    assert torch.equal(out_na.view(torch.uint8), out_ws.view(torch.uint8))

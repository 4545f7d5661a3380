"""Run-to-run determinism at full size: msa_decode repeated 100 times on each
workload gives bitwise the same selections, page tables and outputs.

No kernel of the path uses atomics or a reduction order that depends on
scheduling: every row's selection is ranked by one workgroup, and each
split's partial result lands in its own workspace slot before the merge
reads all splits in a fixed order.  Between repeats the outputs are
overwritten with sentinels and, every tenth repeat, the workspace with
random bytes, so a result cannot be left over from the previous call and
nothing may depend on what the workspace held before.
"""
import pytest
import torch

import block_sparse_attention_10_amd as msa
from synth import CONFIG_ORDER, CONFIGS, EXTRA_CONFIGS, make_workload
from tests.msa_gpu import alloc_outputs, describe_workload

pytestmark = pytest.mark.gpu

DEV = "cuda"
REPEATS = 100


@pytest.mark.parametrize("name", CONFIG_ORDER + EXTRA_CONFIGS)
def test_repeated_decode_is_bitwise_identical(name):
    cfg = CONFIGS[name]
    print(f"determinism {name}: generating", flush=True)
    w = make_workload(cfg, DEV)
    p, t = describe_workload(w)
    o = alloc_outputs(w, p)
    sel, pt, out, ws = o["selected"], o["page_table"], o["out"], o["workspace"]
    g = torch.Generator(device=DEV).manual_seed(cfg.seed)

    msa.msa_decode(p, t, sel, pt, out, ws)
    torch.cuda.synchronize()
    want = (sel.clone(), pt.clone(), out.clone())
    assert not torch.isnan(out).any()
    print(f"determinism {name}: {REPEATS} repeats", flush=True)
    for i in range(REPEATS):
        sel.fill_(-7 - i)
        pt.fill_(-7 - i)
        out.fill_(float("nan") if i % 2 else 1e30)
        if i % 10 == 0:
            ws.copy_(torch.randint(0, 256, ws.shape, generator=g, device=DEV,
                                   dtype=torch.int32).to(torch.uint8))
        msa.msa_decode(p, t, sel, pt, out, ws)
        assert torch.equal(sel, want[0]), f"{name}: repeat {i} selected"
        assert torch.equal(pt, want[1]), f"{name}: repeat {i} page_table"
        assert torch.equal(out, want[2]), f"{name}: repeat {i} out"
    print(f"determinism {name}: ok", flush=True)
    del w, o, want
    torch.cuda.empty_cache()

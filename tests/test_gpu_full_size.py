"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (automatic GEMM path): routing (ids, gates, counts) for every
token against the oracle, and the layer output, token by token, on every token
of the decode batches and on a sample of the prefill batches that the oracle
evaluates one by one (the first and last token of every expert's dispatch
segment, so every tile height an expert's last tile takes is hit, plus the
batch's first and last token).  Weights are generated on the device; the
oracle receives only the experts its sampled tokens use and evaluates the
sample on disjoint token shards in parallel host threads."""
import gc

import numpy as np
import pytest
import torch

import moe_synth
import sparse_mixture_experts_03_amd as moe
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu

# workload -> tokens the oracle evaluates (bounded so each case stays within seconds)
SAMPLE = {
    "tiny-f32-T64-d128-E8": 64,
    "decode-bf16-T8-d8192-E128": 8,
    "prefill-skewed-bf16-T4096-d4096-E16": 48,
    "prefill-balanced-bf16-T2048-d8192-E128": 32,
    "prefill-skewed-bf16-T2048-d8192-E128": 32,
    "int4-decode-T16-d12288-E16": 16,
    "int4-prefill-T8192-d12288-E16": 34,
}


@pytest.mark.parametrize("name", list(SAMPLE))
def test_full_size_parity(oracle, name):
    assert torch.cuda.is_available()
    dev = torch.device("cuda:0")
    cfg = moe_synth.workload(name)
    inp = moe_synth.generate(cfg, device=dev, seed=0)
    out = H.run_forward(cfg, inp, device=dev)
    ref = H.oracle_route(oracle, cfg, inp)
    ids = out["ids"].cpu().numpy()
    amb = H.check_routing(ids, out["gates"].cpu().numpy(), ref, cfg["k"])
    counts = out["counts"].cpu().numpy()
    H.check_forward_counts(oracle, ref["ids"], ids, amb, cfg["E"], counts)
    assert int(counts.sum()) == cfg["T"] * cfg["k"]
    if SAMPLE[name] >= cfg["T"]:
        tokens = np.array([t for t in range(cfg["T"]) if t not in set(amb)], dtype=np.int64)
    else:
        tokens = H.sample_tokens(ref["ids"], cfg["E"], SAMPLE[name], exclude=set(amb))
    y_ref = H.oracle_y(oracle, cfg, inp, ref, tokens)
    err = H.check_y(out["y"], tokens, y_ref, cfg["act"])
    yall = out["y"].float()
    assert bool(torch.isfinite(yall).all())
    print(f"\n{name}: ambiguous {len(amb)}, active experts {(counts > 0).sum()}, max count {counts.max()}, "
          f"count var {np.var(counts):.1f}, sampled {len(tokens)} tokens, worst per-token err {err:.2e}")
    del inp, out, yall
    gc.collect()
    torch.cuda.empty_cache()

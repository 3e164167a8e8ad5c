"""GPU: the no-relay baseline (prefix-shared system pages, context step only) computes
the same exact attention as the relay path and the oracle.  Tolerances as in
test_parity_gpu."""
import pytest
import torch

import oracle
from shared_prompt_kv_amd import baseline, relay as R
import workloads as W
from tests.test_parity_gpu import check, say

pytestmark = pytest.mark.gpu

SPECS = [
    W.config_spec(2).replace(batch=5, sys_len=336, ctx_lo=16, ctx_hi=100),
    W.config_spec(4).replace(batch=9, sys_len=512, ctx_median=60, ctx_cap=200),
    W.config_spec(5).replace(batch=4, sys_len=288, ctx_lo=64, ctx_hi=300),
    W.config_spec(5).replace(name="c5-f32", dtype="f32", batch=3, sys_len=48, ctx_lo=17, ctx_hi=99),
]


@pytest.mark.parametrize("spec", SPECS, ids=[f"{s.name}-B{s.batch}-L{s.sys_len}" for s in SPECS])
def test_baseline_matches_oracle_and_relay(spec):
    say(f"[parity] no-relay baseline {spec}")
    assert torch.cuda.is_available()
    w = W.generate(spec)
    t = R.to_device(w, "cuda")
    relay_out = R.decode_workload(t)
    base_out = R.decode_workload(baseline.prefix_shared(t))
    torch.cuda.synchronize()
    ref, _ = oracle.Problem(w).attention()
    check(base_out.cpu().numpy(), ref, spec.dtype, "baseline")
    check(relay_out.cpu().numpy(), ref, spec.dtype, "relay")

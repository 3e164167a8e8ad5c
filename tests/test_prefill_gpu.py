"""GPU: the offline system-prompt prefill (cache fill with position embedding, the
prompt's causal attention) against the oracle (oracle/rope.py prefill_expect), and the
system cache's save / load round trip."""
import os

import numpy as np
import pytest
import torch

from oracle import rope
from shared_prompt_kv_amd import prefill, relay as R
import workloads as W
from tests.test_parity_gpu import check, say
from tests.test_rope_gpu import assert_stored_close, upload

pytestmark = pytest.mark.gpu

# (dtype, L_s, H_q, H_kv, d, method): bf16 d = 128 runs the causal matrix-core kernel
# ("auto") and, for comparison, the decode path; other inputs only the decode path
CASES = [("bf16", 37, 8, 2, 128, "auto"), ("bf16", 37, 8, 2, 128, "decode"),
         ("bf16", 200, 4, 4, 128, "auto"), ("bf16", 512, 32, 8, 128, "auto"),
         ("bf16", 512, 32, 8, 128, "decode"), ("bf16", 1100, 8, 8, 128, "auto"),
         ("f32", 100, 4, 4, 64, "auto")]


def host(dtype, x):
    x = x.cpu()
    return x.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else x.numpy()


@pytest.mark.parametrize("dtype,L,Hq,Hkv,d,method", CASES)
def test_prefill_matches_oracle_and_cache_round_trips(dtype, L, Hq, Hkv, d, method, tmp_path):
    say(f"[parity] system prefill {dtype} L={L} Hq={Hq} Hkv={Hkv} d={d} method={method}")
    spec = W.config_spec(2).replace(dtype=dtype)
    r = np.random.default_rng(L)
    conv = (lambda x: W.f32_to_bf16_bits(x.astype(np.float32))) if dtype == "bf16" else (lambda x: x.astype(np.float32))
    q, k, v = (conv(r.standard_normal(s)) for s in ((L, Hq, d), (L, Hkv, d), (L, Hkv, d)))
    tab = R.relay_rope_table(L, d)
    scale = 1.0 / np.sqrt(d)
    qd, kd, vd = upload(spec, q), upload(spec, k), upload(spec, v)
    assert prefill.uses_matrix_cores(qd, kd, scale) == (dtype == "bf16")
    sys_k, sys_v, out = prefill.prefill_system(qd, kd, vd, tab, scale, method=method)
    torch.cuda.synchronize()
    ek, ev, eo = rope.prefill_expect(q, k, v, dtype)
    assert_stored_close(spec, host(dtype, sys_k), ek, "system keys")
    assert np.array_equal(host(dtype, sys_v), ev), "system values / tile padding"
    check(out.cpu().numpy(), eo, dtype, "prefill attention")
    # save / load: the same bits, and a decode on the loaded cache gives the same bits
    path = os.path.join(tmp_path, "sys.safetensors")
    prefill.save_system_cache(path, sys_k, sys_v, L)
    k2, v2, L2, base = prefill.load_system_cache(path)
    assert L2 == L and base == 10000.0 and torch.equal(k2, sys_k) and torch.equal(v2, sys_v)
    w = W.generate(spec.replace(batch=3, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, sys_len=L, ctx_lo=5, ctx_hi=40))
    t = R.to_device(w, "cuda")
    a = R.decode_workload(dict(t, sys_k=sys_k, sys_v=sys_v))
    b = R.decode_workload(dict(t, sys_k=k2, sys_v=v2))
    assert torch.equal(a, b)

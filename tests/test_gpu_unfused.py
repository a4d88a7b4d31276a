"""GPU parity of fa_fwd_unfused (the standard three-kernel baseline) against the fp64 oracle,
and its agreement with the fused forward on the same inputs."""

import pytest
import torch

from io_aware_attention_02_amd import fa_fwd, fa_fwd_unfused
from io_aware_attention_02_amd.inputs import prefill_inputs
from oracle import attention_ref

from gpu_common import TOL_LSE, TOL_O_BF16, device, f64, max_abs, say

pytestmark = pytest.mark.gpu

SHAPES = [
    # (B, H, Hkv, N, d, causal)
    (1, 1, 1, 8, 128, False),
    (1, 2, 2, 64, 64, True),
    (2, 4, 1, 136, 128, True),
    (1, 8, 2, 1000, 128, False),
    (1, 2, 2, 2048, 64, True),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{s[0]}H{s[1]}Hkv{s[2]}N{s[3]}d{s[4]}{'c' if s[5] else ''}" for s in SHAPES])
def test_unfused_matches_oracle_and_fused(shape):
    B, H, Hkv, N, d, causal = shape
    say(f"fa_fwd_unfused {shape}")
    dev = device()
    q, k, v, _ = prefill_inputs(B, H, Hkv, N, d, "bf16", seed=401 + N)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = fa_fwd_unfused(qd, kd, vd, causal=causal)
    of, lf = fa_fwd(qd, kd, vd, causal=causal)
    torch.cuda.synchronize()
    ro, rl = attention_ref(f64(q), f64(k), f64(v), 1 / d ** 0.5, causal=causal)
    assert max_abs(f64(o), ro) <= TOL_O_BF16
    assert max_abs(f64(lse), rl) <= TOL_LSE
    assert max_abs(f64(o), f64(of)) <= TOL_O_BF16

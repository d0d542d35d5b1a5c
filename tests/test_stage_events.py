"""moe_opts.stage_events: each stage's kernel reports its own start and end, in launch order and
inside the whole call, and timing leaves the result bit-identical."""
import numpy as np
import pytest

import moe_inputs as mi
from helpers import dev, host, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = {
    # streaming expert GEMMs (small groups)
    "stream_bf16": mi.Workload("stream_bf16", T=300, d=256, F=512, dtype="bf16", seed=621),
    # LDS-tiled expert GEMMs with a split down projection
    "tiled_bf16": mi.Workload("tiled_bf16", T=700, d=256, F=2048, E=4, K=2, dtype="bf16", seed=622),
    # few tokens: the per-token router and the single-wavefront permutation
    "few_bf16": mi.Workload("few_bf16", T=32, d=256, F=512, dtype="bf16", seed=623),
}


@pytest.mark.parametrize("name", list(CASES))
def test_stage_events(name):
    import sparse_mixture_experts_33_amd as M
    w = CASES[name]
    say(f"[stage events] {name} T={w.T} d={w.d} F={w.F} E={w.E} K={w.K}")
    W = mi.layer_weights(w)
    x = dev(mi.tokens(w))
    dW = {k: dev(v) for k, v in W.items() if v is not None}
    dm = M.Dims(w.T, w.d, w.F, w.E, w.K, M.MOE_BF16)
    ws = torch.empty(M.moe_workspace_bytes(dm), dtype=torch.uint8, device="cuda")
    y0 = torch.empty((w.T, w.d), dtype=torch.bfloat16, device="cuda")
    y1 = torch.empty_like(y0)
    M.moe_forward(dm, x, dW["w_gate"], dW["w1"], dW["w3"], dW["w2"], y0, ws)

    n = 2 * M.MOE_NUM_STAGES
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    outer = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in ev:
        e.record()  # torch creates the underlying event on its first record
    torch.cuda.synchronize()
    arr = M.stage_event_array({i: e.cuda_event for i, e in enumerate(ev)})
    assert all(arr[i] for i in range(n))
    outer[0].record()
    M.moe_forward(dm, x, dW["w_gate"], dW["w1"], dW["w3"], dW["w2"], y1, ws, stage_events=arr)
    outer[1].record()
    torch.cuda.synchronize()

    assert np.array_equal(host(y0), host(y1))
    dur = [ev[2 * s].elapsed_time(ev[2 * s + 1]) for s in range(M.MOE_NUM_STAGES)]
    total = outer[0].elapsed_time(outer[1])
    say(f"  stage ms {['%.4f' % t for t in dur]}, whole call {total:.4f} ms")
    assert all(t > 0 for t in dur)
    # stages run in order: stage s ends no later than stage s+1 starts (1 us of timer slack)
    for s in range(M.MOE_NUM_STAGES - 1):
        assert ev[2 * s + 1].elapsed_time(ev[2 * s + 2]) >= -1e-3
    assert sum(dur) <= total + 1e-3

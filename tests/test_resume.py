"""Checkpoint/resume of the balancing state (the only state the layer carries between
steps is the per-expert bias and the step counter, which seeds the next batch).

The skewed balancing loop (Zipf-ranked router offsets, fresh seeded tokens each step,
gamma = 0.01; mpbf.cn "DeepSeek-V3技术报告" section 2.2: the bias moves by gamma after
every step) is run 50 steps straight, and again as 25 steps, a save of the state to a
file, a reload into fresh arrays and 25 more steps: the final biases must be equal bit
for bit.  This runs on the oracle at a reduced width (H = 256, T = 1024, the 256
experts, 8 groups, top-8 of the full layer); the GPU counterpart at the full shape is
in tests/test_gpu_full.py."""
import json

import numpy as np

import oracle
import workloads

W = workloads.get("v3-skew-loop", T=1024, H=256)


def _steps(bias, first, last):
    wr = workloads.to_numpy(workloads.make_router(W)[0])
    for step in range(first, last):
        x = workloads.to_numpy(workloads.make_x(W, step=step))
        _, _, counts, _ = oracle.route(x, wr, bias, W.G, W.M, W.K, W.J)
        bias = oracle.bias_update(counts, W.T, W.K, W.gamma, bias)
    return bias


def test_bias_state_resumes_bit_for_bit(tmp_path):
    b0 = workloads.to_numpy(workloads.make_router(W)[1]).copy()
    straight = _steps(b0.copy(), 0, W.steps)
    half = W.steps // 2
    b_half = _steps(b0.copy(), 0, half)
    path = tmp_path / "moe_state.json"
    # the state as a checkpoint would hold it: step counter and the bias bits
    path.write_text(json.dumps({"step": half, "bias_bits": b_half.view(np.uint32).tolist()}))
    state = json.loads(path.read_text())
    b_loaded = np.array(state["bias_bits"], np.uint32).view(np.float32)
    assert np.array_equal(b_loaded.view(np.uint32), b_half.view(np.uint32))
    resumed = _steps(b_loaded, state["step"], W.steps)
    assert np.array_equal(resumed.view(np.uint32), straight.view(np.uint32))
    # and the run did move the bias (the loop is not trivially constant)
    assert np.abs(straight).max() >= 10 * W.gamma

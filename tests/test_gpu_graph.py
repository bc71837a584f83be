"""The product under HIP graph capture: a serving loop captures its decode
step once and replays it.  With the caller's workspace (zeroed once, outside
the capture) the captured launches allocate nothing and record no memset;
every replay leaves the split-K counters at zero, so each replay equals the
eager call bit for bit (the carries meet in a fixed order).

Each graph is replayed several times, with other eager work on the same
workspace and synchronizations between the replays, and every replay is
compared with the eager result.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_02_amd as q8
from block_quantized_weight_02_amd import inputs

pytestmark = pytest.mark.gpu

from tests import gpu_util as g  # noqa: E402

BF16, Q8 = q8.Q8_ACT_BF16, q8.Q8_ACT_Q8_0


def _nan(m, Npad):
    return torch.full((m, Npad), float("nan"), dtype=torch.float32, device=g.DEV)


@pytest.mark.parametrize("m", [2, 16])
def test_graph_replays_match_eager(m):
    K, N = 4096, 640
    x, q, s = inputs.random_case(m, K, N, seed=900 + m)
    Wq, Ws = g.pack(q, s)
    xd = g.dev(x.view(np.int16))
    Npad = q8.q8_padded_cols(N)
    plans = {act: q8.q8_gemv_default_plan(m, K, N, act) for act in (BF16, Q8)}
    assert plans[BF16].split_k > 1            # the carries meet through the workspace
    need = max(q8.q8_plan_workspace_bytes(p, m, K, N) for p in plans.values())
    ws = torch.zeros(need, dtype=torch.uint8, device=g.DEV)
    xq = g.empty_bytes(q8.q8_act_bytes(m, K))

    def step(y, y8):
        q8.q8_gemv_ws(xd, Wq, Ws, y, m, K, N, BF16, None, ws, need)
        q8.q8_quantize_act(xd, xq, m, K)
        q8.q8_gemv_ws(xq, Wq, Ws, y8, m, K, N, Q8, None, ws, need)

    ye, y8e = _nan(m, Npad), _nan(m, Npad)
    step(ye, y8e)
    torch.cuda.synchronize()
    ye, y8e = ye.cpu().numpy(), y8e.cpu().numpy()

    y, y8 = _nan(m, Npad), _nan(m, Npad)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(y, y8)
    torch.cuda.synchronize()

    # other eager work on the same workspace between the replays
    xo, qo, so = inputs.random_case(3, 2048, 200, seed=910 + m)
    Wo, Wso = g.pack(qo, so)
    yo = _nan(3, q8.q8_padded_cols(200))
    for rep in range(5):
        y.fill_(float("nan"))
        y8.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), ye.view(np.uint32),
                                      err_msg=f"bf16 replay {rep}")
        np.testing.assert_array_equal(y8.cpu().numpy().view(np.uint32), y8e.view(np.uint32),
                                      err_msg=f"int8 replay {rep}")
        q8.q8_gemv_ws(g.dev(xo.view(np.int16)), Wo, Wso, yo, 3, 2048, 200, BF16, None, ws,
                      q8.q8_plan_workspace_bytes(q8.q8_gemv_default_plan(3, 2048, 200, BF16),
                                                 3, 2048, 200))
        torch.cuda.synchronize()

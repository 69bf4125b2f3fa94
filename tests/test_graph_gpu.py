"""The hot path captured in a HIP graph: every replay must equal the eager
result. The library issues only kernel launches (no memset or copy nodes), so
replays are independent; the test replays several times with eager work and
synchronizations in between and compares each replay bit for bit."""

import numpy as np
import pytest
import torch

import gen
from tests.devutil import to_device

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import w4_gemm_vqv_amd as vqv
    vqv.lib()
    c = gen.make_config("tiny")
    d = to_device(c)
    M, N, T = c["M"], c["N"], 8
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    am = torch.empty(T, dtype=torch.int32, device="cuda")
    al = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(vqv.vqv_verify_workspace_bytes(1, T, N), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(3)
    draft = torch.from_numpy(rng.integers(0, N, size=(1, T - 1)).astype(np.int32)).cuda()

    def path(st):
        vqv.vqv_qgemm(d["x"], d["wq"], d["scales"], d["biases"], y=y, stream=st)
        vqv.vqv_verify(y, draft, 1, T, argmax=am, accept_len=al, workspace=ws, stream=st)

    path(None)
    torch.cuda.synchronize()
    want = (y.clone(), am.clone(), al.clone())
    # force the first two drafts to be accepted so the walk is exercised
    draft[0, :2] = want[1][:2]
    path(None)
    torch.cuda.synchronize()
    want = (y.clone(), am.clone(), al.clone())
    assert int(want[2][0]) >= 2

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path(torch.cuda.current_stream())
    for rep in range(4):
        y.fill_(float("nan"))
        am.fill_(-1)
        al.fill_(-1)
        _ = (torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want[0]), f"replay {rep}: y differs"
        assert torch.equal(am, want[1]) and torch.equal(al, want[2]), f"replay {rep}: verify"


@pytest.mark.parametrize("group", [32, 128])
def test_graph_replays_match_eager_other_groups(group):
    """The fused call (projection with the argmax epilogue, then the finishing
    kernel) at groups 32 and 128, captured and replayed."""
    import w4_gemm_vqv_amd as vqv
    vqv.lib()
    c = gen.make_config("tiny", group=group)
    d = to_device(c)
    M, N, T = c["M"], c["N"], 8
    rng = np.random.default_rng(4)
    draft = torch.from_numpy(rng.integers(0, N, size=(1, T - 1)).astype(np.int32)).cuda()
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    am = torch.empty(T, dtype=torch.int32, device="cuda")
    al = torch.empty(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(vqv.vqv_qgemm_verify_workspace_bytes(M, c["K"], N, group, vqv.VQV_BF16),
                     dtype=torch.uint8, device="cuda")

    def path(st):
        vqv.vqv_qgemm_verify(d["x"], d["wq"], d["scales"], d["biases"], draft, 1, T, y=y,
                             argmax=am, accept_len=al, workspace=ws, group=group, stream=st)

    path(None)
    torch.cuda.synchronize()
    draft[0, :3] = am[:3]                              # the walk accepts three drafts
    path(None)
    torch.cuda.synchronize()
    want = (y.clone(), am.clone(), al.clone())
    assert int(want[2][0]) >= 3

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path(torch.cuda.current_stream())
    for rep in range(4):
        y.fill_(float("nan"))
        am.fill_(-1)
        al.fill_(-1)
        _ = (torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want[0]), f"group {group} replay {rep}: y differs"
        assert torch.equal(am, want[1]) and torch.equal(al, want[2]), f"group {group} replay {rep}"

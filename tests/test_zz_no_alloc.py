"""The allocation-free fused call (vqv_qgemm_verify_ex_noalloc) against the
workspace call it mirrors (vqv_qgemm_verify_ex), through the C ABI: every
output bit for bit, on two calls in a row that share the library's static
scratch, the second with a smaller problem."""

import numpy as np
import pytest
import torch

import gen
from tests.devutil import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vqv():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X")
    import w4_gemm_vqv_amd as v
    v.lib()
    return v


def _case(M, K, N, act, B, T, seed):
    rng = np.random.default_rng(seed)
    wq, s, b = gen.make_weights(rng, N, K)
    x = gen.make_x(rng, M, K, act)
    c = dict(x=x, wq=wq, scales=s, biases=b, act=act)
    d = to_device(c)
    draft = torch.from_numpy(rng.integers(0, N, size=(B, max(T - 1, 1))).astype(np.int32)
                             [:, :T - 1].copy()).cuda()
    dl = torch.from_numpy(rng.integers(0, T, size=B).astype(np.int32)).cuda()
    return d, draft, dl


def _both(vqv, d, draft, dl, B, T, with_y):
    """(workspace call, allocation-free call) outputs on the same inputs."""
    M, N = d["x"].shape[0], d["wq"].shape[0]
    ref = vqv.vqv_qgemm_verify_ex(d["x"], d["wq"], d["scales"], d["biases"], draft, B, T,
                                  draft_len=dl, want_y=with_y)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda") if with_y else None
    am = torch.full((B * T,), -7, dtype=torch.int32, device="cuda")
    al = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    mg = torch.full((B * T,), float("nan"), dtype=torch.float32, device="cuda")
    out = vqv.vqv_qgemm_verify_ex_noalloc(d["x"], d["wq"], d["scales"], d["biases"], draft, B, T,
                                          draft_len=dl, y=y, argmax=am, accept_len=al,
                                          margin=mg)
    torch.cuda.synchronize()
    return ref, out


def _same(ref, out, what):
    y0, a0, l0, m0 = ref
    y1, a1, l1, m1 = out
    assert torch.equal(a0, a1), f"{what}: argmax"
    assert torch.equal(l0, l1), f"{what}: accept_len"
    assert np.array_equal(m0.cpu().numpy().view(np.uint32), m1.cpu().numpy().view(np.uint32)), \
        f"{what}: margin bits"
    if y0 is not None:
        assert np.array_equal(y0.cpu().numpy().view(np.uint32), y1.cpu().numpy().view(np.uint32)), \
            f"{what}: y bits"


# (M, K, N, act, B, T, with_y): a larger call, then a smaller one, per kernel
# family (8-row, 16-row and batched vocabulary kernels, fp32 activations).
ROWS8 = [(8, 5120, 17408, "bf16", 1, 8, True), (4, 512, 1000, "fp16", 1, 4, True)]
ROWS16 = [(16, 1024, 5000, "bf16", 2, 8, True), (12, 512, 3000, "bf16", 3, 4, False)]
BATCHED = [(64, 512, 40000, "bf16", 4, 16, False), (32, 512, 33000, "fp16", 2, 16, True)]
FP32 = [(8, 1024, 2048, "fp32", 2, 4, True), (4, 512, 700, "fp32", 1, 4, False)]


@pytest.mark.parametrize("calls", [ROWS8, ROWS16, BATCHED, FP32],
                         ids=["rows8", "rows16", "batched", "fp32"])
def test_noalloc_matches_workspace_call(vqv, calls):
    for i, (M, K, N, act, B, T, with_y) in enumerate(calls):
        d, draft, dl = _case(M, K, N, act, B, T, seed=100 * M + i)
        ref, out = _both(vqv, d, draft, dl, B, T, with_y)
        _same(ref, out, f"call {i}: M={M} K={K} N={N} {act} B={B} T={T} y={with_y}")


def test_noalloc_rejects_oversized_scratch(vqv):
    """A problem whose scratch exceeds the static array is refused before any
    launch: the outputs keep their sentinels."""
    M, K, N, B, T = 8, 64, 1_000_000, 1, 8      # 12,500 work-groups: 1.6 MB of partials
    d, draft, dl = _case(M, K, N, "bf16", B, T, seed=5)
    am = torch.full((B * T,), -7, dtype=torch.int32, device="cuda")
    al = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(vqv.VqvError) as e:
        vqv.vqv_qgemm_verify_ex_noalloc(d["x"], d["wq"], d["scales"], d["biases"], draft, B, T,
                                        argmax=am, accept_len=al)
    assert e.value.status == vqv.VQV_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (am == -7).all() and (al == -7).all()

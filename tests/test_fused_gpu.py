"""GPU parity of vqv_qgemm_verify (projection with the greedy verify fused
into its epilogue) through the C ABI.

The fused call must give exactly what vqv_qgemm followed by vqv_verify gives
on the same inputs (y, argmax and accept_len bit for bit), and its argmax
must equal the oracle's argmax of the GPU's own logits. Every projection
kernel carries the fused epilogue, so the shapes cover each of them: the
8-row kernels (whole-line and half-line), the whole-tile vocabulary kernel
with one or several row sets, the batched vocabulary kernel (17..64 rows on
one weight stream), the 16-row kernel, and the general kernel (more rows at
large K, fp32 activations, K past the 8-row kernels' LDS budget).
"""

import numpy as np
import pytest
import torch

import gen
from oracle import argmax_ref, qgemm_ref, verify_ref
from tests.devutil import assert_close, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vqv():
    import w4_gemm_vqv_amd as v
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    v.lib()
    return v


def case(M, K, N, act, seed, group=64):
    rng = np.random.default_rng(seed)
    wq, s, b = gen.make_weights(rng, N, K, group)
    x = gen.make_x(rng, M, K, act, 1.0, None)
    return dict(M=M, K=K, N=N, act=act, wq=wq, scales=s, biases=b, x=x, seed=seed, group=group)


def drafts_for(vqv, d, B, T, N, seed, accept, group=64):
    """Drafts that realise the given accept lengths against the GPU's own
    argmax (from the separate path)."""
    y = vqv.vqv_qgemm(d["x"], d["wq"], d["scales"], d["biases"], group=group)
    torch.cuda.synchronize()
    a = np.array([argmax_ref(r) for r in y.cpu().numpy()])
    return gen.make_drafts(a, B, T, N, seed=seed, accept=accept)


def compare(vqv, c, B, T, accept=None, want_y=True, ws=None):
    d = to_device(c)
    M, N = c["M"], c["N"]
    if accept is None:
        accept = np.random.default_rng(c["seed"] + 1).integers(0, T, size=B)
    group = c.get("group", 64)
    draft = drafts_for(vqv, d, B, T, N, c["seed"], accept, group)
    dt = torch.from_numpy(draft).cuda() if T > 1 else None
    y1 = vqv.vqv_qgemm(d["x"], d["wq"], d["scales"], d["biases"], group=group)
    a1, l1 = vqv.vqv_verify(y1, dt, B, T)
    y2, a2, l2 = vqv.vqv_qgemm_verify(d["x"], d["wq"], d["scales"], d["biases"], dt, B, T,
                                      want_y=want_y, workspace=ws, group=group)
    torch.cuda.synchronize()
    if want_y:
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)), \
            "fused y differs from vqv_qgemm"
    assert torch.equal(a1, a2), (a1.cpu().numpy(), a2.cpu().numpy())
    assert torch.equal(l1, l2), (l1.cpu().numpy(), l2.cpu().numpy())
    ra, rl = verify_ref(y1.cpu().numpy(), draft, B, T)
    np.testing.assert_array_equal(a2.cpu().numpy(), ra)
    np.testing.assert_array_equal(l2.cpu().numpy(), rl)
    if T > 1:
        np.testing.assert_array_equal(l2.cpu().numpy(), accept)
    return y2, a2, l2


@pytest.mark.parametrize("M,K,N,act,B,T", [
    (8, 512, 1024, "bf16", 1, 8), (8, 512, 1024, "fp16", 2, 4), (4, 1280, 3000, "bf16", 1, 4),
    (1, 64, 17, "bf16", 1, 1), (8, 192, 999, "fp16", 8, 1), (5, 320, 5000, "bf16", 1, 5),
    (8, 2560, 17408, "bf16", 1, 8), (6, 5120, 1000, "bf16", 3, 2), (8, 640, 12000, "fp16", 4, 2),
    # vocabulary widths: the persistent whole-tile kernel's fused epilogue
    (8, 512, 70000, "bf16", 1, 8), (4, 1024, 66001, "fp16", 2, 2), (1, 2560, 66000, "bf16", 1, 1),
])
def test_fused_matches_separate(vqv, M, K, N, act, B, T):
    compare(vqv, case(M, K, N, act, seed=M * 7 + K + N), B, T)


@pytest.mark.parametrize("M,K,N,act,B,T", [
    # 16-row kernel (9..64 rows, K <= 2560)
    (16, 512, 1000, "bf16", 1, 16), (64, 256, 700, "fp16", 4, 16), (12, 2560, 17408, "bf16", 3, 4),
    (40, 640, 3000, "bf16", 5, 8), (9, 128, 40, "fp16", 9, 1),
    # general kernel: more rows at large K, fp32, M <= 8 past the 8-row kernels' LDS
    (16, 5120, 4000, "bf16", 1, 16), (24, 3072, 1500, "fp16", 3, 8), (64, 4096, 1000, "bf16", 4, 16),
    (8, 512, 700, "fp32", 1, 8), (8, 5120, 1024, "fp32", 1, 8), (64, 1024, 3000, "fp32", 4, 16),
    (33, 256, 999, "fp32", 3, 11), (8, 8192, 300, "bf16", 1, 8), (2, 16384, 700, "fp16", 1, 2),
])
def test_general_kernels_match_separate(vqv, M, K, N, act, B, T):
    compare(vqv, case(M, K, N, act, seed=M + K + N), B, T)


@pytest.mark.parametrize("M,K,N,act,B,T", [
    # batched vocabulary kernel (17..64 rows, 8..40 tiles per wave)
    (64, 512, 40000, "bf16", 4, 16), (32, 1024, 33000, "fp16", 2, 16), (48, 256, 151936, "bf16", 3, 16),
    (17, 512, 36000, "bf16", 17, 1),
    # whole-tile kernel: 9..16 rows, and several row sets past the batched kernel's width
    (16, 512, 70000, "bf16", 1, 16), (12, 1024, 66001, "fp16", 2, 6), (32, 512, 200000, "bf16", 2, 16),
])
def test_batched_vocab_matches_separate(vqv, M, K, N, act, B, T):
    compare(vqv, case(M, K, N, act, seed=3 * M + K + N), B, T)


@pytest.mark.parametrize("M,K,N,act,B,T", [
    (8, 512, 1024, "bf16", 1, 8), (8, 2560, 17408, "fp16", 2, 4), (5, 384, 5000, "bf16", 1, 5),
    (8, 512, 70000, "bf16", 1, 8), (1, 2560, 66000, "fp16", 1, 1), (16, 512, 1000, "bf16", 1, 16),
    (8, 512, 700, "fp32", 1, 8),
])
def test_group128_matches_separate(vqv, M, K, N, act, B, T):
    """Group 128 through the fused epilogues of the 8-row, whole-tile, 16-row
    and general kernels; the logits themselves are pinned by the projection
    tests."""
    c = case(M, K, N, act, seed=M * 11 + K + N, group=128)
    y, _, _ = compare(vqv, c, B, T)
    ref = qgemm_ref(c["x"], act, c["wq"], c["scales"], c["biases"], group=128)
    assert_close(y.cpu().numpy(), ref, act, f"group 128 fused M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N,act,B,T", [
    (8, 512, 1024, "bf16", 1, 8), (8, 5120, 17408, "bf16", 1, 8), (4, 1280, 3000, "fp16", 2, 2),
    (16, 512, 1000, "fp32", 1, 16), (8, 2560, 151936, "fp16", 1, 8), (1, 64, 17, "bf16", 1, 1),
    (8, 512, 70000, "bf16", 2, 4), (8, 1280, 70000, "bf16", 1, 8), (64, 512, 40000, "bf16", 4, 16),
    (16, 1024, 2000, "fp16", 2, 8),
])
def test_group32_matches_separate(vqv, M, K, N, act, B, T):
    """Group 32: the fused epilogues of the whole-tile kernel (vocabulary widths,
    K/128 a multiple of 4), the batched vocabulary kernel, the 8-row and 16-row
    kernels and the general kernel (fp32)."""
    c = case(M, K, N, act, seed=M * 13 + K + N, group=32)
    y, _, _ = compare(vqv, c, B, T)
    ref = qgemm_ref(c["x"], act, c["wq"], c["scales"], c["biases"], group=32)
    assert_close(y.cpu().numpy(), ref, act, f"group 32 fused M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N,act,B,T", [
    (8, 1024, 4000, "bf16", 1, 8), (64, 512, 40000, "bf16", 4, 16), (16, 512, 1000, "fp16", 2, 8),
    (16, 5120, 2000, "bf16", 1, 16), (8, 512, 700, "fp32", 1, 8), (16, 512, 70000, "bf16", 1, 16),
])
def test_without_logits(vqv, M, K, N, act, B, T):
    """y = NULL: each kernel family skips the logits and keeps the partials."""
    c = case(M, K, N, act, seed=21 + M)
    y, a, l = compare(vqv, c, B, T, want_y=False)
    assert y is None


def test_workspace_reuse_and_every_accept_length(vqv):
    """One workspace (filled with garbage first) serves many calls."""
    c = case(8, 2560, 20000, "fp16", seed=5)
    need = vqv.vqv_qgemm_verify_workspace_bytes(8, 2560, 20000, 64, vqv.VQV_FP16)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    for L in range(8):
        _, _, l = compare(vqv, c, 1, 8, accept=np.array([L]), ws=ws)
        assert int(l[0]) == L


def test_batched_workspace_reuse_and_every_accept_length(vqv):
    """Four sequences of 16 rows on the batched vocabulary kernel, one garbage-
    filled workspace, every accept length 0..15 in some sequence."""
    c = case(64, 512, 40000, "bf16", seed=6)
    need = vqv.vqv_qgemm_verify_workspace_bytes(64, 512, 40000, 64, vqv.VQV_BF16)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
    for r in range(4):
        accept = np.array([4 * r, 4 * r + 1, 4 * r + 2, 4 * r + 3])
        _, _, l = compare(vqv, c, 4, 16, accept=accept, ws=ws)
        np.testing.assert_array_equal(l.cpu().numpy(), accept)


def test_full_size_target(vqv):
    c = gen.make_config("target")
    compare(vqv, c, 1, 8, accept=np.array([5]))


def test_full_size_vocab(vqv):
    c = gen.make_config("vocab_verify")
    compare(vqv, c, 1, 8, accept=np.array([7]))


def test_full_size_batched(vqv):
    c = gen.make_config("batched_vocab")
    compare(vqv, c, 4, 16, accept=np.array([13, 0, 15, 6]))


def test_full_size_draft_w4a32(vqv):
    c = gen.make_config("draft_w4a32")
    compare(vqv, c, 1, 8, accept=np.array([3]))


def test_logits_within_contract(vqv):
    c = case(8, 1024, 2000, "bf16", seed=3)
    d = to_device(c)
    y, _, _ = vqv.vqv_qgemm_verify(d["x"], d["wq"], d["scales"], d["biases"],
                                   torch.zeros((1, 7), dtype=torch.int32, device="cuda"), 1, 8)
    torch.cuda.synchronize()
    ref = qgemm_ref(c["x"], "bf16", c["wq"], c["scales"], c["biases"])
    assert_close(y.cpu().numpy(), ref, "bf16", "fused logits")


def test_graph_replays(vqv):
    c = case(8, 512, 3000, "bf16", seed=8)
    d = to_device(c)
    draft = torch.zeros((1, 7), dtype=torch.int32, device="cuda")
    need = vqv.vqv_qgemm_verify_workspace_bytes(8, 512, 3000, 64, vqv.VQV_BF16)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    y = torch.empty((8, 3000), dtype=torch.float32, device="cuda")
    a = torch.empty(8, dtype=torch.int32, device="cuda")
    l = torch.empty(1, dtype=torch.int32, device="cuda")

    def run(st):
        vqv.vqv_qgemm_verify(d["x"], d["wq"], d["scales"], d["biases"], draft, 1, 8, y=y,
                             argmax=a, accept_len=l, workspace=ws, stream=st)

    run(None)
    torch.cuda.synchronize()
    draft[0, :3] = a[:3]
    run(None)
    torch.cuda.synchronize()
    want = (y.clone(), a.clone(), l.clone())
    assert int(want[2][0]) >= 3
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(torch.cuda.current_stream())
    for rep in range(4):
        y.fill_(float("nan"))
        a.fill_(-1)
        l.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want[0]) and torch.equal(a, want[1]) and torch.equal(l, want[2]), rep


@pytest.mark.parametrize("name,B,T", [("vocab_verify", 1, 8), ("batched_vocab", 4, 16)])
def test_full_size_without_logits(vqv, name, B, T):
    """The logits-free fused call at the vocabulary and batched workloads'
    full sizes (the call `bench.py` times beside the step): its argmax and
    accept lengths equal the two-call path's and the oracle walk's."""
    c = gen.make_config(name)
    y, _, _ = compare(vqv, c, B, T, want_y=False)
    assert y is None

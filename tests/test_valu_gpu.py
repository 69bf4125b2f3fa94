"""GPU parity of the vector-ALU kernel (qgemm_w4_v: one or two activation
rows, a K-major dot2 matvec) through the C ABI, pinned with
VQV_FORCE_VARIANT=v: every output against the CPU oracle, the fused verify
bit for bit against the separate path on the same kernel.
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


@pytest.fixture
def pin_v(monkeypatch):
    monkeypatch.setenv("VQV_FORCE_VARIANT", "v")


def case(M, K, N, act, seed, group=64):
    rng = np.random.default_rng(seed)
    wq, s, b = gen.make_weights(rng, N, K, group)
    x = gen.make_x(rng, M, K, act, 1.0, None)
    return dict(M=M, K=K, N=N, act=act, wq=wq, scales=s, biases=b, x=x, group=group)


ACT = {"bf16": 0, "fp16": 1}

# K: one group, odd group counts, partial and whole chunk rounds of 1024
# code bytes (K = 2048 per round), up to four rounds; N: a single column,
# ragged counts, fewer columns than waves and many columns per wave.
SHAPES = [(1, 64, 1), (1, 192, 17), (2, 128, 1000), (1, 2048, 3000), (2, 2560, 999),
          (1, 5120, 17408), (2, 5120, 4097), (1, 6144, 500), (2, 8192, 300), (1, 4160, 65)]


@pytest.mark.parametrize("act", ["bf16", "fp16"])
@pytest.mark.parametrize("M,K,N", SHAPES)
@pytest.mark.parametrize("group", [64, 128])
def test_valu_parity(vqv, pin_v, act, M, K, N, group):
    if K % group:
        pytest.skip("K not a multiple of the group")
    assert vqv.vqv_qgemm_kernel(M, K, N, group, ACT[act]) == "qgemm_w4_v"
    c = case(M, K, N, act, seed=M * 100 + K + N + group, group=group)
    d = to_device(c)
    y = vqv.vqv_qgemm(d["x"], d["wq"], d["scales"], d["biases"], group=group)
    torch.cuda.synchronize()
    ref = qgemm_ref(c["x"], act, c["wq"], c["scales"], c["biases"], group=group)
    assert_close(y.cpu().numpy(), ref, act, f"valu M={M} K={K} N={N} {act} group {group}")


def test_valu_deterministic(vqv, pin_v):
    c = case(1, 5120, 17408, "bf16", seed=3)
    d = to_device(c)
    ys = [vqv.vqv_qgemm(d["x"], d["wq"], d["scales"], d["biases"]) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(ys[0].view(torch.int32), t.view(torch.int32)) for t in ys[1:])


@pytest.mark.parametrize("M,K,N,act,B,T", [
    (1, 5120, 17408, "bf16", 1, 1), (2, 2560, 5000, "fp16", 1, 2), (2, 512, 1000, "bf16", 2, 1),
    (1, 64, 1, "bf16", 1, 1), (2, 8192, 300, "bf16", 1, 2),
])
def test_valu_fused_matches_separate(vqv, pin_v, M, K, N, act, B, T):
    c = case(M, K, N, act, seed=7 * M + K + N)
    d = to_device(c)
    y1 = vqv.vqv_qgemm(d["x"], d["wq"], d["scales"], d["biases"])
    torch.cuda.synchronize()
    a_gpu = np.array([argmax_ref(r) for r in y1.cpu().numpy()])
    accept = np.full(B, T - 1)
    draft = gen.make_drafts(a_gpu, B, T, N, seed=K, accept=accept) if T > 1 else None
    dt = torch.from_numpy(draft).cuda() if draft is not None else None
    a1, l1, m1 = vqv.vqv_verify_ex(y1, dt, B, T)
    y2, a2, l2, m2 = vqv.vqv_qgemm_verify_ex(d["x"], d["wq"], d["scales"], d["biases"], dt, B, T)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    assert torch.equal(a1, a2) and torch.equal(l1, l2)
    assert np.array_equal(m1.cpu().numpy().view(np.uint32), m2.cpu().numpy().view(np.uint32))
    ra, rl = verify_ref(y1.cpu().numpy(), draft, B, T)
    np.testing.assert_array_equal(a2.cpu().numpy(), ra)
    np.testing.assert_array_equal(l2.cpu().numpy(), rl)

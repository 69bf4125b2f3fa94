"""GPU parity of vqv_qgemm_swiglu (gate/up projection with its SwiGLU
activation) against the CPU oracle, through the C ABI.

h = silu(x . Wg^T) * (x . Wu^T) with W = [Wg; Wu] stacked along N. The
tolerance follows from the projection's contract |dy| <= tau*(1+|y|) on the
gate g and the up value u by first-order propagation through
h = silu(g)*u (|silu'| <= 1.1), plus the fp32 evaluation of the epilogue:
    |dh| <= tau*(1.1*|u|*(1+|g|) + |silu(g)|*(1+|u|) + 1.1*tau*(1+|g|)*(1+|u|))
            + 2^-20*|h|,
with g, u, h the oracle's float64 values. Shapes cover the fused kernel
(16-bit activations, K <= 2560, row sets of 16: several tiles, ragged tails,
odd group counts, M below 8 and up to 64) and the two-step fallback (fp32
activations, larger K).
"""

import numpy as np
import pytest
import torch

import gen
from oracle import qgemm_ref, silu_ref
from tests.devutil import TOL, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vqv():
    import w4_gemm_vqv_amd as v
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    v.lib()
    return v


def case(M, K, N, act, seed, sigma=1.0, group=64):
    rng = np.random.default_rng(seed)
    wq, s, b = gen.make_weights(rng, N, K, group)
    x = gen.make_x(rng, M, K, act, sigma, None)
    return dict(M=M, K=K, N=N, act=act, wq=wq, scales=s, biases=b, x=x, group=group)


def gate_up_ref(c, cols=None):
    """float64 gate g, up u and h = silu(g)*u for hidden columns `cols`."""
    nh = c["N"] // 2
    idx = np.arange(nh) if cols is None else np.asarray(cols)
    group = c.get("group", 64)
    g = qgemm_ref(c["x"], c["act"], c["wq"], c["scales"], c["biases"], group, cols=idx)
    u = qgemm_ref(c["x"], c["act"], c["wq"], c["scales"], c["biases"], group, cols=nh + idx)
    return g, u, silu_ref(g) * u


def assert_swiglu_close(h_gpu, g, u, h_ref, act, what):
    tau = TOL[act]
    ag, au = np.abs(g), np.abs(u)
    allow = tau * (1.1 * au * (1 + ag) + np.abs(silu_ref(g)) * (1 + au)
                   + 1.1 * tau * (1 + ag) * (1 + au)) + 2.0 ** -20 * np.abs(h_ref)
    err = np.abs(h_gpu.astype(np.float64) - h_ref)
    bad = ~(err <= allow)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside the bound; first "
                             f"{i} gpu={h_gpu[i]!r} ref={h_ref[i]!r} allow={allow[i]!r}")
    return float(np.max(err / allow)) if err.size else 0.0


def run(vqv, c, M=None):
    d = to_device(c)
    x = d["x"] if M is None else d["x"][:M].contiguous()
    h = vqv.vqv_qgemm_swiglu(x, d["wq"], d["scales"], d["biases"], group=c.get("group", 64))
    torch.cuda.synchronize()
    return h.cpu().numpy()


FUSED = [(16, 512, 2 * 1000, "bf16"), (16, 2560, 2 * 3000, "bf16"), (12, 640, 2 * 777, "fp16"),
         (9, 64, 2 * 5, "bf16"), (1, 512, 2 * 300, "bf16"), (8, 192, 2 * 1234, "fp16"),
         (16, 1280, 2 * 6000, "fp16"), (5, 448, 2 * 41, "bf16"), (16, 128, 2, "bf16")]
FUSED += [(32, 512, 2 * 500, "bf16"), (64, 256, 2 * 130, "fp16"), (48, 2560, 2 * 2100, "bf16"),
          (17, 640, 2 * 999, "fp16")]
FALLBACK = [(16, 512, 2 * 300, "fp32"), (16, 5120, 2 * 200, "bf16"), (3, 4096, 2 * 77, "fp32"),
            (40, 3072, 2 * 150, "fp16")]


@pytest.mark.parametrize("M,K,N,act", FUSED + FALLBACK)
def test_swiglu_parity(vqv, M, K, N, act):
    c = case(M, K, N, act, seed=M * 100 + K + N)
    h = run(vqv, c)
    assert h.shape == (M, N // 2)
    g, u, ref = gate_up_ref(c)
    worst = assert_swiglu_close(h, g, u, ref, act, f"M={M} K={K} N={N} {act}")
    print(f"M={M} K={K} N={N} {act}: worst error/allowance {worst:.3g}")


@pytest.mark.parametrize("M,K,N,act", [(16, 512, 2 * 1000, "bf16"), (12, 640, 2 * 777, "fp16"),
                                        (16, 2560, 2 * 3000, "bf16"), (64, 256, 2 * 130, "fp16"),
                                        (16, 512, 2 * 300, "fp32"), (40, 3072, 2 * 150, "fp16")])
def test_swiglu_group128(vqv, M, K, N, act):
    c = case(M, K, N, act, seed=M * 100 + K + N + 128, group=128)
    h = run(vqv, c)
    g, u, ref = gate_up_ref(c)
    assert_swiglu_close(h, g, u, ref, act, f"group 128 M={M} K={K} N={N} {act}")


@pytest.mark.parametrize("M,K,N,act", [(16, 512, 2 * 1000, "bf16"), (9, 192, 2 * 77, "fp16"),
                                        (40, 1280, 2 * 150, "fp32")])
def test_swiglu_group32(vqv, M, K, N, act):
    c = case(M, K, N, act, seed=M * 100 + K + N + 32, group=32)
    h = run(vqv, c)
    g, u, ref = gate_up_ref(c)
    assert_swiglu_close(h, g, u, ref, act, f"group 32 M={M} K={K} N={N} {act}")


def test_fused_workspace_is_zero(vqv):
    assert vqv.vqv_qgemm_swiglu_workspace_bytes(16, 2560, 18432, 64, vqv.VQV_BF16) == 0
    assert vqv.vqv_qgemm_swiglu_workspace_bytes(64, 2560, 18432, 64, vqv.VQV_BF16) == 0
    assert vqv.vqv_qgemm_swiglu_workspace_bytes(16, 2560, 18432, 64, vqv.VQV_FP32) > 0


def test_matches_plain_projection(vqv):
    """Against silu(g)*u formed in float64 from vqv_qgemm's own gate and up
    outputs: both sides sum in fp32, so they agree far inside the contract."""
    c = case(16, 1024, 2 * 2500, "bf16", seed=31)
    d = to_device(c)
    h = vqv.vqv_qgemm_swiglu(d["x"], d["wq"], d["scales"], d["biases"])
    y = vqv.vqv_qgemm(d["x"], d["wq"], d["scales"], d["biases"])
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    nh = c["N"] // 2
    ref = silu_ref(y[:, :nh]) * y[:, nh:]
    err = np.abs(h.cpu().numpy() - ref)
    assert np.all(err <= 1e-5 * (1 + np.abs(ref))), float(err.max())


def test_full_size_gate_up(vqv):
    """The gate/up workload, M=16, K=2560, N=2x9216, every output."""
    c = gen.make_config("gate_up")
    h = run(vqv, c)
    g, u, ref = gate_up_ref(c)
    worst = assert_swiglu_close(h, g, u, ref, c["act"], "gate_up")
    print(f"gate_up: worst error/allowance {worst:.3g}")


def test_deterministic_and_writes_only_h(vqv):
    c = case(16, 2560, 2 * 4000, "bf16", seed=7)
    d = to_device(c)
    out = torch.full((16 + 2, 4000), 7.5, dtype=torch.float32, device="cuda")
    h = out[1:17]
    vqv.vqv_qgemm_swiglu(d["x"], d["wq"], d["scales"], d["biases"], h=h)
    first = h.clone()
    vqv.vqv_qgemm_swiglu(d["x"], d["wq"], d["scales"], d["biases"], h=h)
    torch.cuda.synchronize()
    assert torch.equal(first, h)
    assert (out[0] == 7.5).all() and (out[17] == 7.5).all()


def test_graph_replays(vqv):
    c = case(16, 2560, 2 * 3000, "bf16", seed=9)
    d = to_device(c)
    h = torch.empty((16, 3000), dtype=torch.float32, device="cuda")
    vqv.vqv_qgemm_swiglu(d["x"], d["wq"], d["scales"], d["biases"], h=h)
    torch.cuda.synchronize()
    eager = h.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vqv.vqv_qgemm_swiglu(d["x"], d["wq"], d["scales"], d["biases"], h=h,
                             stream=torch.cuda.current_stream())
    for _ in range(3):
        h.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h, eager)

"""A seeded sweep of random shapes through the C ABI against the oracle.

The hand-picked shapes elsewhere aim at each kernel's edges; this sweep draws
M, K, N, the group size and the activation type at random (K and N
log-uniform, within the documented limits), so the dispatcher's choice of
kernel and every ragged tail it meets are exercised in combinations nobody
picked. Each case checks vqv_qgemm against the oracle element by element and,
on a factorisation M = B*T, vqv_qgemm_verify's logits against the oracle and
its argmax and accept lengths bit for bit against the oracle's verify of the
same logits; vqv_qgemm_verify_ex the same, with random valid draft counts
(some outside 0..T-1) and the margins bit for bit. Where N is even, vqv_qgemm_swiglu's h is checked against the
oracle's silu(gate) * up of the same projection, N/2 columns each.
"""

import numpy as np
import pytest
import torch

import gen
from oracle import argmax_ref, qgemm_ref, silu_ref, verify_ref
from tests.devutil import assert_close, to_device
from tests.test_swiglu_gpu import assert_swiglu_close
from tests.test_verify_ex_gpu import bits

pytestmark = pytest.mark.gpu

ROWS = [1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 17, 24, 31, 32, 33, 48, 63, 64]


def sweep_cases(n, seed, n_lo=1, n_hi=80000, max_nk=12_000_000, first=0):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        group = int(rng.choice([32, 64, 128]))
        act = str(rng.choice(["bf16", "fp16", "fp32"]))
        M = int(rng.choice(ROWS))
        unit = 128 if group == 128 else 64
        kmax = 8192 if group == 32 else 16384
        K = unit * max(1, int(round(np.exp(rng.uniform(0.0, np.log(kmax // unit))))))
        N = max(1, int(np.exp(rng.uniform(np.log(n_lo), np.log(n_hi)))))
        if N * K > max_nk:
            continue
        divisors = [t for t in range(1, M + 1) if M % t == 0]
        T = int(rng.choice(divisors))
        out.append((M, K, N, group, act, M // T, T, first + len(out)))
    return out


# Small and mid-sized outputs, then vocabulary-like widths (the whole-tile
# and row-set kernels).
CASES = (sweep_cases(96, 2026) +
         sweep_cases(64, 2027, n_lo=8000, n_hi=160000, max_nk=40_000_000, first=96))


@pytest.fixture(scope="module")
def vqv():
    import w4_gemm_vqv_amd as v
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    v.lib()
    return v


@pytest.mark.parametrize("M,K,N,group,act,B,T,i", CASES)
def test_sweep(vqv, M, K, N, group, act, B, T, i):
    what = f"sweep case {i}: M={M} K={K} N={N} group={group} {act} B={B} T={T}"
    print(what, flush=True)
    rng = np.random.default_rng((2026, i))
    wq, s, b = gen.make_weights(rng, N, K, group)
    x = gen.make_x(rng, M, K, act, 1.0, None)
    c = dict(act=act, x=x, wq=wq, scales=s, biases=b)
    d = to_device(c)
    ref = qgemm_ref(x, act, wq, s, b, group=group)

    y = vqv.vqv_qgemm(d["x"], d["wq"], d["scales"], d["biases"], group=group)
    torch.cuda.synchronize()
    y_np = y.cpu().numpy()
    assert_close(y_np, ref, act, what)

    a_own = np.array([argmax_ref(r) for r in y_np])
    accept = rng.integers(0, T, size=B)
    draft = gen.make_drafts(a_own, B, T, N, seed=i, accept=accept)
    dt = torch.from_numpy(draft).cuda() if T > 1 else None
    y2, am, al = vqv.vqv_qgemm_verify(d["x"], d["wq"], d["scales"], d["biases"], dt, B, T,
                                      group=group)
    torch.cuda.synchronize()
    y2_np = y2.cpu().numpy()
    assert_close(y2_np, ref, act, what + " (fused call)")
    ra, rl = verify_ref(y2_np, draft, B, T)
    np.testing.assert_array_equal(am.cpu().numpy(), ra, err_msg=what)
    np.testing.assert_array_equal(al.cpu().numpy(), rl, err_msg=what)

    draft_len = rng.integers(-1, T + 1, size=B).astype(np.int32)
    lt = torch.from_numpy(draft_len).cuda()
    y3, am3, al3, mg3 = vqv.vqv_qgemm_verify_ex(d["x"], d["wq"], d["scales"], d["biases"], dt,
                                                B, T, draft_len=lt, group=group)
    torch.cuda.synchronize()
    y3_np = y3.cpu().numpy()
    assert_close(y3_np, ref, act, what + " (fused call with margins)")
    ra, rl, rm = verify_ref(y3_np, draft, B, T, draft_len=draft_len, margin=True)
    np.testing.assert_array_equal(am3.cpu().numpy(), ra, err_msg=what)
    np.testing.assert_array_equal(al3.cpu().numpy(), rl, err_msg=what)
    np.testing.assert_array_equal(bits(mg3.cpu().numpy()), bits(rm), err_msg=what)

    if N % 2 == 0:
        h = vqv.vqv_qgemm_swiglu(d["x"], d["wq"], d["scales"], d["biases"], group=group)
        torch.cuda.synchronize()
        g, u = ref[:, :N // 2], ref[:, N // 2:]
        assert_swiglu_close(h.cpu().numpy(), g, u, silu_ref(g) * u, act, what + " (SwiGLU)")

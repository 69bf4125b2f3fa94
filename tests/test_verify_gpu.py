"""GPU parity of vqv_verify against the CPU oracle (through the C ABI).

Verify alone is fed the same fp32 logits on both sides and must match bit
for bit. End to end (GPU qgemm -> GPU verify against fp64 oracle -> oracle
verify) the argmax is exact where the oracle's top-1/top-2 gap exceeds 1e-3;
near ties accept any index within 1e-3 of the maximum, and the accept length
must then equal the oracle walk over the GPU's own argmax.
"""

import numpy as np
import pytest
import torch

import gen
from oracle import accept_walk_ref, argmax_ref, qgemm_ref, verify_ref
from tests.devutil import sha, to_device, top2_gap

pytestmark = pytest.mark.gpu

NEAR_TIE = 1e-3


@pytest.fixture(scope="module")
def vqv():
    import w4_gemm_vqv_amd as v
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    v.lib()
    return v


def gpu_verify(vqv, logits: np.ndarray, draft, B, T):
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    d = None if draft is None else torch.from_numpy(np.ascontiguousarray(draft, np.int32)).cuda()
    a, acc = vqv.vqv_verify(lg, d, B, T)
    torch.cuda.synchronize()
    return a.cpu().numpy(), acc.cpu().numpy()


def check_exact(vqv, logits, draft, B, T):
    a, acc = gpu_verify(vqv, logits, draft, B, T)
    ra, racc = verify_ref(logits, draft, B, T)
    np.testing.assert_array_equal(a, ra)
    np.testing.assert_array_equal(acc, racc)
    return a, acc


@pytest.mark.parametrize("B,T,N", [(1, 8, 1024), (4, 16, 5000), (1, 1, 7), (3, 5, 1),
                                   (2, 8, 4097), (1, 8, 151936), (4, 16, 151936), (64, 2, 333),
                                   (1, 64, 8193), (7, 3, 12289)])
def test_random_logits_bit_exact(vqv, B, T, N):
    rng = np.random.default_rng(B * 100 + T * 10 + N)
    logits = rng.standard_normal((B * T, N)).astype(np.float32)
    a_ref = np.array([argmax_ref(r) for r in logits])
    L = rng.integers(0, T, size=B)
    draft = gen.make_drafts(a_ref, B, T, N, seed=N, accept=L) if T > 1 else None
    a, acc = check_exact(vqv, logits, draft, B, T)
    if T > 1:
        np.testing.assert_array_equal(acc, L)


def test_planted_ties_lowest_index(vqv):
    """Equal maxima in different chunks, lanes and waves: lowest index wins."""
    N, T = 20000, 8
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((T, N)).astype(np.float32)
    spots = [(0, [5, 17000]), (1, [4095, 4096]), (2, [19999, 0]), (3, [300, 301, 302]),
             (4, [8191, 12288, 16384]), (5, [63, 64]), (6, [1, 19998]), (7, [2048, 10])]
    for r, idx in spots:
        logits[r, idx] = 9.5
    a, _ = check_exact(vqv, logits, np.zeros((1, T - 1), np.int32), 1, T)
    assert a.tolist() == [min(i) for _, i in spots]


def test_nan_inf_signed_zero(vqv):
    N = 9000
    inf, nan = np.float32(np.inf), np.float32(np.nan)
    rows = np.full((10, N), -5.0, dtype=np.float32)
    rows[0, [100, 8000]] = nan            # first NaN
    rows[1, [7000]] = nan; rows[1, 10] = inf   # NaN beats +inf
    rows[2, [4500, 4600]] = inf           # first +inf
    rows[3, :] = -inf                     # all -inf -> 0
    rows[4, :] = -0.0; rows[4, 5000] = 0.0   # -0 and +0 tie -> 0
    rows[5, :] = -1.0; rows[5, 6000] = 0.0; rows[5, 50] = -0.0  # -0 at 50 ties +0 at 6000
    rows[6, :] = -inf; rows[6, 8999] = -3.0
    rows[7, :] = np.float32(3.4e38); rows[7, 1] = inf
    rows[8, 4096] = nan; rows[8, 4095] = inf
    rows[9, :] = np.float32(1e-45); rows[9, 2] = np.float32(3e-45)  # denormals
    a, _ = check_exact(vqv, rows, np.zeros((1, 9), np.int32), 1, 10)
    assert a.tolist() == [100, 7000, 4500, 0, 0, 50, 8999, 1, 4096, 2]


def test_walk_cases(vqv):
    T, N = 8, 3000
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((T, N)).astype(np.float32)
    a = np.array([argmax_ref(r) for r in logits])
    cases = {"all": a[:7].copy(), "first_miss": np.r_[a[0] + 1, a[1:7]]}
    for j in range(7):
        d = a[:7].copy()
        d[j] = (a[j] + 1) % N
        cases[f"miss_{j}"] = d
    oor = a[:7].copy()
    oor[3] = -1
    cases["negative_id"] = oor
    oor2 = a[:7].copy()
    oor2[0] = N + 5
    cases["id_beyond_N"] = oor2
    expect = {"all": 7, "first_miss": 0, "negative_id": 3, "id_beyond_N": 0}
    expect.update({f"miss_{j}": j for j in range(7)})
    for k, d in cases.items():
        _, acc = check_exact(vqv, logits, d[None, :].astype(np.int32), 1, T)
        assert acc[0] == expect[k], k


def test_identical_sequences_control(vqv):
    B, T, N = 8, 16, 4000
    rng = np.random.default_rng(3)
    one = rng.standard_normal((T, N)).astype(np.float32)
    a = np.array([argmax_ref(r) for r in one])
    d = np.tile(np.r_[a[:11], (a[11] + 7) % N, a[12:15]], (B, 1)).astype(np.int32)
    _, acc = check_exact(vqv, np.concatenate([one] * B), d, B, T)
    assert acc.tolist() == [11] * B


def test_outputs_exactly_sized(vqv):
    """argmax and accept_len are written in place; guard words stay intact."""
    B, T, N = 2, 4, 100
    logits = torch.randn(B * T, N, device="cuda")
    draft = torch.zeros(B, T - 1, dtype=torch.int32, device="cuda")
    buf = torch.full((B * T + 16,), -77, dtype=torch.int32, device="cuda")
    abuf = torch.full((B + 16,), -77, dtype=torch.int32, device="cuda")
    vqv.vqv_verify(logits, draft, B, T, argmax=buf[8:8 + B * T], accept_len=abuf[8:8 + B])
    torch.cuda.synchronize()
    bb, ab = buf.cpu().numpy(), abuf.cpu().numpy()
    assert (bb[:8] == -77).all() and (bb[8 + B * T:] == -77).all()
    assert (ab[:8] == -77).all() and (ab[8 + B:] == -77).all()
    np.testing.assert_array_equal(bb[8:8 + B * T], logits.argmax(dim=1).cpu().numpy())


def test_deterministic(vqv):
    rng = np.random.default_rng(4)
    lg = torch.from_numpy(rng.standard_normal((64, 151936)).astype(np.float32)).cuda()
    d = torch.from_numpy(rng.integers(0, 151936, size=(4, 15)).astype(np.int32)).cuda()
    hs = set()
    for _ in range(3):
        a, acc = vqv.vqv_verify(lg, d, 4, 16)
        torch.cuda.synchronize()
        hs.add(sha(a) + sha(acc))
    assert len(hs) == 1


# ---------------------------------------------------------------- end to end


def e2e(vqv, c, M, B, T, accept=None, force_first=None):
    d = to_device(c)
    y = vqv.vqv_qgemm(d["x"][:M].contiguous(), d["wq"], d["scales"], d["biases"])
    torch.cuda.synchronize()
    y_ref = qgemm_ref(c["x"][:M], c["act"], c["wq"], c["scales"], c["biases"])
    a_ref = np.array([argmax_ref(r) for r in y_ref])
    draft = gen.make_drafts(a_ref, B, T, c["N"], seed=c["seed"], accept=accept,
                            force_first=force_first)
    a, acc = vqv.vqv_verify(y, torch.from_numpy(draft).cuda(), B, T)
    torch.cuda.synchronize()
    a, acc = a.cpu().numpy(), acc.cpu().numpy()
    y_gpu = y.cpu().numpy()
    # verify alone, same fp32 logits: bit-exact
    ra32, racc32 = verify_ref(y_gpu, draft, B, T)
    np.testing.assert_array_equal(a, ra32)
    np.testing.assert_array_equal(acc, racc32)
    # against the fp64 oracle, with the near-tie rule
    for r in range(B * T):
        if top2_gap(y_ref[r]) > NEAR_TIE:
            assert a[r] == a_ref[r], (r, a[r], a_ref[r])
        else:
            assert y_ref[r, a[r]] >= y_ref[r].max() - NEAR_TIE, r
    for b in range(B):
        rows = range(b * T, b * T + T)
        L_ref = accept_walk_ref(a_ref[b * T:(b + 1) * T], draft[b], T)
        walked = [r for r in rows][:min(L_ref, T - 2) + 1]
        if all(top2_gap(y_ref[r]) > NEAR_TIE for r in walked):
            assert acc[b] == L_ref, (b, acc[b], L_ref)
        else:
            assert acc[b] == accept_walk_ref(a[b * T:(b + 1) * T], draft[b], T)
    return a, acc, draft


def test_e2e_tiny(vqv):
    c = gen.make_config("tiny")
    a, acc, _ = e2e(vqv, c, 8, 1, 8, force_first=3)
    assert acc[0] >= 3


@pytest.fixture(scope="module")
def vocab_cfg():
    return gen.make_config("vocab_verify")


@pytest.mark.parametrize("L", range(8))
def test_e2e_vocab_all_accept_lengths(vqv, vocab_cfg, L):
    _, acc, _ = e2e(vqv, vocab_cfg, 8, 1, 8, accept=np.array([L]))
    assert acc[0] == L


def test_e2e_batched(vqv):
    c = gen.make_config("batched_vocab")
    L = gen.accept_lengths(c["seed"], 4, 16)
    _, acc, _ = e2e(vqv, c, 64, 4, 16, accept=L)
    np.testing.assert_array_equal(acc, L)

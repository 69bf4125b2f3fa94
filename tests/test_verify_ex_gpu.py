"""GPU parity of the verify extras through the C ABI: per-sequence valid
draft counts (draft_len) and the top-1 minus top-2 margin of each row.

vqv_verify_ex is fed the same fp32 logits as the oracle's verify_ref and must
match it bit for bit: argmax, accept_len and margin (every NaN counts as one
NaN). vqv_qgemm_verify_ex must equal vqv_qgemm followed by vqv_verify_ex on
every projection kernel's fused epilogue (1..64 rows), and the oracle's
verify of the GPU's own logits.
"""

import numpy as np
import pytest
import torch

import gen
from oracle import argmax_ref, verify_ref
from tests.devutil import to_device

pytestmark = pytest.mark.gpu

NAN_BITS = np.uint32(0x7FC00000)


@pytest.fixture(scope="module")
def vqv():
    import w4_gemm_vqv_amd as v
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    v.lib()
    return v


def bits(m: np.ndarray) -> np.ndarray:
    """fp32 bit patterns with every NaN folded onto one pattern."""
    m = np.asarray(m, dtype=np.float32)
    return np.where(np.isnan(m), NAN_BITS, m.view(np.uint32))


def dev_i32(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def verify_ex(vqv, logits, draft, B, T, draft_len):
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    a, acc, m = vqv.vqv_verify_ex(lg, dev_i32(draft), B, T, draft_len=dev_i32(draft_len))
    torch.cuda.synchronize()
    return a.cpu().numpy(), acc.cpu().numpy(), m.cpu().numpy()


def check_exact(vqv, logits, draft, B, T, draft_len):
    a, acc, m = verify_ex(vqv, logits, draft, B, T, draft_len)
    ra, racc, rm = verify_ref(logits, draft, B, T, draft_len=draft_len, margin=True)
    np.testing.assert_array_equal(a, ra)
    np.testing.assert_array_equal(acc, racc)
    np.testing.assert_array_equal(bits(m), bits(rm))
    return a, acc, m


@pytest.mark.parametrize("B,T,N", [(1, 8, 1024), (4, 16, 5000), (1, 1, 7), (3, 5, 1),
                                   (2, 8, 4097), (1, 8, 151936), (4, 16, 151936), (64, 2, 333),
                                   (1, 64, 8193), (7, 3, 12289)])
def test_random_logits_bit_exact(vqv, B, T, N):
    rng = np.random.default_rng(B * 1000 + T * 10 + N)
    logits = rng.standard_normal((B * T, N)).astype(np.float32)
    a_ref = np.array([argmax_ref(r) for r in logits])
    L = rng.integers(0, T, size=B)
    draft = gen.make_drafts(a_ref, B, T, N, seed=N + 1, accept=L) if T > 1 else None
    dl = rng.integers(-2, T + 3, size=B).astype(np.int32)
    _, acc, _ = check_exact(vqv, logits, draft, B, T, dl)
    np.testing.assert_array_equal(acc, np.minimum(L, np.clip(dl, 0, T - 1)))


def test_without_draft_len_matches_verify(vqv):
    """draft_len NULL walks all T-1 drafts, exactly as vqv_verify."""
    B, T, N = 3, 8, 3000
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((B * T, N)).astype(np.float32)
    a_ref = np.array([argmax_ref(r) for r in logits])
    draft = gen.make_drafts(a_ref, B, T, N, seed=5, accept=np.array([7, 0, 4]))
    a, acc, m = check_exact(vqv, logits, draft, B, T, None)
    lg = torch.from_numpy(logits).cuda()
    a0, acc0 = vqv.vqv_verify(lg, dev_i32(draft), B, T)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a0.cpu().numpy(), a)
    np.testing.assert_array_equal(acc0.cpu().numpy(), acc)
    assert acc.tolist() == [7, 0, 4]


def test_draft_len_edges(vqv):
    """Every draft matches; draft_len alone decides the walk (clamped to 0..T-1)."""
    T, N = 8, 2048
    lens = [-5, 0, 1, 3, 6, 7, 8, 1 << 30]
    B = len(lens)
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((B * T, N)).astype(np.float32)
    a_ref = np.array([argmax_ref(r) for r in logits])
    draft = gen.make_drafts(a_ref, B, T, N, seed=2, accept=np.full(B, T - 1))
    _, acc, _ = check_exact(vqv, logits, draft, B, T, np.array(lens, np.int32))
    assert acc.tolist() == [0, 0, 1, 3, 6, 7, 7, 7]


def test_margin_special_rows(vqv):
    N = 9000
    inf, nan = np.float32(np.inf), np.float32(np.nan)
    rows = np.full((16, N), -5.0, dtype=np.float32)
    rows[0, [3, 8500]] = 2.0                      # tie in different chunks: 0
    rows[1, 4000] = 0.0; rows[1, 4100] = -0.0     # -0 ties +0 (rest negative): 0
    rows[2, [10, 8999]] = inf                     # two +inf: 0
    rows[3, 77] = inf                             # +inf over finite: inf
    rows[4, 6000] = nan                           # NaN: NaN
    rows[5, :] = -inf                             # all -inf: tie, 0
    rows[6, :] = -3e38; rows[6, 1] = 3e38         # difference overflows: inf
    rows[7, 5] = 1.5; rows[7, 4096] = 1.25        # exact 0.25
    rows[8, 100] = np.float32(2.8e-45); rows[8, :100] = -0.0; rows[8, 101:] = np.float32(1.4e-45)
    rows[9, 0] = 1.0; rows[9, 1] = np.nextafter(np.float32(1.0), np.float32(0.0))  # one ulp
    rows[10, :] = -2.0; rows[10, [4095, 4096]] = -1.0  # tie across a chunk edge: 0
    rows[11, :] = np.linspace(-1, 1, N, dtype=np.float32)
    rows[12, 8191] = 7.0; rows[12, 8190] = 6.0    # best and second in one lane block
    rows[13, 0] = 1e-3; rows[13, 1] = -1e-3       # others -5
    rows[14, :] = 0.0                             # all zeros: 0
    rows[15, 123] = 4.0; rows[15, 124] = nan; rows[15, 125] = inf
    check_exact(vqv, rows, np.zeros((2, 7), np.int32), 2, 8, np.array([7, 7], np.int32))


def test_margin_one_column(vqv):
    """N == 1: no second value, +inf."""
    logits = np.array([[1.0], [-2.0], [np.nan], [0.0]], dtype=np.float32)
    _, _, m = check_exact(vqv, logits, np.zeros((1, 3), np.int32), 1, 4, None)
    assert np.isposinf(m[[0, 1, 3]]).all() and np.isnan(m[2])


# ------------------------------------------------- projection + verify extras


def case(M, K, N, act, seed):
    rng = np.random.default_rng(seed)
    wq, s, b = gen.make_weights(rng, N, K)
    x = gen.make_x(rng, M, K, act, 1.0, None)
    return dict(M=M, K=K, N=N, act=act, wq=wq, scales=s, biases=b, x=x, seed=seed)


def compare_fused(vqv, c, B, T, accept=None, draft_len=None, want_y=True, ws=None):
    d = to_device(c)
    N = c["N"]
    rng = np.random.default_rng(c["seed"] + 1)
    if accept is None:
        accept = rng.integers(0, T, size=B)
    if draft_len is None:
        draft_len = rng.integers(-1, T + 2, size=B).astype(np.int32)
    y1 = vqv.vqv_qgemm(d["x"], d["wq"], d["scales"], d["biases"])
    torch.cuda.synchronize()
    y_np = y1.cpu().numpy()
    a_gpu = np.array([argmax_ref(r) for r in y_np])
    draft = gen.make_drafts(a_gpu, B, T, N, seed=c["seed"], accept=accept)
    dt, lt = dev_i32(draft) if T > 1 else None, dev_i32(draft_len)
    a1, l1, m1 = vqv.vqv_verify_ex(y1, dt, B, T, draft_len=lt)
    y2, a2, l2, m2 = vqv.vqv_qgemm_verify_ex(d["x"], d["wq"], d["scales"], d["biases"], dt, B, T,
                                            draft_len=lt, want_y=want_y, workspace=ws)
    torch.cuda.synchronize()
    if want_y:
        assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)), \
            "fused y differs from vqv_qgemm"
    assert torch.equal(a1, a2)
    assert torch.equal(l1, l2), (l1.cpu().numpy(), l2.cpu().numpy())
    np.testing.assert_array_equal(bits(m2.cpu().numpy()), bits(m1.cpu().numpy()))
    ra, rl, rm = verify_ref(y_np, draft, B, T, draft_len=draft_len, margin=True)
    np.testing.assert_array_equal(a2.cpu().numpy(), ra)
    np.testing.assert_array_equal(l2.cpu().numpy(), rl)
    np.testing.assert_array_equal(bits(m2.cpu().numpy()), bits(rm))
    if T > 1:
        np.testing.assert_array_equal(l2.cpu().numpy(),
                                      np.minimum(accept, np.clip(draft_len, 0, T - 1)))
    return y2, a2, l2, m2


@pytest.mark.parametrize("M,K,N,act,B,T", [
    (8, 512, 1024, "bf16", 1, 8), (8, 512, 1024, "fp16", 2, 4), (4, 1280, 3000, "bf16", 1, 4),
    (1, 64, 17, "bf16", 1, 1), (8, 192, 999, "fp16", 8, 1), (5, 320, 5000, "bf16", 1, 5),
    (8, 2560, 17408, "bf16", 1, 8), (6, 5120, 1000, "bf16", 3, 2), (8, 640, 12000, "fp16", 4, 2),
    (2, 128, 1, "bf16", 1, 2), (8, 512, 70000, "fp16", 2, 4), (3, 1024, 66001, "bf16", 1, 3),
])
def test_fused_ex_matches_separate(vqv, M, K, N, act, B, T):
    compare_fused(vqv, case(M, K, N, act, seed=M * 11 + K + N), B, T)


@pytest.mark.parametrize("M,K,N,act,B,T", [
    # 16-row kernel, general kernel (large K, fp32), batched vocabulary kernel,
    # whole-tile kernel with 16 rows and with two row sets
    (16, 512, 1000, "bf16", 1, 16), (64, 256, 700, "fp16", 4, 16), (32, 2560, 5000, "bf16", 2, 16),
    (16, 5120, 3000, "bf16", 2, 8), (48, 3072, 900, "fp16", 3, 16), (8, 512, 700, "fp32", 1, 8),
    (64, 512, 2000, "fp32", 4, 16), (8, 8192, 300, "bf16", 1, 8),
    (64, 512, 40000, "bf16", 4, 16), (32, 1024, 151936, "fp16", 2, 16), (20, 256, 30000, "bf16", 4, 5),
    (16, 1024, 66001, "bf16", 1, 16), (32, 512, 200000, "fp16", 4, 8),
])
def test_rows_beyond_8_ex_matches_separate(vqv, M, K, N, act, B, T):
    compare_fused(vqv, case(M, K, N, act, seed=M + K + N + 3), B, T)


@pytest.mark.parametrize("M,K,N,act,B,T", [
    (8, 5120, 17408, "bf16", 1, 8), (8, 512, 70000, "fp16", 1, 8), (64, 512, 40000, "bf16", 4, 16),
    (16, 512, 1000, "bf16", 2, 8), (16, 5120, 3000, "bf16", 1, 16), (8, 512, 700, "fp32", 1, 8),
    (32, 512, 200000, "bf16", 2, 16), (4, 1280, 3000, "fp16", 2, 2),
])
def test_fused_ex_nan_columns(vqv, M, K, N, act, B, T):
    """NaN scales in three columns make those logits NaN in every row: each
    kernel family's epilogue must report the first of them as the argmax and a
    NaN margin, as the separate path and the oracle do."""
    c = case(M, K, N, act, seed=M * 5 + K + N)
    s = c["scales"].copy()
    cols = sorted({N // 3, N // 3 + 17, N - 2})
    for col in cols:
        s[col, 0] = np.uint16(0x7E00)                # fp16 NaN
    c["scales"] = s
    _, a, _, m = compare_fused(vqv, c, B, T)
    assert (a.cpu().numpy() == cols[0]).all()
    assert np.isnan(m.cpu().numpy()).all()


def test_fused_ex_without_logits_and_reused_workspace(vqv):
    c = case(8, 2560, 20000, "fp16", seed=15)
    need = vqv.vqv_qgemm_verify_workspace_bytes(8, 2560, 20000, 64, vqv.VQV_FP16)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    for L, dl in [(3, 3), (3, 1), (2, 3), (0, 0), (3, -1), (1, 100)]:
        y, _, l, _ = compare_fused(vqv, c, 2, 4, accept=np.array([L, 3]),
                                   draft_len=np.array([dl, 2], np.int32), want_y=False, ws=ws)
        assert y is None
        assert l.cpu().tolist() == [min(L, max(dl, 0), 3), 2]


def test_full_size_target_ex(vqv):
    compare_fused(vqv, gen.make_config("target"), 1, 8, accept=np.array([6]),
                  draft_len=np.array([4], np.int32))


def test_full_size_vocab_ex(vqv):
    compare_fused(vqv, gen.make_config("vocab_verify"), 1, 8, accept=np.array([7]),
                  draft_len=np.array([7], np.int32))


def test_full_size_batched_ex(vqv):
    compare_fused(vqv, gen.make_config("batched_vocab"), 4, 16,
                  accept=np.array([15, 9, 0, 4]), draft_len=np.array([15, 12, 3, 2], np.int32))

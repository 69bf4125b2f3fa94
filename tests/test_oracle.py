"""Pins for the CPU oracle.

Each check reaches the expected value by a route that does not reuse the
oracle's code: exact rational brute force with its own bit decoding, closed
forms over group sums, numpy's argmax, and hand-built walks. A plausible slip
in the oracle (a dropped bias term, a swapped nibble, a wrong group index, a
transposed operand, a sign error, a tie broken the wrong way) fails at least
one of them.
"""

import struct
from fractions import Fraction

import numpy as np
import pytest

import gen
from oracle import (margin_ref, accept_walk_ref, argmax_ref, decode_act, dequantize, qgemm_ref,
                    qgemm_swiglu_ref, silu_ref, swiglu_ref, unpack_codes, verify_ref)

# ---------------------------------------------------------------- brute force


def _f16(bits: int) -> Fraction:
    return Fraction(struct.unpack("<e", int(bits).to_bytes(2, "little"))[0])


def _bf16(bits: int) -> Fraction:
    return Fraction(struct.unpack("<f", (int(bits) << 16).to_bytes(4, "little"))[0])


def _act(x, act, m, k) -> Fraction:
    if act == "bf16":
        return _bf16(x[m][k])
    if act == "fp16":
        return _f16(x[m][k])
    return Fraction(float(x[m][k]))


def _brute_qgemm(x, act, wq, scales, biases, M, K, N, group=64):
    """Exact rational y[m][n] = sum_k x*(s*q + b), with nothing shared with the
    oracle: nibbles read one at a time, fp16/bf16 decoded by struct."""
    xs, wb, sb, bb = x.tolist(), wq.tolist(), scales.tolist(), biases.tolist()
    y = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        for k in range(K):
            byte = wb[n][k // 2]
            q = (byte & 15) if k % 2 == 0 else (byte >> 4)
            w = _f16(sb[n][k // group]) * q + _f16(bb[n][k // group])
            for m in range(M):
                y[m][n] += _act(xs, act, m, k) * w
    return y


@pytest.mark.parametrize("act", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("M,K,N,seed", [(1, 64, 1, 0), (2, 128, 3, 1), (3, 192, 5, 2),
                                         (3, 64, 4, 3)])
def test_brute_force_tiny(act, M, K, N, seed):
    rng = np.random.default_rng(seed)
    wq, s, b = gen.make_weights(rng, N, K)
    x = gen.make_x(rng, M, K, act)
    y = qgemm_ref(x, act, wq, s, b)
    exact = _brute_qgemm(x, act, wq, s, b, M, K, N)
    for m in range(M):
        for n in range(N):
            e = float(exact[m][n])
            assert abs(y[m, n] - e) <= 1e-12 * (1.0 + abs(e)), (m, n, y[m, n], e)


@pytest.mark.parametrize("act", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("M,K,N,seed", [(1, 128, 2, 20), (2, 384, 3, 21)])
def test_brute_force_tiny_group128(act, M, K, N, seed):
    """Group 128: one scale and bias per 128 contiguous k."""
    rng = np.random.default_rng(seed)
    wq, s, b = gen.make_weights(rng, N, K, group=128)
    assert s.shape == (N, K // 128)
    x = gen.make_x(rng, M, K, act)
    y = qgemm_ref(x, act, wq, s, b, group=128)
    exact = _brute_qgemm(x, act, wq, s, b, M, K, N, group=128)
    for m in range(M):
        for n in range(N):
            e = float(exact[m][n])
            assert abs(y[m, n] - e) <= 1e-12 * (1.0 + abs(e)), (m, n, y[m, n], e)


@pytest.mark.parametrize("act", ["bf16", "fp32"])
@pytest.mark.parametrize("M,K,N,seed", [(1, 64, 2, 24), (2, 192, 3, 25)])
def test_brute_force_tiny_group32(act, M, K, N, seed):
    """Group 32: one scale and bias per 32 contiguous k."""
    rng = np.random.default_rng(seed)
    wq, s, b = gen.make_weights(rng, N, K, group=32)
    assert s.shape == (N, K // 32)
    x = gen.make_x(rng, M, K, act)
    y = qgemm_ref(x, act, wq, s, b, group=32)
    exact = _brute_qgemm(x, act, wq, s, b, M, K, N, group=32)
    for m in range(M):
        for n in range(N):
            e = float(exact[m][n])
            assert abs(y[m, n] - e) <= 1e-12 * (1.0 + abs(e)), (m, n, y[m, n], e)


def test_group64_is_group32_with_equal_halves():
    """Group 32 with both halves of every 64-group sharing one entry is group 64."""
    rng = np.random.default_rng(26)
    wq, s, b = gen.make_weights(rng, 7, 384, group=64)
    x = gen.make_x(rng, 3, 384, "fp16")
    y64 = qgemm_ref(x, "fp16", wq, s, b, group=64)
    y32 = qgemm_ref(x, "fp16", wq, np.repeat(s, 2, axis=1), np.repeat(b, 2, axis=1), group=32)
    np.testing.assert_allclose(y32, y64, rtol=1e-13, atol=1e-13)


def test_dequantize_group32_boundary():
    """k=31 and k=32 sit in different 32-groups."""
    wq = np.full((1, 32), 0x22, dtype=np.uint8)  # every code 2
    s = np.array([[np.float16(0.5).view(np.uint16), np.float16(4.0).view(np.uint16)]],
                 dtype=np.uint16)
    b = np.array([[np.float16(1.0).view(np.uint16), np.float16(-2.0).view(np.uint16)]],
                 dtype=np.uint16)
    w = dequantize(wq, s, b, group=32)
    assert w[0, 0] == 2.0 and w[0, 31] == 2.0 and w[0, 32] == 6.0 and w[0, 63] == 6.0


def test_group128_is_group64_with_each_entry_twice():
    """A 128-group's scale and bias cover both of its 64-halves."""
    rng = np.random.default_rng(22)
    wq, s, b = gen.make_weights(rng, 9, 512, group=128)
    x = gen.make_x(rng, 4, 512, "bf16")
    y128 = qgemm_ref(x, "bf16", wq, s, b, group=128)
    y64 = qgemm_ref(x, "bf16", wq, np.repeat(s, 2, axis=1), np.repeat(b, 2, axis=1), group=64)
    np.testing.assert_allclose(y128, y64, rtol=1e-13, atol=1e-13)


def test_group_size_must_match_table():
    rng = np.random.default_rng(23)
    wq, s, b = gen.make_weights(rng, 3, 256, group=64)
    with pytest.raises(ValueError):
        dequantize(wq, s, b, group=128)
    with pytest.raises(ValueError):
        dequantize(wq[:, :96], s[:, :3], b[:, :3], group=128)   # K = 192


# ---------------------------------------------------------------- closed forms


def _group_sums(xd, K):
    return xd.reshape(xd.shape[0], K // 64, 64).sum(axis=2)


def _rand(seed, M=3, K=256, N=7, act="bf16"):
    rng = np.random.default_rng(seed)
    wq, s, b = gen.make_weights(rng, N, K)
    x = gen.make_x(rng, M, K, act)
    return x, wq, s, b


def _f16arr(bits):
    return np.array([[float(_f16(v)) for v in row] for row in bits.tolist()])


def test_zero_codes_give_bias_times_group_sums():
    """All-zero codes: y[m,n] = sum_g b[n,g] * sum_{k in g} x[m,k]."""
    x, wq, s, b = _rand(10)
    wq[:] = 0
    K = wq.shape[1] * 2
    xd = decode_act(x, "bf16")
    expect = _group_sums(xd, K) @ _f16arr(b).T
    np.testing.assert_allclose(qgemm_ref(x, "bf16", wq, s, b), expect, rtol=1e-12,
                               atol=1e-12)


@pytest.mark.parametrize("c", [1, 7, 15])
def test_constant_code(c):
    """Every code equal to c: y = sum_g (c*s + b) * xsum_g."""
    x, wq, s, b = _rand(11 + c)
    wq[:] = c | (c << 4)
    K = wq.shape[1] * 2
    xd = decode_act(x, "bf16")
    expect = _group_sums(xd, K) @ (c * _f16arr(s) + _f16arr(b)).T
    np.testing.assert_allclose(qgemm_ref(x, "bf16", wq, s, b), expect, rtol=1e-12,
                               atol=1e-12)


def test_one_hot_rows_read_single_weights():
    """x = e_k reads one weight: y[n] = s[n,k//64]*q[n,k] + b[n,k//64], with
    the nibble taken from byte k//2 (low nibble for even k)."""
    _, wq, s, b = _rand(20, K=192, N=5)
    K = 192
    ks = [0, 1, 2, 63, 64, 65, 127, 128, 191]
    x = np.zeros((len(ks), K), dtype=np.float32)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    y = qgemm_ref(x, "fp32", wq, s, b)
    sf, bf = _f16arr(s), _f16arr(b)
    for i, k in enumerate(ks):
        for n in range(5):
            byte = int(wq[n, k // 2])
            q = (byte >> (4 * (k % 2))) & 15
            assert y[i, n] == sf[n, k // 64] * q + bf[n, k // 64]


def test_nibble_order_hand_case():
    """Hand case: byte 0 = 0x21, s = 1, b = 0. k=0 reads the low nibble (1),
    k=1 the high nibble (2); a swapped unpack gives 2 and 1."""
    wq = np.zeros((1, 32), dtype=np.uint8)
    wq[0, 0] = 0x21
    one = np.float16(1.0).view(np.uint16)
    s = np.full((1, 1), one, dtype=np.uint16)
    b = np.zeros((1, 1), dtype=np.uint16)
    x = np.zeros((2, 64), dtype=np.float32)
    x[0, 0] = 1.0
    x[1, 1] = 1.0
    assert qgemm_ref(x, "fp32", wq, s, b)[:, 0].tolist() == [1.0, 2.0]
    assert unpack_codes(wq)[0, :3].tolist() == [1, 2, 0]


def test_all_ones_x():
    """x = 1 everywhere: y[n] = sum_g (s[n,g]*sum_{k in g} q + 64*b[n,g])."""
    _, wq, s, b = _rand(30, K=320, N=6)
    x = np.ones((1, 320), dtype=np.float32)
    q = np.array([[(byte >> sh) & 15 for byte in row for sh in (0, 4)]
                  for row in wq.tolist()], dtype=np.float64)
    qsum = q.reshape(6, 5, 64).sum(axis=2)
    expect = (_f16arr(s) * qsum + 64.0 * _f16arr(b)).sum(axis=1)
    np.testing.assert_allclose(qgemm_ref(x, "fp32", wq, s, b)[0], expect, rtol=1e-13)


def test_linear_in_x():
    rng = np.random.default_rng(40)
    wq, s, b = gen.make_weights(rng, 9, 256)
    # quarter-integer activations so that x1 + x2 is exact in float32
    x1 = (rng.integers(-64, 65, size=(2, 256)) / 4).astype(np.float32)
    x2 = (rng.integers(-64, 65, size=(2, 256)) / 4).astype(np.float32)
    y1 = qgemm_ref(x1, "fp32", wq, s, b)
    y2 = qgemm_ref(x2, "fp32", wq, s, b)
    np.testing.assert_allclose(qgemm_ref(x1 + x2, "fp32", wq, s, b), y1 + y2,
                               rtol=1e-12, atol=1e-12)
    # scaling x by a power of two scales y exactly
    np.testing.assert_array_equal(qgemm_ref(x1 * np.float32(4), "fp32", wq, s, b), 4 * y1)
    np.testing.assert_array_equal(qgemm_ref(-x1, "fp32", wq, s, b), -y1)
    np.testing.assert_allclose(qgemm_ref(np.concatenate([x1, x2]), "fp32", wq, s, b),
                               np.concatenate([y1, y2]), rtol=1e-13)


def test_group_permutation_invariance():
    """Permuting whole groups of k together with their scale/bias columns
    leaves y unchanged (up to float64 summation order); permuting only the
    codes changes it (the group index matters)."""
    x, wq, s, b = _rand(50, K=384, N=4)
    perm = np.array([3, 0, 5, 1, 4, 2])
    wq_p = wq.reshape(4, 6, 32)[:, perm].reshape(4, 192)
    y = qgemm_ref(x, "bf16", wq, s, b)
    yp = qgemm_ref(x[:, (perm[:, None] * 64 + np.arange(64)).ravel()], "bf16", wq_p,
                   s[:, perm], b[:, perm])
    np.testing.assert_allclose(yp, y, rtol=1e-12, atol=1e-12)
    y_wrong = qgemm_ref(x[:, (perm[:, None] * 64 + np.arange(64)).ravel()], "bf16",
                        wq_p, s, b)
    assert not np.allclose(y_wrong, y)


def test_integer_exact_case_matches_integer_arithmetic():
    """s = 1, integer biases and integer x: y is an integer computed here with
    Python ints, and the float64 oracle must equal it exactly."""
    rng = np.random.default_rng(60)
    M, K, N = 4, 256, 6
    wq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = np.full((N, K // 64), np.float16(1.0).view(np.uint16), dtype=np.uint16)
    bint = rng.integers(-8, 1, size=(N, K // 64))
    b = bint.astype(np.float16).view(np.uint16)
    xint = rng.integers(-8, 9, size=(M, K))
    x = gen.f32_to_bf16_bits(xint.astype(np.float32))
    y = qgemm_ref(x, "bf16", wq, s, b)
    for m in range(M):
        for n in range(N):
            tot = 0
            for k in range(K):
                byte = int(wq[n, k // 2])
                q = (byte >> (4 * (k & 1))) & 15
                tot += int(xint[m, k]) * (q + int(bint[n, k // 64]))
            assert y[m, n] == tot


def test_decode_act_bit_patterns():
    assert decode_act(np.array([0x3F80, 0xC000, 0x0000, 0x8000], np.uint16), "bf16"
                      ).tolist() == [1.0, -2.0, 0.0, -0.0]
    assert decode_act(np.array([0x3C00, 0xC000, 0x7BFF], np.uint16), "fp16"
                      ).tolist() == [1.0, -2.0, 65504.0]


def test_dequantize_group_boundary():
    """k=63 and k=64 sit in different groups."""
    wq = np.full((1, 64), 0x11, dtype=np.uint8)  # every code 1
    s = np.array([[np.float16(2.0).view(np.uint16), np.float16(3.0).view(np.uint16)]],
                 dtype=np.uint16)
    b = np.array([[np.float16(-1.0).view(np.uint16), np.float16(0.5).view(np.uint16)]],
                 dtype=np.uint16)
    w = dequantize(wq, s, b)
    assert w[0, 63] == 1.0 and w[0, 64] == 3.5 and w[0, 0] == 1.0 and w[0, 127] == 3.5


def test_dequantize_group128_boundary():
    """k=127 and k=128 sit in different 128-groups; k=63 and k=64 share one."""
    wq = np.full((1, 128), 0x11, dtype=np.uint8)  # every code 1
    s = np.array([[np.float16(2.0).view(np.uint16), np.float16(3.0).view(np.uint16)]],
                 dtype=np.uint16)
    b = np.array([[np.float16(-1.0).view(np.uint16), np.float16(0.5).view(np.uint16)]],
                 dtype=np.uint16)
    w = dequantize(wq, s, b, group=128)
    assert w[0, 63] == 1.0 and w[0, 64] == 1.0 and w[0, 127] == 1.0
    assert w[0, 128] == 3.5 and w[0, 255] == 3.5


def test_chunking_and_column_subset_agree():
    x, wq, s, b = _rand(70, M=2, K=128, N=50)
    full = qgemm_ref(x, "bf16", wq, s, b, chunk=7)
    np.testing.assert_allclose(full, qgemm_ref(x, "bf16", wq, s, b, chunk=4096), rtol=1e-14)
    cols = [49, 0, 13, 13, 31]
    np.testing.assert_array_equal(qgemm_ref(x, "bf16", wq, s, b, cols=cols), full[:, cols])


# ---------------------------------------------------------------- argmax


def _scan_argmax(row):
    """Pure-Python scan: NaN wins (first one); otherwise strictly greater
    replaces, so the first maximum is kept."""
    best = 0
    for i, v in enumerate(row):
        if v != v:
            return i
        if v > row[best]:
            best = i
    return best


@pytest.mark.parametrize("seed", range(5))
def test_argmax_matches_numpy_on_random_rows(seed):
    rng = np.random.default_rng(seed)
    for _ in range(20):
        v = rng.standard_normal(int(rng.integers(1, 300))).astype(np.float32)
        assert argmax_ref(v) == int(np.argmax(v)) == _scan_argmax(v.tolist())


def test_argmax_ties_lowest_index():
    v = np.array([0.0, 3.0, 1.0, 3.0, 3.0], dtype=np.float32)
    assert argmax_ref(v) == 1 == int(np.argmax(v))
    v = np.full(1000, 2.5, dtype=np.float32)
    assert argmax_ref(v) == 0


def test_argmax_signed_zero_ties():
    v = np.array([-1.0, -0.0, 0.0, -2.0], dtype=np.float32)
    assert argmax_ref(v) == 1 == int(np.argmax(v))
    v = np.array([-1.0, 0.0, -0.0], dtype=np.float32)
    assert argmax_ref(v) == 1


def test_argmax_nan_and_inf():
    inf, nan = np.inf, np.nan
    cases = [
        [1.0, nan, 5.0, nan],  # first NaN
        [nan, inf],
        [1.0, inf, 2.0, inf],  # +inf is an ordinary maximum, first one
        [-inf, -inf, -inf],  # all -inf -> 0
        [-inf, -3.0, -inf],
        [3.0, -inf, inf, nan],
    ]
    for c in cases:
        v = np.array(c, dtype=np.float32)
        assert argmax_ref(v) == int(np.argmax(v)) == _scan_argmax(c), c


# ---------------------------------------------------------------- accept walk


def test_walk_hand_cases():
    T = 8
    a = np.array([5, 9, 2, 2, 7, 1, 0, 4])
    assert accept_walk_ref(a, a[:7], T) == 7  # all accepted
    d = a[:7].copy()
    d[0] = 6
    assert accept_walk_ref(a, d, T) == 0  # first draft misses
    for j in range(7):
        d = a[:7].copy()
        d[j] = a[j] + 1
        assert accept_walk_ref(a, d, T) == j  # miss at j
    assert accept_walk_ref(np.array([3]), np.array([], dtype=np.int32), 1) == 0  # T=1
    # a later match after a miss does not count
    d = a[:7].copy()
    d[2] = 100
    assert accept_walk_ref(a, d, T) == 2


def test_walk_tie_draft_is_higher_tied_index():
    """Row 0 ties at indices 2 and 5; the argmax is 2, so a draft of 5 misses."""
    T, N = 3, 8
    logits = np.zeros((T, N), dtype=np.float32)
    logits[0, [2, 5]] = 4.0
    logits[1, 6] = 1.0
    logits[2, 1] = 1.0
    a, acc = verify_ref(logits, np.array([[5, 6]], dtype=np.int32), 1, T)
    assert a.tolist() == [2, 6, 1] and acc.tolist() == [0]
    a, acc = verify_ref(logits, np.array([[2, 6]], dtype=np.int32), 1, T)
    assert acc.tolist() == [2]


def test_identical_sequences_control():
    rng = np.random.default_rng(5)
    T, N, B = 16, 300, 4
    one = rng.standard_normal((T, N)).astype(np.float32)
    logits = np.concatenate([one] * B)
    a1 = np.array([argmax_ref(r) for r in one])
    d = np.tile(np.concatenate([a1[:9], [a1[9] + 1], a1[10:15]]), (B, 1)).astype(np.int32)
    a, acc = verify_ref(logits, d, B, T)
    assert acc.tolist() == [9] * B
    assert a.tolist() == a1.tolist() * B


def test_verify_out_of_range_drafts_never_match():
    logits = np.eye(4, dtype=np.float32)
    a, acc = verify_ref(logits, np.array([[-1, 4, 2]], dtype=np.int32), 1, 4)
    assert a.tolist() == [0, 1, 2, 3] and acc.tolist() == [0]


def test_drafts_builder_realises_accept_lengths():
    """gen.make_drafts with accept=L yields exactly L under the oracle walk."""
    B, T, N = 4, 16, 1000
    rng = np.random.default_rng(3)
    a = rng.integers(0, N, size=B * T)
    L = gen.accept_lengths(9, B, T)
    d = gen.make_drafts(a, B, T, N, seed=9, accept=L)
    for b in range(B):
        assert accept_walk_ref(a[b * T:(b + 1) * T], d[b], T) == L[b]
    for L0 in range(T):
        d = gen.make_drafts(a, B, T, N, seed=1, accept=np.full(B, L0))
        assert all(accept_walk_ref(a[b * T:(b + 1) * T], d[b], T) == L0 for b in range(B))


# ---------------------------------------------------------------- margin


@pytest.mark.parametrize("seed", range(6))
def test_margin_matches_sorted_top_two(seed):
    """Rows with distinct values: the two largest from a library sort."""
    rng = np.random.default_rng(seed)
    for n in (2, 3, 17, 1000):
        v = rng.standard_normal(n).astype(np.float32)
        v = np.unique(v)  # distinct values (sorted); shuffle them back
        rng.shuffle(v)
        srt = np.sort(v)
        assert margin_ref(v) == np.float32(srt[-1]) - np.float32(srt[-2])


def test_margin_hand_cases():
    f = np.float32
    assert margin_ref(np.array([1, 3, 2], f)) == f(1.0)
    assert margin_ref(np.array([3, 3, 1], f)) == f(0.0)            # tied maximum
    assert margin_ref(np.array([-0.0, 0.0], f)) == f(0.0)          # signed zeros tie
    assert margin_ref(np.array([np.inf, np.inf, 1], f)) == f(0.0)  # tied +inf
    assert margin_ref(np.array([-np.inf, -np.inf], f)) == f(0.0)   # tied -inf
    assert margin_ref(np.array([np.inf, 1], f)) == f(np.inf)
    assert margin_ref(np.array([2, -np.inf], f)) == f(np.inf)
    assert margin_ref(np.array([5], f)) == f(np.inf)                # no competitor
    assert np.isnan(margin_ref(np.array([1, np.nan, 3], f)))
    assert margin_ref(np.array([-1, -4, -2], f)) == f(1.0)
    # fp32 rounding of the difference: 1 - 2^-30 is not representable
    assert margin_ref(np.array([1.0, 2.0 ** -30], f)) == f(1.0)


def test_margin_through_verify():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((6, 50)).astype(np.float32)
    a, acc, m = verify_ref(lg, np.zeros((2, 2), np.int32), 2, 3, margin=True)
    for r in range(6):
        top = np.sort(lg[r])[-2:]
        assert m[r] == np.float32(top[1]) - np.float32(top[0])


# ---------------------------------------------------------------- valid draft length


def test_walk_draft_len_caps_the_walk():
    a = np.array([5, 6, 7, 8, 9])
    d = np.array([5, 6, 7, 8])       # every draft matches: natural walk 4 (T=5)
    assert accept_walk_ref(a, d, 5) == 4
    assert [accept_walk_ref(a, d, 5, L) for L in range(6)] == [0, 1, 2, 3, 4, 4]
    assert accept_walk_ref(a, d, 5, -3) == 0      # clamped to 0
    assert accept_walk_ref(a, d, 5, 99) == 4      # clamped to T-1
    d2 = np.array([5, 0, 7, 8])      # miss at 1: the cap never extends a walk
    assert [accept_walk_ref(a, d2, 5, L) for L in range(5)] == [0, 1, 1, 1, 1]


def test_verify_draft_len_per_sequence():
    rng = np.random.default_rng(9)
    B, T, N = 3, 6, 40
    lg = rng.standard_normal((B * T, N)).astype(np.float32)
    a = np.array([int(np.argmax(r)) for r in lg])
    draft = np.stack([a[b * T:b * T + T - 1] for b in range(B)])  # full accept
    _, acc = verify_ref(lg, draft, B, T)
    assert acc.tolist() == [T - 1] * B
    _, acc = verify_ref(lg, draft, B, T, draft_len=np.array([0, 3, 5]))
    assert acc.tolist() == [0, 3, 5]


# ---------------------------------------------------------------- gate/up SwiGLU


def test_silu_closed_forms():
    """sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4; silu(0) = 0;
    silu(g) - silu(-g) = g; silu(g) -> g for large g."""
    ln3 = np.log(3.0)
    assert silu_ref(0.0) == 0.0
    assert abs(silu_ref(ln3) - 0.75 * ln3) <= 1e-15
    assert abs(silu_ref(-ln3) + 0.25 * ln3) <= 1e-15
    assert abs(silu_ref(np.log(1.0 / 3.0)) + 0.25 * ln3) <= 1e-15
    g = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(silu_ref(g) - silu_ref(-g), g, rtol=0, atol=1e-13)
    assert silu_ref(60.0) == 60.0            # sigmoid(60) rounds to 1 in float64
    assert -1e-20 < silu_ref(-60.0) < 0.0    # -60 * e^-60


def test_silu_against_library_logistic():
    """g * expit(g), scipy's logistic routine, on random and large values."""
    from scipy.special import expit
    rng = np.random.default_rng(5)
    g = np.concatenate([rng.standard_normal(1000) * 4, [-700.0, -40.0, 40.0, 700.0]])
    np.testing.assert_allclose(silu_ref(g), g * expit(g), rtol=1e-14, atol=1e-300)


def test_swiglu_halves_are_gate_then_up():
    """h = silu(gate) * up with the gate in the first half of the columns:
    an asymmetric hand case that a swapped or interleaved split fails."""
    y = np.array([[1.0, 2.0, -3.0, 5.0, 7.0, 0.5]])
    s1, s2 = 1.0 / (1.0 + np.exp(-1.0)), 2.0 / (1.0 + np.exp(-2.0))
    s3 = -3.0 / (1.0 + np.exp(3.0))
    np.testing.assert_allclose(swiglu_ref(y), [[s1 * 5.0, s2 * 7.0, s3 * 0.5]], rtol=1e-15)
    assert swiglu_ref(np.zeros((2, 4))).shape == (2, 2)
    with pytest.raises(ValueError):
        swiglu_ref(np.zeros((1, 3)))


@pytest.mark.parametrize("act", ["bf16", "fp16"])
def test_qgemm_swiglu_brute_force(act):
    """Exact rational gate and up columns, then silu by math.exp."""
    import math
    M, K, NH = 2, 128, 3
    rng = np.random.default_rng(12)
    wq, s, b = gen.make_weights(rng, 2 * NH, K)
    x = gen.make_x(rng, M, K, act)
    y = _brute_qgemm(x, act, wq, s, b, M, K, 2 * NH)
    h = qgemm_swiglu_ref(x, act, wq, s, b)
    for m in range(M):
        for j in range(NH):
            g, u = float(y[m][j]), float(y[m][NH + j])
            e = g / (1.0 + math.exp(-g)) * u
            assert abs(h[m, j] - e) <= 1e-12 * (1.0 + abs(e)), (m, j, h[m, j], e)


def test_qgemm_swiglu_column_subset():
    x, wq, s, b = _rand(21, M=4, K=192, N=10)
    full = qgemm_swiglu_ref(x, "bf16", wq, s, b)
    cols = [4, 0, 3]
    np.testing.assert_array_equal(qgemm_swiglu_ref(x, "bf16", wq, s, b, cols=cols),
                                  full[:, cols])


def test_qgemm_swiglu_zero_gate_and_zero_up():
    """Zero codes and zero biases in the gate half give h = 0 whatever the up
    half is; the same in the up half gives h = 0 too."""
    x, wq, s, b = _rand(22, M=3, K=128, N=8)
    for rows in (slice(0, 4), slice(4, 8)):
        wq2, b2 = wq.copy(), b.copy()
        wq2[rows] = 0
        b2[rows] = 0
        np.testing.assert_array_equal(qgemm_swiglu_ref(x, "bf16", wq2, s, b2),
                                      np.zeros((3, 4)))

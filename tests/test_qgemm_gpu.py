"""GPU parity of vqv_qgemm against the CPU oracle (through the C ABI).

Small cases compare every output; the full-size workloads compare sampled
columns (the oracle computes those one by one), in the launch configuration
the benchmark uses.
"""

import numpy as np
import pytest
import torch

import gen
from oracle import qgemm_ref
from tests.devutil import assert_close, sha, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vqv():
    import w4_gemm_vqv_amd as v
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    v.lib()  # fails loudly if the HIP library is missing
    return v


def run(vqv, c, M=None):
    d = to_device(c)
    x = d["x"] if M is None else d["x"][:M].contiguous()
    y = vqv.vqv_qgemm(x, d["wq"], d["scales"], d["biases"], group=c.get("group", 64))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def case(M, K, N, act, seed, sigma=1.0, real_rows=None, group=64):
    rng = np.random.default_rng(seed)
    wq, s, b = gen.make_weights(rng, N, K, group)
    x = gen.make_x(rng, M, K, act, sigma, real_rows)
    return dict(M=M, K=K, N=N, act=act, wq=wq, scales=s, biases=b, x=x, group=group)


# Shapes span several column tiles and work-group splits, ragged N tails,
# odd group counts (K/64 odd), and M across row-set boundaries.
SHAPES = [
    (8, 512, 1024), (8, 64, 3), (1, 128, 17), (4, 192, 65), (5, 320, 1000), (8, 1088, 129),
    (3, 5120, 200), (9, 256, 70), (16, 640, 300), (17, 128, 64), (32, 256, 96), (33, 384, 50),
    (64, 512, 130), (7, 4096, 64), (8, 8192, 77), (8, 16384, 40), (16, 16320, 33),
    (64, 2560, 96), (5, 5120, 1000),
    # Work-groups of several column tiles (the column share of a CU spans
    # 2, 3 and 5 tiles, the last one partial): runs that cross a tile.
    (8, 512, 5000), (8, 1280, 12000), (5, 640, 17000), (8, 2560, 17408),
    # One row set of 9..16 rows (the 16-row kernel for 16-bit activations):
    # several tiles per work-group, ragged tails, G = 1 and odd G.
    (16, 512, 5000), (12, 1280, 12000), (10, 192, 4001), (16, 64, 300), (13, 2560, 17408),
    (16, 2560, 2000), (11, 448, 777),
    # Row sets of 16 (17..64 rows): several column groups per XCD, ragged
    # last row set, a padded grid.
    (64, 2560, 5000), (48, 1280, 3001), (20, 512, 12000), (64, 64, 99), (40, 2560, 17408),
    # Wide outputs (at least two column tiles per wave): waves own whole
    # tiles (one row set, a ragged last tile, three and four row sets).
    (8, 512, 70000), (16, 1024, 66000), (12, 2560, 66001), (48, 512, 30000), (64, 1536, 25000),
    (3, 2560, 66001),
    # 17..64 rows at vocabulary widths, every row set on one weight stream:
    # two, three and four row sets, K in whole and partial chunks of 5 pairs,
    # ragged last tile and row set.
    (64, 2560, 70000), (40, 1280, 40001), (17, 768, 33000), (33, 384, 36000),
]


@pytest.mark.parametrize("act", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_parity_small(vqv, act, M, K, N):
    c = case(M, K, N, act, seed=M * 1000 + K + N)
    y = run(vqv, c)
    ref = qgemm_ref(c["x"], act, c["wq"], c["scales"], c["biases"])
    assert_close(y, ref, act, f"M={M} K={K} N={N} {act}")


# Group 128 through every kernel: the target projection and the 8-row kernel,
# the generic kernel (K/64 not a multiple of 8, odd K/128), the 16-row kernel
# with and without 16-byte table units, row sets on one weight stream
# (partial chunks), whole-tile waves, and the narrow draft projection.
SHAPES_G128 = [
    (8, 5120, 17408), (8, 512, 1024), (4, 1280, 12000), (1, 128, 17), (5, 384, 1000),
    (16, 640, 300), (16, 1024, 5000), (12, 2560, 17408), (48, 1280, 3001),
    (64, 2560, 70000), (40, 1280, 40001), (33, 384, 36000),
    (8, 512, 70000), (16, 1024, 66000), (48, 512, 30000), (1, 5120, 1024), (8, 5120, 1000),
]


@pytest.mark.parametrize("act", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("M,K,N", SHAPES_G128)
def test_parity_group128(vqv, act, M, K, N):
    c = case(M, K, N, act, seed=M * 1000 + K + N + 128, group=128)
    y = run(vqv, c)
    ref = qgemm_ref(c["x"], act, c["wq"], c["scales"], c["biases"], group=128)
    assert_close(y, ref, act, f"group 128 M={M} K={K} N={N} {act}")


@pytest.mark.parametrize("act", ["bf16", "fp32"])
@pytest.mark.parametrize("M,K,N", SHAPES_G128[::2])
def test_group128_equals_group64_twice(vqv, act, M, K, N):
    """A 128-group's entry serves both 64-halves in the kernels: the result
    equals, bit for bit, group 64 with every entry repeated."""
    c = case(M, K, N, act, seed=M + K + N, group=128)
    y128 = run(vqv, c)
    c64 = dict(c, group=64, scales=np.repeat(c["scales"], 2, axis=1),
               biases=np.repeat(c["biases"], 2, axis=1))
    np.testing.assert_array_equal(y128, run(vqv, c64))


# Group 32 runs on the 8-row kernel (M <= 8), the 16-row, row-set and
# whole-tile kernels and the generic kernel in every configuration its dispatch
# takes: one row set with the whole K range staged (64-80 column shares and
# wide N), narrow outputs, chunked staging at large K, two, four and eight row
# sets, the small fallbacks, and an odd count of 64-groups.
SHAPES_G32 = [
    (8, 5120, 17408), (8, 5120, 1024), (1, 640, 300), (4, 1280, 30000), (5, 192, 65),
    (8, 8192, 300), (16, 640, 300), (12, 8192, 100), (9, 448, 777), (32, 256, 96),
    (20, 1280, 500), (64, 512, 130), (40, 8192, 70), (64, 64, 99),
    # The 8-row kernel at its edges: one 64-group, an odd group count with a
    # ragged tail, runs across tiles, and K at its staging limit.
    (8, 64, 3), (3, 64, 1000), (7, 320, 4001), (8, 1088, 129), (2, 2560, 66001),
    # The 16-row kernel: one to four row sets, several tiles per work-group,
    # K at its staging limit, 16-bit table loads (K/32 not a multiple of 8).
    (16, 512, 5000), (12, 2560, 17408), (64, 2560, 5000), (48, 1280, 3001), (33, 384, 9000),
    # The row-set kernel at vocabulary widths: two, three and four row sets,
    # whole and partial chunks, ragged last tile and row set.
    (64, 2560, 70000), (40, 1280, 40001), (17, 768, 33000), (33, 384, 36000),
    # The whole-tile kernel (K/128 a multiple of 4): one row set, a ragged
    # last tile.
    (8, 512, 70000), (16, 1024, 66000), (12, 2560, 66001),
]


@pytest.mark.parametrize("act", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("M,K,N", SHAPES_G32)
def test_parity_group32(vqv, act, M, K, N):
    c = case(M, K, N, act, seed=M * 1000 + K + N + 32, group=32)
    y = run(vqv, c)
    ref = qgemm_ref(c["x"], act, c["wq"], c["scales"], c["biases"], group=32)
    assert_close(y, ref, act, f"group 32 M={M} K={K} N={N} {act}")


@pytest.mark.parametrize("act", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("M,K,N", [(8, 512, 1024), (3, 192, 37), (16, 1280, 96), (64, 256, 40)])
def test_integer_case_bit_exact_group32(vqv, act, M, K, N):
    """Integer-exact inputs with one scale and bias per 32 k, the two halves
    of a 64-group given different biases: bit for bit against the oracle."""
    rng = np.random.default_rng(27 + M + K + N)
    wq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    G = K // 32
    s = np.full((N, G), np.float16(1.0).view(np.uint16), dtype=np.uint16)
    b = rng.integers(-8, 1, size=(N, G)).astype(np.float16).view(np.uint16)
    xi = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    x = {"bf16": lambda: gen.f32_to_bf16_bits(xi), "fp16": lambda: xi.astype(np.float16).view(np.uint16),
         "fp32": lambda: xi}[act]()
    c = dict(M=M, K=K, N=N, act=act, wq=wq, scales=s, biases=b, x=x, group=32)
    np.testing.assert_array_equal(run(vqv, c), qgemm_ref(x, act, wq, s, b, group=32)
                                  .astype(np.float32))


def test_group32_halves_use_their_own_scale(vqv):
    """Scale 1 on the first 32-k half of every group and 0 on the second, zero
    biases: y is the product over the first halves only."""
    M, K, N = 8, 512, 200
    rng = np.random.default_rng(28)
    wq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = np.zeros((N, K // 32), dtype=np.float16)
    s[:, 0::2] = 1.0
    s = s.view(np.uint16)
    b = np.zeros((N, K // 32), dtype=np.uint16)
    xi = rng.integers(-4, 5, size=(M, K)).astype(np.float32)
    x = gen.f32_to_bf16_bits(xi)
    c = dict(M=M, K=K, N=N, act="bf16", wq=wq, scales=s, biases=b, x=x, group=32)
    y = run(vqv, c)
    q = np.empty((N, K), np.float64)
    q[:, 0::2] = wq & 15
    q[:, 1::2] = wq >> 4
    first = (np.arange(K) // 32) % 2 == 0
    np.testing.assert_array_equal(y, (xi[:, first] @ q[:, first].T).astype(np.float32))


@pytest.mark.parametrize("act", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("M,K,N", [(8, 512, 1024), (3, 384, 37), (16, 1280, 96), (64, 256, 40)])
def test_integer_case_bit_exact_group128(vqv, act, M, K, N):
    """Integer-exact inputs with one scale and bias per 128 k: fp32 is exact in
    any order, so the GPU equals the oracle bit for bit."""
    rng = np.random.default_rng(17 + M + K + N)
    wq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    G = K // 128
    s = np.full((N, G), np.float16(1.0).view(np.uint16), dtype=np.uint16)
    b = rng.integers(-8, 1, size=(N, G)).astype(np.float16).view(np.uint16)
    xi = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    x = {"bf16": lambda: gen.f32_to_bf16_bits(xi), "fp16": lambda: xi.astype(np.float16).view(np.uint16),
         "fp32": lambda: xi}[act]()
    c = dict(M=M, K=K, N=N, act=act, wq=wq, scales=s, biases=b, x=x, group=128)
    np.testing.assert_array_equal(run(vqv, c), qgemm_ref(x, act, wq, s, b, group=128)
                                  .astype(np.float32))


@pytest.mark.parametrize("act", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("M,K,N", [(8, 512, 1024), (3, 192, 37), (16, 1280, 96), (64, 256, 40)])
def test_integer_case_bit_exact(vqv, act, M, K, N):
    """s = 1, integer biases, integer x in [-8, 8]: every partial sum is an
    integer below 2^24, so fp32 is exact in any order and the GPU must equal
    the oracle bit for bit. Pins unpacking, indexing, group mapping, tails."""
    rng = np.random.default_rng(7 + M + K + N)
    wq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    G = K // 64
    s = np.full((N, G), np.float16(1.0).view(np.uint16), dtype=np.uint16)
    b = rng.integers(-8, 1, size=(N, G)).astype(np.float16).view(np.uint16)
    xi = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    x = {"bf16": lambda: gen.f32_to_bf16_bits(xi), "fp16": lambda: xi.astype(np.float16).view(np.uint16),
         "fp32": lambda: xi}[act]()
    c = dict(M=M, K=K, N=N, act=act, wq=wq, scales=s, biases=b, x=x)
    y = run(vqv, c)
    ref = qgemm_ref(x, act, wq, s, b)
    np.testing.assert_array_equal(y, ref.astype(np.float32))


def test_dyadic_scales_bit_exact(vqv):
    """s = 2^-6 and b = -8*2^-6: still exact in fp32 (dyadic, small)."""
    M, K, N = 8, 1024, 300
    rng = np.random.default_rng(11)
    wq = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = np.full((N, K // 64), np.float16(2.0 ** -6).view(np.uint16), dtype=np.uint16)
    b = np.full((N, K // 64), np.float16(-8 * 2.0 ** -6).view(np.uint16), dtype=np.uint16)
    x = gen.f32_to_bf16_bits(rng.integers(-8, 9, size=(M, K)).astype(np.float32))
    c = dict(M=M, K=K, N=N, act="bf16", wq=wq, scales=s, biases=b, x=x)
    np.testing.assert_array_equal(run(vqv, c), qgemm_ref(x, "bf16", wq, s, b).astype(np.float32))


def test_zero_padded_rows_are_exact_zero(vqv):
    """W4A32 draft projection: 1 real row + 7 zero rows; padding gives 0.0."""
    c = gen.make_config("draft_w4a32", N=512, K=1024)
    y = run(vqv, c)
    assert np.all(y[1:] == 0.0)
    ref = qgemm_ref(c["x"], "fp32", c["wq"], c["scales"], c["biases"])
    assert_close(y, ref, "fp32", "draft_w4a32 scaled")


def test_zero_codes_identity(vqv):
    """All-zero codes: y = sum_g b * xsum_g (the bias-only identity)."""
    c = case(8, 512, 256, "bf16", seed=5)
    c["wq"][:] = 0
    y = run(vqv, c)
    ref = qgemm_ref(c["x"], "bf16", c["wq"], c["scales"], c["biases"])
    assert_close(y, ref, "bf16", "zero codes")


def test_rows_independent_of_M(vqv):
    """Row r computed at M=1, 4 and 8 from the same x rows: each within the
    contract. Bit equality across M is reported, not required."""
    c = case(8, 1024, 500, "bf16", seed=9)
    ref = qgemm_ref(c["x"], "bf16", c["wq"], c["scales"], c["biases"])
    ys = {M: run(vqv, c, M=M) for M in (1, 4, 8)}
    for M, y in ys.items():
        assert_close(y, ref[:M], "bf16", f"M={M}")
    same = np.array_equal(ys[1][0], ys[8][0]) and np.array_equal(ys[4], ys[8][:4])
    print(f"row results bit-identical across M=1/4/8: {same}")


# Shapes that reach each projection kernel: qgemm_w4_m8 (M <= 8), the 16-row
# kernel (9..64 rows), the whole-tile kernel (vocabulary widths), the
# all-row-sets kernel (17..64 rows at vocabulary widths) and the generic
# kernel (fp32 activations).
KERNEL_SHAPES = [(8, 2048, 4096, "bf16"), (16, 1024, 3000, "fp16"), (16, 1024, 66000, "bf16"),
                 (64, 1280, 40000, "bf16"), (8, 512, 300, "fp32")]


@pytest.mark.parametrize("M,K,N,act", KERNEL_SHAPES)
def test_deterministic_fingerprint(vqv, M, K, N, act):
    c = case(M, K, N, act, seed=12)
    d = to_device(c)
    hs = set()
    for _ in range(3):
        y = vqv.vqv_qgemm(d["x"], d["wq"], d["scales"], d["biases"])
        torch.cuda.synchronize()
        hs.add(sha(y))
    assert len(hs) == 1


def _set_act(c, m, k, value):
    """Write one activation (given as a float) in the config's own encoding."""
    if c["act"] == "fp32":
        c["x"][m, k] = value
    elif c["act"] == "fp16":
        c["x"][m, k] = np.float16(value).view(np.uint16)
    else:
        c["x"][m, k] = np.uint16(np.float32(value).view(np.uint32) >> 16)


@pytest.mark.parametrize("M,K,N,act", [(4, 256, 64, "fp32"), (4, 256, 64, "bf16"),
                                       (12, 256, 64, "fp16"), (12, 1024, 66000, "bf16")])
def test_nonfinite_activation_propagates(vqv, M, K, N, act):
    c = case(M, K, N, act, seed=13)
    _set_act(c, 1, 70, np.nan)
    _set_act(c, 2, 3, np.inf)
    y = run(vqv, c)
    assert np.isnan(y[1]).all()
    assert (~np.isfinite(y[2])).all()
    rows = [r for r in range(M) if r not in (1, 2)]
    ref = qgemm_ref(c["x"][rows], act, c["wq"], c["scales"], c["biases"])
    assert_close(y[rows], ref, act, "finite rows")


@pytest.mark.parametrize("M,K,N,act", [(5, 256, 70, "bf16"), (13, 256, 70, "fp16"),
                                       (16, 1024, 66001, "bf16"), (5, 256, 70, "fp32")])
def test_writes_only_its_output(vqv, M, K, N, act):
    """y is written exactly in [M, N]; guard bytes around it stay untouched."""
    c = case(M, K, N, act, seed=14)
    d = to_device(c)
    buf = torch.full((M * N + 64,), 123.0, dtype=torch.float32, device="cuda")
    y = buf[32:32 + M * N].view(M, N)
    vqv.vqv_qgemm(d["x"], d["wq"], d["scales"], d["biases"], y=y)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(b[:32] == 123.0) and np.all(b[32 + M * N:] == 123.0)
    ref = qgemm_ref(c["x"], act, c["wq"], c["scales"], c["biases"])
    assert_close(y.cpu().numpy(), ref, act, "offset output")


# ---------------------------------------------------------------- full sizes

FULL = [("target", 8), ("target", 4), ("target", 1), ("draft_w4a32", 8), ("vocab_verify", 8),
        ("batched_vocab", 64), ("gate_up", 16)]


@pytest.fixture(scope="module")
def full_cfgs():
    return {}


# Workloads small enough for the oracle to compute every column in seconds;
# the two vocabulary-width workloads are checked on sampled columns.
EVERY_COLUMN = ("target", "draft_w4a32", "gate_up")


@pytest.mark.parametrize("name,M", FULL)
def test_full_size_columns(vqv, full_cfgs, name, M):
    if name not in full_cfgs:
        full_cfgs.clear()  # keep one large workload in host memory at a time
        full_cfgs[name] = gen.make_config(name)
    c = full_cfgs[name]
    y = run(vqv, c, M=M)
    N = c["N"]
    if name in EVERY_COLUMN:
        # All rows of the workload once (rows are independent), then the first M.
        if "ref" not in c:
            c["ref"] = qgemm_ref(c["x"], c["act"], c["wq"], c["scales"], c["biases"])
        cols, ref = np.arange(N), c["ref"][:M]
    else:
        rng = np.random.default_rng(99)
        cols = np.unique(np.concatenate([[0, 1, 15, 16, N // 2, N - 2, N - 1],
                                         rng.integers(0, N, size=1024)]))
        ref = qgemm_ref(c["x"][:M], c["act"], c["wq"], c["scales"], c["biases"], cols=cols)
    worst = assert_close(y[:, cols], ref, c["act"], f"{name} M={M}")
    print(f"{name} M={M}: worst error/allowance {worst:.3g}")
    if c.get("real_rows"):
        assert np.all(y[c["real_rows"]:] == 0.0)

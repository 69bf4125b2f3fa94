"""The C ABI: the library loads, exports every symbol include/vqv.h declares,
and rejects bad arguments on the host with the documented status before any
launch. The CPU tests pass fabricated (never dereferenced) pointers, which is
safe because validation happens before anything touches the device."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vqv.h")

OK, ARG, UNSUP, ALIGN, WS, HIP = range(6)
BF16, FP16, FP32 = range(3)


@pytest.fixture(scope="module")
def L():
    from w4_gemm_vqv_amd import vqv
    if not os.path.exists(vqv.LIB_PATH):
        from w4_gemm_vqv_amd.build import build
        build(verbose=False)
    return vqv.lib()


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return sorted(set(re.findall(r"^\s*[\w\s\*]+?\b(vqv_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_calls():
    assert declared_functions() == sorted(
        ["vqv_abi_version", "vqv_status_string", "vqv_qgemm_kernel", "vqv_qgemm_workspace_bytes",
         "vqv_qgemm",
         "vqv_verify_workspace_bytes", "vqv_verify", "vqv_verify_ex",
         "vqv_qgemm_verify_workspace_bytes", "vqv_qgemm_verify", "vqv_qgemm_verify_ex",
         "vqv_qgemm_swiglu_workspace_bytes", "vqv_qgemm_swiglu", "vqv_qgemm_verify_ex_noalloc"])


def test_exports_every_declared_symbol(L):
    from w4_gemm_vqv_amd import vqv
    out = subprocess.run(["nm", "-D", "--defined-only", vqv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (vqv_\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)
    assert set(vqv.EXPORTS) == set(declared_functions())


def test_version_and_strings(L):
    assert L.vqv_abi_version() == 6
    for s in range(6):
        assert L.vqv_status_string(s)
    assert L.vqv_status_string(99) == b"unknown status"


def test_workspace_queries(L):
    assert L.vqv_qgemm_workspace_bytes(8, 5120, 17408, 64, BF16) == 0
    assert L.vqv_qgemm_workspace_bytes(8, 5120, 1024, 64, FP32) == 0
    # one 16-byte top-two partial per (row, chunk of 4096 logits)
    assert L.vqv_verify_workspace_bytes(1, 8, 17408) == 8 * 5 * 16
    assert L.vqv_verify_workspace_bytes(4, 16, 151936) == 64 * 38 * 16
    assert L.vqv_verify_workspace_bytes(1, 1, 1) == 16
    assert L.vqv_verify_workspace_bytes(0, 8, 10) == 0


def test_kernel_query(L):
    """The kernel a problem runs on, planned for 256 CUs without a GPU."""
    L.vqv_qgemm_kernel.restype = ctypes.c_char_p
    k = lambda *a: L.vqv_qgemm_kernel(*a)
    assert k(8, 5120, 17408, 64, BF16) == b"qgemm_w4_m8q"
    assert k(64, 2560, 151936, 64, BF16) == b"qgemm_w4_rows"
    assert k(8, 2560, 151936, 64, FP16) == b"qgemm_w4_wide"
    assert k(16, 2560, 18432, 64, BF16) == b"qgemm_w4_m16"
    assert k(8, 5120, 1024, 64, FP32) == b"qgemm_w4"
    assert k(8, 5120, 1024, 64, BF16) == b"qgemm_w4_m8q"
    assert k(8, 5120, 17408, 32, BF16) == b"qgemm_w4_m8"
    assert k(1, 5120, 17408, 64, BF16) == b"qgemm_w4_v"
    assert k(1, 2560, 151936, 64, FP16) == b"qgemm_w4_wide"
    assert k(1, 5120, 17408, 32, BF16) == b"qgemm_w4_m8"
    assert k(2, 5120, 17408, 64, BF16) == b"qgemm_w4_m8q"
    assert k(0, 5120, 17408, 64, BF16) is None
    assert k(8, 5120, 17408, 16, BF16) is None
    assert k(8, 5120, 17408, 64, 9) is None


def test_variant_switch(L, monkeypatch):
    """VQV_FORCE_VARIANT is read per call: "v" pins the vector-ALU kernel where
    it applies (one or two rows of 16-bit activations), "m8q" and "m8" the
    8-row MFMA kernels; other shapes ignore it."""
    L.vqv_qgemm_kernel.restype = ctypes.c_char_p
    monkeypatch.setenv("VQV_FORCE_VARIANT", "v")
    assert L.vqv_qgemm_kernel(1, 5120, 17408, 64, BF16) == b"qgemm_w4_v"
    assert L.vqv_qgemm_kernel(2, 2560, 1000, 128, FP16) == b"qgemm_w4_v"
    assert L.vqv_qgemm_kernel(8, 5120, 17408, 64, BF16) == b"qgemm_w4_m8q"
    assert L.vqv_qgemm_kernel(1, 5120, 1024, 64, FP32) == b"qgemm_w4"
    assert L.vqv_qgemm_kernel(1, 5120, 1024, 32, BF16) != b"qgemm_w4_v"
    assert L.vqv_qgemm_kernel(1, 2560, 151936, 64, BF16) == b"qgemm_w4_v"
    monkeypatch.setenv("VQV_FORCE_VARIANT", "m8q")
    assert L.vqv_qgemm_kernel(1, 5120, 17408, 64, BF16) == b"qgemm_w4_m8q"
    assert L.vqv_qgemm_kernel(1, 2560, 151936, 64, BF16) == b"qgemm_w4_wide"
    monkeypatch.setenv("VQV_FORCE_VARIANT", "m8")
    assert L.vqv_qgemm_kernel(1, 5120, 17408, 64, BF16) == b"qgemm_w4_m8"


def test_fused_workspace_queries(L):
    """The fused call's scratch is a 256-byte head and one 16-byte top-two
    partial per (row, work-group covering the row): never room for logits.
    Without a GPU the library plans for 256 CUs."""
    head = 256
    fused = L.vqv_qgemm_verify_workspace_bytes(8, 5120, 17408, 64, BF16)
    assert head < fused <= head + 8 * 256 * 16
    # the batched vocabulary projection: 250 work-groups of 38 column tiles each
    assert L.vqv_qgemm_verify_workspace_bytes(64, 2560, 151936, 64, BF16) == head + 64 * 250 * 16
    # 16 rows on the 16-row kernel (250 workers), fp32 on 16-column work-groups
    assert L.vqv_qgemm_verify_workspace_bytes(16, 512, 1000, 64, BF16) == head + 16 * 250 * 16
    assert L.vqv_qgemm_verify_workspace_bytes(8, 512, 1000, 64, FP32) == head + 8 * 63 * 16
    for M, K, N, group, act in [(16, 5120, 4000, 64, FP16), (64, 256, 700, 64, BF16),
                                (32, 512, 200000, 64, BF16), (8, 512, 1000, 32, BF16),
                                (40, 3072, 2000, 128, FP32), (1, 16384, 100, 64, BF16)]:
        n = L.vqv_qgemm_verify_workspace_bytes(M, K, N, group, act)
        assert head < n and (n - head) % (16 * M) == 0, (M, K, N, group, act, n)
    assert L.vqv_qgemm_verify_workspace_bytes(0, 512, 1000, 64, BF16) == 0
    assert L.vqv_qgemm_verify_workspace_bytes(65, 512, 1000, 64, BF16) == 0
    assert L.vqv_qgemm_verify_workspace_bytes(8, 512, 1000, 16, BF16) == 0
    assert L.vqv_qgemm_verify_workspace_bytes(8, 512, 1000, 64, 7) == 0
    # group 128 takes the same paths as group 64
    assert (L.vqv_qgemm_verify_workspace_bytes(8, 5120, 17408, 128, BF16) ==
            L.vqv_qgemm_verify_workspace_bytes(8, 5120, 17408, 64, BF16))
    assert L.vqv_qgemm_verify_workspace_bytes(8, 512, 1000, 256, BF16) == 0


# Fabricated, well-aligned and non-overlapping device addresses.
X, W, S, B_, Y, WSP = (0x10000000 * i for i in range(1, 7))


def q(L, x=X, wq=W, s=S, b=B_, y=Y, M=8, K=512, N=1024, group=64, act=BF16, ws=None, wsb=0):
    return L.vqv_qgemm(x, wq, s, b, y, M, K, N, group, act, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), ARG), (dict(wq=None), ARG), (dict(s=None), ARG), (dict(b=None), ARG),
    (dict(y=None), ARG), (dict(M=0), ARG), (dict(M=65), ARG), (dict(N=0), ARG), (dict(K=0), ARG),
    (dict(K=32), ARG), (dict(K=100), ARG), (dict(group=16), UNSUP), (dict(group=256), UNSUP),
    (dict(group=32, K=96), UNSUP), (dict(group=32, K=8192 + 64), UNSUP),
    (dict(group=128, K=192), ARG), (dict(group=128, s=S + 1), ALIGN),
    (dict(act=3), ARG), (dict(act=-1), ARG), (dict(x=X + 8), ALIGN), (dict(wq=W + 4), ALIGN),
    (dict(s=S + 1), ALIGN), (dict(y=Y + 2), ALIGN), (dict(y=X), ARG), (dict(y=W + 64), ARG),
    (dict(y=S), ARG), (dict(M=64, K=64 * 2 ** 20, act=FP32), UNSUP), (dict(K=16384 + 64), UNSUP),
])
def test_qgemm_rejects(L, kw, status):
    assert q(L, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(logits=None), ARG), (dict(argmax=None), ARG), (dict(acc=None), ARG),
    (dict(B=0), ARG), (dict(T=0), ARG), (dict(T=65), ARG), (dict(N=0), ARG),
    (dict(draft=None), ARG), (dict(B=2 ** 20, T=64, N=64), ARG), (dict(logits=X + 4), ALIGN),
    (dict(argmax=Y + 2), ALIGN), (dict(ws=None), WS), (dict(wsb=8), WS), (dict(ws=WSP + 4), WS),
    (dict(ws=WSP + 8), WS),
    (dict(argmax=X + 64), ARG), (dict(acc=X), ARG), (dict(ws=X), ARG),
])
def test_verify_rejects(L, kw, status):
    a = dict(logits=X, draft=W, B=1, T=8, N=1024, argmax=Y, acc=S, ws=WSP, wsb=1 << 20)
    a.update(kw)
    assert L.vqv_verify(a["logits"], a["draft"], a["B"], a["T"], a["N"], a["argmax"], a["acc"],
                        a["ws"], a["wsb"], None) == status


DR, AM, AC = 0x70000000, 0x80000000, 0x90000000


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), ARG), (dict(am=None), ARG), (dict(ac=None), ARG), (dict(dr=None), ARG),
    (dict(B=2), ARG), (dict(T=4), ARG), (dict(M=65, B=65, T=1), ARG), (dict(group=16), UNSUP),
    (dict(group=128, K=320), ARG),
    (dict(K=100), ARG), (dict(y=Y + 4), ALIGN), (dict(am=AM + 2), ALIGN), (dict(ws=None), WS),
    (dict(wsb=8), WS), (dict(ws=WSP + 16), WS), (dict(am=X), ARG), (dict(ws=W), ARG),
    (dict(y=DR), ARG), (dict(ac=AM + 16), ARG), (dict(K=16384 + 64), UNSUP),
])
def test_fused_rejects(L, kw, status):
    a = dict(x=X, wq=W, s=S, b=B_, y=Y, M=8, K=512, N=1024, group=64, act=BF16, dr=DR, B=1, T=8,
             am=AM, ac=AC, ws=WSP, wsb=1 << 20)
    a.update(kw)
    assert L.vqv_qgemm_verify(a["x"], a["wq"], a["s"], a["b"], a["y"], a["M"], a["K"], a["N"],
                              a["group"], a["act"], a["dr"], a["B"], a["T"], a["am"], a["ac"],
                              a["ws"], a["wsb"], None) == status


LEN, MG = 0xA0000000, 0xB0000000


@pytest.mark.parametrize("kw,status", [
    (dict(dl=LEN + 2), ALIGN), (dict(mg=MG + 2), ALIGN), (dict(mg=Y), ARG), (dict(mg=S), ARG),
    (dict(mg=X + 64), ARG), (dict(mg=WSP), ARG), (dict(dl=Y), ARG), (dict(dl=S), ARG),
    (dict(dl=WSP + 32), ARG), (dict(mg=MG + 8, B=2, T=4, dl=MG + 16), ARG), (dict(mg=LEN), ARG),
])
def test_verify_ex_rejects(L, kw, status):
    a = dict(logits=X, draft=W, dl=LEN, B=1, T=8, N=1024, argmax=Y, acc=S, mg=MG, ws=WSP,
             wsb=1 << 20)
    a.update(kw)
    assert L.vqv_verify_ex(a["logits"], a["draft"], a["dl"], a["B"], a["T"], a["N"], a["argmax"],
                           a["acc"], a["mg"], a["ws"], a["wsb"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dl=LEN + 2), ALIGN), (dict(mg=MG + 2), ALIGN), (dict(mg=AM), ARG), (dict(mg=Y), ARG),
    (dict(mg=X), ARG), (dict(mg=WSP + 64), ARG), (dict(dl=AM), ARG), (dict(dl=AC), ARG),
    (dict(dl=Y + 128), ARG), (dict(dl=WSP), ARG), (dict(mg=LEN), ARG), (dict(x=None), ARG),
])
def test_fused_ex_rejects(L, kw, status):
    a = dict(x=X, wq=W, s=S, b=B_, y=Y, M=8, K=512, N=1024, group=64, act=BF16, dr=DR, dl=LEN,
             B=1, T=8, am=AM, ac=AC, mg=MG, ws=WSP, wsb=1 << 20)
    a.update(kw)
    assert L.vqv_qgemm_verify_ex(a["x"], a["wq"], a["s"], a["b"], a["y"], a["M"], a["K"], a["N"],
                                 a["group"], a["act"], a["dr"], a["dl"], a["B"], a["T"], a["am"],
                                 a["ac"], a["mg"], a["ws"], a["wsb"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), ARG), (dict(B=2), ARG), (dict(group=16), UNSUP), (dict(am=AM + 2), ALIGN),
    (dict(mg=Y), ARG), (dict(dl=AM), ARG), (dict(y=X), ARG), (dict(K=16384 + 64), UNSUP),
    # scratch beyond VQV_NOALLOC_SCRATCH_BYTES: the partials of very wide
    # projections on 64- or 80-column work-groups
    (dict(K=5120, N=1_000_000, wq=1 << 36, s=2 << 36, b=3 << 36, y=4 << 36), WS),
    (dict(M=64, B=4, T=16, K=5120, N=300_000, wq=1 << 36, s=2 << 36, b=3 << 36, y=4 << 36,
          dr=5 << 36, dl=6 << 36, am=7 << 36, ac=8 << 36, mg=9 << 36), WS),
])
def test_noalloc_rejects(L, kw, status):
    """Rejections of the allocation-free call come before it looks up its
    scratch or launches anything (so they run without a GPU)."""
    a = dict(x=X, wq=W, s=S, b=B_, y=Y, M=8, K=512, N=1024, group=64, act=BF16, dr=DR, dl=LEN,
             B=1, T=8, am=AM, ac=AC, mg=MG)
    a.update(kw)
    assert L.vqv_qgemm_verify_ex_noalloc(a["x"], a["wq"], a["s"], a["b"], a["y"], a["M"], a["K"],
                                         a["N"], a["group"], a["act"], a["dr"], a["dl"], a["B"],
                                         a["T"], a["am"], a["ac"], a["mg"], None) == status


def test_swiglu_workspace_queries(L):
    # fused into the 16-row kernel (row sets of 16): no workspace
    assert L.vqv_qgemm_swiglu_workspace_bytes(16, 2560, 18432, 64, BF16) == 0
    assert L.vqv_qgemm_swiglu_workspace_bytes(4, 512, 1000, 64, FP16) == 0
    assert L.vqv_qgemm_swiglu_workspace_bytes(64, 512, 1000, 64, BF16) == 0
    # fallbacks hold the stacked output
    assert L.vqv_qgemm_swiglu_workspace_bytes(32, 512, 1000, 64, FP32) >= 32 * 1000 * 4
    assert L.vqv_qgemm_swiglu_workspace_bytes(16, 512, 1000, 64, FP32) >= 16 * 1000 * 4
    assert L.vqv_qgemm_swiglu_workspace_bytes(16, 5120, 1000, 64, BF16) >= 16 * 1000 * 4
    # invalid: odd N, group, M
    assert L.vqv_qgemm_swiglu_workspace_bytes(16, 512, 1001, 64, BF16) == 0
    assert L.vqv_qgemm_swiglu_workspace_bytes(16, 512, 1000, 16, BF16) == 0
    assert L.vqv_qgemm_swiglu_workspace_bytes(16, 512, 1000, 32, BF16) == 0  # fused too
    assert L.vqv_qgemm_swiglu_workspace_bytes(16, 512, 1000, 32, FP32) >= 16 * 1000 * 4
    assert L.vqv_qgemm_swiglu_workspace_bytes(64, 512, 1000, 128, BF16) == 0
    assert L.vqv_qgemm_swiglu_workspace_bytes(16, 512, 1000, 256, BF16) == 0
    assert L.vqv_qgemm_swiglu_workspace_bytes(0, 512, 1000, 64, BF16) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), ARG), (dict(h=None), ARG), (dict(N=1001), ARG), (dict(N=0), ARG),
    (dict(M=65), ARG), (dict(K=100), ARG), (dict(group=16), UNSUP), (dict(act=3), ARG),
    (dict(group=128, K=448), ARG),
    (dict(x=X + 8), ALIGN), (dict(h=Y + 2), ALIGN), (dict(h=X), ARG), (dict(h=W + 64), ARG),
    (dict(h=S), ARG), (dict(K=16384 + 64), UNSUP),
    (dict(act=FP32, ws=None), WS), (dict(act=FP32, wsb=64), WS),
    (dict(act=FP32, ws=WSP + 16), WS), (dict(act=FP32, ws=X), ARG),
    (dict(act=FP32, h=WSP + 256), ARG),
])
def test_swiglu_rejects(L, kw, status):
    a = dict(x=X, wq=W, s=S, b=B_, h=Y, M=16, K=512, N=1000, group=64, act=BF16, ws=WSP,
             wsb=1 << 20)
    a.update(kw)
    assert L.vqv_qgemm_swiglu(a["x"], a["wq"], a["s"], a["b"], a["h"], a["M"], a["K"], a["N"],
                              a["group"], a["act"], a["ws"], a["wsb"], None) == status


def test_python_binding_raises_with_status(L):
    from w4_gemm_vqv_amd import vqv
    with pytest.raises(vqv.VqvError) as e:
        vqv._check(ARG)
    assert e.value.status == ARG


def test_binding_has_no_cpu_path():
    """The binding and the library never import the oracle."""
    pkg = os.path.join(ROOT, "w4_gemm_vqv_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("oracle's", ""), f
                assert "import gen" not in text, f


def test_binding_checks_tensor_sizes(L):
    """The binding refuses a caller's tensor of the wrong size, dtype or device
    before the call: the library sees only its pointer, so a short buffer would
    be read or written past its end on the GPU."""
    import torch
    from w4_gemm_vqv_amd import vqv
    M, K, N = 8, 128, 64
    x = torch.zeros(M, K, dtype=torch.bfloat16)
    wq = torch.zeros(N, K // 2, dtype=torch.uint8)
    s = torch.zeros(N, K // 64, dtype=torch.float16)
    dr = torch.zeros(1, 7, dtype=torch.int32)
    logits = torch.zeros(M, N)
    bad = [
        (lambda: vqv.vqv_qgemm(x, wq, s, s, y=torch.empty(M, N - 1)), "y must hold"),
        (lambda: vqv.vqv_qgemm(x, wq, s, s, y=torch.empty(M, N, dtype=torch.float16)),
         "y must hold"),
        (lambda: vqv.vqv_qgemm(x, wq, s, s, y=torch.empty(M, N, device="meta")), "y is on meta"),
        (lambda: vqv.vqv_qgemm(x, wq.to("meta"), s, s), "wq is on meta"),
        (lambda: vqv.vqv_qgemm_swiglu(x, wq, s, s, h=torch.empty(M, N)), "h must hold"),
        (lambda: vqv.vqv_verify(logits, dr, 2, 8), "logits must hold"),
        (lambda: vqv.vqv_verify(logits, dr[:, :6], 1, 8), "draft must hold"),
        (lambda: vqv.vqv_verify(logits, dr.long(), 1, 8), "draft must hold"),
        (lambda: vqv.vqv_verify(logits, dr, 1, 8, accept_len=torch.empty(2, dtype=torch.int32)),
         "accept_len must hold"),
        (lambda: vqv.vqv_verify_ex(logits, dr, 1, 8, draft_len=torch.zeros(2, dtype=torch.int32)),
         "draft_len must hold"),
        (lambda: vqv.vqv_qgemm_verify(x, wq, s, s, dr, 1, 8,
                                      argmax=torch.empty(4, dtype=torch.int32)), "argmax must hold"),
        (lambda: vqv.vqv_qgemm_verify(x, wq, s, s, dr, 1, 8, y=torch.empty(M * N + 1)),
         "y must hold"),
        (lambda: vqv.vqv_qgemm_verify_ex(x, wq, s, s, dr, 1, 8, margin=torch.empty(7)),
         "margin must hold"),
    ]
    for call, msg in bad:
        with pytest.raises(ValueError, match=msg):
            call()
    # Right sizes on the CPU get as far as the device check.
    with pytest.raises(ValueError, match="device tensor"):
        vqv.vqv_qgemm(x, wq, s, s, y=torch.empty(M, N))


# ---------------------------------------------------------------- on the GPU


@pytest.mark.gpu
def test_rejected_calls_write_nothing():
    import torch
    from w4_gemm_vqv_amd import vqv
    Lg = vqv.lib()
    x = torch.zeros(8, 512, dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros(1024, 256, dtype=torch.uint8, device="cuda")
    s = torch.zeros(1024, 8, dtype=torch.float16, device="cuda")
    y = torch.full((8, 1024), 7.0, device="cuda")
    for M, K, group in [(0, 512, 64), (8, 512, 16), (8, 500, 64), (8, 96, 32)]:
        st = Lg.vqv_qgemm(x.data_ptr(), wq.data_ptr(), s.data_ptr(), s.data_ptr(), y.data_ptr(),
                          M, K, 1024, group, BF16, None, 0, None)
        assert st != OK
    lg = torch.zeros(8, 1024, device="cuda")
    am = torch.full((8,), -3, dtype=torch.int32, device="cuda")
    ac = torch.full((1,), -3, dtype=torch.int32, device="cuda")
    ws = torch.zeros(8, dtype=torch.uint8, device="cuda")
    st = Lg.vqv_verify(lg.data_ptr(), None, 1, 8, 1024, am.data_ptr(), ac.data_ptr(),
                       ws.data_ptr(), 8, None)
    assert st == ARG
    torch.cuda.synchronize()
    assert (y == 7.0).all() and (am == -3).all() and (ac == -3).all()


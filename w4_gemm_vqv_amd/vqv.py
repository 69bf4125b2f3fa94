"""Thin Python binding of libvqv (include/vqv.h) through ctypes.

The functions carry the C names and only marshal arguments: tensor data
pointers, sizes and the stream handle go to the library, which checks them
and launches its HIP kernels. There is no other code path; if the library is
missing the import of any call fails loudly.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvqv.so")

VQV_BF16, VQV_FP16, VQV_FP32 = 0, 1, 2
VQV_OK, VQV_ERR_ARG, VQV_ERR_UNSUPPORTED, VQV_ERR_ALIGN, VQV_ERR_WORKSPACE, VQV_ERR_HIP = range(6)
EXPORTS = ("vqv_abi_version", "vqv_status_string", "vqv_qgemm_kernel",
           "vqv_qgemm_workspace_bytes", "vqv_qgemm",
           "vqv_verify_workspace_bytes", "vqv_verify", "vqv_verify_ex",
           "vqv_qgemm_verify_workspace_bytes", "vqv_qgemm_verify", "vqv_qgemm_verify_ex",
           "vqv_qgemm_swiglu_workspace_bytes", "vqv_qgemm_swiglu", "vqv_qgemm_verify_ex_noalloc")
VQV_NOALLOC_SCRATCH_BYTES = 1 << 20

_DTYPES = {torch.bfloat16: VQV_BF16, torch.float16: VQV_FP16, torch.float32: VQV_FP32}
_lib = None


class VqvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"vqv status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libvqv (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m w4_gemm_vqv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.vqv_abi_version.restype = i
        L.vqv_abi_version.argtypes = []
        L.vqv_status_string.restype = ctypes.c_char_p
        L.vqv_status_string.argtypes = [i]
        L.vqv_qgemm_kernel.restype = ctypes.c_char_p
        L.vqv_qgemm_kernel.argtypes = [i, i, i, i, i]
        L.vqv_qgemm_workspace_bytes.restype = sz
        L.vqv_qgemm_workspace_bytes.argtypes = [i, i, i, i, i]
        L.vqv_qgemm.restype = i
        L.vqv_qgemm.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, sz, vp]
        L.vqv_verify_workspace_bytes.restype = sz
        L.vqv_verify_workspace_bytes.argtypes = [i, i, i]
        L.vqv_verify.restype = i
        L.vqv_verify.argtypes = [vp, vp, i, i, i, vp, vp, vp, sz, vp]
        L.vqv_qgemm_verify_workspace_bytes.restype = sz
        L.vqv_qgemm_verify_workspace_bytes.argtypes = [i, i, i, i, i]
        L.vqv_qgemm_verify.restype = i
        L.vqv_qgemm_verify.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, i, i, vp, vp, vp, sz,
                                       vp]
        L.vqv_verify_ex.restype = i
        L.vqv_verify_ex.argtypes = [vp, vp, vp, i, i, i, vp, vp, vp, vp, sz, vp]
        L.vqv_qgemm_swiglu_workspace_bytes.restype = sz
        L.vqv_qgemm_swiglu_workspace_bytes.argtypes = [i, i, i, i, i]
        L.vqv_qgemm_swiglu.restype = i
        L.vqv_qgemm_swiglu.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, sz, vp]
        L.vqv_qgemm_verify_ex.restype = i
        L.vqv_qgemm_verify_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, i, i, vp, vp,
                                          vp, vp, sz, vp]
        L.vqv_qgemm_verify_ex_noalloc.restype = i
        L.vqv_qgemm_verify_ex_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, i, i,
                                                  vp, vp, vp, vp]
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != VQV_OK:
        raise VqvError(status, lib().vqv_status_string(status).decode())


def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev(t: torch.Tensor, name: str) -> int:
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous device tensor")
    return t.data_ptr()


def _need(t: torch.Tensor | None, name: str, numel: int, dtype: torch.dtype,
          device: torch.device) -> None:
    """A tensor the library reads or writes must hold exactly what the call
    covers, in the stated dtype and on the device of the call's main input:
    the library sees only a pointer, so a shorter buffer would be accessed past
    its end on the GPU."""
    if t is None:
        return
    if t.dtype != dtype or t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} {dtype} values, got {t.numel()} {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the call's inputs on {device}")


def _check_weight(wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, K: int,
                  group: int) -> None:
    """The library reads N*K/2 code bytes and N*K/group table entries: the
    tensors must hold that much."""
    rows = wq.shape[0]
    if wq.numel() * wq.element_size() != rows * (K // 2):
        raise ValueError(f"wq must hold [N, K/2] = [{rows}, {K // 2}] bytes")
    if group > 0 and K % group == 0:
        for t, name in ((scales, "scales"), (biases, "biases")):
            if t.numel() != rows * (K // group) or t.element_size() != 2:
                raise ValueError(f"{name} must hold [N, K/group] = [{rows}, {K // group}] "
                                 "16-bit entries")


def vqv_abi_version() -> int:
    return lib().vqv_abi_version()


def vqv_status_string(status: int) -> str:
    return lib().vqv_status_string(status).decode()


def vqv_qgemm_kernel(M: int, K: int, N: int, group: int = 64,
                     act_dtype: int = VQV_BF16) -> str | None:
    """Name of the projection kernel these sizes run on (None if rejected)."""
    r = lib().vqv_qgemm_kernel(M, K, N, group, act_dtype)
    return r.decode() if r is not None else None


def vqv_qgemm_workspace_bytes(M: int, K: int, N: int, group: int = 64,
                              act_dtype: int = VQV_BF16) -> int:
    return lib().vqv_qgemm_workspace_bytes(M, K, N, group, act_dtype)


def vqv_qgemm(x: torch.Tensor, wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor,
              y: torch.Tensor | None = None, group: int = 64,
              workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y[M,N] fp32 = x[M,K] . W^T with W given as packed codes [N,K/2] uint8 and
    fp16 scales/biases [N,K/group] (float16, or int16 bit patterns)."""
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported activation dtype {x.dtype}")
    M, K = x.shape
    N = wq.shape[0]
    _check_weight(wq, scales, biases, K, group)
    for t, name in ((wq, "wq"), (scales, "scales"), (biases, "biases")):
        _need(t, name, t.numel(), t.dtype, x.device)
    _need(y, "y", M * N, torch.float32, x.device)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    act = _DTYPES[x.dtype]
    need = vqv_qgemm_workspace_bytes(M, K, N, group, act)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().vqv_qgemm(_dev(x, "x"), _dev(wq, "wq"), _dev(scales, "scales"),
                           _dev(biases, "biases"), _dev(y, "y"), M, K, N, group, act,
                           ws_ptr, ws_bytes, _stream_handle(stream)))
    return y


def vqv_verify_workspace_bytes(B: int, T: int, N: int) -> int:
    return lib().vqv_verify_workspace_bytes(B, T, N)


def _verify_io(logits, draft, B, T, N, dev, argmax, accept_len, draft_len=None, margin=None):
    """Sizes of the verify's tensors: logits [B*T, N] fp32, drafts [B, T-1]
    int32, valid counts [B] int32, argmax and margin [B*T], accept_len [B]."""
    if logits is not None:
        _need(logits, "logits", B * T * N, torch.float32, dev)
    if draft is not None and draft.numel():
        _need(draft, "draft", B * (T - 1), torch.int32, dev)
    _need(draft_len, "draft_len", B, torch.int32, dev)
    _need(argmax, "argmax", B * T, torch.int32, dev)
    _need(accept_len, "accept_len", B, torch.int32, dev)
    _need(margin, "margin", B * T, torch.float32, dev)


def vqv_verify(logits: torch.Tensor, draft: torch.Tensor | None, B: int, T: int,
               argmax: torch.Tensor | None = None, accept_len: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, stream=None):
    """(argmax [B*T] int32, accept_len [B] int32) of fp32 logits [B*T, N]
    against int32 drafts [B, T-1]."""
    N = logits.shape[-1]
    dev = logits.device
    _verify_io(logits, draft, B, T, N, dev, argmax, accept_len)
    if argmax is None:
        argmax = torch.empty(B * T, dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(vqv_verify_workspace_bytes(B, T, N), 16), dtype=torch.uint8,
                                device=dev)
    dptr = _dev(draft, "draft") if (draft is not None and draft.numel()) else None
    _check(lib().vqv_verify(_dev(logits, "logits"), dptr, B, T, N, _dev(argmax, "argmax"),
                            _dev(accept_len, "accept_len"), _dev(workspace, "workspace"),
                            workspace.numel() * workspace.element_size(),
                            _stream_handle(stream)))
    return argmax, accept_len


def vqv_verify_ex(logits: torch.Tensor, draft: torch.Tensor | None, B: int, T: int,
                  draft_len: torch.Tensor | None = None, want_margin: bool = True,
                  argmax: torch.Tensor | None = None, accept_len: torch.Tensor | None = None,
                  margin: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                  stream=None):
    """(argmax [B*T] int32, accept_len [B] int32, margin [B*T] fp32 or None):
    vqv_verify with per-sequence valid draft counts (int32 [B], or None) and
    the top-1 minus top-2 margin of each row."""
    N = logits.shape[-1]
    dev = logits.device
    _verify_io(logits, draft, B, T, N, dev, argmax, accept_len, draft_len, margin)
    if argmax is None:
        argmax = torch.empty(B * T, dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if margin is None and want_margin:
        margin = torch.empty(B * T, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(vqv_verify_workspace_bytes(B, T, N), 16), dtype=torch.uint8,
                                device=dev)
    dptr = _dev(draft, "draft") if (draft is not None and draft.numel()) else None
    lptr = _dev(draft_len, "draft_len") if draft_len is not None else None
    mptr = _dev(margin, "margin") if margin is not None else None
    _check(lib().vqv_verify_ex(_dev(logits, "logits"), dptr, lptr, B, T, N,
                               _dev(argmax, "argmax"), _dev(accept_len, "accept_len"), mptr,
                               _dev(workspace, "workspace"),
                               workspace.numel() * workspace.element_size(),
                               _stream_handle(stream)))
    return argmax, accept_len, margin


def vqv_qgemm_verify_workspace_bytes(M: int, K: int, N: int, group: int = 64,
                                     act_dtype: int = VQV_BF16) -> int:
    return lib().vqv_qgemm_verify_workspace_bytes(M, K, N, group, act_dtype)


def vqv_qgemm_verify(x: torch.Tensor, wq: torch.Tensor, scales: torch.Tensor,
                     biases: torch.Tensor, draft: torch.Tensor | None, B: int, T: int,
                     y: torch.Tensor | None = None, want_y: bool = True,
                     argmax: torch.Tensor | None = None, accept_len: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, group: int = 64, stream=None):
    """(y or None, argmax [B*T] int32, accept_len [B] int32) of the projection
    followed by the greedy verify."""
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported activation dtype {x.dtype}")
    M, K = x.shape
    N = wq.shape[0]
    _check_weight(wq, scales, biases, K, group)
    dev = x.device
    act = _DTYPES[x.dtype]
    for t, name in ((wq, "wq"), (scales, "scales"), (biases, "biases")):
        _need(t, name, t.numel(), t.dtype, dev)
    _need(y, "y", M * N, torch.float32, dev)
    _verify_io(None, draft, B, T, N, dev, argmax, accept_len)
    if y is None and want_y:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    if argmax is None:
        argmax = torch.empty(B * T, dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if workspace is None:
        need = vqv_qgemm_verify_workspace_bytes(M, K, N, group, act)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    dptr = _dev(draft, "draft") if (draft is not None and draft.numel()) else None
    _check(lib().vqv_qgemm_verify(_dev(x, "x"), _dev(wq, "wq"), _dev(scales, "scales"),
                                  _dev(biases, "biases"), _dev(y, "y") if y is not None else None,
                                  M, K, N, group, act, dptr, B, T, _dev(argmax, "argmax"),
                                  _dev(accept_len, "accept_len"), _dev(workspace, "workspace"),
                                  workspace.numel() * workspace.element_size(),
                                  _stream_handle(stream)))
    return y, argmax, accept_len


def vqv_qgemm_verify_ex(x: torch.Tensor, wq: torch.Tensor, scales: torch.Tensor,
                        biases: torch.Tensor, draft: torch.Tensor | None, B: int, T: int,
                        draft_len: torch.Tensor | None = None, want_margin: bool = True,
                        y: torch.Tensor | None = None, want_y: bool = True,
                        argmax: torch.Tensor | None = None,
                        accept_len: torch.Tensor | None = None,
                        margin: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, group: int = 64, stream=None):
    """(y or None, argmax, accept_len, margin or None): vqv_qgemm_verify with
    vqv_verify_ex's valid draft counts and margins."""
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported activation dtype {x.dtype}")
    M, K = x.shape
    N = wq.shape[0]
    _check_weight(wq, scales, biases, K, group)
    dev = x.device
    act = _DTYPES[x.dtype]
    for t, name in ((wq, "wq"), (scales, "scales"), (biases, "biases")):
        _need(t, name, t.numel(), t.dtype, dev)
    _need(y, "y", M * N, torch.float32, dev)
    _verify_io(None, draft, B, T, N, dev, argmax, accept_len, draft_len, margin)
    if y is None and want_y:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    if argmax is None:
        argmax = torch.empty(B * T, dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if margin is None and want_margin:
        margin = torch.empty(B * T, dtype=torch.float32, device=dev)
    if workspace is None:
        need = vqv_qgemm_verify_workspace_bytes(M, K, N, group, act)
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    dptr = _dev(draft, "draft") if (draft is not None and draft.numel()) else None
    lptr = _dev(draft_len, "draft_len") if draft_len is not None else None
    mptr = _dev(margin, "margin") if margin is not None else None
    _check(lib().vqv_qgemm_verify_ex(
        _dev(x, "x"), _dev(wq, "wq"), _dev(scales, "scales"), _dev(biases, "biases"),
        _dev(y, "y") if y is not None else None, M, K, N, group, act, dptr, lptr, B, T,
        _dev(argmax, "argmax"), _dev(accept_len, "accept_len"), mptr,
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream_handle(stream)))
    return y, argmax, accept_len, margin


def vqv_qgemm_verify_ex_noalloc(x: torch.Tensor, wq: torch.Tensor, scales: torch.Tensor,
                                biases: torch.Tensor, draft: torch.Tensor | None, B: int, T: int,
                                draft_len: torch.Tensor | None = None,
                                y: torch.Tensor | None = None,
                                argmax: torch.Tensor | None = None,
                                accept_len: torch.Tensor | None = None,
                                margin: torch.Tensor | None = None, group: int = 64,
                                stream=None):
    """(y, argmax, accept_len, margin) as vqv_qgemm_verify_ex, with the
    library's static per-GPU scratch instead of a workspace. Outputs the
    caller leaves as None are not produced (y, margin) or are allocated here
    (argmax, accept_len) -- pass them in to allocate nothing."""
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported activation dtype {x.dtype}")
    M, K = x.shape
    N = wq.shape[0]
    _check_weight(wq, scales, biases, K, group)
    dev = x.device
    act = _DTYPES[x.dtype]
    for t, name in ((wq, "wq"), (scales, "scales"), (biases, "biases")):
        _need(t, name, t.numel(), t.dtype, dev)
    _need(y, "y", M * N, torch.float32, dev)
    _verify_io(None, draft, B, T, N, dev, argmax, accept_len, draft_len, margin)
    if argmax is None:
        argmax = torch.empty(B * T, dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    dptr = _dev(draft, "draft") if (draft is not None and draft.numel()) else None
    lptr = _dev(draft_len, "draft_len") if draft_len is not None else None
    mptr = _dev(margin, "margin") if margin is not None else None
    _check(lib().vqv_qgemm_verify_ex_noalloc(
        _dev(x, "x"), _dev(wq, "wq"), _dev(scales, "scales"), _dev(biases, "biases"),
        _dev(y, "y") if y is not None else None, M, K, N, group, act, dptr, lptr, B, T,
        _dev(argmax, "argmax"), _dev(accept_len, "accept_len"), mptr, _stream_handle(stream)))
    return y, argmax, accept_len, margin


def vqv_qgemm_swiglu_workspace_bytes(M: int, K: int, N: int, group: int = 64,
                                     act_dtype: int = VQV_BF16) -> int:
    return lib().vqv_qgemm_swiglu_workspace_bytes(M, K, N, group, act_dtype)


def vqv_qgemm_swiglu(x: torch.Tensor, wq: torch.Tensor, scales: torch.Tensor,
                     biases: torch.Tensor, h: torch.Tensor | None = None, group: int = 64,
                     workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """h [M, N/2] fp32 = silu(x . Wg^T) * (x . Wu^T) for a stacked gate/up
    weight ([N, K/2] codes, gate rows first)."""
    if x.dtype not in _DTYPES:
        raise ValueError(f"unsupported activation dtype {x.dtype}")
    M, K = x.shape
    N = wq.shape[0]
    _check_weight(wq, scales, biases, K, group)
    act = _DTYPES[x.dtype]
    for t, name in ((wq, "wq"), (scales, "scales"), (biases, "biases")):
        _need(t, name, t.numel(), t.dtype, x.device)
    _need(h, "h", M * (N // 2), torch.float32, x.device)
    if h is None:
        h = torch.empty((M, N // 2), dtype=torch.float32, device=x.device)
    need = vqv_qgemm_swiglu_workspace_bytes(M, K, N, group, act)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().vqv_qgemm_swiglu(_dev(x, "x"), _dev(wq, "wq"), _dev(scales, "scales"),
                                  _dev(biases, "biases"), _dev(h, "h"), M, K, N, group, act,
                                  ws_ptr, ws_bytes, _stream_handle(stream)))
    return h

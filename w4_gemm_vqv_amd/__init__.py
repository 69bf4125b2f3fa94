"""libvqv: W4 verify projection and greedy verify for MI355X (gfx950).

The compute path is the HIP library ``libvqv.so`` (C ABI in include/vqv.h);
``w4_gemm_vqv_amd.vqv`` is its Python binding. Build with
``python -m w4_gemm_vqv_amd.build``.
"""

from .vqv import (EXPORTS, LIB_PATH, VQV_BF16, VQV_ERR_ALIGN, VQV_ERR_ARG, VQV_ERR_HIP,
                  VQV_ERR_UNSUPPORTED, VQV_ERR_WORKSPACE, VQV_FP16, VQV_FP32, VQV_OK, VqvError,
                  VQV_NOALLOC_SCRATCH_BYTES, lib, vqv_abi_version, vqv_qgemm, vqv_qgemm_kernel,
                  vqv_qgemm_swiglu,
                  vqv_qgemm_swiglu_workspace_bytes, vqv_qgemm_verify, vqv_qgemm_verify_ex,
                  vqv_qgemm_verify_ex_noalloc,
                  vqv_qgemm_verify_workspace_bytes, vqv_qgemm_workspace_bytes, vqv_status_string,
                  vqv_verify, vqv_verify_ex, vqv_verify_workspace_bytes)

__all__ = ["EXPORTS", "LIB_PATH", "VQV_BF16", "VQV_ERR_ALIGN", "VQV_ERR_ARG", "VQV_ERR_HIP",
           "VQV_ERR_UNSUPPORTED", "VQV_ERR_WORKSPACE", "VQV_FP16", "VQV_FP32", "VQV_OK",
           "VQV_NOALLOC_SCRATCH_BYTES", "VqvError", "lib", "vqv_abi_version", "vqv_qgemm",
           "vqv_qgemm_kernel", "vqv_qgemm_swiglu",
           "vqv_qgemm_swiglu_workspace_bytes", "vqv_qgemm_verify",
           "vqv_qgemm_verify_ex", "vqv_qgemm_verify_ex_noalloc",
           "vqv_qgemm_verify_workspace_bytes", "vqv_qgemm_workspace_bytes",
           "vqv_status_string", "vqv_verify", "vqv_verify_ex", "vqv_verify_workspace_bytes"]

"""Hadamard-rotated INT8 quantized linear layer for AMD Instinct MI355X (gfx950).

The public API is the C ABI of ``libsdnq_hip.so`` (``include/sdnq_hip.h``); the
functions below are its ctypes binding, with the same names.
"""
from ._binding import (  # noqa: F401
    SDNQ_ERR_INVALID_ARG,
    SDNQ_ERR_LAUNCH,
    SDNQ_ERR_UNSUPPORTED,
    SDNQ_ERR_WORKSPACE,
    SDNQ_OK,
    SdnqError,
    lib,
    sdnq_attention_int8,
    sdnq_attention_workspace_bytes,
    sdnq_attention_workspace_offset,
    sdnq_gemm_fp8_f32,
    sdnq_gemm_i8_i32,
    sdnq_qlinear_backward_input,
    sdnq_qlinear_backward_input_fp8,
    sdnq_qlinear_forward,
    sdnq_qlinear_forward_noalloc,
    SDNQ_NOALLOC_SCRATCH_BYTES,
    sdnq_qlinear_forward_fp8,
    sdnq_qlinear_forward_fp8_quantized,
    sdnq_qlinear_forward_quantized,
    sdnq_rotate_quantize_act,
    sdnq_rotate_quantize_act_fp8,
    sdnq_rotate_quantize_weight,
    sdnq_rotate_quantize_weight_fp8,
    sdnq_svd_quantize_weight,
    sdnq_svd_workspace_bytes,
    sdnq_svd_workspace_q_offset,
    sdnq_qlinear_weight_grad,
    sdnq_weight_grad_workspace_offset,
    sdnq_weight_grad_workspace_bytes,
    sdnq_workspace_bytes,
    status_string,
)

"""FP32 matrix multiply C = A x B for the AMD Instinct MI355X (gfx950), plus the
sliding window sum that the same pages use to introduce cooperative staging,
and two cases of tiling beyond GEMM: the 2-D convolution run as an implicit
product and blockwise attention.

The product runs in libsgemm.so (hand-written HIP kernels behind the C ABI
in include/sgemm.h); this package only passes tensors' device addresses,
leading dimensions and the current stream to it.
"""
from .api import (SPLITK_HEADER_BYTES, SPLITK_MAX_TILES, attention, attention_raw, autotune, autotune_raw, config_has_general_form, config_info,
                  conv2d_config_available, conv2d_nhwc, conv2d_nhwc_raw, conv2d_output_size,
                  conv2d_select_config, conv2d_config_has_splitk, conv2d_nhwc_splitk,
                  conv2d_nhwc_splitk_raw, conv2d_splitk_plan,
                  config_selectable, num_configs, predict_us, select_config,
                  select_general_config, sgemm, sgemm_ex, sgemm_ex_raw, sgemm_raw,
                  config_has_splitk, sgemm_splitk, sgemm_splitk_noalloc, splitk_plan,
                  splitk_plan_full_tiles, splitk_workspace, config_has_general_splitk,
                  ex_splitk_plan, ex_splitk_plan_full_tiles, sgemm_ex_splitk, sgemm_ex_splitk_raw,
                  sgemm_strided_batched, sgemm_strided_batched_raw, window_sum,
                  window_sum_raw, workgroups_per_cu)
from ._native import SgemmError, status_string

__all__ = ["sgemm", "sgemm_strided_batched", "sgemm_raw", "sgemm_strided_batched_raw",
           "num_configs", "config_info", "select_config", "config_selectable", "predict_us",
           "autotune", "autotune_raw", "sgemm_ex", "sgemm_ex_raw", "config_has_general_form",
           "select_general_config", "window_sum", "window_sum_raw", "conv2d_nhwc",
           "conv2d_nhwc_raw", "conv2d_output_size", "conv2d_config_available",
           "conv2d_select_config", "conv2d_config_has_splitk", "conv2d_nhwc_splitk",
           "conv2d_nhwc_splitk_raw", "conv2d_splitk_plan", "workgroups_per_cu", "attention", "attention_raw",
           "sgemm_splitk", "sgemm_splitk_noalloc", "splitk_plan", "splitk_plan_full_tiles",
           "splitk_workspace", "config_has_splitk", "config_has_general_splitk",
           "ex_splitk_plan", "ex_splitk_plan_full_tiles", "sgemm_ex_splitk",
           "sgemm_ex_splitk_raw",
           "SPLITK_HEADER_BYTES", "SPLITK_MAX_TILES", "SgemmError",
           "status_string"]

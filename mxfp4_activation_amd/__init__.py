"""MI355X-native WUSH online activation path (fused per-block transform + 4-bit
quantization), as a C-ABI HIP library with a thin PyTorch binding.

    from mxfp4_activation_amd import quant_mxfp4
    codes, scales = quant_mxfp4(X_bf16, T_bf16)

The transform banks come from ``mxfp4_activation_amd.transforms`` (offline
construction in the library, on the device) or from the caller.
"""

from ._lib import FMT, LIB_PATH, WushError, load  # noqa: F401

__all__ = [
    "load", "WushError", "quant", "quant_mxfp4", "quant_nvfp4", "quant_int4", "transform_f32",
    "absmax_transformed", "nvfp4_global_scale", "e2m1_encode", "build_transforms", "fixed_transforms",
    "f64_to_bf16", "dequant", "gemm_mxfp4",
]


def __getattr__(name):
    # torch-dependent wrappers are imported on first use
    if name in __all__:
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)

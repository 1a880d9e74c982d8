"""MI355X-native FP8 block-scaled NT GEMM with M-grouped MoE variants.

The compute runs in the HIP library libdg.so (hand-written gfx950 kernels
behind a C ABI declared in include/dg.h); the Python layer only passes
device pointers, sizes and the current HIP stream.  The binding is loaded on
first use and raises if the library has not been built.
"""

__all__ = [
    "fp8_gemm_nt",
    "m_grouped_fp8_gemm_nt_contiguous",
    "m_grouped_fp8_gemm_nt_masked",
    "quantize_e4m3_1x128",
    "quantize_e4m3_128x128",
    "get_mk_alignment_for_contiguous_layout",
    "set_mk_alignment_for_contiguous_layout",
    "get_sf_aligned_size",
    "set_num_cus",
    "get_num_cus",
    "last_config",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)

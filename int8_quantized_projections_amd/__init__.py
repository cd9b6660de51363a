"""Q8_0 quantized projections for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libq8proj.so`` (C ABI in
``include/q8proj.h``). ``q8lib`` is a thin ctypes binding over it that only
marshals torch tensors into pointers and the current HIP stream.
"""
from . import q8lib  # noqa: F401
from .q8lib import (  # noqa: F401
    LAYOUT_PLANE64,
    LAYOUT_ROW,
    Q4KWeights,
    Q8Error,
    Q8Weights,
    act_bytes,
    alloc_act,
    gemv_plan,
    launch_counts,
    launch_counts_reset,
    q4k_gemm,
    q8_gemm,
    q8_gemm_shared_multi,
    q8_gemv,
    q8_gemv_f32,
    q8_gemv_shared_multi,
    q8_gemv_shared_multi_plus_f32,
    q8_quantize,
    q8_weights_repack,
    rmsnorm_quant,
    rmsnorm_quant_gemv_shared_multi_plus_f32,
    swiglu_quant,
)

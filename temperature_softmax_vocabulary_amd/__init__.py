"""MI355X-native (gfx950) temperature softmax over an LLM vocabulary, with
inverse-CDF token draws.

The computation lives in libtsoftmax.so (HIP kernels behind a C-ABI, see
include/tsoftmax.h); this package is a thin ctypes binding over it plus the
seeded workload generator. Build the library with
``python -m temperature_softmax_vocabulary_amd.build``.
"""
from .binding import (  # noqa: F401
    CHUNKS,
    LIB_PATH,
    TS_ERR_HIP,
    TS_ERR_INVALID_ARGUMENT,
    TS_ERR_NOT_RESERVED,
    TS_ERR_OUT_OF_MEMORY,
    TS_ERR_SYNC_TIMEOUT,
    TS_OK,
    TS_VARIANT_AUTO,
    TS_VARIANT_FUSED,
    TS_VARIANT_ROWWISE,
    TS_VARIANT_SPLIT,
    VARIANT_NAMES,
    TsError,
    lib,
    ts_abi_version,
    ts_copy_f32,
    ts_debug_set_resident_cap,
    ts_debug_set_spin_limit,
    ts_device_errors,
    ts_device_memory_params,
    ts_plan,
    ts_reserve,
    ts_sample,
    ts_softmax,
    ts_softmax_masked,
    ts_softmax_noalloc,
    ts_softmax_sample,
    ts_softmax_variant,
    ts_status_string,
)

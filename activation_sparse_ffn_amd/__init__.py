"""MI355X-native predictor-gated activation-sparse FFN step (libsfx).

The compute lives in libsfx.so (HIP kernels for gfx950 behind the C ABI in
include/sfx.h); this package is its ctypes binding plus buffer orchestration.
Build with `python -m activation_sparse_ffn_amd.build`.
"""
from ._abi import (SFX_BF16, SFX_F16, SFX_F32, SFX_MAX_B, SFX_MAX_GROUPS, SFX_Q4G32,  # noqa: F401
                   SFX_REGLU, SFX_RELU, SfxError, abi_version, load, sfx_compact, sfx_compact_ws,
                   sfx_predict, sfx_predict_ws, sfx_sparse_down, sfx_sparse_down_ws, sfx_sparse_up,
                   sfx_tam_update, sfx_tam_ws, status_str, workspace)
from ._abi import layer_descriptors, sfx_ffn_step, sfx_ffn_step_ws  # noqa: F401
from ._abi import sfx_ffn_pipeline, sfx_ffn_pipeline_ws, sfx_sparse_down_noalloc  # noqa: F401
from ._abi import sfx_hot_update, sfx_topk_now_update  # noqa: F401
from .step import HotRegion, StackStep, StepBuffers, TamState, TopKNowState, run_layer  # noqa: F401

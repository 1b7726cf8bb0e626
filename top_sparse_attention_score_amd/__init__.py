"""MI355X-native QSA top-k sparse attention: index scores + top-k, split-KV
attention over an int8 KV cache with fp16 scales, and the partial merge.

The computation lives in libqsa.so (hand-written HIP for gfx950, C ABI in
include/qsa.h); ``qsa`` is the ctypes binding.
"""
from .qsa import (QSA_ATTEND_AUTO, QSA_ATTEND_MATRIX, QSA_ATTEND_VECTOR,  # noqa: F401
                  QSA_F16, QSA_F32, QSA_NOALLOC_WORKSPACE_BYTES,  # noqa: F401
                  AppendDesc, AttnDesc, IndexDesc, QsaError,  # noqa: F401
                  QsaPath, append_desc, attn_desc, index_desc, path_for, qsa_attend,
                  qsa_attend_merge, qsa_step, qsa_step_workspace, StepCall,
                  qsa_decode_window, qsa_decode_window_workspace,
                  qsa_index_topk, qsa_index_topk_noalloc, qsa_kv_append, qsa_merge_gated,
                  qsa_index_topk_workspace, qsa_merge, qsa_partials_floats, to_device)

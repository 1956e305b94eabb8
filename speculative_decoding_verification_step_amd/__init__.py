"""MI355X-native speculative-decoding verification step.

The step streams the target weights once over all B*(K+1) drafted positions
(RMSNorm -> up -> SiLU -> down blocks, final RMSNorm, LM head) and then applies
modified rejection sampling per request.  All of it runs in the HIP kernels of
``libspecverify.so`` (C ABI in ``include/spec_verify.h``; the host-side
draft-length choice in ``include/spec_verify_kselect.h``, the paged attention of
the verified positions in ``include/spec_verify_attn.h``, a mixture-of-experts
target in ``include/spec_verify_moe.h``, the draft loop and the whole
speculative cycle in ``include/spec_verify_cycle.h``); this package is the
ctypes binding and the in-tree build.
"""
from .binding import (  # noqa: F401
    KV_BLOCK, KVPool, LIB_PATH, Model, MoEModel, SpecVerifyError, accept, accept_noalloc,
    accept_workspace_bytes, attention,
    attention_workspace_bytes, choose_k, cycle, cycle_workspace_bytes, embed, kv_append, kv_commit,
    lib, pack, profile_begin, profile_end, profile_pause, sample, sample_workspace_bytes, window_k, workspace,
    SV_OK, SV_ERR_INVALID_ARG, SV_ERR_UNSUPPORTED, SV_ERR_WORKSPACE, SV_ERR_HIP,
)

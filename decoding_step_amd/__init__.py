"""MI355X-native decode step of a masked diffusion LM (LM head + confidence + commit).

The compute path is the HIP library ``libdlm.so`` (C ABI in ``include/dlm.h``);
this package only binds it (``_native``), builds it (``build``), provides
device-memory helpers (``device``), the seeded synthetic inputs (``synth``)
and the workload table (``workloads``).
"""
from ._native import (  # noqa: F401
    DLM_AUTO_ADVANCE, DLM_BF16, DLM_CREDIT, DLM_CREDIT_SLOTS, DLM_F32, DLM_HIERARCHICAL, DLM_MAX_L,
    DLM_MAX_RULES, DLM_MAX_SEQS, DLM_OK, DLM_THRESHOLD, DlmError, StepPolicy,
    dlm_commit, dlm_decode_step, dlm_last_error, dlm_token_stats, dlm_version,
    dlm_workspace_bytes, dlm_workspace_init,
)

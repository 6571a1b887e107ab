"""CPU oracle for the masked-diffusion decode step -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check of ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (the HIP library and its Python binding) never imports, links or calls
it, and it imports nothing from the product path.

See :mod:`oracle.reference` for the definitions and the pages they follow.
"""
from .reference import (  # noqa: F401
    THRESHOLD, HIERARCHICAL, CREDIT, SLOTS,
    as_f64, lm_head_logits, token_stats, topk_candidates, shard_stats, merge_shards,
    commit_threshold, commit_hierarchical, commit_credit,
    RUNNING, FINISHED, EOS_IN_BLOCK, early_stop,
    decode_step,
)

"""CPU oracle for the DFlash drafter hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library.
"""
from .dflash_oracle import (  # noqa: F401
    OracleCache, accept, accept_ragged, attention, draft_forward, draft_forward_blocks,
    draft_forward_ragged,
    fuse_context, gumbel_pick, lm_head_argmax_ragged,
    inject_kv, lm_head_argmax, log_softmax_t, logsumexp_t, rmsnorm,
    sample_accept, sample_drafts, silu, store, to_bf16,
)

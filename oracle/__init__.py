"""fp64 CPU oracle (test infrastructure only; the HIP library never imports it).

See ``oracle.fa_oracle`` for what is computed and which page each step follows.
"""
from .fa_oracle import (  # noqa: F401
    NEG_INF,
    attention,
    attention_head,
    decode,
    gather_pages,
    is_visible,
    logsumexp,
    lse_merge,
    online_softmax_fa1,
    online_softmax_fa2,
    safe_softmax,
    split_partials,
    visible_mask,
)

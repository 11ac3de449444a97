"""CPU oracle of the KV-cached Talker forward (test infrastructure only).

Imported only by the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; the HIP library never uses it.
"""
from .talker import (  # noqa: F401
    TalkerOracle,
    causal_gqa_attention,
    rms_norm,
    rope_inv_freq,
    rope_neox,
    round_kv,
    silu,
    swiglu,
)

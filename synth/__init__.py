"""Seeded synthetic inputs shared by the CPU oracle side and the HIP side.

This package holds shapes, seeds and random draws only: it contains none of
the Talker forward's arithmetic.  See ``synth.talker_inputs``.
"""
from .talker_inputs import (  # noqa: F401
    TalkerShape,
    WORKLOADS,
    workload,
    make_weights,
    prefill_embeddings,
    step_embedding,
    batch_lengths,
    outlier_channels,
    round_to_bf16,
    embedding_tables,
    overlay_row,
)

"""Seeded synthetic inputs shared by the HIP path and the CPU oracle.

This module holds data generation only: random tensors, the per-cell offset
field that gives video tokens spatial locality, and random block selections
for the externally indexed modes.  It contains none of the method's
arithmetic (no tiling tables, pooling, routing, TopK or attention), so that
both sides can read the same values without sharing any computation.

Every generator takes an explicit ``device`` and draws from a
``torch.Generator`` seeded with the workload's seed, in the order documented
in each function.  Values on a CUDA device and on the CPU come from different
generator streams, so a comparison always hands the oracle a host copy of
exactly the tensors the device computed on.
"""

from .configs import WORKLOADS, workload, scaled
from .gen import vsa_inputs, nsa_inputs, msa_inputs, kept_lists, coarse_gate, h3_inputs

__all__ = [
    "kept_lists",
    "coarse_gate",
    "WORKLOADS",
    "workload",
    "scaled",
    "vsa_inputs",
    "h3_inputs",
    "nsa_inputs",
    "msa_inputs",
]

"""Seeded synthetic inputs for the KV-cache eviction step.

This package only draws random numbers and lays them out in the shapes the
eviction step consumes.  It holds none of the step's arithmetic (no rotary
embedding, no attention, no selection, no sampling): both the CPU oracle and
the GPU library receive the same tensors from here and do their own work.
"""
from .specs import Workload, WORKLOADS, get_workload  # noqa: F401
from .gen import make_layer, make_append, make_traces, request_lengths, initial_recent_obs, make_sentences, \
    random_layer, random_rows  # noqa: F401

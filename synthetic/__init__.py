"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package holds only random-number generation and dtype rounding. It holds
none of the attention arithmetic, so neither side can borrow the other's
computation through it.
"""
from .inputs import GlobalProblem, global_problem, WORKLOADS, workload, doc_starts

__all__ = ["GlobalProblem", "global_problem", "WORKLOADS", "workload", "doc_starts"]

"""Seeded synthetic inputs for the routed-expert MoE layer.

This package is shared by the CPU oracle, the tests and the benchmark.  It
only *creates* inputs (weights, activations, router matrices or logits,
routing traces, slot permutations) and holds none of the layer's arithmetic:
no dequantisation, routing, FFN or combine.
"""
from .inputs import *  # noqa: F401,F403

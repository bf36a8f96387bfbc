"""Seeded synthetic inputs for the expert-cached MoE layer.

This package draws the inputs that both the fp64 oracle and the HIP path
consume: expert weights in their storage format, activations, router logits and
decode routing traces.  It holds none of the layer's arithmetic (no routing, no
expert FFN, no cache policy); it only draws numbers and stores them in the
element formats the layer reads (fp32, bf16 bit patterns, MXFP4 codes+scales).
"""
from .gen import *  # noqa: F401,F403

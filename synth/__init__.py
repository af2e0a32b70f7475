"""Seeded synthetic workloads for the KV4-RL decode-attention path.

This package only draws inputs: context lengths, page tables, slot ids and
BF16 query/key/value tensors.  It holds none of the method's arithmetic (no
rotation, no quantizer, no attention); both the CPU oracle and the HIP path
consume what it produces.

Workload shapes follow the KV4-RL pages (paper.rainbus.top summary, "研究动机"
and "方法步骤详情"; onedev.kr summary, "어떻게 동작하나"): GQA decode with
head_dim 128, page size 16, a length-biased response-position law (the
inspection paradox behind KV concentration, Prop. 4.1) and K values with a few
fixed outlier channels, the situation the Hadamard rotation is there for.
"""
from .lengths import lognormal_moments_to_params, sample_contexts, law_mean_context
from .configs import CONFIGS, Workload, make_workload
from .values import draw_values, outlier_channels

__all__ = [
    "lognormal_moments_to_params", "sample_contexts", "law_mean_context",
    "CONFIGS", "Workload", "make_workload", "draw_values", "outlier_channels",
]

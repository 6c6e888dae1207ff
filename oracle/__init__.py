"""CPU oracle of the sparse MoE layer -- test infrastructure only.

Importable by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py``; never by the GPU library.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (F64, precision, biased_logits, build_index, combine,  # noqa: F401
                         combine_backward, count_tokens, gate_backward,
                         gate_weights, grouped_matmul, grouped_matmul_backward,
                         layer_backward, layer_forward, permute,
                         permute_backward, rel_fro, route, router_backward,
                         router_logits, sigmoid, silu, softmax, swiglu,
                         swiglu_backward, topk_experts)

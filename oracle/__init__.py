"""CPU oracle for the DBO expert-parallel MoE layer — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it and
shares no code with it: it is a plain, slow, float64 restatement of what the
layer computes, used to check the GPU path.

What it follows:
  * the split of a batch into two microbatches whose MoE results are simply
    stacked ("[Core/DBO][1/N] Add Dual-Batch Overlap mechanism to VLLM",
    Purpose; the second microbatch continues a request the first one began,
    "[Core/DBO][2/N] ... Prefill support", Purpose);
  * dispatch -> experts -> combine, the prepare/experts/finalize chain of the
    fused-MoE layer ("[Core/DBO][2/N]", review of modular_kernel.py);
  * the SwiGLU expert the pages name through its act-and-mul kernel
    ("[Core/DBO][1/N]", performance discussion) and the fused SiLU-mul op
    ("[Core/DBO][1/N]", CI discussion);
  * worst-case dispatch capacity of tokens x dispatchers ("DeepEP HT: full
    decode CUDA graphs via worst-token dispatch", bot review 2).
The pages print no routing formula, no top-k rule, no fp8 scaling rule and no
worked example; every such step here is one stated reading (the readings table
of the design notes), and the module docstrings name which.

Parity status: every function is pinned by the ``-m "not gpu"`` tests
(closed forms, brute force on tiny inputs, library special cases, invariants,
hand-derived golden values under tests/golden/).  None is "parity unpinned".
"""
from .numerics import fp8_e4m3fn_value, FP8_E4M3FN_TABLE, decode, dequant_fp8_blocks
from .routing import router_logits, softmax_rows, sigmoid, select_topk, select_grouped, route
from .dispatch import dispatch_ref
from .ffn import silu, swiglu_expert, grouped_ffn_ref
from .quant import (fp8_e4m3fn_encode, group_exponent, quant_rows_fp8, dequant_rows_fp8,
                    fp8_roundtrip_rows, swiglu_expert_fp8act, grouped_ffn_fp8act_ref)
from .layer import (split_point, expert_weights, shared_weights, moe_layer_token,
                    moe_layer_expert, moe_layer_microbatched, combine_ref, slice_view)

__all__ = [
    "fp8_e4m3fn_value", "FP8_E4M3FN_TABLE", "decode", "dequant_fp8_blocks",
    "router_logits", "softmax_rows", "sigmoid", "select_topk", "select_grouped", "route",
    "dispatch_ref", "silu", "swiglu_expert", "grouped_ffn_ref",
    "fp8_e4m3fn_encode", "group_exponent", "quant_rows_fp8", "dequant_rows_fp8",
    "fp8_roundtrip_rows", "swiglu_expert_fp8act", "grouped_ffn_fp8act_ref",
    "split_point", "expert_weights", "shared_weights", "moe_layer_token", "moe_layer_expert",
    "moe_layer_microbatched", "combine_ref", "slice_view",
]

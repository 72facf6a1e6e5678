"""CPU: the benchmark's roofline accounting, pinned to numbers the pages print.

bench.py prices the dominant kernel (the routed experts' first projection)
and the whole layer by algorithmic bytes and flops.  The per-expert weight
sizes those formulas imply must be the expert tensors of 24 MiB (fused gate
and up projection) and 12 MiB (down projection) in bf16 that the miles page
lists for Step-5-Preview (section 5.3 Optimizer), at the Model Architecture
table's hidden size 4096 and expert width 1536; the totals below are those
sizes written out by hand for the 8192-token prefill.
"""
import json
import os

import bench
import moe_inputs as mi

HERE = os.path.dirname(os.path.abspath(__file__))
FACTS = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))
MIB = 2 ** 20


def test_expert_tensor_sizes_match_the_page():
    arch, routing = FACTS["step5_architecture"], FACTS["step5_routing"]
    c = mi.WORKLOADS["step5_prefill"].cfg
    assert (c.hidden_size, c.moe_intermediate_size, c.num_experts, c.top_k) == (
        arch["hidden_size"], arch["expert_intermediate_size"], arch["routed_experts"], arch["top_k"])
    w2_mib, w13_mib = routing["fp8_expert_tensor_mib"]
    assert c.hidden_size * c.moe_intermediate_size * 2 == w2_mib * MIB
    assert 2 * c.moe_intermediate_size * c.hidden_size * 2 == w13_mib * MIB


def test_first_projection_bytes():
    wl = mi.WORKLOADS["step5_prefill"]
    touched = 284
    T, k = 8192, 8
    want = (touched * 24 * MIB          # W13 of every touched expert, once
            + T * 4096 * 2              # x, once
            + T * k * 1536 * 2)         # h of the routed rows, written once
    assert bench.up_kernel_bytes(wl, touched) == want == 7_415_529_472


def test_layer_bytes_and_flops():
    wl = mi.WORKLOADS["step5_prefill"]
    touched, T, E, H, I, k = 284, 8192, 352, 4096, 1536, 8
    want_bytes = (touched * 36 * MIB + 36 * MIB   # routed experts touched, shared expert
                  + E * H * 2 + E * 4             # router weight, bias
                  + T * H * 2 + T * H * 4)        # x in, fp32 out
    assert bench.layer_bytes(wl, touched) == want_bytes
    # router GEMM + three projections of every routed pair + the shared expert's
    want_flops = 2 * T * E * H + 3 * (2 * T * k * H * I) + 3 * (2 * T * H * I)
    assert bench.layer_flops(wl, touched) == want_flops


def test_fp8_first_projection_bytes():
    wl = mi.WORKLOADS["step5_fp8_prefill"]
    touched, T, H, I, k = 284, 8192, 4096, 1536, 8
    # one byte per code, one fp32 scale per 128 x 128 block; h as codes plus
    # one fp32 scale per 128 columns of a row
    w13 = 2 * I * H + (2 * I // 128) * (H // 128) * 4
    want = touched * w13 + T * H * 2 + T * k * (I + I // 128 * 4)
    assert w13 == 12 * MIB + 3072
    assert bench.up_kernel_bytes(wl, touched) == want

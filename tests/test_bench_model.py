"""CPU: the benchmark's roofline accounting, pinned to numbers the pages print.

bench.py prices the dominant kernel (the routed experts' first projection,
with the shared expert as one more group of the launch) and the whole layer
by algorithmic bytes and flops: weights once, activations in once, outputs
out once; intermediates (h, the expert rows) are not counted.  The per-expert weight
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
    T = 8192
    want = (touched * 24 * MIB          # W13 of every touched expert, once
            + 24 * MIB                  # the shared expert's, a group of the same launch
            + T * 4096 * 2)             # x, once (h is an intermediate: not counted)
    assert bench.up_kernel_bytes(wl, touched) == want == 7_239_368_704
    # its flops: the routed pairs' and the shared expert's rows, gate and up
    assert bench.up_kernel_flops(wl) == 2 * (T * 8 + T) * 2 * 1536 * 4096


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
    touched, T, H, I = 284, 8192, 4096, 1536
    # one byte per code, one fp32 scale per 128 x 128 block; x read once as
    # codes with one fp32 scale per 128 columns of a row (the shared expert
    # runs in bf16 launches of its own)
    w13 = 2 * I * H + (2 * I // 128) * (H // 128) * 4
    want = touched * w13 + T * H + T * (H // 128) * 4
    assert w13 == 12 * MIB + 3072
    assert bench.up_kernel_bytes(wl, touched) == want


def test_fp8_layer_bytes_count_block_scales():
    wl = mi.WORKLOADS["step5_fp8_prefill"]
    touched, T, E, H, I = 284, 8192, 352, 4096, 1536
    scales = touched * ((2 * I // 128) * (H // 128) + (H // 128) * (I // 128)) * 4
    want = touched * 18 * MIB + scales + 36 * MIB + E * H * 2 + E * 4 + T * H * 2 + T * H * 4
    assert bench.layer_bytes(wl, touched) == want


def test_counter_summaries_carry_traffic_and_source_hash():
    """Each committed counter summary that bench.py reads for `traffic` names
    the bytes per launch and the SHA-256 of the kernel source it was taken
    on (bench.py reports the bytes only while that source is unchanged)."""
    import re
    for name, (summary, src) in bench.TRAFFIC_FILES.items():
        assert name in mi.WORKLOADS
        text = open(summary).read()
        t = re.search(r"^traffic_bytes_per_launch:\s*(\d+)$", text, re.M)
        h = re.search(r"^kernel_source_sha256:\s*([0-9a-f]{64})$", text, re.M)
        assert t and h, summary
        assert 1e9 < int(t.group(1)) < 2e10
        assert os.path.exists(src)

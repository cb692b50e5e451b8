"""Byte accounting pinned to the memory table the pages print."""
import os

import pytest

from block_diffusion_drafter_ctx_amd import roofline as rf

GOLD = os.path.join(os.path.dirname(__file__), "golden", "jp_memory_table.txt")


def _golden():
    out = {}
    for line in open(GOLD, encoding="utf-8"):
        line = line.split("#")[0].strip()
        if line:
            k, v, rel = line.split()[:3]
            out[k] = (float(v), rel)
    return out


def test_memory_table():
    g = _golden()
    D, T, n, gamma = 2048, 2048, 5, 16
    assert rf.w_c_bytes(D, n) == 5 * 2048 * 2048 * 2 == 41_943_040
    ours = {
        "w_c_params": rf.w_c_bytes(D, n),
        "projection_input": rf.fusion_input_bytes(T, D, n),
        "projection_output": rf.fusion_output_bytes(T, D),
    }
    for k, val in ours.items():
        printed, rel = g[k]
        assert rel == "approx"
        # the page rounds to whole MB (its 40 MB input is 40 MiB = 41.9 MB)
        assert abs(val - printed) / printed < 0.06, (k, val, printed)
    # decode-time temporaries at block 16: the block's residual, normed input and
    # attention output rows in bf16 stay below the page's bound
    printed, rel = g["decode_temporaries_block16"]
    assert rel == "below"
    assert 3 * gamma * D * 2 < printed


def test_stage_formulas_closed_forms():
    # Qwen3-8B-shaped drafter layer: 192.94 M parameters incl. gains
    assert rf.layer_weight_elems(4096, 32, 8, 128, 12288) == 192_946_176
    assert rf.fuse_flops(2048, 4096) == 2 * 2048 * 5 * 4096 * 4096
    assert rf.inject_bytes(0, 4096, 5, 8, 128) == 2 * 5 * 8 * 128 * 4096 * 2
    b = rf.draft_forward_bytes(4096, 5, 32, 8, 128, 12288, 151936, 1, 16, [2048])
    assert 3.2e9 < b < 3.25e9


@pytest.mark.parametrize("gamma", [8, 16, 32])
def test_draft_bytes_nearly_flat_in_gamma(gamma):
    # The pages' claim that a parallel draft costs about one forward whatever
    # the block size shows up as weight bytes dominating the traffic.
    b8 = rf.draft_forward_bytes(4096, 8, 32, 8, 128, 12288, 151936, 4, 8, [8192] * 4)
    bg = rf.draft_forward_bytes(4096, 8, 32, 8, 128, 12288, 151936, 4, gamma, [8192] * 4)
    assert bg / b8 < 1.01

"""Writes tests/golden/v3_skew_bias.txt: the routing bias of the load-skewed
V3 prefill workload (T=16384, 256 experts, top-8 of 8 groups / 4 kept).

Calls only ``synth`` and ``oracle``: the oracle routes a seeded calibration
batch (tensor id 5, 4096 tokens, same distribution as the workload's x) with
the router weights of the workload, and adjusts the per-expert bias by the
overloaded/underloaded rule (onlylabs "DeepSeek v3 and R1 Model
Architecture", section "Local Balanced Routing to Experts") toward a Zipf(1.2)
load profile capped at 20x the mean, with 16 empty experts.

Run from the repository root:  python tests/golden/make_skew_bias.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import calibrate, route  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "v3_skew_bias.txt")
CAL_TOKENS = 4096


def main():
    s = synth.V3_SKEW
    x = synth.bf16_bits_to_f32(synth.gen_x(s, tokens=CAL_TOKENS, tensor_id=synth.T_CAL))
    wr = synth.bf16_bits_to_f32(synth.gen_router_w(s))
    scores = route.sigmoid_scores(route.router_logits(x, wr))
    target = synth.zipf_targets(CAL_TOKENS, s.top_k, s.n_experts)
    bias, ld = calibrate.calibrate(scores, target, s.n_group, s.topk_group, s.top_k)
    mean = ld.mean()
    with open(OUT, "w") as f:
        f.write("# routing bias (fp32 bit patterns, one per expert) of the load-skewed V3 prefill workload\n")
        f.write(f"# written by tests/golden/make_skew_bias.py; calibration batch {CAL_TOKENS} tokens\n")
        f.write(f"# achieved on the calibration batch: top/mean {ld.max() / mean:.2f}, empty {int((ld == 0).sum())}, "
                f"min non-empty {int(ld[ld > 0].min())}, max {int(ld.max())}\n")
        for v in bias:
            f.write(f"{int(np.float32(v).view(np.uint32)):08x}\n")
    print(open(OUT).read().splitlines()[2])


if __name__ == "__main__":
    main()

"""Writes tests/golden/skew_t64k_expert_bias.txt: the expert bias of the skewed
65536-token workload, derived from the oracle's first routing pass (no bias)
over that workload's synthetic router inputs, by the oracle's expert-bias
update from a zero bias at rate 0.1:
    bias_e = -0.1 * (count_e - mean) / max_e |count_e - mean|,  mean = T*k/E.
Calls only oracle/ and the seeded input generator.

    python tests/golden/make_skew_bias.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from group_limited_top_amd import synth  # noqa: E402


def skew_bias():
    shape = synth.WORKLOADS["skew_t64k"]
    x, wr, _ = synth.router_inputs(shape)
    idx, _, flag, _ = oracle.route(synth.to_numpy_bits(x), wr.numpy(), None, shape.n_group,
                                   shape.topk_group, shape.top_k, shape.scale)
    assert not flag.any()
    counts = np.bincount(idx.reshape(-1), minlength=shape.E).astype(np.int32)
    bias = oracle.bias_update(counts, None, 0.1)
    return counts, bias


if __name__ == "__main__":
    counts, bias = skew_bias()
    out = os.path.join(HERE, "skew_t64k_expert_bias.txt")
    with open(out, "w") as f:
        f.write("# expert bias of the skew_t64k workload (written by make_skew_bias.py from the\n")
        f.write("# oracle's unbiased routing counts; one fp32 value per expert, repr-exact)\n")
        for v in bias:
            f.write(f"{float(v)!r}\n")
    top = np.sort(counts)[::-1]
    print(f"wrote {out}; hottest expert {top[0]} hits, top-20 share {top[:20].sum() / counts.sum():.3f}")

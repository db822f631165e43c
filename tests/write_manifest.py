"""Write tests/manifest.json: the seeded workloads, their shapes, and the parity bars.

Everything here is read from synth (seeds, shapes) and from the oracle's
comparison module (tolerances); test_manifest_matches checks that the committed
file is what this script writes.  Run from the repository root:
python3 tests/write_manifest.py
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def manifest():
    dense = {name: {"seed": c.seed, "m": c.m, "n": c.n, "k": c.k, "group": c.group,
                    "weights": f"fp32 N(0, {synth.WEIGHT_STD}^2) [n, k], drawn first",
                    "activations": "fp32 N(0, 1) [m, k] cast to fp16 (round to nearest even)"
                                   + ("; drawn as [4096, k], the first m rows" if name.startswith("gemm_") else "")}
             for name, c in synth.DENSE_CASES.items()}
    moe = {name: {"seed": c.seed, "tokens": c.tokens, "experts": c.experts, "topk": c.topk, "n": c.n, "k": c.k,
                  "group": c.group,
                  "recipe": "per-expert fp32 weights e = 0..E-1, then fp16 x [tokens, k], then for each token in "
                            "order topk distinct experts uniformly; pairs sorted by (expert, token)"}
           for name, c in synth.MOE_CASES.items()}
    extra = {
        "batched_decode_m16": "weights of gemv_np4_4x5120x17408_g128; x fp16 [16, 5120] from default_rng(seed + 100)",
        "swiglu_gate_up": "gate then up fp32 weights [17408, 5120] from default_rng(seed of gemv_up_1x5120x17408_g128 "
                          "+ 200), rows interleaved (gate 2i, up 2i + 1); x [m, 5120] from the same generator",
        "moe_router_weights": "softmax over N(0, 1) logits [tokens, topk] from default_rng(moe seed + 500), fp32",
    }
    return {
        "generator": "numpy.random.default_rng(seed) (PCG64)",
        "dense": dense,
        "moe": moe,
        "other_workloads": extra,
        "parity": {
            "floating_point": {"elementwise": f"|y - y_ref| <= {oracle.ELEM_TOL} * max|y_ref|",
                               "per_row": f"||y_row - y_ref_row||_2 <= {oracle.ROW_TOL} * ||y_ref_row||_2",
                               "reference": "fp64 oracle (dequantise, then matrix product), y_ref rounded to fp16 "
                                            "for comparison only where stated"},
            "bit_exact": "integer activations in [-2, 2], codes in [-8, 7], power-of-two scales: every sum is "
                         "exact, so the fp16 outputs must equal the oracle's bit for bit",
            "integer_work": "pack / unpack / quantise codes, MoE routing offsets: bit-exact",
            "unordered": "rows inside one expert after routing: any order; checked as a valid permutation",
        },
    }


def main():
    path = os.path.join(ROOT, "tests", "manifest.json")
    with open(path, "w") as f:
        json.dump(manifest(), f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()

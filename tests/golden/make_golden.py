"""Writes the oracle's outputs for small seeded workloads as regression fixtures.

Run from the repository root:  python tests/golden/make_golden.py
Only `synth` (inputs) and `oracle` (expected values) are used.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json")


def main():
    cases = []
    for run in range(4):
        x = synth.make_config(1, run)
        o = oracle.verify_chain(x.logits, x.q, x.tokens, x.u, x.temperature, x.logit_dtype)
        cases.append(dict(kind="chain", config=1, run=run,
                          accepted_len=o["accepted_len"].tolist(),
                          out_tokens=o["out_tokens"].tolist(), status=o["status"].tolist(),
                          flagged=o["flagged"].tolist()))
    for run in range(2):
        x = synth.make_config(4, run, B=8, gamma=6, V=300)
        o = oracle.verify_greedy(x.logits, x.tokens, x.logit_dtype)
        cases.append(dict(kind="greedy", config=4, run=run, override=dict(B=8, gamma=6, V=300),
                          accepted_len=o["accepted_len"].tolist(),
                          out_tokens=o["out_tokens"].tolist(), status=o["status"].tolist()))
    for run in range(2):
        x = synth.make_config(5, run, B=4, N=15, V=64, boost=6.0)
        o = oracle.verify_tree(x.logits, x.parents, x.node_tokens, x.u, x.temperature, x.logit_dtype)
        cases.append(dict(kind="tree", config=5, run=run, override=dict(B=4, N=15, V=64, boost=6.0),
                          accepted_len=o["accepted_len"].tolist(),
                          out_tokens=o["out_tokens"].tolist(), out_nodes=o["out_nodes"].tolist(),
                          status=o["status"].tolist()))
    for run in range(2):
        x = synth.make_config(6, run, B=6, N=13, V=48, per_child=bool(run))
        o = oracle.verify_tree_residual(x.logits, x.q, x.parents, x.node_tokens, x.u_acc, x.u_draw,
                                        x.temperature, x.logit_dtype)
        cases.append(dict(kind="tree_residual", config=6, run=run,
                          override=dict(B=6, N=13, V=48, per_child=bool(run)),
                          accepted_len=o["accepted_len"].tolist(),
                          out_tokens=o["out_tokens"].tolist(), out_nodes=o["out_nodes"].tolist(),
                          status=o["status"].tolist()))
    with open(OUT, "w") as f:
        json.dump(dict(note="written by tests/golden/make_golden.py from oracle/ outputs", cases=cases),
                  f, indent=1)
    print("wrote", OUT)


if __name__ == "__main__":
    main()

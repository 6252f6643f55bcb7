"""Writes the stored expected values under tests/golden/ by calling only the oracle.

    python tests/golden/make_golden.py

gpt2_124m_b4t64_fp32_steps.json: the float64 oracle's loss before each of 10
consecutive forward+backward+AdamW steps over one fixed batch of the GPT-2
124M shape at B=4, T=64 (the over-fit-one-batch run described in
"1000 行 C 代码完成 GPT-2 训练的 LLM.c", section 快速开始吧！), with the seeded
synthetic weights and tokens, plus checksums of the final parameters.
"""
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def ten_steps(name="gpt2_124m_b4t64_fp32", steps=10):
    w = synth.WORKLOADS[name]
    o = oracle.Oracle(w.model, w.B, w.T, "f64")
    o.set("params", synth.init_params(w.model))
    x, y = synth.inputs_targets(w)
    losses = []
    for t in range(1, steps + 1):
        t0 = time.time()
        losses.append(o.step(x, y, w, t))
        print(f"step {t}: loss {losses[-1]:.12f} ({time.time() - t0:.1f} s)", flush=True)
    p = o.get("params")
    return {
        "_source": "written by tests/golden/make_golden.py from the float64 oracle",
        "workload": name,
        "losses": losses,
        "final_params_sum": float(p.sum()),
        "final_params_abs_sum": float(np.abs(p).sum()),
    }


if __name__ == "__main__":
    out = ten_steps()
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gpt2_124m_b4t64_fp32_steps.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)

"""Writes tests/golden/tiny_layer.json: expected values of one small fp32 MoE
layer (T 12, H 64, E 6, top-2, I 32, gated shared expert with Is 32,
sqrtsoftplus scores with an fp32 selection bias, renorm), computed by the
oracle alone from the seeded CPU inputs of workloads.make_inputs.

The pages print no worked numeric example of the layer, so the stored values
are the oracle's: the router ("mstar.model.components.moe", Router contract;
"Sparse MoE FFN for DFlash-family drafters", What's here: MoEGate), the
counting-sort dispatch ("feat: Phase 43", dispatch path) and the dense-masked
layer output ("feat: Phase 43", equivalence of the sparse path with the
dense-masked one).  Run from the repository root:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import moe_ref as R  # noqa: E402
from workloads import Workload, make_inputs  # noqa: E402

WORKLOAD = Workload("golden_tiny", T=12, H=64, E=6, k=2, I=32, Is=32, score=2, renorm=True, shared_gated=True,
                    dtype="fp32", bias_var=0.5, seed=7)
PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_layer.json")


def compute():
    w = WORKLOAD
    inp = {k: v.numpy().astype(np.float64) for k, v in make_inputs(w, device="cpu").items()}
    res = R.layer_forward(inp["x"], inp["w_router"], w.k, w.score, w.renorm, inp["w_gate_up"], inp["w_down"],
                          inp["ws_gate_up"], inp["ws_down"], inp["w_shared_gate"],
                          sel_bias=inp["sel_bias"].astype(np.float32))
    d = R.dispatch(res["ids"], w.E)
    return {
        "workload": {k: getattr(w, k) for k in ("T", "H", "E", "k", "I", "Is", "score", "renorm", "shared_gated",
                                                "dtype", "bias_var", "seed")},
        "logits32": res["logits"].astype(np.float32).astype(np.float64).tolist(),
        "ids": res["ids"].astype(np.int64).tolist(),
        "weights": res["weights"].tolist(),
        "counts": d["counts"].astype(np.int64).tolist(),
        "offsets": d["offsets"].astype(np.int64).tolist(),
        "perm": d["perm"].astype(np.int64).tolist(),
        "pos": d["pos"].astype(np.int64).tolist(),
        "out": res["out"].tolist(),
    }


if __name__ == "__main__":
    with open(PATH, "w") as f:
        json.dump(compute(), f, indent=None, separators=(",", ":"))
        f.write("\n")
    print("wrote", PATH)

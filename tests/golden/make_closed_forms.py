"""Writes the hand-derived fixtures in this folder.

closed_forms.json: tiny attention cases whose outputs follow in closed form
from the definition (scores, row softmax, product with V; gradients by the
chain rule).  The derivation of every number is stored next to it.  Nothing
here calls the oracle or the GPU path: these values are what both are
checked against.

worked_example_memory.json: the sizes stated on the glossary page "Flash
Attention", sections "Worked example" and "Check your understanding".

Run from the repository root:  python tests/golden/make_closed_forms.py
"""

import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def closed_forms():
    e = math.e
    ln2, ln3 = math.log(2.0), math.log(3.0)
    return {
        "citation": (
            "Closed forms of the attention definition (score matrix, row softmax, "
            "product with V) as described on 'How Flash Attention Improves "
            "Transformer Memory Efficiency ...', sections 'Full Matrix Construction' "
            "and 'Intermediate Tensor Storage'; causal mask per the glossary page "
            "'Flash Attention', FAQ on attention masks. Values worked out by hand; "
            "see 'derivation'."),
        "forward": {
            "scale": 1.0,
            "q": [[1.0, 0.0], [0.0, 1.0]],
            "k": [[0.0, 0.0], [ln2, 0.0], [ln3, 1.0]],
            "v": [[6.0, 0.0], [0.0, 6.0], [6.0, 6.0]],
            "derivation": [
                "row 0 scores (0, ln2, ln3) -> exp (1, 2, 3), sum 6: "
                "P=(1/6, 2/6, 3/6), lse=ln 6, O=(1+3, 2+3)=(4, 5)",
                "row 1 scores (0, 0, 1) -> exp (1, 1, e), sum 2+e: lse=ln(2+e), "
                "O=((6+6e)/(2+e), (6+6e)/(2+e))",
                "causal: row 0 sees key 0 only -> O=V0=(6,0), lse=S00=0; row 1 sees "
                "keys 0,1 with scores (0,0) -> P=(1/2,1/2), O=(3,3), lse=ln 2",
            ],
            "noncausal": {
                "O": [[4.0, 5.0], [(6 + 6 * e) / (2 + e)] * 2],
                "lse": [math.log(6.0), math.log(2.0 + e)],
            },
            "causal": {"O": [[6.0, 0.0], [3.0, 3.0]], "lse": [0.0, ln2]},
        },
        "backward": {
            "scale": 1.0,
            "q": [[1.0]],
            "k": [[0.0], [ln2]],
            "v": [[0.0], [3.0]],
            "dO": [[1.0]],
            "derivation": [
                "scores (0, ln2) -> P=(1/3, 2/3), O=2",
                "dV_j = P_j dO = (1/3, 2/3); dP_j = dO v_j = (0, 3); D = dO*O = 2",
                "dS_j = P_j (dP_j - D) = (-2/3, 2/3); dQ = scale * sum_j dS_j k_j = "
                "(2/3) ln 2; dK_j = scale * dS_j q = (-2/3, 2/3)",
            ],
            "dq": [[2.0 / 3.0 * ln2]],
            "dk": [[-2.0 / 3.0], [2.0 / 3.0]],
            "dv": [[1.0 / 3.0], [2.0 / 3.0]],
        },
    }


def worked_example_memory():
    return {
        "citation": (
            "Glossary page 'Flash Attention', sections 'Worked example' and 'Check "
            "your understanding': one head, one 4,096-token sequence, two bytes per "
            "stored score"),
        "L": 4096,
        "elements": 16777216,
        "bytes_per_element": 2,
        "bytes": 33554432,
        "MiB": 32,
        "L_doubled": 8192,
        "MiB_doubled": 128,
        "growth_when_L_doubles": 4,
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "closed_forms.json"), "w") as f:
        json.dump(closed_forms(), f, indent=1)
    with open(os.path.join(HERE, "worked_example_memory.json"), "w") as f:
        json.dump(worked_example_memory(), f, indent=1)

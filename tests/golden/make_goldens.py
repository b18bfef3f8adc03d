"""Write the stored expected values under tests/golden/ from the oracle's
60-digit brute force (oracle/bruteforce.py) alone.

    python tests/golden/make_goldens.py

two_class.json: rows z = (0, d) with target column 1, i.e. a target margin
of d over a single competitor, for margins on both sides of the collapse
margin the torchtitan PR "[loss] fix softmax collapse with improved ce perf"
names in its opening summary (about 16.6, where fp32 rounds p_t to exactly 1;
every margin here is exact in bf16 and fp32)
and up to 40.  Stored as decimal strings with 30 significant digits.

equal_competitors.json: rows of V - 1 equal non-targets at 0 and the target
at d (the collapse regime with a large vocabulary).
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle.bruteforce import ce_row  # noqa: E402

MARGINS = [0.5, 4.0, 10.0, 16.5, 16.625, 16.75, 20.0, 25.0, 30.0, 40.0]


def main():
    rows = []
    for d in MARGINS:
        loss, g = ce_row([0.0, d], 1)
        rows.append({"z": [0.0, d], "target": 1, "loss": f"{loss:.30e}",
                     "grad": [f"{v:.30e}" for v in g]})
    with open(os.path.join(HERE, "two_class.json"), "w") as f:
        json.dump({"source": "oracle/bruteforce.py (decimal, 60 digits)", "rows": rows}, f,
                  indent=1)
    rows = []
    for V, d in [(8, 20.0), (1000, 25.0), (32000, 30.0), (128256, 40.0)]:
        z = [0.0] * V
        z[V // 2] = d
        loss, g = ce_row(z, V // 2)
        rows.append({"V": V, "target": V // 2, "margin": d, "loss": f"{loss:.30e}",
                     "grad_target": f"{g[V // 2]:.30e}", "grad_other": f"{g[0]:.30e}"})
    with open(os.path.join(HERE, "equal_competitors.json"), "w") as f:
        json.dump({"source": "oracle/bruteforce.py (decimal, 60 digits)", "rows": rows}, f,
                  indent=1)


if __name__ == "__main__":
    main()

"""Write tests/golden/tiny_rope_oracle.json from the fp64 oracle alone.

The pages print no worked example for the rotary embedding (neither the
Chronicals abstract nor the Unsloth articles give numbers per element), so
this fixture is a regression lock on the oracle: small fixed inputs, the
oracle's float64 outputs (forward and backward) and their bfloat16 roundings.
It calls only ``oracle`` and numpy.  Re-run it only when a change to the
oracle's arithmetic is justified by a reading of the pages.

    python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402


def main():
    T, H, D, theta = 6, 2, 8, 10000.0
    cu = [0, 3, 3, 5]  # an empty segment, and token 5 outside every sequence
    # exactly representable inputs: multiples of 1/8 in [-2, 2]
    x = ((np.arange(T * H * D).reshape(T, H, D) * 7) % 33 - 16) / 8.0
    out = {
        "what": "rotate_half RoPE of a tiny packed batch, fp64 oracle outputs",
        "T": T, "H": H, "D": D, "theta": theta, "cu_seqlens": cu,
        "x": x.tolist(),
    }
    for name, d in (("fwd", 1), ("bwd", -1)):
        y = oracle.rope(x, np.array(cu), theta, d)
        out[name] = [float.hex(float(v)) for v in y.ravel()]
        out[name + "_bf16_bits"] = [int(b) for b in oracle.bf16_bits(oracle.bf16_rne(y)).ravel()]
    out["positions"] = [int(p) for p in oracle.segment_positions(np.array(cu), T)]
    with open(os.path.join(HERE, "tiny_rope_oracle.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()

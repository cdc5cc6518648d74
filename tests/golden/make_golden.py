"""Writes tests/golden/tiny_e4_h64_f128.json from the CPU oracle only.

The pages print no worked numeric example for this path, so this fixture is
a regression guard: the SHA-256 of the oracle's bf16 outputs on the seeded
4-expert workload (expert 2 empty), plus a handful of values.  Run
``python tests/golden/make_golden.py`` to regenerate after a change that a
cited passage justifies.
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workload  # noqa: E402


def summarize():
    c = workload.draw_case(workload.by_name("tiny_e4_h64_f128"))
    fw = oracle.forward(c.x, c.offsets, c.w1, c.w2)
    dg = oracle.dgrad(c.dy, fw["h1"], c.offsets, c.w1, c.w2)
    out = {"counts": [int(v) for v in c.counts], "offsets": [int(v) for v in c.offsets]}
    inputs = hashlib.sha256()
    for t in (c.x, c.w1, c.w2, c.dy):
        inputs.update(t.contiguous().view(dtype=__import__("torch").int16).numpy().tobytes())
    out["inputs_sha256"] = inputs.hexdigest()
    for name, arr in (("h1", fw["h1"]), ("a", fw["a"]), ("y", fw["y"]), ("dh1", dg["dh1"]),
                      ("dx", dg["dx"])):
        bits = oracle.f32_to_bf16_bits_exact(arr)
        out[name + "_sha256"] = hashlib.sha256(bits.tobytes()).hexdigest()
        out[name + "_first"] = [float(v) for v in arr.reshape(-1)[:4]]
    return out


if __name__ == "__main__":
    path = os.path.join(HERE, "tiny_e4_h64_f128.json")
    with open(path, "w") as fh:
        json.dump(summarize(), fh, indent=1)
        fh.write("\n")
    print("wrote", path)

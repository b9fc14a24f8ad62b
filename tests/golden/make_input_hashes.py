"""Writes tests/golden/input_hashes.json: a SHA-256 of every named workload's
storage arrays (q, k, v) plus its scale and, for e4m3, its descales.

The hashes pin the seeded input generator (SplitMix64 stream, Box-Muller normals,
fill order, scaling, single rounding to the storage type): a change anywhere in it
changes the inputs every parity test and benchmark line is quoted on.  They are
not expected results of the method: this script calls only the input module.

    python tests/golden/make_input_hashes.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import fa_inputs as G  # noqa: E402

OUT = os.path.join(HERE, "input_hashes.json")


def digest(x) -> dict:
    out = {}
    for name in ("q", "k", "v"):
        a = getattr(x, name)
        out[name] = {"shape": list(a.shape), "dtype": str(a.dtype),
                     "sha256": hashlib.sha256(a.tobytes()).hexdigest()}
    out["scale"] = float(x.scale).hex()
    descale = getattr(x, "descale", None)
    if descale is not None:
        out["descale"] = [float(v).hex() for v in descale]
    return out


def all_digests() -> dict:
    return {name: digest(G.workload(name)) for name in (*G.WORKLOADS, *G.DECODE_WORKLOADS)}


if __name__ == "__main__":
    with open(OUT, "w") as f:
        json.dump(all_digests(), f, indent=1, sort_keys=True)
        f.write("\n")
    print("wrote", OUT)

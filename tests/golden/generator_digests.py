"""SHA-256 digests of every array the seeded generator draws for the five
named workloads.

Run ``python tests/golden/generator_digests.py --write`` to (re)write
``generator_sha256.json`` beside this file; the test suite recomputes the
digests and compares. A change of draw order, distribution, rounding or
seed changes every digest it touches, so it cannot slip by unnoticed.

Each workload gets one digest per array, keyed by name: x, W, the shared
VeRA pair, the token assignment (as int32), and every adapter's parameter
arrays (``a<id>.<field>``) plus its scalar c (as the float64 bytes). Values
are hashed as little-endian float64 (the generator's exact rounded values).
"""

from __future__ import annotations

import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from synth import make_config  # noqa: E402

OUT = os.path.join(HERE, "generator_sha256.json")
FIELDS = ("A", "B", "m", "l", "vd", "ve", "Q", "R", "s", "b", "d", "e")


def _h(arr, dtype="<f8") -> str:
    a = np.ascontiguousarray(np.asarray(arr).astype(dtype))
    return hashlib.sha256(a.tobytes()).hexdigest()


def digests(idx: int) -> dict:
    wl = make_config(idx)
    out = {"x": _h(wl.x), "W": _h(wl.W), "token_adapter": _h(wl.token_adapter, "<i4")}
    if wl.A_sh is not None:
        out["A_sh"] = _h(wl.A_sh)
        out["B_sh"] = _h(wl.B_sh)
    # adapters: one digest over all of them (2048 on the FFN-up workload),
    # fed field by field in id order
    h = hashlib.sha256()
    for a in wl.adapters:
        h.update(f"{a.id}:{a.method}:{a.rank}:{a.blk}:".encode())
        h.update(np.float64(a.c).astype("<f8").tobytes())
        for f in FIELDS:
            v = getattr(a, f)
            if v is not None:
                h.update(f.encode())
                h.update(np.ascontiguousarray(np.asarray(v).astype("<f8")).tobytes())
    out["adapters"] = h.hexdigest()
    out["name"] = wl.name
    return out


def all_digests() -> dict:
    return {str(i): digests(i) for i in range(5)}


if __name__ == "__main__":
    d = all_digests()
    if "--write" in sys.argv:
        with open(OUT, "w") as f:
            json.dump(d, f, indent=1, sort_keys=True)
            f.write("\n")
        print(f"wrote {OUT}")
    else:
        print(json.dumps(d, indent=1, sort_keys=True))

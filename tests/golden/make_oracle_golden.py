"""Write tests/golden/oracle_tiny_decode.json from the oracle alone.

Run from the repository root: ``python tests/golden/make_oracle_golden.py``.
It calls only ``oracle/`` and the seeded input generator; nothing from the HIP
path. The fixture guards the oracle against unnoticed changes.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import workload  # noqa: E402


def main():
    w = workload(1)
    out = oracle.decode_attention(w.q, w.k_pool, w.v_pool, w.block_table, w.lens(0), w.scale, w.P)
    path = os.path.join(ROOT, "tests", "golden", "oracle_tiny_decode.json")
    with open(path, "w") as f:
        json.dump({"workload": 1, "shape": list(out.shape), "values": [float(x) for x in out.ravel()]}, f)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()

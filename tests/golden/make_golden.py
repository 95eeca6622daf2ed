"""Writes tests/golden/tiny_decode_oracle.json from the CPU oracle alone.

The pages print no worked numeric example of the attention output, so this file
is not a value from the pages: it freezes the oracle's own result on the tiny
decode workload (B=2, Hq=8, Hkv=2, 128 keys per row, seed 1000) so that any later
change to the oracle's arithmetic shows up as a diff that must be justified.

Run from the repository root:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle      # noqa: E402
import workloads   # noqa: E402


def compute():
    b = workloads.tiny_decode()
    args, kwargs = b.oracle_args()
    out, lse = oracle.paged_attention(*args, **kwargs)
    return b, out, lse


def main():
    b, out, lse = compute()
    doc = {
        "workload": "tiny_decode seed 1000: B=2, Sq=1, Hq=8, Hkv=2, D=128, 128 keys per row, page 16",
        "inputs_sha256": hashlib.sha256(b.q.tobytes() + b.k_cache.tobytes() + b.v_cache.tobytes()).hexdigest(),
        "lse": [[float(x) for x in row] for row in lse[:, :, 0]],
        "out_bf16_bits": out[:, :, 0, :].astype(int).tolist(),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_decode_oracle.json")
    with open(path, "w") as f:
        json.dump(doc, f)
    print("wrote", path)


if __name__ == "__main__":
    main()

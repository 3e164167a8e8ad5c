"""Writes workload_sha256.json: SHA-256 of the seeded generator's output for small specs.

These are determinism fixtures for the inputs (not expected outputs).  Run from the
repository root: ``python tests/golden/make_workload_hashes.py``.
"""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import workloads as W  # noqa: E402
from tests.test_workloads import _hash_specs  # noqa: E402

if __name__ == "__main__":
    out = {name: W.generate(spec).sha256() for name, spec in _hash_specs().items()}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workload_sha256.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(json.dumps(out, indent=1))

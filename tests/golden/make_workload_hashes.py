"""Write workload_sha256.txt: SHA-256 of the bfloat16 bytes of each synthetic input shard.

Calls only the input generators (no part of the method).  Run from the repository root:
    python tests/golden/make_workload_hashes.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from workloads import CONFIGS, make_shard, sha256_bits  # noqa: E402

# (config, shard) pairs recorded; the CPU suite regenerates each and compares.
RECORDED = [(1, 0), (2, 0), (3, 0), (3, 3), (4, 0), (5, 0), (5, 7)]

if __name__ == "__main__":
    lines = ["# config shard sha256(bfloat16 bytes) -- written by make_workload_hashes.py"]
    for cid, p in RECORDED:
        lines.append(f"{cid} {p} {sha256_bits(make_shard(cid, p))}")
        print(lines[-1], file=sys.stderr)
    with open(os.path.join(HERE, "workload_sha256.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

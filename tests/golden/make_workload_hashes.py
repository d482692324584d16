"""Write workload_sha256.txt: SHA-256 of the bfloat16 bytes of each synthetic input shard.

Calls only the input generators (no part of the method).  Run from the repository root:
    python tests/golden/make_workload_hashes.py
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from workloads import GPT2_7B, GPT6_7B, GPT13B_GRAD, QWEN7B, TINY, make_shard, sha256_bits  # noqa: E402

# (workload, shard) pairs recorded; the CPU suite regenerates each and compares.
RECORDED = [(TINY, 0), (GPT2_7B, 0), (GPT6_7B, 0), (GPT6_7B, 3), (GPT13B_GRAD, 0), (QWEN7B, 0),
            (QWEN7B, 7)]

if __name__ == "__main__":
    lines = ["# workload shard sha256(bfloat16 bytes) -- written by make_workload_hashes.py"]
    for key, p in RECORDED:
        lines.append(f"{key} {p} {sha256_bits(make_shard(key, p))}")
        print(lines[-1], file=sys.stderr)
    with open(os.path.join(HERE, "workload_sha256.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

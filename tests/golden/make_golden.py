"""Writes tests/golden/tiny_oracle.json: the oracle's result on the seeded
4-user fp32 toy workload (regression fixture; calls only the oracle and the
input generator)."""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from full_catalog_ranking_amd import synth  # noqa: E402
from oracle import oracle as O  # noqa: E402


def main():
    d = synth.make_workload("tiny")
    r = O.full(d["H"], d["E"], d["K"])
    out = dict(workload="tiny", seed=0, idx=r["idx"].tolist(),
               score=r["score"].tolist(), lse=r["lse"].tolist())
    with open(os.path.join(HERE, "tiny_oracle.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()

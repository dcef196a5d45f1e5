"""Writes graft_tau.json: Graft checkpoint thresholds for the B=16, V=152064
hybrid-tree workload, calibrated on 20 warm-up rounds of the seeded generator
with the oracle's draft phase (25th percentile of c_d among rows still active
at each checkpoint).  Calls only oracle/ and gen/."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from gen import configs  # noqa: E402
from tests.harness import calibrate_tau  # noqa: E402

SEED, ROUNDS = 1004, 20

if __name__ == "__main__":
    w = configs.C4
    tau = calibrate_tau(w, SEED, ROUNDS)
    out = {"workload": w.name, "seed": SEED, "warmup_rounds": ROUNDS, "percentile": 25,
           "ck_depth": list(w.graft.ck_depth), "tau": tau}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "graft_tau.json")
    json.dump(out, open(path, "w"), indent=1)
    print(out)

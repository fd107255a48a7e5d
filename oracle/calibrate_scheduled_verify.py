"""Total-variation distances behind the scheduled ragged verify's confidences (test infrastructure).

The scheduled verify workload asks for per-position confidences from a logistic
model of the draft-target gap. The DSpark study notes (section 5.1) train the
confidence head against the acceptance probability of a drafted position, which
is 1 - TV(p, q), the total-variation distance between the target and draft
distributions. This script computes TV_{i,k} = 1/2 sum_v |p_v - q_v| with the
oracle's fp64 softmax for every (request, position) of the workload, p the
target row that predicts position k and q the draft row of position k, and
writes them to workloads/scheduled_tv.json together with a hash of the logits
they were computed from. The generator turns them into confidences
c_{i,k} = sigmoid(4 - 8 TV_{i,k} + 0.25 eta_{i,k}), eta ~ N(0, 1) its own noise.
It calls only the oracle and the seeded generator.

    python -m oracle.calibrate_scheduled_verify
"""
import hashlib
import json
import os

import numpy as np

import workloads
from oracle.verify import log_softmax


def tv_table(c):
    R, K = c["R"], c["K"]
    tv = np.zeros((R, K))
    for i in range(R):
        t = workloads.values(c["t"][i], "bf16")
        d = workloads.values(c["d"][i], "bf16")
        for k in range(1, K + 1):
            p = np.exp(log_softmax(t[k - 1], 1.0))
            q = np.exp(log_softmax(d[k - 1], 1.0))
            tv[i, k - 1] = 0.5 * np.abs(p - q).sum()
    return tv


def main():
    c = workloads.scheduled_verify(with_conf=False)
    tv = tv_table(c)
    out = os.path.join(os.path.dirname(workloads.__file__), "scheduled_tv.json")
    with open(out, "w") as f:
        json.dump({"R": c["R"], "K": c["K"], "logits_sha256": workloads.scheduled_logits_hash(c),
                   "method": "TV_{i,k} = 1/2 sum_v |softmax(t_{i,k-1}) - softmax(d_{i,k})|, oracle fp64 softmax",
                   "tv": [[round(float(v), 7) for v in row] for row in tv]}, f)
        f.write("\n")
    print("wrote", out, "mean TV", tv.mean(), "min", tv.min(), "max", tv.max())


if __name__ == "__main__":
    main()

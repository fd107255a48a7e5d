"""Choose the draft-noise scale of the dense-vocab verify workload (test infrastructure).

The workload asks for draft logits d = t + sigma * eps whose one-token acceptance
rate is about 0.8. The one-token acceptance rate of a draft distribution q
against a target p is sum_v min(p_v, q_v) = 1 - TV(p, q) (DSpark study notes,
section 5.1: the confidence label is this rate, expressed through the total
variation distance). This script bisects sigma on [0.01, 5] until the mean of
that rate over all R*K position pairs of the workload is within 0.005 of 0.8,
using the oracle's fp64 log-softmax, and writes the result to
workloads/calibration.json. It calls only the oracle and the seeded generator.

    python -m oracle.calibrate_dense_verify
"""
import json
import os

import numpy as np

import workloads
from oracle.verify import log_softmax


def mean_acceptance(sigma):
    c = workloads.verify_case(64, 7, workloads.V_QWEN3, dtype="bf16", seed=1002, t_sigma=3.0,
                              boost_p=0.01, boost=8.0, d_sigma=sigma)
    acc = []
    for i in range(c["R"]):
        t = workloads.values(c["t"][i], "bf16")
        d = workloads.values(c["d"][i], "bf16")
        for k in range(1, c["K"] + 1):
            p = np.exp(log_softmax(t[k - 1], 1.0))
            q = np.exp(log_softmax(d[k - 1], 1.0))
            acc.append(np.minimum(p, q).sum())
    return float(np.mean(acc))


def main():
    lo, hi = 0.01, 5.0
    a_lo, a_hi = mean_acceptance(lo), mean_acceptance(hi)
    assert a_lo > 0.8 > a_hi, (a_lo, a_hi)
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        a = mean_acceptance(mid)
        print(f"sigma={mid:.6f} acceptance={a:.6f}", flush=True)
        if abs(a - 0.8) <= 0.005:
            break
        if a > 0.8:
            lo = mid
        else:
            hi = mid
    out = os.path.join(os.path.dirname(workloads.__file__), "calibration.json")
    with open(out, "w") as f:
        json.dump({"dense_verify_sigma": round(mid, 6), "dense_verify_mean_acceptance": round(a, 6),
                   "method": "bisection of sigma on [0.01, 5] for mean sum_v min(p, q) = 0.80 +- 0.005 "
                             "over the 448 (target, draft) row pairs, oracle fp64 softmax"}, f, indent=1)
        f.write("\n")
    print("wrote", out)


if __name__ == "__main__":
    main()

"""GPU parity of the calibration metric (ECE of the confidences against the verify's
outcomes, dsp_verify_calibration) against the oracle: fp64 values within 1e-12 (the
two sides sum in different orders), observation counts exact."""
import json
import os

import numpy as np
import pytest
import torch

import block_drafting_verification_amd as dsp
import workloads
from oracle import calibration as ocal
from oracle import verify as ov
from parity import cu_from_windows, host, packed_from_dense, to_gpu, values

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _check(conf, cu, decided, B):
    print(f"calibration R={conf.shape[0]} K={conf.shape[1]} bins={B}", flush=True)
    g = dsp.verify_calibration(to_gpu(np.ascontiguousarray(conf, np.float32)), to_gpu(np.asarray(cu, np.int32)),
                               to_gpu(np.asarray(decided, np.int32)), B)
    torch.cuda.synchronize()
    o = ocal.verify_ece(np.asarray(conf, np.float32), cu, decided, B)
    np.testing.assert_array_equal(host(g["n_obs"]), o["n_obs"])
    np.testing.assert_allclose(host(g["ece"]), o["ece"], rtol=0, atol=1e-12)
    assert abs(float(host(g["ece_batch"])[0]) - o["ece_batch"]) < 1e-12
    np.testing.assert_array_equal(host(g["bin_count"]), o["bin_count"])
    np.testing.assert_allclose(host(g["bin_conf"]), o["bin_conf"], rtol=1e-13, atol=1e-12)
    np.testing.assert_array_equal(host(g["bin_out"]), o["bin_out"])
    return g, o


def test_hand_worked_case():
    gl = json.load(open(os.path.join(GOLD, "ece_case.json")))
    g, _ = _check(np.array(gl["conf"], np.float32), gl["cu_seqlens"], gl["decided"], gl["n_bins"])
    np.testing.assert_allclose(host(g["ece"]), gl["expected"]["ece"], rtol=0, atol=1e-15)


@pytest.mark.parametrize("R,K,B", [(1, 1, 1), (37, 7, 10), (300, 16, 10), (1000, 64, 64), (5, 3, 7)])
def test_random_cases(R, K, B):
    rng = np.random.Generator(np.random.PCG64(R * 13 + K))
    conf = rng.random((R, K)).astype(np.float32)
    conf[rng.random((R, K)) < 0.05] = 1.0
    conf[rng.random((R, K)) < 0.05] = 0.0
    w = rng.integers(0, K + 1, size=R)
    decided = np.array([rng.integers(-1, n + 1) if n > 0 else rng.integers(-1, 1) for n in w])
    _check(conf, cu_from_windows(w), decided, B)


def test_scheduled_workload_outcomes():
    """The scheduled verify workload's confidences against the oracle's own verify decisions
    (compact windows from the scheduler, and the cap-accept ceiling of the full block)."""
    c = workloads.scheduled_verify()
    R, K = c["R"], c["K"]
    from oracle import schedule as osch
    w = osch.schedule_windows(c["conf"], c["cost"])["windows"]
    cu = cu_from_windows(w)
    tv = values(packed_from_dense(c["t"], w), "bf16")
    dv = values(c["d"], "bf16")
    o = ov.verify_chain(tv, cu, dv, c["x"], 1.0, seed=0, rnd=3)
    _check(c["conf"], cu, o["accepted_len"], 10)
    # the full-block ceiling (cap-accept) as the outcomes of every scheduled request
    full = np.full(R, K)
    sel = np.arange(0, R, 8)
    cuf = cu_from_windows(full[sel])
    of = ov.verify_chain(values(c["t"][sel].reshape(-1, c["V"]), "bf16"), cuf, dv[sel], c["x"][sel], 1.0, seed=0,
                         rnd=3, req_id=sel, cap=w[sel])
    _check(c["conf"][sel], cuf, of["ceiling"], 10)

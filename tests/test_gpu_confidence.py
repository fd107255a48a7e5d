"""GPU parity of the confidence head (DSpark study notes, section 5.1; SGLang article, STS)."""
import numpy as np
import pytest
import torch

import block_drafting_verification_amd as dsp
import workloads
from oracle import confidence as oc
from parity import host, to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu


def _check(c, dt="bf16", temps=True, pad=0):
    R, K, H = c["R"], c["K"], c["H"]
    h32 = workloads.bf16_bits_to_f32(c["h"])
    w32 = workloads.bf16_bits_to_f32(c["w"])
    if dt == "bf16":
        hb = c["h"]
        if pad:
            hb = np.concatenate([hb, np.zeros((R, K, pad), np.uint16)], axis=2)
        hg = to_gpu_bf16(hb)[..., :H]
        wg = to_gpu_bf16(c["w"])
    else:
        hf = h32
        if pad:
            hf = np.concatenate([hf, np.zeros((R, K, pad), np.float32)], axis=2)
        hg = to_gpu(hf)[..., :H]
        wg = to_gpu(w32)
    tg = to_gpu(c["temps"]) if temps else None
    print(f"confidence R={R} K={K} H={H} dtype={dt} sts={temps} pad={pad}", flush=True)
    g = dsp.confidence_head(hg, wg, c["bias"], tg)
    torch.cuda.synchronize()
    assert int(host(g["status"])[0]) == 0
    ref = oc.confidence_head(h32, w32, c["bias"], c["temps"] if temps else None)
    np.testing.assert_allclose(host(g["conf"]).astype(np.float64), ref, rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("R,K,H", [(3, 5, 64), (7, 3, 1000), (64, 7, 4096), (5, 16, 4099), (2, 2, 3)])
def test_confidence_small(R, K, H):
    c = workloads.confidence_case(R, K, H, seed=R * 100 + H)
    _check(c)
    _check(c, temps=False)
    _check(c, dt="f32", pad=5)
    _check(c, pad=3)  # rows not 16-byte aligned: the element path


def test_confidence_cycle_shape():
    """256 requests x 16 positions, hidden size 4096 (the cycle's shape)."""
    c = workloads.confidence_case(256, 16, 4096, seed=1007)
    _check(c)

"""GPU parity of the RNN sequential head (dsp_draft_rnn_step) against the oracle: tokens
exact except counted argmax near-ties (the oracle replays the GPU's tokens, so every step
is checked locally), log-probabilities within 1e-5."""
import numpy as np
import pytest
import torch

import block_drafting_verification_amd as dsp
import workloads
from oracle import rnn as orn
from parity import ARGMAX_BAND, TieCounter, host, to_gpu, to_gpu_bf16, to_gpu_bf16_token_major

pytestmark = pytest.mark.gpu


def _f(bits):
    return workloads.bf16_bits_to_f32(bits).astype(np.float64)


def _check_rnn(c, want_logq=True, requests=None, token_major=False):
    R, B, V, r, H = c["R"], c["B"], c["V"], c["rank"], c["H"]
    print(f"rnn R={R} B={B} V={V} rank={r} H={H} token_major={token_major}", flush=True)
    Wot = np.ascontiguousarray(c["Wo"].T)
    Lg = to_gpu_bf16_token_major(c["L"]) if token_major else to_gpu_bf16(c["L"])
    g = dsp.draft_rnn_step(Lg, to_gpu_bf16(c["h"]), to_gpu_bf16(c["Gt"]), to_gpu_bf16(c["A"]),
                           to_gpu_bf16(c["E"]), to_gpu_bf16(Wot), to_gpu(c["anchors"].astype(np.int32)),
                           bias=to_gpu(c["bias"]), want_logq=want_logq)
    torch.cuda.synchronize()
    assert int(host(g["status"])[0]) == 0
    y = host(g["y"]).astype(np.int64)
    sel = np.arange(R) if requests is None else np.asarray(requests)
    L = _f(c["L"][sel])
    o = orn.rnn_chain(L, _f(c["h"][sel]), _f(c["A"]), _f(c["E"]), _f(c["Gt"]).T, c["bias"].astype(np.float64),
                      _f(c["Wo"]), c["anchors"][sel], forced=y[sel])
    assert not o["memo_tie"].any(), "a memo entry sits on a bf16 rounding midpoint"
    ties = TieCounter()
    ties.decisions += y[sel].size
    for ii, d in np.argwhere(o["y"] != y[sel]):
        # the oracle's winner against the GPU's choice, both in fp64 under the same memo:
        # their log-probabilities differ by exactly their z difference
        gap = o["logq"][ii, d] - o["logq_forced"][ii, d]
        assert gap < ARGMAX_BAND * max(1.0, abs(o["zmax"][ii, d])), (sel[ii], d, gap)
        ties.near += 1
    ties.check()
    if want_logq:
        np.testing.assert_allclose(host(g["logq"]).astype(np.float64)[sel], o["logq_forced"], rtol=1e-5, atol=1e-5)
    return y, o, g


@pytest.mark.parametrize("R,B,V,rank,H", [(5, 4, 1000, 32, 48), (130, 3, 4099, 64, 96), (7, 5, 30000, 256, 512),
                                          (300, 2, 129, 96, 16), (3, 2, 2000, 512, 64), (64, 6, 9001, 128, 4096)])
def test_rnn_small(R, B, V, rank, H):
    c = workloads.rnn_case(R, B, V, rank=rank, H=H, seed=R + V, wo_scale=100.0)  # corrections that change choices
    y, o, _ = _check_rnn(c)
    # the correction matters at this scale: the tokens are not the base logits' arg-maxes
    assert not np.array_equal(o["y"], np.argmax(workloads.bf16_bits_to_f32(c["L"]), axis=-1))
    c = workloads.rnn_case(R, B, V, rank=rank, H=H, seed=R + V + 1)
    _check_rnn(c, want_logq=False)


def test_rnn_memory_fixture():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "rnn_memory.json")))
    V, r = g["vocab"], 32
    L = np.array(g["L"], np.float32)
    R, B, _ = L.shape
    E = np.zeros((V, r), np.float32)
    E[:, :2] = np.array(g["E"], np.float32)
    A = np.zeros((r, r), np.float32)
    A[:2, :2] = np.array(g["A"], np.float32)
    Wo = np.zeros((r, V), np.float32)
    Wo[:2] = np.array(g["Wo"], np.float32)
    c = dict(L=workloads.f32_to_bf16_bits(L), h=np.zeros((R, B, 8), np.uint16), Gt=np.zeros((r, 8), np.uint16),
             A=workloads.f32_to_bf16_bits(A), E=workloads.f32_to_bf16_bits(E), Wo=workloads.f32_to_bf16_bits(Wo),
             bias=np.zeros(r, np.float32), anchors=np.full(R, g["anchor"], np.int32), R=R, B=B, V=V, rank=r, H=8)
    y, _, _ = _check_rnn(c)
    assert y.tolist() == g["expected"]


def test_rnn_c4_shape_sampled_requests():
    """256 requests x 16 positions, V = 151,936, rank 256, H = 4096 (the Markov-chain
    workload's shape with backbone states): 8 requests checked through all 16 steps."""
    c = workloads.rnn_case(256, 16, workloads.V_QWEN3, 256, H=4096, seed=1007)
    _check_rnn(c, requests=[0, 1, 63, 64, 128, 200, 254, 255])


def test_rnn_token_major_layout():
    """RNN head from token-major base logits: oracle parity, and tokens and logq
    bit-identical to the row-major call's."""
    c = workloads.rnn_case(24, 4, 9001, rank=256, H=96, seed=33, wo_scale=100.0)
    ya, _, ga = _check_rnn(c)
    yb, _, gb = _check_rnn(c, token_major=True)
    np.testing.assert_array_equal(ya, yb)
    np.testing.assert_array_equal(host(ga["logq"]).view(np.uint32), host(gb["logq"]).view(np.uint32))


def test_rnn_bad_previous_token_sets_status():
    c = workloads.rnn_case(4, 2, 500, 32, H=16, seed=9)
    a = c["anchors"].astype(np.int32).copy()
    a[2] = 500
    g = dsp.draft_rnn_step(to_gpu_bf16(c["L"]), to_gpu_bf16(c["h"]), to_gpu_bf16(c["Gt"]), to_gpu_bf16(c["A"]),
                           to_gpu_bf16(c["E"]), to_gpu_bf16(np.ascontiguousarray(c["Wo"].T)), to_gpu(a))
    torch.cuda.synchronize()
    assert int(host(g["status"])[0]) & dsp.DSP_STATUS_TOKEN_RANGE

"""The allocation-free verify entry point (dsp_verify_rejection_noalloc) against the
workspace entry point (dsp_verify_rejection): both run the same kernels on the same
inputs, so every output must be bit-identical. Two calls in a row through the
library's fixed scratch, the second on a smaller batch (the scratch keeps the first
call's contents), for the sampled, greedy chain and greedy tree verify; a batch whose
scratch need exceeds the fixed size is refused before anything is launched."""
import numpy as np
import pytest
import torch

import block_drafting_verification_amd as dsp
import workloads
from parity import cu_from_windows, host, logits_to_gpu, packed_from_dense, to_gpu

pytestmark = pytest.mark.gpu

KEYS = ("accepted_len", "out_tokens", "stop_pos", "p_x", "q_x", "status")


def _pair(case, windows, T, seed, rnd, parent=None, **kw):
    R, K, V, dt = case["R"], case["K"], case["V"], case["dtype"]
    tp = packed_from_dense(case["t"], windows)
    tg = logits_to_gpu(tp, dt)
    dg = logits_to_gpu(case["d"], dt) if T > 0 else None
    xg = to_gpu(case["x"].astype(np.int32))
    cu = to_gpu(cu_from_windows(windows))
    pg = None if parent is None else to_gpu(parent)
    print(f"noalloc pair R={R} K={K} V={V} T={T} tree={parent is not None}", flush=True)
    a = dsp.verify_rejection(tg, cu, xg, drf=dg, parent=pg, temperature=T, seed=seed, round=rnd, **kw)
    b = dsp.verify_rejection_noalloc(tg, cu, xg, drf=dg, parent=pg, temperature=T, seed=seed, round=rnd, **kw)
    torch.cuda.synchronize()
    for k in KEYS:
        if a.get(k) is None:
            assert b.get(k) is None
            continue
        np.testing.assert_array_equal(host(b[k]), host(a[k]), err_msg=k)
    assert int(host(a["status"])[0]) == 0
    return a


def test_sampled_two_calls_second_smaller():
    big = workloads.verify_case(256, 7, 40000, dtype="bf16", seed=71, t_sigma=3.0, d_sigma=0.5)
    rng = np.random.Generator(np.random.PCG64(1))
    _pair(big, rng.integers(0, 8, size=256), 1.0, 3, 5)   # 256 requests: decide / residual / draw
    small = workloads.verify_case(5, 3, 3001, dtype="f32", seed=72, t_sigma=2.0, d_sigma=0.4)
    _pair(small, np.array([3, 0, 2, 3, 1]), 0.8, 4, 6)
    mid = workloads.verify_case(40, 16, 20011, dtype="bf16", seed=73, t_sigma=3.0, d_sigma=0.3)
    _pair(mid, np.full(40, 16), 1.0, 5, 7, cap=to_gpu(np.arange(40, dtype=np.int32) % 18))


def test_greedy_chain_and_tree_two_calls():
    c = workloads.verify_case(64, 6, 30011, dtype="bf16", seed=74, t_sigma=3.0, d_sigma=0.5, temperature=0.0)
    _pair(c, np.full(64, 6), 0.0, 0, 0, want_probs=False)
    t = workloads.verify_case(6, 5, 5003, dtype="bf16", seed=75, t_sigma=3.0, d_sigma=0.5, temperature=0.0)
    par = np.array([[-1, 0, 0, 1, 3]] * 6, dtype=np.int32)
    _pair(t, np.full(6, 5), 0.0, 0, 0, parent=par, want_probs=False)


def test_oversized_batch_is_refused_before_launch():
    R, K, V = 2000, 64, workloads.V_QWEN3
    dev = torch.device("cuda", 0)
    tg = torch.zeros(R, V, dtype=torch.bfloat16, device=dev)
    cu = torch.arange(R + 1, dtype=torch.int32, device=dev)
    x = torch.zeros(R, K, dtype=torch.int32, device=dev)
    need = dsp.lib().dsp_verify_rejection_workspace_size(R, K, V, R, dsp.DSP_BF16, dsp.DSP_BF16)
    assert need > (8 << 20)
    out = dict(accepted_len=torch.full((R,), 7, dtype=torch.int32, device=dev))
    with pytest.raises(dsp.DspError, match="allocation-free"):
        dsp.verify_rejection_noalloc(tg, cu, x, temperature=0.0, out=out, want_probs=False)
    torch.cuda.synchronize()
    assert int(out["accepted_len"][0].item()) == 7  # nothing ran

"""Helpers for GPU-vs-oracle parity tests: tensor conversion and near-tie accounting.

Decisions must match the oracle exactly, except where the oracle's own fp64
margin says the decision is a near-tie:
  accept/reject        |u - ratio| < 1e-6
  inverse-CDF draw     the target lies within 1e-6 * total of a CDF boundary
  argmax / top-k       winner vs. runner-up gap < 1e-6 * max(1, |value|)
Near-ties are counted; they must stay below 0.01 % of the decisions checked.
"""
import numpy as np
import torch

import workloads

ACCEPT_BAND = 1e-6
SAMPLE_BAND = 1e-6
ARGMAX_BAND = 1e-6
MAX_NEAR_TIE_FRACTION = 1e-4


def dev():
    return torch.device("cuda", 0)


def to_gpu_bf16(bits):
    """uint16 bfloat16 bit patterns (numpy) -> torch.bfloat16 on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def to_gpu_bf16_token_major(bits):
    """[R, B, V] bfloat16 bits -> a [B, V, R] GPU buffer viewed as [R, B, V] (unit stride
    over requests: the chain's token-major base-logit layout)."""
    return to_gpu_bf16(np.ascontiguousarray(np.transpose(bits, (1, 2, 0)))).permute(2, 0, 1)


def to_gpu(arr, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(arr))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev())


def logits_to_gpu(arr, dtype):
    return to_gpu_bf16(arr) if dtype == "bf16" else to_gpu(arr.astype(np.float32))


def host(t):
    return t.detach().cpu().numpy()


class TieCounter:
    def __init__(self):
        self.decisions = 0
        self.near = 0
        self.notes = []

    def check(self, max_fraction=MAX_NEAR_TIE_FRACTION, min_decisions_for_fraction=10000):
        if self.near == 0:
            return
        # with few decisions a single counted near-tie is reported but tolerated
        if self.decisions >= min_decisions_for_fraction:
            assert self.near / self.decisions < max_fraction, (self.near, self.decisions, self.notes[:5])
        else:
            assert self.near <= 1, (self.near, self.decisions, self.notes[:5])


def rounding_bands(res, eps, tok_dev, T):
    """Accept and draw bands of a verify whose draft rows may differ from the oracle's at
    bf16 rounding near-ties (the sampled chain's emitted rows; oracle.markov.chain_sampled
    gives eps and tok_dev per row and the bound derivations).

    Accept at position k: ratio = p(x)/q(x) and q(x) moves by a factor within exp(+-eta),
    eta = tok_dev / T + log(1 / (1 - eps)), so |ratio' - ratio| <= ratio * expm1(eta).
    Residual draw at the stop k: sum_v |q'_v - q_v| <= dq = 2 eps / (1 - eps), hence every
    residual CDF boundary and the target u' * sum(r) move by at most dq each, and the
    decision stands while the oracle's relative margin exceeds 2 dq / sum(r).
    A bonus draw reads the target rows only. The base bands cover the arithmetic itself.
    Returns (accept_band [R, K], sample_band [R]).
    """
    e = np.minimum(np.asarray(eps, dtype=np.float64), 0.5)
    eta = np.asarray(tok_dev, dtype=np.float64) / T - np.log1p(-e)
    accept = ACCEPT_BAND + res["ratio"] * np.expm1(eta)
    dq = 2.0 * e / (1.0 - e)
    R = dq.shape[0]
    sample = np.full(R, SAMPLE_BAND)
    for i in range(R):
        k = int(res["stop_pos"][i])
        if res["resid_mass"][i] > 0:
            sample[i] += 2.0 * dq[i, k - 1] / res["resid_mass"][i]
    return accept, sample


def compare_chain_verify(gpu, orc_fn, R, K, windows, ties, p_rtol=1e-5, draft_bounds=None):
    """Compare a sampled / greedy chain verify result against the oracle with replay.

    orc_fn(forced_len) -> oracle result dict. The oracle is first run on its own;
    where the accepted length differs, the disagreement must be a counted accept
    near-tie and the oracle is replayed along the GPU's decisions to check the
    drawn token. draft_bounds = (eps, tok_dev, T) (optional) widens the bands per
    decision by ``rounding_bands`` where the draft rows themselves may differ
    slightly between the two sides.
    """
    acc = host(gpu["accepted_len"]).astype(np.int64)
    toks = host(gpu["out_tokens"]).astype(np.int64)
    own = orc_fn(None)
    rep = own
    if np.any(acc != own["accepted_len"]):
        rep = orc_fn(acc)
    if draft_bounds is None:
        accept_band, sample_band = np.full((R, K), ACCEPT_BAND), np.full(R, SAMPLE_BAND)
    else:
        accept_band, _ = rounding_bands(own, *draft_bounds)
        _, sample_band = rounding_bands(rep, *draft_bounds)
    for i in range(R):
        n = int(windows[i])
        decided = min(n, int(own["accepted_len"][i]) + 1)
        ties.decisions += decided + 1
        if acc[i] != own["accepted_len"][i]:
            k = int(min(acc[i], own["accepted_len"][i])) + 1  # first differing decision
            m = own["accept_margin"][i, k - 1]
            band = accept_band[i, k - 1]
            assert m < band, f"request {i}: accepted {acc[i]} vs oracle {own['accepted_len'][i]} (margin {m})"
            ties.near += 1
            ties.notes.append(("accept", i, k, m))
        r = rep
        np.testing.assert_array_equal(toks[i, :acc[i]], r["out_tokens"][i, :acc[i]])
        if toks[i, acc[i]] != r["out_tokens"][i, acc[i]]:
            m = r["sample_margin"][i]
            band = sample_band[i]
            assert m < band, f"request {i}: drawn token {toks[i, acc[i]]} vs {r['out_tokens'][i, acc[i]]} (margin {m})"
            ties.near += 1
            ties.notes.append(("sample", i, m))
        assert np.all(toks[i, acc[i] + 1:] == -1)
    if gpu.get("p_x") is not None and "p_x" in own:
        px, qx = host(gpu["p_x"]), host(gpu["q_x"])
        np.testing.assert_allclose(px, own["p_x"], rtol=p_rtol, atol=1e-30)
        np.testing.assert_allclose(qx, own["q_x"], rtol=p_rtol, atol=1e-30)


def packed_from_dense(t, windows):
    """Rows of a dense [R, K+1, V] target buffer packed front to back by windows (host side)."""
    rows = [t[i, :int(windows[i]) + 1] for i in range(t.shape[0])]
    return np.concatenate(rows, axis=0)


def cu_from_windows(windows):
    return np.concatenate([[0], np.cumsum(np.asarray(windows) + 1)]).astype(np.int32)


def values(arr, dtype):
    return workloads.values(arr, dtype)

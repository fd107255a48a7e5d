"""MI355X (gfx950) hot path of confidence-scheduled speculative decoding.

Thin torch-tensor binding of libdsp's C ABI (include/dsp.h). Every function
here only checks and marshals arguments (device pointers, strides, the current
HIP stream, a workspace from torch's allocator); all arithmetic runs in the HIP
kernels of libdsp.so. The library must be built first
(``python -m block_drafting_verification_amd.build``); nothing here falls back
to another implementation.

Calls (same names as the C entry points without the ``dsp_`` prefix):
  confidence_head    -- per-position confidences (linear projection + sigmoid, STS temperatures)
  schedule_windows   -- survival products + hardware-aware prefix scheduler
  pack_ragged        -- front-packed cu_seqlens verify buffer
  verify_rejection   -- batched ragged rejection / greedy / tree verify
  verify_rejection_noalloc -- the same with the library's fixed scratch (allocates nothing)
  verify_calibration -- ECE of the confidences against a verify's outcomes
  draft_markov_step  -- Markov-head greedy chain
  draft_markov_sample -- Markov-head sampled chain emitting its bf16 draft logits
  draft_rnn_step     -- greedy chain with the RNN sequential head
  tree_expand        -- PCTree expansion
  philox_uniforms    -- the counter-based uniforms the verify step draws
  TierGraphs         -- one captured verify graph per packed-row tier, replayed by the pack's tier
"""
import ctypes

import torch

from . import _abi
from ._abi import (DSP_BF16, DSP_BF16_TOKEN_MAJOR, DSP_F32, DSP_SCHED_ARGMAX, DSP_SCHED_EARLY_STOP, DSP_SCHED_THRESHOLD,
                   DSP_SCHED_TOP_M, DSP_STATUS_NONFINITE, DSP_STATUS_TIMEOUT, DSP_STATUS_TOKEN_RANGE,
                   DSP_STATUS_WINDOW_RANGE,
                   DspError, KERNELS)
from .tiers import TierGraphs

__all__ = ["PreparedCall", "TierGraphs", "confidence_head", "schedule_windows", "pack_ragged", "verify_rejection",
           "verify_rejection_noalloc", "verify_calibration", "draft_markov_step", "draft_rnn_step",
           "draft_markov_sample", "tree_expand", "schedule_pack",
           "philox_uniforms", "stream_read", "set_option", "prof_enable", "prof_reset", "prof_query", "DspError", "lib",
           "DSP_SCHED_EARLY_STOP", "DSP_SCHED_ARGMAX", "DSP_SCHED_TOP_M", "DSP_SCHED_THRESHOLD",
           "DSP_STATUS_TOKEN_RANGE",
           "DSP_STATUS_WINDOW_RANGE", "DSP_STATUS_NONFINITE", "DSP_STATUS_TIMEOUT"]


def lib():
    return _abi.load()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return DSP_BF16
    if t.dtype == torch.float32:
        return DSP_F32
    raise TypeError(f"logits must be bfloat16 or float32, got {t.dtype}")


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _on_gpu(*ts):
    for t in ts:
        if t is not None:
            _need(t.is_cuda, "tensors must live on the GPU")


def _take(o, key, make):
    t = o.get(key)
    return make() if t is None else t


_ws_cache = {}


def _call_stream(stream):
    return torch.cuda.current_stream() if stream is None else stream


def _is_current(stream, device):
    return stream.cuda_stream == torch.cuda.current_stream(device).cuda_stream


def _workspace(nbytes, device, private=False, stream=None):
    """A device byte buffer of at least nbytes.

    Prepared calls get a private buffer, kept for their lifetime. One-shot calls on
    the current stream share one buffer per (device, stream): calls on one stream run
    in order, and a grown cache entry is freed on the stream it was allocated on. A
    one-shot call on another stream gets a buffer of its own, recorded on that stream
    so the caching allocator does not reuse it before the call's kernels finish.
    """
    if private:
        return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    s = _call_stream(stream)
    if not _is_current(s, device):
        buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        buf.record_stream(s)
        return buf
    key = (device.index if device.index is not None else torch.cuda.current_device(), s.cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < max(nbytes, 1):
        buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


class PreparedCall:
    """A libdsp call whose arguments were checked and marshalled once.

    Calling it issues exactly one C ABI call on the stream captured at
    preparation time, with the same device buffers (results land in
    ``outputs``). Suitable for tight loops and HIP graph capture.
    """

    def __init__(self, fn, args, keep, outputs):
        self._fn = fn
        self._args = tuple(args)
        self._keep = keep
        self.outputs = outputs

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            _abi.check(rc)
        return self.outputs


def _finish(fn, args, outputs, prepare, keep, stream=None):
    if prepare:
        return PreparedCall(fn, args, keep, outputs)
    _abi.check(fn(*args))
    if stream is not None:
        # outputs allocated on the current stream but written on another: keep the
        # allocator from handing their memory out again before that stream is done
        for t in outputs.values():
            if isinstance(t, torch.Tensor) and not _is_current(stream, t.device):
                t.record_stream(stream)
    return outputs


def philox_uniforms(ctr, seed, stream=None):
    """ctr: uint64-valued int64 tensor [n, 4] on the GPU -> float64 [n, 4] uniforms."""
    _on_gpu(ctr)
    _need(ctr.dim() == 2 and ctr.shape[1] == 4 and ctr.is_contiguous(), "ctr must be contiguous [n, 4]")
    out = torch.empty(ctr.shape, dtype=torch.float64, device=ctr.device)
    _abi.check(lib().dsp_philox_uniforms(_ptr(ctr), ctr.shape[0], seed, _ptr(out), _stream(stream)))
    return out


def confidence_head(h, w, bias, sts_temp=None, out=None, status=None, stream=None, prepare=False):
    """Confidence head: h [R, K, H] (bf16/fp32, unit inner stride), w [H], scalar bias,
    sts_temp float32 [K] or None. Returns dict(conf float32 [R, K], status)."""
    _on_gpu(h, w, sts_temp)
    _need(h.dim() == 3 and h.stride(2) == 1, "h: [R, K, H] with unit inner stride")
    R, K, H = h.shape
    _need(w.dim() == 1 and w.numel() == H and w.is_contiguous(), "w: contiguous [H]")
    _need(sts_temp is None or (sts_temp.dtype == torch.float32 and sts_temp.numel() == K
                               and sts_temp.is_contiguous()), "sts_temp: float32 [K]")
    dev = h.device
    o = out or {}
    conf = _take(o, "conf", lambda: torch.empty(R, K, dtype=torch.float32, device=dev))
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    args = (_ptr(h), _dtype_code(h), h.stride(0), h.stride(1), _ptr(w), _dtype_code(w), float(bias),
            _ptr(sts_temp), R, K, H, _ptr(conf), _ptr(status), _stream(stream))
    return _finish(lib().dsp_confidence_head, args, dict(conf=conf, status=status), prepare, (h, w, sts_temp), stream=stream)


def schedule_windows(conf, cost, mode=DSP_SCHED_EARLY_STOP, max_tokens=-1, threshold=0.0, want_survival=True,
                     out=None, stream=None, prepare=False):
    """conf: float32 [R, K]; cost: float64 [>= R*K+1] (both on the GPU).

    mode: DSP_SCHED_EARLY_STOP, DSP_SCHED_ARGMAX, DSP_SCHED_TOP_M (capacity max_tokens)
    or DSP_SCHED_THRESHOLD (survival >= threshold).

    Returns dict(windows int32 [R], survival float64 [R, K] or None, stats float64 [4]).
    """
    _on_gpu(conf, cost)
    _need(conf.dtype == torch.float32 and conf.dim() == 2 and conf.is_contiguous(), "conf: contiguous float32 [R, K]")
    _need(cost.dtype == torch.float64 and cost.is_contiguous(), "cost: contiguous float64")
    R, K = conf.shape
    dev = conf.device
    o = out or {}
    windows = _take(o, "windows", lambda: torch.empty(R, dtype=torch.int32, device=dev))
    survival = _take(o, "survival", lambda: torch.empty(R, K, dtype=torch.float64, device=dev)) if want_survival else None
    stats = _take(o, "stats", lambda: torch.empty(4, dtype=torch.float64, device=dev))
    ws = _workspace(lib().dsp_schedule_windows_workspace_size(R, K), dev, prepare, stream)
    args = (_ptr(conf), R, K, _ptr(cost), cost.numel(), mode, max_tokens, float(threshold), _ptr(windows),
            _ptr(survival),
            _ptr(stats), _ptr(ws), ws.numel(), _stream(stream))
    res = dict(windows=windows, survival=survival, stats=stats)
    return _finish(lib().dsp_schedule_windows, args, res, prepare, (conf, cost, ws), stream=stream)


def pack_ragged(windows, anchors, drafts, tiers=None, out=None, status=None, stream=None, prepare=False):
    """windows int32 [R], anchors int32 [R], drafts int32 [R, K] (GPU); tiers: host list.

    Returns dict(cu_seqlens [R+1], tokens/row_req/row_pos [R*(K+1)], total_and_tier [2], status [1]).
    """
    _on_gpu(windows, anchors, drafts)
    for t in (windows, anchors, drafts):
        _need(t.dtype == torch.int32, "pack_ragged takes int32 tensors")
    _need(drafts.dim() == 2 and drafts.stride(1) == 1, "drafts: [R, K] with unit inner stride")
    R, K = drafts.shape
    dev = drafts.device
    o = out or {}
    cu = _take(o, "cu_seqlens", lambda: torch.empty(R + 1, dtype=torch.int32, device=dev))
    tokens = _take(o, "tokens", lambda: torch.empty(R * (K + 1), dtype=torch.int32, device=dev))
    row_req = _take(o, "row_req", lambda: torch.empty(R * (K + 1), dtype=torch.int32, device=dev))
    row_pos = _take(o, "row_pos", lambda: torch.empty(R * (K + 1), dtype=torch.int32, device=dev))
    tt = _take(o, "total_and_tier", lambda: torch.empty(2, dtype=torch.int32, device=dev))
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    tl = list(tiers or [])
    arr = (ctypes.c_int32 * max(len(tl), 1))(*tl) if tl else None
    args = (_ptr(windows), _ptr(anchors), _ptr(drafts), drafts.stride(0), R, K,
            ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None, len(tl),
            _ptr(cu), _ptr(tokens), _ptr(row_req), _ptr(row_pos), _ptr(tt), _ptr(status), _stream(stream))
    res = dict(cu_seqlens=cu, tokens=tokens, row_req=row_req, row_pos=row_pos, total_and_tier=tt, status=status)
    return _finish(lib().dsp_pack_ragged, args, res, prepare, (windows, anchors, drafts, arr), stream=stream)


def schedule_pack(conf, cost, anchors, drafts, mode=DSP_SCHED_EARLY_STOP, max_tokens=-1, threshold=0.0,
                  want_survival=True, tiers=None, out=None, status=None, stream=None, prepare=False):
    """schedule_windows then pack_ragged on its windows, in one call (one launch fewer).

    conf float32 [R, K], cost float64 [>= R*K+1], anchors int32 [R], drafts int32 [R, K] (GPU).
    Returns the union of both calls' dicts.
    """
    _on_gpu(conf, cost, anchors, drafts)
    _need(conf.dtype == torch.float32 and conf.dim() == 2 and conf.is_contiguous(), "conf: contiguous float32 [R, K]")
    _need(cost.dtype == torch.float64 and cost.is_contiguous(), "cost: contiguous float64")
    for t in (anchors, drafts):
        _need(t.dtype == torch.int32, "anchors and drafts are int32")
    _need(drafts.dim() == 2 and drafts.stride(1) == 1 and tuple(drafts.shape) == tuple(conf.shape),
          "drafts: [R, K] like conf, unit inner stride")
    R, K = conf.shape
    dev = conf.device
    o = out or {}
    windows = _take(o, "windows", lambda: torch.empty(R, dtype=torch.int32, device=dev))
    survival = _take(o, "survival", lambda: torch.empty(R, K, dtype=torch.float64, device=dev)) if want_survival else None
    stats = _take(o, "stats", lambda: torch.empty(4, dtype=torch.float64, device=dev))
    cu = _take(o, "cu_seqlens", lambda: torch.empty(R + 1, dtype=torch.int32, device=dev))
    tokens = _take(o, "tokens", lambda: torch.empty(R * (K + 1), dtype=torch.int32, device=dev))
    row_req = _take(o, "row_req", lambda: torch.empty(R * (K + 1), dtype=torch.int32, device=dev))
    row_pos = _take(o, "row_pos", lambda: torch.empty(R * (K + 1), dtype=torch.int32, device=dev))
    tt = _take(o, "total_and_tier", lambda: torch.empty(2, dtype=torch.int32, device=dev))
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    tl = list(tiers or [])
    arr = (ctypes.c_int32 * max(len(tl), 1))(*tl) if tl else None
    ws = _workspace(lib().dsp_schedule_windows_workspace_size(R, K), dev, prepare, stream)
    args = (_ptr(conf), R, K, _ptr(cost), cost.numel(), mode, max_tokens, float(threshold), _ptr(windows),
            _ptr(survival), _ptr(stats), _ptr(anchors), _ptr(drafts), drafts.stride(0),
            ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None, len(tl),
            _ptr(cu), _ptr(tokens), _ptr(row_req), _ptr(row_pos), _ptr(tt), _ptr(status), _ptr(ws), ws.numel(),
            _stream(stream))
    res = dict(windows=windows, survival=survival, stats=stats, cu_seqlens=cu, tokens=tokens, row_req=row_req,
               row_pos=row_pos, total_and_tier=tt, status=status)
    return _finish(lib().dsp_schedule_pack, args, res, prepare, (conf, cost, anchors, drafts, ws, arr), stream=stream)


def verify_rejection_noalloc(tgt, cu_seqlens, draft_tok, drf=None, parent=None, temperature=1.0, seed=0,
                             round=0, req_id=None, max_rows=0, want_probs=True, out=None, status=None,
                             stream=None, round_dev=None, row_req=None, row_pos=None, cap=None,
                             want_ceiling=False, prepare=False):
    """verify_rejection through the allocation-free entry point: the library's fixed
    per-GPU scratch replaces the workspace (batches needing more than 8 MiB of it raise
    DspError). Pass every output in `out` to allocate nothing here either; calls that
    overlap on one GPU share that scratch and must not be issued."""
    return verify_rejection(tgt, cu_seqlens, draft_tok, drf, parent, temperature, seed, round, req_id, max_rows,
                            want_probs, out, status, stream, round_dev, row_req, row_pos, cap, want_ceiling,
                            prepare, _noalloc=True)


def verify_rejection(tgt, cu_seqlens, draft_tok, drf=None, parent=None, temperature=1.0, seed=0,
                     round=0, req_id=None, max_rows=0, want_probs=True, out=None, status=None,
                     stream=None, round_dev=None, row_req=None, row_pos=None, cap=None, want_ceiling=False,
                     prepare=False, _noalloc=False):
    """Batched ragged verify.

    tgt: packed target logits [T_rows, V] (bf16/fp32, unit inner stride);
    cu_seqlens: int32 [R+1]; draft_tok: int32 [R, K]; drf: draft logits [R, K, V]
    (T > 0); parent: int32 [R, K] selects the greedy tree walk (T must be 0).
    row_req/row_pos: the pack's packed-row maps (optional; locate draft rows directly).
    cap: int32 [R] cap-accept commit windows (chain only); want_ceiling (implied by cap)
    adds 'ceiling' [R], the drafts accepted over the whole packed window.
    Returns dict(accepted_len, out_tokens [R, K+1], stop_pos, p_x, q_x, status[, ceiling]).
    """
    _on_gpu(tgt, cu_seqlens, draft_tok, drf, parent, req_id, round_dev, row_req, row_pos, cap)
    if row_req is not None or row_pos is not None:
        _need(row_req is not None and row_pos is not None and row_req.dtype == torch.int32 and
              row_pos.dtype == torch.int32, "row_req and row_pos: int32, together")
    if round_dev is not None:
        _need(round_dev.dtype == torch.int64 and round_dev.numel() == 1, "round_dev: one int64 on the GPU")
    _need(tgt.dim() == 2 and tgt.stride(1) == 1, "tgt: [rows, V] with unit inner stride")
    _need(cu_seqlens.dtype == torch.int32 and cu_seqlens.is_contiguous(), "cu_seqlens: contiguous int32")
    _need(draft_tok.dtype == torch.int32 and draft_tok.dim() == 2 and draft_tok.stride(1) == 1,
          "draft_tok: int32 [R, K] with unit inner stride")
    R, K = draft_tok.shape
    V = tgt.shape[1]
    _need(cu_seqlens.numel() == R + 1, "cu_seqlens must have R+1 entries")
    t_dt = _dtype_code(tgt)
    greedy = float(temperature) == 0.0
    d_dt, ld_dr, ld_dk = DSP_BF16, 0, 0
    if drf is not None:
        _need(drf.dim() == 3 and drf.shape[0] == R and drf.shape[1] >= K and drf.shape[2] == V and drf.stride(2) == 1,
              "drf: [R, >=K, V] with unit inner stride")
        d_dt, ld_dr, ld_dk = _dtype_code(drf), drf.stride(0), drf.stride(1)
    else:
        _need(greedy, "draft logits are required when temperature > 0")
    if parent is not None:
        _need(parent.dtype == torch.int32 and parent.shape == draft_tok.shape and parent.stride() == draft_tok.stride(),
              "parent: int32 with the layout of draft_tok")
    if req_id is not None:
        _need(req_id.dtype == torch.int64 and req_id.numel() == R and req_id.is_contiguous(), "req_id: int64 [R]")
    dev = tgt.device
    o = out or {}
    acc = _take(o, "accepted_len", lambda: torch.empty(R, dtype=torch.int32, device=dev))
    toks = _take(o, "out_tokens", lambda: torch.empty(R, K + 1, dtype=torch.int32, device=dev))
    stop = _take(o, "stop_pos", lambda: torch.empty(R, dtype=torch.int32, device=dev))
    p_x = _take(o, "p_x", lambda: torch.empty(R, K, dtype=torch.float32, device=dev)) if want_probs else None
    q_x = _take(o, "q_x", lambda: torch.empty(R, K, dtype=torch.float32, device=dev)) if want_probs else None
    if cap is not None:
        _need(cap.dtype == torch.int32 and cap.numel() == R and cap.is_contiguous(), "cap: int32 [R]")
    ceiling = _take(o, "ceiling", lambda: torch.empty(R, dtype=torch.int32, device=dev)) \
        if (cap is not None or want_ceiling) else None
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    # bound the rows the device may read by what the target tensor holds
    rows_cap = min(R * (K + 1), tgt.shape[0])
    max_rows = rows_cap if not max_rows else min(int(max_rows), rows_cap)
    args = (_ptr(tgt), t_dt, tgt.stride(0), _ptr(cu_seqlens), _ptr(drf), d_dt, ld_dr, ld_dk,
            _ptr(draft_tok), draft_tok.stride(0), _ptr(parent), R, K, V, max_rows, float(temperature),
            int(seed), int(round), _ptr(round_dev), _ptr(req_id), _ptr(row_req), _ptr(row_pos), _ptr(cap),
            _ptr(ceiling), _ptr(acc), _ptr(toks), _ptr(stop), _ptr(p_x), _ptr(q_x), _ptr(status))
    res = dict(accepted_len=acc, out_tokens=toks, stop_pos=stop, p_x=p_x, q_x=q_x, status=status)
    if ceiling is not None:
        res["ceiling"] = ceiling
    keep = (tgt, cu_seqlens, drf, draft_tok, parent, req_id, round_dev, row_req, row_pos, cap)
    if _noalloc:
        return _finish(lib().dsp_verify_rejection_noalloc, args + (_stream(stream),), res, prepare, keep,
                       stream=stream)
    nbytes = lib().dsp_verify_rejection_workspace_size(R, K, V, max_rows, t_dt, d_dt)
    ws = _workspace(nbytes, dev, prepare, stream)
    return _finish(lib().dsp_verify_rejection, args + (_ptr(ws), ws.numel(), _stream(stream)), res, prepare,
                   keep + (ws,), stream=stream)


def verify_calibration(conf, cu_seqlens, decided, n_bins=10, out=None, stream=None, prepare=False):
    """ECE of the confidences conf float32 [R, K] against a verify's outcomes: cu_seqlens
    int32 [R+1] (the packing verified), decided int32 [R] (accepted_len, or the cap-accept
    ceiling). Returns dict(ece float64 [R], n_obs int32 [R], ece_batch, bin_count, bin_conf,
    bin_out (float64 [n_bins] each, views of one 'batch' buffer))."""
    _on_gpu(conf, cu_seqlens, decided)
    _need(conf.dtype == torch.float32 and conf.dim() == 2 and conf.stride(1) == 1,
          "conf: float32 [R, K] with unit inner stride")
    R, K = conf.shape
    _need(cu_seqlens.dtype == torch.int32 and cu_seqlens.numel() == R + 1 and cu_seqlens.is_contiguous(),
          "cu_seqlens: contiguous int32 [R+1]")
    _need(decided.dtype == torch.int32 and decided.numel() == R and decided.is_contiguous(), "decided: int32 [R]")
    dev = conf.device
    o = out or {}
    ece = _take(o, "ece", lambda: torch.empty(R, dtype=torch.float64, device=dev))
    nobs = _take(o, "n_obs", lambda: torch.empty(R, dtype=torch.int32, device=dev))
    batch = _take(o, "batch", lambda: torch.empty(1 + 3 * n_bins, dtype=torch.float64, device=dev))
    args = (_ptr(conf), conf.stride(0), _ptr(cu_seqlens), _ptr(decided), R, K, int(n_bins), _ptr(ece), _ptr(nobs),
            _ptr(batch), _stream(stream))
    res = dict(ece=ece, n_obs=nobs, batch=batch, ece_batch=batch[0:1], bin_count=batch[1:1 + n_bins],
               bin_conf=batch[1 + n_bins:1 + 2 * n_bins], bin_out=batch[1 + 2 * n_bins:])
    return _finish(lib().dsp_verify_calibration, args, res, prepare, (conf, cu_seqlens, decided), stream=stream)


def _chain_l(L):
    """Layout code and strides of the chain's base logits L [R, B, V]: row-major (unit
    stride over the vocabulary) or token-major (unit stride over requests, e.g. a
    [B, V, R] buffer viewed through permute(2, 0, 1))."""
    _need(L.dtype == torch.bfloat16 and L.dim() == 3, "L: bf16 [R, B, V]")
    if L.stride(2) == 1:
        return DSP_BF16, L.stride(0), L.stride(1)
    _need(L.stride(0) == 1, "L: unit stride over the vocabulary or over requests")
    return DSP_BF16_TOKEN_MAJOR, L.stride(2), L.stride(1)


def _check_markov(L, U, Wt, chain=False):
    _on_gpu(L, U, Wt)
    if chain:
        _chain_l(L)
    else:
        _need(L.dtype == torch.bfloat16 and L.dim() == 3 and L.stride(2) == 1, "L: bf16 [R, B, V], unit inner stride")
    _need(U.dtype == torch.bfloat16 and U.dim() == 2 and U.is_contiguous(), "U: contiguous bf16 [V, rank]")
    _need(Wt.dtype == torch.bfloat16 and Wt.shape == U.shape and Wt.is_contiguous(),
          "Wt: contiguous bf16 [V, rank] (the second factor stored vocab-major)")


def draft_markov_step(L, U, Wt, prev_tok, n_steps=None, want_logq=False, out=None, status=None, stream=None,
                      prepare=False):
    """Greedy Markov chain. L: bf16 [R, B, V]; U, Wt: bf16 [V, rank]; prev_tok: int32 [R].

    Returns dict(y int32 [R, n], logq float32 [R, n] or None, status).
    """
    _check_markov(L, U, Wt, chain=True)
    l_dt, ldl_r, ldl_d = _chain_l(L)
    R, B, V = L.shape
    n = B if n_steps is None else int(n_steps)
    _need(1 <= n <= B, "n_steps must be in [1, B]")
    rank = U.shape[1]
    _need(prev_tok.dtype == torch.int32 and prev_tok.numel() == R and prev_tok.is_contiguous(), "prev_tok: int32 [R]")
    dev = L.device
    o = out or {}
    y = _take(o, "y", lambda: torch.empty(R, n, dtype=torch.int32, device=dev))
    logq = _take(o, "logq", lambda: torch.empty(R, n, dtype=torch.float32, device=dev)) if want_logq else None
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = _workspace(lib().dsp_draft_markov_step_workspace_size(R, V, rank, n, int(want_logq)), dev, prepare, stream)
    args = (_ptr(L), l_dt, ldl_r, ldl_d, _ptr(U), _ptr(Wt), V, rank, _ptr(prev_tok), R, n,
            _ptr(y), y.stride(0), _ptr(logq), _ptr(status), _ptr(ws), ws.numel(), _stream(stream))
    return _finish(lib().dsp_draft_markov_step, args, dict(y=y, logq=logq, status=status), prepare,
                   (L, U, Wt, prev_tok, ws), stream=stream)


def draft_rnn_step(L, h, Gt, A, E, Wot, prev_tok, bias=None, n_steps=None, want_logq=False, out=None, status=None,
                   stream=None, prepare=False):
    """Greedy chain with the RNN head. L: bf16 [R, B, V]; h: bf16 [R, B, H] backbone states;
    Gt: bf16 [r, H]; A: bf16 [r, r]; E, Wot: bf16 [V, r]; bias: float32 [r] or None;
    prev_tok: int32 [R]. Returns dict(y int32 [R, n], logq float32 [R, n] or None, status)."""
    _on_gpu(L, h, Gt, A, E, Wot, prev_tok, bias)
    l_dt, ldl_r, ldl_d = _chain_l(L)
    R, B, V = L.shape
    _need(h.dtype == torch.bfloat16 and h.dim() == 3 and h.shape[:2] == (R, B) and h.stride(2) == 1,
          "h: bf16 [R, B, H], unit inner stride")
    H = h.shape[2]
    rank = A.shape[0]
    _need(A.dtype == torch.bfloat16 and A.shape == (rank, rank) and A.is_contiguous(), "A: contiguous bf16 [r, r]")
    _need(Gt.dtype == torch.bfloat16 and Gt.shape == (rank, H) and Gt.is_contiguous(), "Gt: contiguous bf16 [r, H]")
    for t, nm in ((E, "E"), (Wot, "Wot")):
        _need(t.dtype == torch.bfloat16 and t.shape == (V, rank) and t.is_contiguous(), f"{nm}: contiguous bf16 [V, r]")
    _need(bias is None or (bias.dtype == torch.float32 and bias.numel() == rank and bias.is_contiguous()),
          "bias: float32 [r]")
    n = B if n_steps is None else int(n_steps)
    _need(1 <= n <= B, "n_steps must be in [1, B]")
    _need(prev_tok.dtype == torch.int32 and prev_tok.numel() == R and prev_tok.is_contiguous(), "prev_tok: int32 [R]")
    dev = L.device
    o = out or {}
    y = _take(o, "y", lambda: torch.empty(R, n, dtype=torch.int32, device=dev))
    logq = _take(o, "logq", lambda: torch.empty(R, n, dtype=torch.float32, device=dev)) if want_logq else None
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = _workspace(lib().dsp_draft_rnn_step_workspace_size(R, V, rank, n), dev, prepare, stream)
    args = (_ptr(L), l_dt, ldl_r, ldl_d, _ptr(h), DSP_BF16, h.stride(0), h.stride(1), H, _ptr(Gt),
            _ptr(A), _ptr(E), _ptr(bias), _ptr(Wot), V, rank, _ptr(prev_tok), R, n, _ptr(y), y.stride(0),
            _ptr(logq), _ptr(status), _ptr(ws), ws.numel(), _stream(stream))
    return _finish(lib().dsp_draft_rnn_step, args, dict(y=y, logq=logq, status=status), prepare,
                   (L, h, Gt, A, E, Wot, prev_tok, bias, ws), stream=stream)


def draft_markov_sample(L, U, Wt, prev_tok, temperature, seed=0, round=0, round_dev=None, req_id=None,
                        n_steps=None, want_logq=True, out=None, status=None, stream=None, prepare=False):
    """Sampled Markov chain. L: bf16 [R, B, V]; U, Wt: bf16 [V, rank]; prev_tok: int32 [R].

    Returns dict(y int32 [R, n], logq float32 [R, n] or None, z bf16 [R, n, V] (the
    emitted draft logits), status).
    """
    _check_markov(L, U, Wt, chain=True)
    l_dt, ldl_r, ldl_d = _chain_l(L)
    R, B, V = L.shape
    n = B if n_steps is None else int(n_steps)
    _need(1 <= n <= B, "n_steps must be in [1, B]")
    rank = U.shape[1]
    _need(prev_tok.dtype == torch.int32 and prev_tok.numel() == R and prev_tok.is_contiguous(), "prev_tok: int32 [R]")
    _on_gpu(round_dev, req_id)
    _need(round_dev is None or (round_dev.dtype == torch.int64 and round_dev.numel() == 1),
          "round_dev: int64 [1]")
    _need(req_id is None or (req_id.dtype == torch.int64 and req_id.numel() == R and req_id.is_contiguous()),
          "req_id: int64 [R]")
    dev = L.device
    o = out or {}
    y = _take(o, "y", lambda: torch.empty(R, n, dtype=torch.int32, device=dev))
    logq = _take(o, "logq", lambda: torch.empty(R, n, dtype=torch.float32, device=dev)) if want_logq else None
    vpad = (V + 7) // 8 * 8
    z = _take(o, "z", lambda: torch.empty(R, n, vpad, dtype=torch.bfloat16, device=dev)[..., :V])
    _need(z.dtype == torch.bfloat16 and z.dim() == 3 and z.stride(2) == 1, "z: bf16 [R, n, V] with unit stride")
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = _workspace(lib().dsp_draft_markov_sample_workspace_size(R, V, rank, n), dev, prepare, stream)
    args = (_ptr(L), l_dt, ldl_r, ldl_d, _ptr(U), _ptr(Wt), V, rank, _ptr(prev_tok), R, n,
            float(temperature), int(seed), int(round), _ptr(round_dev), _ptr(req_id), _ptr(y), y.stride(0),
            _ptr(logq), _ptr(z), z.stride(0), z.stride(1), _ptr(status), _ptr(ws), ws.numel(), _stream(stream))
    return _finish(lib().dsp_draft_markov_sample, args, dict(y=y, logq=logq, z=z, status=status), prepare,
                   (L, U, Wt, prev_tok, round_dev, req_id, ws), stream=stream)


def tree_expand(L, U, Wt, anchor, topk, frontier, topN, want_mask=False, out=None, status=None, stream=None,
                prepare=False):
    """PCTree expansion. Returns dict(node_token, node_parent, node_depth [R, topN] int32,
    node_score float64 [R, topN], n_nodes int32 [R], anc_mask int64 [R, topN, ceil(topN/64)]
    (uint64 bit sets: node o's ancestors and itself) or None, status)."""
    _check_markov(L, U, Wt)
    R, D, V = L.shape
    rank = U.shape[1]
    _need(anchor.dtype == torch.int32 and anchor.numel() == R and anchor.is_contiguous(), "anchor: int32 [R]")
    dev = L.device
    o = out or {}
    tok = _take(o, "node_token", lambda: torch.empty(R, topN, dtype=torch.int32, device=dev))
    par = _take(o, "node_parent", lambda: torch.empty(R, topN, dtype=torch.int32, device=dev))
    dep = _take(o, "node_depth", lambda: torch.empty(R, topN, dtype=torch.int32, device=dev))
    sc = _take(o, "node_score", lambda: torch.empty(R, topN, dtype=torch.float64, device=dev))
    nn = _take(o, "n_nodes", lambda: torch.empty(R, dtype=torch.int32, device=dev))
    words = (topN + 63) // 64
    mask = _take(o, "anc_mask", lambda: torch.empty(R, topN, words, dtype=torch.int64, device=dev)) \
        if want_mask else None
    if status is None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    nbytes = lib().dsp_tree_expand_workspace_size(R, D, V, rank, topk, frontier, topN)
    ws = _workspace(nbytes, dev, prepare, stream)
    args = (_ptr(L), DSP_BF16, L.stride(0), L.stride(1), _ptr(U), _ptr(Wt), V, rank, _ptr(anchor), R, D, topk,
            frontier, topN, _ptr(tok), _ptr(par), _ptr(dep), _ptr(sc), _ptr(nn), _ptr(mask), _ptr(status),
            _ptr(ws), ws.numel(), _stream(stream))
    res = dict(node_token=tok, node_parent=par, node_depth=dep, node_score=sc, n_nodes=nn, anc_mask=mask,
               status=status)
    return _finish(lib().dsp_tree_expand, args, res, prepare, (L, U, Wt, anchor, ws), stream=stream)


def stream_read(t, sink=None, stream=None):
    """Read every byte of the contiguous GPU tensor t (16-byte aligned, size a multiple of 16)
    with the library's streaming-read probe; returns the sink word tensor."""
    _on_gpu(t)
    _need(t.is_contiguous(), "t must be contiguous")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=t.device)
    _abi.check(lib().dsp_stream_read(_ptr(t), t.numel() * t.element_size(), _ptr(sink), _stream(stream)))
    return sink


def set_option(option, value):
    """Set a library option: "chain_persistent" (1 = the greedy chain may run all steps in
    one persistent launch, 0 = one launch per step, the default), "spin_limit" (polls of a
    persistent launch's grid barrier before it gives up with DSP_STATUS_TIMEOUT) or
    "tree_split" (1 = the tree's GEMM runs its depths whose row blocks span at most 16
    requests on the kernel with direct-to-LDS stages and a fixed issue order, the default;
    0 = the general GEMM everywhere; outputs are bit-identical) or "chain_sched" (1 = the
    greedy chain's arg-max steps run on the GEMM with direct-to-LDS stages; 0 = the general
    GEMM, the default; outputs are bit-identical)."""
    code = {"chain_persistent": _abi.DSP_OPT_CHAIN_PERSISTENT, "spin_limit": _abi.DSP_OPT_SPIN_LIMIT,
            "tree_split": _abi.DSP_OPT_TREE_SPLIT, "chain_sched": _abi.DSP_OPT_CHAIN_SCHED}[option]
    _abi.check(lib().dsp_set_option(code, int(value)))


def prof_enable(on=True, kernels=None):
    """Time every kernel (on=True), none (False), or only the named kernels."""
    if not on:
        mask = 0
    elif kernels is None:
        mask = -1
    else:
        mask = 0
        for k in kernels:
            mask |= 1 << KERNELS.index(k)
    _abi.check(lib().dsp_prof_enable(mask))


def prof_reset():
    _abi.check(lib().dsp_prof_reset())


def prof_query(kernel):
    """(total milliseconds, launches) recorded for a kernel name from KERNELS since the last reset."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _abi.check(lib().dsp_prof_query(KERNELS.index(kernel), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value

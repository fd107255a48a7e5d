"""Per-tier HIP graph replay of the ragged verify.

The SGLang article's "Ragged verify" section rounds the packed row total up to one
of a few captured sizes (tiers) and replays the graph captured for that size, so a
short batch does not pay for launches sized to the longest one. Here the pack
(``pack_ragged`` / ``schedule_pack`` with ``tiers=``) writes
``total_and_tier = (T, smallest tier >= T)`` on the device; a ``TierGraphs`` holds
one captured graph per tier and replays the one the pack chose.

The tier is known only once the scheduler's kernels have run, so choosing a graph
on the host costs a read-back of those two integers (through pinned host memory)
and a wait for it. The alternative that needs no read-back is one graph captured
at the largest size, whose kernels skip the rows past the device-side total.

Only host plumbing lives here: no arithmetic of the path.
"""
import torch


class TierGraphs:
    """One captured HIP graph per row tier.

    make(tier) returns a zero-argument callable that issues, on the current stream,
    work sized for `tier` packed rows (for example a prepared ``verify_rejection``
    with ``max_rows=tier``); it is called once per tier, inside the capture. The
    buffers those calls use must stay alive and at fixed addresses for as long as
    the graphs are replayed.
    """

    def __init__(self, tiers, make, stream=None):
        ts = sorted({int(t) for t in tiers})
        if not ts or ts[0] < 1:
            raise ValueError("tiers must be positive integers")
        self.tiers = ts
        self.stream = torch.cuda.current_stream() if stream is None else stream
        self._host = torch.zeros(2, dtype=torch.int32, pin_memory=True)
        self._ready = torch.cuda.Event()
        self.graphs = {}
        self._calls = {}
        for t in ts:
            fn = make(t)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.stream):
                fn()
            self.graphs[t] = g
            self._calls[t] = fn

    def tier_of(self, total_and_tier):
        """Read (T, tier) back once the work already queued on the stream has written it;
        returns the tier. Raises if the pack found no tier large enough (tier -1)."""
        with torch.cuda.stream(self.stream):
            self._host.copy_(total_and_tier, non_blocking=True)
            self._ready.record(self.stream)
        self._ready.synchronize()
        total, tier = int(self._host[0]), int(self._host[1])
        if tier < 0 or tier not in self.graphs:
            raise ValueError(f"packed total {total} has no captured tier (tiers {self.tiers})")
        return tier

    def replay(self, total_and_tier):
        """Replay the graph of the tier in total_and_tier (device int32 [2]); returns it."""
        tier = self.tier_of(total_and_tier)
        with torch.cuda.stream(self.stream):
            self.graphs[tier].replay()
        return tier

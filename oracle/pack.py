"""Front-packed ragged verify buffer -- oracle side (test infrastructure).

Follows the SGLang article (winzheng.jp), section "Ragged verify": each
request's verify window is packed front to back into one compact buffer with
cu_seqlens-style offsets, and the packed total is rounded up to the nearest
captured graph tier. The target writes the anchor and then checks the drafts
(DSpark study notes, section 3, Figure 1), so request i occupies n_i + 1 rows:
its anchor followed by its first n_i draft tokens, in request order.

Pinned by: cumsum special case, row-map bijection and total = R + sum n_i
invariants, and a hand-worked fixture (tests/test_oracle_pack.py).
"""
import numpy as np


def pack_ragged(windows, anchors, drafts, tiers=None):
    """Return dict(cu_seqlens [R+1], tokens [T], row_req [T], row_pos [T], total T, tier).

    windows: [R] int (0 <= n_i <= K); anchors: [R]; drafts: [R, K].
    tier: smallest entry of ``tiers`` (ascending) that is >= T, -1 if none;
    T itself when no tier list is given.
    """
    windows = np.asarray(windows, dtype=np.int64)
    anchors = np.asarray(anchors, dtype=np.int64)
    drafts = np.asarray(drafts, dtype=np.int64)
    R = windows.shape[0]
    cu = [0]
    for i in range(R):
        cu.append(cu[-1] + int(windows[i]) + 1)
    T = cu[-1]
    tokens = np.empty(T, dtype=np.int32)
    row_req = np.empty(T, dtype=np.int32)
    row_pos = np.empty(T, dtype=np.int32)
    for i in range(R):
        base = cu[i]
        tokens[base] = anchors[i]
        row_req[base] = i
        row_pos[base] = 0
        for k in range(1, int(windows[i]) + 1):
            tokens[base + k] = drafts[i, k - 1]
            row_req[base + k] = i
            row_pos[base + k] = k
    if tiers is None:
        tier = T
    else:
        tier = -1
        for t in tiers:
            if t >= T:
                tier = int(t)
                break
    return dict(cu_seqlens=np.array(cu, dtype=np.int32), tokens=tokens, row_req=row_req,
                row_pos=row_pos, total=T, tier=tier)

"""Open top-K score gaps in generated inputs.

TEST INFRASTRUCTURE ONLY (tests, the smoke check): it calls only the oracle.

Selection is compared bit-exactly, so every compared row must have a clear
boundary: when a row has more candidates than K, the K-th and (K+1)-th best
block scores (oracle, fp64) must differ by more than `min_gap`. A row that
misses the bar gets fresh query rows for its token (all G heads of the group,
keyed by attempt, same shared direction); other rows are untouched.
"""
import numpy as np

import synth


def boundary_gaps(R, Cn, K, relative=False):
    gaps = np.full(len(Cn), np.inf)
    for r, c in enumerate(Cn):
        if c > K:
            s = np.sort(R[r, :c])[::-1]
            gaps[r] = s[K - 1] - s[K]
            if relative:
                gaps[r] /= abs(s[K - 1])
    return gaps


def open_gaps(d, orc, group_rows=None, min_gap=1e-3, max_attempts=64, kbar=None, pos=None,
              score_fn=None, relative=False):
    """Redraw query tokens in-place in d["q"] until every listed row clears min_gap (relative to
    the K-th score when `relative`; scores from score_fn, default the oracle's raw scores).

    Returns (kbar, number of token redraws, smallest gap seen after fixing)."""
    w = d["workload"]
    G, K = w.group, w.top_k
    if kbar is None:
        kbar = orc.pool(d["k"], d["kv_len"])
    if pos is None:
        pos = orc.positions(w.mode, d["n_q"], d["q_pos0"])
    pending = orc.all_group_rows(w.batch, w.n_kv_heads, d["n_q"]) if group_rows is None else \
        np.asarray(group_rows, dtype=np.int32).reshape(-1, 3)
    redrawn = 0
    min_seen = np.inf
    for attempt in range(max_attempts):
        R, Cn = (score_fn or orc.scores)(d["q"], kbar, pos, pending, w.n_kv_heads)
        gaps = boundary_gaps(R, Cn, K, relative)
        bad = pending[gaps <= min_gap]
        ok = gaps[gaps > min_gap]
        if len(ok):
            min_seen = min(min_seen, ok.min())
        if len(bad) == 0:
            return kbar, redrawn, min_seen
        for b, g, i in bad:
            d["q"][b, g * G:(g + 1) * G, i] = synth.redraw_q_token(w, d["seed"], int(b), int(g), int(i), attempt)
            redrawn += 1
        pending = bad
    raise RuntimeError(f"{len(pending)} rows still within {min_gap} of a top-K tie after {max_attempts} redraws")

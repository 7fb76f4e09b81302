"""Plain CPU oracle of the DSA top-k position selector.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Follows page "mlx-bun 0.2.0 -> 0.4.0", file glm52-dsa.ts,
selectGlm52DsaDevice (the deterministic device form of the threshold-ties
selection), with the dense fallback of the indexer on page
"mlx-bun 0.4.0 -> 1.0.0", file glm52.ts: a row whose context is not longer
than top_k attends densely (no selection).

Selection of one row of float32 scores s[0..n):
  1. rank key: the order-preserving map of the float bits to uint32 (negative
     values flip every bit, others flip the sign bit), then inverted, so an
     ascending sort of the keys orders scores descending;
  2. a stable ascending sort of the keys: equal keys (equal score bits) keep
     ascending positions; the first top_k positions are selected;
  3. threshold = the minimum selected score;
  4. output order: the selected positions whose score is strictly greater
     than the threshold, ascending, then the remaining selected positions
     (the threshold ties), ascending.
The comparisons of step 4 are float comparisons (+0 and -0 are equal), the
ranking of steps 1-2 is by bits (+0 ranks above -0).  Scores must not be NaN
(the pages do not define that case); the oracle rejects it.
"""

from __future__ import annotations

import numpy as np

from .mla_oracle import OracleError


def dsa_rank_keys(scores: np.ndarray) -> np.ndarray:
    """uint32 keys whose ascending order is the descending order of the float32 scores."""
    s = np.ascontiguousarray(scores, dtype=np.float32)
    bits = s.view(np.uint32)
    negative = (bits & np.uint32(0x80000000)) != 0
    ascending = np.where(negative, ~bits, bits ^ np.uint32(0x80000000)).astype(np.uint32)
    return (~ascending).astype(np.uint32)


def dsa_select(scores: np.ndarray, top_k: int):
    """Selected positions (int32, in the output order) of one row, or None when
    the row is not longer than top_k (dense attention)."""
    s = np.asarray(scores, dtype=np.float32)
    if s.ndim != 1:
        raise OracleError("one row of scores expected")
    if top_k < 1:
        raise OracleError("top_k must be positive")
    if np.isnan(s).any():
        raise OracleError("NaN scores have no defined selection")
    n = s.shape[0]
    if n <= top_k:
        return None
    order = np.argsort(dsa_rank_keys(s), kind="stable")
    chosen = order[:top_k]
    threshold = s[chosen].min()
    above = np.sort(chosen[s[chosen] > threshold])
    ties = np.sort(chosen[~(s[chosen] > threshold)])
    return np.concatenate([above, ties]).astype(np.int32)


def dsa_select_rows(scores, row_len, top_k: int):
    """Rows b < B of scores[b, :row_len[b]] -> (sel_idx concatenated over the
    selected rows, sel_count per row: top_k, or -1 for a dense row)."""
    counts, parts = [], []
    for b, n in enumerate(row_len):
        sel = dsa_select(np.asarray(scores[b])[: int(n)], top_k)
        if sel is None:
            counts.append(-1)
        else:
            counts.append(top_k)
            parts.append(sel)
    idx = np.concatenate(parts).astype(np.int32) if parts else np.zeros(0, dtype=np.int32)
    return idx, np.array(counts, dtype=np.int32)

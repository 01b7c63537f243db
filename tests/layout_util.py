"""Row-subset helper for checking sampled rows of a large training layout."""
import numpy as np


def key_closure(rows, K, sample):
    """Kept rows that one layer of the sampled rows depends on: the sample,
    the depth-0 rows up to the largest sampled position (those up to the
    largest anchor are keys) and each sampled row's chain.  Visibility
    depends only on (position, depth), so with one layer
    the oracle over this chain-closed subset gives the sampled rows' exact
    results.  Returns (subset rows, indices of the sample in the subset)."""
    P, D = rows // K, rows % K
    pmax = int(np.max(P[sample]))
    need = set(int(r) for r in rows[sample])
    need.update(p * K for p in range(pmax + 1))
    for i in sample:
        a = int(P[i] - D[i])
        need.update((a + j) * K + j for j in range(1, int(D[i]) + 1))
    sub = np.array(sorted(need), dtype=np.int64)
    lm = np.searchsorted(sub, rows[sample])
    return sub, lm

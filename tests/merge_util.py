"""fp64 merge of attention results over disjoint key subsets through their
log-sum-exp: o = sum_r exp(lse_r) o_r / sum_r exp(lse_r) and
lse = log sum_r exp(lse_r) (what a caller combining sequence shards does)."""
import numpy as np


def merge(parts):
    """parts: [(o [B,S,H,D], lse [B,H,S]), ...] -> (o, lse) in fp64."""
    lses = np.stack([np.asarray(l, np.float64) for _, l in parts])   # [R,B,H,S]
    m = lses.max(axis=0)
    w = np.exp(lses - m)
    den = w.sum(axis=0)
    num = sum(np.transpose(w[r], (0, 2, 1))[..., None] * np.asarray(parts[r][0], np.float64)
              for r in range(len(parts)))
    return num / np.transpose(den, (0, 2, 1))[..., None], m + np.log(den)

"""Small statistics helpers shared by the oracle pins."""
import numpy as np


def chi2_pooled(counts, probs, min_expected=5.0):
    """Pearson statistic with cells of expected count < min_expected pooled
    (smallest first).  Returns (statistic, degrees of freedom).  A count in a
    cell of probability zero is an error of the sampler, not noise."""
    counts = np.asarray(counts, dtype=float)
    probs = np.asarray(probs, dtype=float)
    if (counts[probs <= 0] > 0).any():
        raise AssertionError("draws landed in a cell of probability zero")
    n = counts.sum()
    e = probs * n
    order = np.argsort(e)
    pooled_c, pooled_e = [], []
    acc_c = acc_e = 0.0
    for c, x in zip(counts[order], e[order]):
        acc_c += c
        acc_e += x
        if acc_e >= min_expected:
            pooled_c.append(acc_c)
            pooled_e.append(acc_e)
            acc_c = acc_e = 0.0
    if acc_e > 0 or acc_c > 0:
        if pooled_e:
            pooled_c[-1] += acc_c
            pooled_e[-1] += acc_e
        else:
            pooled_c.append(acc_c)
            pooled_e.append(acc_e)
    pc, pe = np.array(pooled_c), np.array(pooled_e)
    return float(((pc - pe) ** 2 / pe).sum()), len(pc) - 1

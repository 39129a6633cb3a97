"""Small statistics helpers shared by the CPU law tests."""
import numpy as np
from scipy import stats


def chisquare_pvalue(counts, probs, min_expected=5.0):
    """Pearson chi-square goodness of fit of integer counts against probs.

    Bins whose expected count is below min_expected are pooled into one bin
    (and that bin is dropped if it is still below the threshold)."""
    counts = np.asarray(counts, dtype=np.float64)
    probs = np.asarray(probs, dtype=np.float64)
    n = counts.sum()
    exp = probs / probs.sum() * n
    big = exp >= min_expected
    obs_b, exp_b = list(counts[big]), list(exp[big])
    if (~big).any():
        rest_o, rest_e = counts[~big].sum(), exp[~big].sum()
        if rest_e >= min_expected:
            obs_b.append(rest_o)
            exp_b.append(rest_e)
        elif rest_o > max(10.0, 10 * rest_e):
            return 0.0  # mass where almost none is expected
    obs_b = np.array(obs_b)
    exp_b = np.array(exp_b)
    exp_b *= obs_b.sum() / exp_b.sum()
    if len(obs_b) < 2:
        return 1.0
    return float(stats.chisquare(obs_b, exp_b).pvalue)

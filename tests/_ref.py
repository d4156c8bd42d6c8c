"""Small textbook references used to pin the oracle (numpy, float64).

These are independent of the oracle's code: textbook softmax attention with a
mask, and a log-sum-exp from scipy.
"""
import numpy as np
from scipy.special import logsumexp

import hils_synth as hs


def f64(a):
    return hs.as_f64(np.asarray(a))


def masked_attention(q, k, v, mask, tau):
    """Softmax attention of each row of q over the keys where mask is True.
    q [n,d], k/v [T,d], mask [n,T] -> [n,d]."""
    logits = tau * (q @ k.T)
    logits = np.where(mask, logits, -np.inf)
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = w / w.sum(axis=1, keepdims=True)
    return w @ v


def causal_attention_rows(q, k, v, pos, tau):
    T = k.shape[0]
    mask = np.arange(T)[None, :] <= np.asarray(pos)[:, None]
    return masked_attention(q, k, v, mask, tau)


def lse(x):
    return logsumexp(x)

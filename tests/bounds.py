"""The logit bound that selects the attention kernels' softmax mode, restated for the tests, and weights built to
land on either side of its limits.

QK-RMSNorm bounds every logit: RoPE rotates each channel pair rigidly, so in base-2 units
|q^ . k^| log2(e) / sqrt(d) <= log2(e) sqrt(d) max_i u_i v_i, with u_i, v_i the larger |weight| of channel pair
i in w_q, w_k (the kernels add a 2% margin for their own rounding).  Up to 48 the static mode takes exp2 of the
logits as they are; up to 80 it subtracts the constant bound - 48 (through the accumulator input of the logit
MFMAs); past 80 (or for NaN weights) the running-maximum kernel runs.
"""
import numpy as np

UNSHIFTED_LIMIT = 48.0
STATIC_LIMIT = 80.0
ONLINE_TARGET = 90.0       # a bound past the static limit with some margin, logits still moderate


def pair_bound(wq, wk, d):
    u = np.maximum(np.abs(wq[0::2]), np.abs(wq[1::2])).astype(np.float64)
    v = np.maximum(np.abs(wk[0::2]), np.abs(wk[1::2])).astype(np.float64)
    return np.log2(np.e) * np.sqrt(d) * float(np.max(u * v)) * 1.02


def mode(wq, wk, d):
    b = pair_bound(wq, wk, d)
    return "static" if b <= STATIC_LIMIT else "online"


def spike_to_bound(wq, wk, d, channel, target=ONLINE_TARGET):
    """A copy of wq with one channel raised so that the pairwise bound equals `target` (that channel's pair then
    holds the maximum): the rest of the weights, and so the typical logits, stay as they were."""
    p = channel // 2
    v = max(abs(float(wk[2 * p])), abs(float(wk[2 * p + 1])))
    w = np.array(wq, dtype=np.float32, copy=True)
    w[channel] = np.float32(target / (np.log2(np.e) * np.sqrt(d) * 1.02 * v))
    b = pair_bound(w, wk, d)
    assert abs(b - target) < 1e-3 * target, (b, target)
    return w

"""The logit bound that selects the static-shift softmax, checked on the CPU with the oracle's RMSNorm
and 3D RoPE: log2(e) sqrt(d) max_i u_i v_i, with u_i, v_i the larger |weight| of channel pair i of w_q
and w_k.  The kernels take exp2 of logits without a shift when this bound (times a 2% margin) is at
most 48, and of the logits less the constant bound - 48 when it is at most 80, so it must hold for every
input, and it should be tight: an input concentrated on the best pair reaches it."""
import numpy as np

from oracle import attention as A

D = 96


def pair_bound(wq, wk, d=D):
    u = np.maximum(np.abs(wq[0::2]), np.abs(wq[1::2]))
    v = np.maximum(np.abs(wk[0::2]), np.abs(wk[1::2]))
    return np.sqrt(d) * float(np.max(u * v))          # natural-log units, no margin


def weights(seed):
    rng = np.random.default_rng(seed)
    wq = 1 + 0.3 * rng.standard_normal(D)
    wk = 1 + 0.3 * rng.standard_normal(D)
    wq[10] = 3.0                                      # the largest |w_q| and |w_k| sit in different pairs,
    wk[40] = 2.5                                      # where the pairwise bound is the tighter one
    return wq, wk


def test_bound_holds_for_random_and_adversarial_inputs():
    wq, wk = weights(0)
    b = pair_bound(wq, wk)
    assert b < np.sqrt(D) * np.abs(wq).max() * np.abs(wk).max()
    rng = np.random.default_rng(1)
    T, H, W = 2, 6, 10
    N = T * H * W
    for trial in range(4):
        q = rng.standard_normal((N, 1, D))
        k = rng.standard_normal((N, 1, D))
        if trial >= 2:                                 # spikes on the large channels
            q[:, 0, 10] *= 30
            k[:, 0, 40] *= 30
        L = A.logits(q, k, wq, wk, T, H, W, 0)
        assert np.abs(L).max() <= b * (1 + 1e-12)


def test_bound_is_reached_by_an_input_on_the_best_pair():
    """q and k each put all their energy on the channel of the best pair with the larger weight (the same
    channel for both here), at the same grid position: the rotation cancels and the logit is
    sqrt(d) u_i v_i up to the norm's eps."""
    wq, wk = weights(2)
    u = np.maximum(np.abs(wq[0::2]), np.abs(wq[1::2]))
    v = np.maximum(np.abs(wk[0::2]), np.abs(wk[1::2]))
    i = int(np.argmax(u * v))
    c = 2 * i + int(np.abs(wq[2 * i + 1]) > np.abs(wq[2 * i]))
    wk[c] = np.sign(wk[c]) * v[i] if wk[c] != 0 else v[i]     # the larger |w_k| of the pair on channel c too
    q = np.zeros((4, 1, D))
    k = np.zeros((4, 1, D))
    q[:, 0, c] = 1.0
    k[:, 0, c] = np.sign(wq[c] * wk[c])
    L = A.logits(q, k, wq, wk, 1, 2, 2, 0, eps=0.0)
    b = pair_bound(wq, wk)
    assert np.isclose(np.diag(L).min(), b, rtol=1e-12)
    assert np.abs(L).max() <= b * (1 + 1e-12)


def test_bench_names_the_kernel_the_weights_select():
    """bench.py labels its roofline with the kernel the weights select: the 1 + 0.1 N(0,1) weights and the
    1.75 times larger ones (bound 59.6, shifted) take the static kernel, one w_q channel at 6 (bound 89.9) the
    running-maximum one; equal weights c give the bound log2(e) sqrt(d) c^2 (times the 2% margin), which
    decides on either side of 80."""
    import importlib.util
    import os

    from synth import WORKLOADS, norm_weights
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    for name, want in (("v5", "static"), ("v5s", "static"), ("v5d128", "static"), ("v5w", "static"),
                       ("v5sw", "static"), ("v5o", "online"), ("v5so", "online")):
        wq, wk = norm_weights(name)
        assert bench.softmax_mode(wq, wk, WORKLOADS[name].head_dim) == want, name
    for d in (96, 128):
        c_edge = np.sqrt(80.0 / (np.log2(np.e) * np.sqrt(d) * 1.02))
        for f, want in ((0.999, "static"), (1.001, "online")):
            w = np.full(d, c_edge * f, dtype=np.float32)
            assert bench.softmax_mode(w, w, d) == want

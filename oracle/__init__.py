"""fp64 CPU oracle for the DiT self-attention hot path.

TEST INFRASTRUCTURE ONLY: the plain, slow, obviously-correct definition the
HIP kernels are checked against.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code
with the HIP path and never imports it.

* ``attention``  -- RMSNorm + 3D RoPE + dense / block-sparse softmax attention (fp64),
                    and joint attention over explicit per-token positions
* ``router``     -- fp32-exact block router (pool, score, top-k), plus an
                    independent float32 evaluation and an exact fp64 variant
* ``block_ops``  -- the operators around attention: AdaLN update, gated residual,
                    SwiGLU (fp64)
* ``brute``      -- pure-Python scalar versions of the above for tiny inputs

Pins: every function is pinned in tests/test_oracle_*.py against closed forms,
invariants, brute force and special cases; parity with a trained H3 model is
unpinned (no weights or reference activations exist for it).
"""
from . import attention, block_ops, brute, router  # noqa: F401

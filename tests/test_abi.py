"""C-ABI contract tests that need no GPU: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments on the host before
queueing any work (so no device is touched)."""
import ctypes
import os
import re

import pytest

import image_diffusion_transformer_amd as dit
from image_diffusion_transformer_amd import _binding as B

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADERS = [os.path.join(INCLUDE, "dit_attn.h"), os.path.join(INCLUDE, "dit_block.h")]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from image_diffusion_transformer_amd.build import build
        build()
    return B.load_library()


def header_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(dit_\w+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert getattr(lib, n) is not None
        assert hasattr(dit, n), n           # the Python binding keeps the C names


def test_keep_count_matches_golden(lib):
    assert dit.dit_attn_keep_count(977, 0.75) == 245
    assert dit.dit_attn_keep_count(1922, 0.80) == 385
    assert dit.dit_attn_keep_count(512, 0.75) == 128
    assert dit.dit_attn_keep_count(977, 0.0) == 977
    assert dit.dit_attn_keep_count(1, 0.8) == 1
    assert dit.dit_attn_keep_count(10, 1.0) == -1
    assert dit.dit_attn_keep_count(0, 0.5) == -1


def test_workspace_bytes(lib):
    n = dit.dit_attn_workspace_bytes(31, 48, 84, 56)
    assert n == dit.dit_attn_workspace_bytes(31, 48, 84, 56, 96, 128, 0.75)   # covers any mask: no sparsity term
    N, nb = 124992, 977
    assert n >= 56 * nb * 48 * 1024 + 2 * 56 * nb * 96 * 4 + 56 * nb * nb * 4   # images + router: pooled, scores
    big = dit.dit_attn_workspace_bytes(1, 640, 820, 1)    # 4100 blocks: no score matrix
    assert big < 4100 * 48 * 1024 + 2 * 4100 * 96 * 4 + 4100 * 4100 * 4
    assert n >= 56 * -(-N // 512) * nb * 4                  # sparse: KV lists per 512-token query tile
    assert n >= 56 * nb * 48 * 1024 + 56 * -(-N // 512) * nb * 4   # K^/V fragment images + sparse lists
    nqt, words = -(-N // 512), -(-nb // 64)
    sched = (56 * nqt * nb * 4 + 56 * nqt * nb + 56 * nqt * 4 + 56 * nqt * 4 * 4   # lists, flags, counts, slots
             + 56 * nb * words * 8)                                                  # packed mask rows
    assert n >= 56 * nb * 48 * 1024 + sched
    assert dit.dit_attn_workspace_bytes(31, 48, 84, 56, 64) == 0    # head_dim 64 unsupported
    n128 = dit.dit_attn_workspace_bytes(31, 48, 84, 42, 128)        # 42 heads x 128: 64 KB tile images
    assert n128 >= 42 * nb * 64 * 1024 + 2 * 42 * nb * 128 * 4 + 42 * nb * nb * 4
    assert dit.dit_attn_workspace_bytes(31, 48, 84, 56, 96, 64) == 0
    assert dit.dit_attn_workspace_bytes(0, 48, 84, 56) == 0
    for bad in (1.0, -0.1, float("nan"), float("inf")):                 # sparsity outside [0, 1)
        assert dit.dit_attn_workspace_bytes(31, 48, 84, 56, 96, 128, bad) == 0


def test_workspace_bytes_signature_matches_header():
    text = re.sub(r"/\*.*?\*/", "", open(HEADERS[0]).read(), flags=re.S)
    decl = re.search(r"size_t\s+dit_attn_workspace_bytes\s*\(([^)]*)\)", text).group(1)
    params = [p.split()[-1] for p in decl.split(",")]
    assert params == ["T", "H", "W", "heads", "head_dim", "block", "sparsity"]
    assert "float sparsity" in decl


# Stand-in addresses, aligned, non-null and 16 MB apart (every buffer of these shapes fits in 16 MB, the
# workspace bound the size checks use excepted); validation fails before anything dereferences them.
FAKE = 1 << 24
Q, K, V, WQ, WK, O, MASK, WS, QP, KP = ((i + 1) << 24 for i in range(10))
WS = 1 << 40     # far above the others: the workspace bytes a call needs may exceed 16 MB


def _dense(lib, **kw):
    a = dict(q=Q, k=K, v=V, wq=WQ, wk=WK, T=2, H=4, W=4, heads=2, d=96, theta=1e4, eps=1e-6,
             o=O, ws=WS, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.dit_attn_dense(a["q"], a["k"], a["v"], a["wq"], a["wk"], a["T"], a["H"], a["W"], a["heads"], a["d"],
                              a["theta"], a["eps"], a["o"], a["ws"], a["wsb"], a["stream"])


def _route(lib, **kw):
    a = dict(q=Q, k=K, wq=WQ, wk=WK, T=2, H=4, W=4, heads=2, d=96, theta=1e4, eps=1e-6, s=0.75,
             block=128, mask=MASK, ws=WS, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.dit_attn_route(a["q"], a["k"], a["wq"], a["wk"], a["T"], a["H"], a["W"], a["heads"], a["d"],
                              a["theta"], a["eps"], a["s"], a["block"], a["mask"], a["ws"], a["wsb"], a["stream"])


def _sparse(lib, **kw):
    a = dict(q=Q, k=K, v=V, wq=WQ, wk=WK, T=2, H=4, W=4, heads=2, d=96, theta=1e4, eps=1e-6,
             block=128, mask=MASK, o=O, ws=WS, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.dit_attn_block_sparse(a["q"], a["k"], a["v"], a["wq"], a["wk"], a["T"], a["H"], a["W"], a["heads"],
                                     a["d"], a["theta"], a["eps"], a["block"], a["mask"], a["o"], a["ws"], a["wsb"],
                                     a["stream"])


@pytest.mark.parametrize("call", [_dense, _route, _sparse])
@pytest.mark.parametrize("kw,status,text", [
    (dict(q=None), B.DIT_ERR_INVALID_ARG, "null"),
    (dict(k=None), B.DIT_ERR_INVALID_ARG, "null"),
    (dict(wq=None), B.DIT_ERR_INVALID_ARG, "null"),
    (dict(q=Q + 2), B.DIT_ERR_INVALID_ARG, "aligned"),
    (dict(T=0), B.DIT_ERR_INVALID_ARG, "grid"),
    (dict(heads=-1), B.DIT_ERR_INVALID_ARG, "grid"),
    (dict(d=64), B.DIT_ERR_UNSUPPORTED, "head_dim"),
    (dict(T=4000, H=4000, W=4), B.DIT_ERR_UNSUPPORTED, "exceeds"),
    (dict(T=1, H=1, W=1, heads=70000), B.DIT_ERR_UNSUPPORTED, "heads 70000 exceeds"),
    (dict(theta=0.0), B.DIT_ERR_INVALID_ARG, "rope_theta"),
    (dict(theta=float("inf")), B.DIT_ERR_INVALID_ARG, "rope_theta"),
    (dict(eps=-1.0), B.DIT_ERR_INVALID_ARG, "eps"),
    (dict(eps=float("nan")), B.DIT_ERR_INVALID_ARG, "eps"),
    (dict(ws=None), B.DIT_ERR_WORKSPACE, "workspace"),
    (dict(wsb=100), B.DIT_ERR_WORKSPACE, "need"),
    (dict(ws=WS + 16), B.DIT_ERR_INVALID_ARG, "256-byte"),
])
def test_validation_errors(lib, call, kw, status, text):
    assert call(lib, **kw) == status
    assert text in B.dit_attn_last_error()


@pytest.mark.parametrize("kw,status,text", [
    (dict(s=1.0), B.DIT_ERR_INVALID_ARG, "sparsity"),
    (dict(s=-0.1), B.DIT_ERR_INVALID_ARG, "sparsity"),
    (dict(s=float("nan")), B.DIT_ERR_INVALID_ARG, "sparsity"),
    (dict(block=64), B.DIT_ERR_UNSUPPORTED, "block"),
    (dict(mask=None), B.DIT_ERR_INVALID_ARG, "mask"),
])
def test_route_specific_errors(lib, kw, status, text):
    assert _route(lib, **kw) == status
    assert text in B.dit_attn_last_error()


@pytest.mark.parametrize("kw,status,text", [
    (dict(v=None), B.DIT_ERR_INVALID_ARG, "null"),
    (dict(o=None), B.DIT_ERR_INVALID_ARG, "null"),
    (dict(mask=None), B.DIT_ERR_INVALID_ARG, "null"),
    (dict(block=256), B.DIT_ERR_UNSUPPORTED, "block"),
])
def test_sparse_specific_errors(lib, kw, status, text):
    assert _sparse(lib, **kw) == status
    assert text in B.dit_attn_last_error()


def test_python_binding_raises(lib):
    with pytest.raises(dit.DitAttnError) as e:
        B._check(_dense(lib, d=64))
    assert e.value.status == B.DIT_ERR_UNSUPPORTED


def test_missing_library_fails_loudly(tmp_path):
    saved = B._lib
    try:
        B._lib = None
        with pytest.raises(RuntimeError, match="not built"):
            B.load_library(str(tmp_path / "libditattn.so"))
    finally:
        B._lib = saved


def _joint(lib, **kw):
    a = dict(q=Q, k=K, v=V, wq=WQ, wk=WK, qp=QP, kp=KP, nq=20, nk=50, heads=2, d=96, maxp=16,
             theta=1e4, eps=1e-6, o=O, ws=WS, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.dit_attn_joint(a["q"], a["k"], a["v"], a["wq"], a["wk"], a["qp"], a["kp"], a["nq"], a["nk"], a["heads"],
                              a["d"], a["maxp"], a["theta"], a["eps"], a["o"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status,text", [
    (dict(qp=None), B.DIT_ERR_INVALID_ARG, "null"),
    (dict(kp=None), B.DIT_ERR_INVALID_ARG, "null"),
    (dict(v=None), B.DIT_ERR_INVALID_ARG, "null"),
    (dict(q=None), B.DIT_ERR_INVALID_ARG, "null"),
    (dict(qp=QP + 2), B.DIT_ERR_INVALID_ARG, "4-byte"),
    (dict(v=V + 8), B.DIT_ERR_INVALID_ARG, "aligned"),
    (dict(nq=0), B.DIT_ERR_INVALID_ARG, "token counts"),
    (dict(nk=-3), B.DIT_ERR_INVALID_ARG, "token counts"),
    (dict(maxp=0), B.DIT_ERR_INVALID_ARG, "max_pos"),
    (dict(maxp=(1 << 20) + 1), B.DIT_ERR_UNSUPPORTED, "max_pos"),
    (dict(d=64), B.DIT_ERR_UNSUPPORTED, "head_dim"),
    (dict(nk=30_000_000), B.DIT_ERR_UNSUPPORTED, "exceeds"),
    (dict(nq=1, nk=1, heads=70000), B.DIT_ERR_UNSUPPORTED, "heads 70000 exceeds"),
    (dict(theta=-1.0), B.DIT_ERR_INVALID_ARG, "rope_theta"),
    (dict(ws=None), B.DIT_ERR_WORKSPACE, "workspace"),
    (dict(wsb=64), B.DIT_ERR_WORKSPACE, "need"),
    (dict(ws=WS + 128), B.DIT_ERR_INVALID_ARG, "256-byte"),
])
def test_joint_validation_errors(lib, kw, status, text):
    assert _joint(lib, **kw) == status
    assert text in B.dit_attn_last_error()


# Buffers a call writes may not overlap any other buffer of the call; read-only inputs may alias.
@pytest.mark.parametrize("call,kw,text", [
    (_dense, dict(o=Q), "q overlaps o"),
    (_dense, dict(o=V + 4096), "v overlaps o"),                 # partial overlap (o starts inside v)
    (_dense, dict(o=WK), "wk overlaps o"),
    (_dense, dict(ws=(K // 256) * 256), "k overlaps workspace"),
    (_dense, dict(o=WS + (1 << 16)), "o overlaps workspace"),
    (_route, dict(mask=K + 256), "k overlaps mask"),
    (_route, dict(ws=WQ - 4096), "wq overlaps workspace"),
    (_sparse, dict(o=MASK), "mask overlaps o"),
    (_sparse, dict(ws=MASK - 256), "mask overlaps workspace"),
    (_joint, dict(o=KP), "k_pos overlaps o"),
    (_joint, dict(ws=QP), "q_pos overlaps workspace"),
])
def test_written_buffers_must_not_overlap(lib, call, kw, text):
    assert call(lib, **kw) == B.DIT_ERR_INVALID_ARG
    assert text in B.dit_attn_last_error()


NO_THROW_PROBE = r'''
import ctypes, resource, sys
sys.path.insert(0, ROOT)
from image_diffusion_transformer_amd import _binding as B
lib = B.load_library()
vm = int(open("/proc/self/status").read().split("VmSize:")[1].split()[0]) * 1024
# 128 MB of address space beyond what the process holds: the RoPE table of a joint call at head dim 128
# with 2^20 positions per axis (3 x 2^20 rows x 44 floats = 554 MB) cannot be allocated.
resource.setrlimit(resource.RLIMIT_AS, (vm + (128 << 20), resource.RLIM_INFINITY))
big = (1 << 40)
st = lib.dit_attn_joint(1 << 24, 2 << 24, 3 << 24, 4 << 24, 5 << 24, 6 << 24, 7 << 24, 20, 50, 2, 128, 1 << 20,
                        1e4, 1e-6, 8 << 24, big, 1 << 36, None)
print(st, B.dit_attn_last_error())
'''


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present: were the address-space limit to fail to "
                    "take, the call would go on to a device copy to a stand-in address")
def test_host_allocation_failure_returns_status_not_exception():
    """A host allocation failure inside an entry point (the RoPE table) comes back as DIT_ERR_HOST with a message:
    no C++ exception crosses the C ABI (it would terminate the process)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = f"ROOT = {root!r}\n" + NO_THROW_PROBE
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    status, _, msg = r.stdout.strip().partition(" ")
    assert int(status) == B.DIT_ERR_HOST, r.stdout
    assert "host memory" in msg


def test_workspace_covers_the_tail_split_partials(lib):
    # 7 heads of the 5 s grid: 1715 query tiles, 215 per XCD run = 6 rounds of 32 and 23 more, which the dense
    # call cuts into 4 key-range pieces each: 8 x 23 x 4 fp32 partials of 8 waves x 2 blocks x (3 x 16 + 2) x 64
    nb = 977
    partials = 8 * 23 * 4 * (8 * 2 * 50 * 64 * 4)
    n = dit.dit_attn_workspace_bytes(31, 48, 84, 7)
    assert n >= 7 * nb * 48 * 1024 + partials
    # the same tiles as one joint call (queries = keys = the grid tokens) split the same way
    assert dit.dit_attn_joint_workspace_bytes(124992, 124992, 7, 96, 84) >= 7 * nb * 48 * 1024 + partials


def test_calls_within_the_noalloc_scratch_never_split_their_last_round(lib):
    # The dense tail split (restated: 8 XCD runs of ceil(tiles / 8), 32 CUs each; at least 4 full rounds, at
    # least 16 key tiles, 2-4 pieces, at least 1% saved) needs many more query tiles than the 64 MiB static
    # scratch of dit_attn_dense_noalloc can hold fragment images for, so that entry point needs no partials.
    import math
    cap = dit.NOALLOC_SCRATCH_BYTES

    def splits(total, nt):
        per = (total + 7) // 8
        rounds, rem = divmod(per, 32)
        if rounds < 4 or rem == 0 or nt < 16:
            return False
        return min(math.ceil(rem * p / 32) / p for p in (2, 3, 4)) <= 1 - 0.01 * (rounds + 1)

    for d, bq, tile in ((96, 512, 48 * 1024), (128, 256, 64 * 1024)):
        for nb in range(16, 1400):
            heads_max = cap // (nb * tile)
            for heads in range(1, heads_max + 1):
                assert not splits(heads * -(-nb * 128 // bq), nb), (d, nb, heads)


def test_joint_workspace_bytes(lib):
    n = dit.dit_attn_joint_workspace_bytes(65536, 197120, 56, 96, 515)
    assert n >= 56 * 1540 * 48 * 1024 + 515 * 32 * 4          # fragment images of 1540 key tiles + table
    assert dit.dit_attn_joint_workspace_bytes(10, 10, 2, 96, 0) == 0
    assert dit.dit_attn_joint_workspace_bytes(10, 0, 2, 96, 4) == 0


# ---------------------------------------------------------------------------------- operators around attention
def _adaln(lib, **kw):
    a = dict(x=FAKE, shift=FAKE, scale=FAKE, tokens=10, hidden=5376, eps=1e-6, h=FAKE + (1 << 24), stream=None)
    a.update(kw)
    return lib.dit_adaln_modulate(a["x"], a["shift"], a["scale"], a["tokens"], a["hidden"], a["eps"], a["h"],
                                  a["stream"])


def _resid(lib, **kw):
    a = dict(x=FAKE, y=FAKE + (1 << 24), gate=FAKE, shift=FAKE, scale=FAKE, tokens=10, hidden=5376, eps=1e-6,
             x_out=FAKE, h=FAKE + (2 << 24), stream=None)
    a.update(kw)
    return lib.dit_gated_residual(a["x"], a["y"], a["gate"], a["shift"], a["scale"], a["tokens"], a["hidden"],
                                  a["eps"], a["x_out"], a["h"], a["stream"])


def _swiglu(lib, **kw):
    a = dict(gu=FAKE, tokens=10, ffn=14336, out=FAKE + (1 << 24), stream=None)
    a.update(kw)
    return lib.dit_swiglu(a["gu"], a["tokens"], a["ffn"], a["out"], a["stream"])


@pytest.mark.parametrize("call,kw,status,text", [
    (_adaln, dict(x=None), B.DIT_ERR_INVALID_ARG, "null"),
    (_adaln, dict(hidden=5370), B.DIT_ERR_INVALID_ARG, "multiple of 8"),
    (_adaln, dict(hidden=0), B.DIT_ERR_INVALID_ARG, "multiple of 8"),
    (_adaln, dict(hidden=8200), B.DIT_ERR_UNSUPPORTED, "exceeds"),
    (_adaln, dict(tokens=-1), B.DIT_ERR_INVALID_ARG, "tokens"),
    (_adaln, dict(eps=float("nan")), B.DIT_ERR_INVALID_ARG, "eps"),
    (_adaln, dict(scale=FAKE + 4), B.DIT_ERR_INVALID_ARG, "aligned"),
    (_adaln, dict(h=FAKE + 1024), B.DIT_ERR_INVALID_ARG, "overlaps"),
    (_resid, dict(gate=None), B.DIT_ERR_INVALID_ARG, "null"),
    (_resid, dict(shift=None), B.DIT_ERR_INVALID_ARG, "shift and scale"),
    (_resid, dict(x_out=FAKE + 1024), B.DIT_ERR_INVALID_ARG, "x itself"),
    (_resid, dict(x_out=FAKE + (1 << 24)), B.DIT_ERR_INVALID_ARG, "overlaps y"),
    (_resid, dict(h=FAKE + 64), B.DIT_ERR_INVALID_ARG, "h overlaps"),
    (_resid, dict(y=FAKE + (1 << 24) + 8), B.DIT_ERR_INVALID_ARG, "aligned"),
    (_swiglu, dict(ffn=12), B.DIT_ERR_INVALID_ARG, "multiple of 8"),
    (_swiglu, dict(out=FAKE + 4096), B.DIT_ERR_INVALID_ARG, "overlaps"),
    (_swiglu, dict(gu=None), B.DIT_ERR_INVALID_ARG, "null"),
])
def test_block_validation_errors(lib, call, kw, status, text):
    assert call(lib, **kw) == status
    assert text in B.dit_attn_last_error()


def test_block_zero_tokens_queue_nothing(lib):
    # valid arguments with no rows: success without touching a device
    assert _adaln(lib, tokens=0) == B.DIT_OK
    assert _resid(lib, tokens=0) == B.DIT_OK
    assert _resid(lib, tokens=0, h=None, shift=None, scale=None) == B.DIT_OK
    assert _swiglu(lib, tokens=0) == B.DIT_OK


def test_product_package_never_imports_the_oracle():
    """The oracle is test infrastructure: importing and loading the product must not pull it in."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys; import image_diffusion_transformer_amd as d; d.load_library(); "
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')]; "
            "assert not bad, bad")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]


def test_launch_order_values(lib):
    """The diagnostic workgroup order takes 0 or 1 only (host-side; no device is touched)."""
    assert lib.dit_attn_set_launch_order(2) == B.DIT_ERR_INVALID_ARG
    assert "launch order" in B.dit_attn_last_error()
    assert lib.dit_attn_set_launch_order(-1) == B.DIT_ERR_INVALID_ARG
    assert lib.dit_attn_set_launch_order(1) == B.DIT_OK
    assert lib.dit_attn_set_launch_order(0) == B.DIT_OK
    assert B.dit_attn_last_error() == ""


def _noalloc(lib, **kw):
    a = dict(q=Q, k=K, v=V, wq=WQ, wk=WK, T=1, H=128, W=342, heads=4, d=96, theta=1e4, eps=1e-6, o=O, stream=None)
    a.update(kw)
    return lib.dit_attn_dense_noalloc(a["q"], a["k"], a["v"], a["wq"], a["wk"], a["T"], a["H"], a["W"], a["heads"],
                                      a["d"], a["theta"], a["eps"], a["o"], a["stream"])


@pytest.mark.parametrize("kw", [dict(), dict(T=1, H=128, W=512, heads=2, d=128), dict(T=31, H=48, W=84, heads=56)])
def test_noalloc_rejects_calls_past_the_static_scratch(lib, kw):
    """Sizes past the 64 MiB static scratch are refused on the host, before any HIP call: one tile image more
    than fits at each head dim (4 x 342 blocks at 96, 2 x 512 at 128) and the full 5 s video layer."""
    assert _noalloc(lib, **kw) == B.DIT_ERR_UNSUPPORTED
    assert "static scratch" in B.dit_attn_last_error()
    assert str(B.NOALLOC_SCRATCH_BYTES) in B.dit_attn_last_error()


@pytest.mark.parametrize("kw,status,text", [
    (dict(q=None), B.DIT_ERR_INVALID_ARG, "null"),
    (dict(o=None), B.DIT_ERR_INVALID_ARG, "null"),
    (dict(d=64), B.DIT_ERR_UNSUPPORTED, "head_dim"),
    (dict(eps=float("nan")), B.DIT_ERR_INVALID_ARG, "eps"),
])
def test_noalloc_validation_errors(lib, kw, status, text):
    assert _noalloc(lib, **kw) == status
    assert text in B.dit_attn_last_error()


def test_noalloc_scratch_size_matches_header():
    text = open(HEADERS[0]).read()
    assert re.search(r"#define DIT_ATTN_NOALLOC_SCRATCH_BYTES \(\(size_t\)64 << 20\)", text)
    assert B.NOALLOC_SCRATCH_BYTES == 64 << 20

"""The HBM-traffic figures bench.py reports are tied to the kernel source they were measured on by a hash
of its code: comment and whitespace edits keep the hash, any change to the code itself changes it."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_code_hash_ignores_comments_and_whitespace(tmp_path):
    b = bench()
    src = "// header\nint f(int x) {\n  return x & 0xffffff;  // mask\n}\n/* block\n comment */\n"
    same = "// other header\n\nint f(int x)   {\n return x & 0xffffff;\n}\n"
    changed = "int f(int x) {\n  return x & 0xfffff;\n}\n"
    paths = []
    for i, text in enumerate((src, same, changed)):
        p = tmp_path / f"k{i}.hip"
        p.write_text(text)
        paths.append(str(p))
    h = [b.kernel_source_sha256(p) for p in paths]
    assert h[0] == h[1]
    assert h[0] != h[2]


"""Host-side checks of bench.py's bookkeeping (no GPU needed)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_source_digest_ignores_comments_only(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("// header\nint f(int x) {\n  return x + 1;  // one\n}\n/* block\n comment */\n")
    b = tmp_path / "b.hip"
    b.write_text("// another header\nint f(int x)   {\n    return x + 1;\n}\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.source_digest(str(a)) == bench.source_digest(str(b))
    assert bench.source_digest(str(a)) != bench.source_digest(str(c))


"""Host logic of bench.py: the source digest that ties a measured HBM traffic figure to the code it
was measured on. A comment or layout edit keeps the digest; any change to code, a string literal
included, changes it."""
import os
import sys

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), ".."))
import bench  # noqa: E402

SRC = 'int f(int a) { // sum\n  /* two\n lines */ return a + 1; }\nconst char* s = "x // y";\n'


def _digest(tmp_path, text):
    p = tmp_path / "k.hip"
    p.write_text(text)
    return bench.code_digest([str(p)])


def test_comment_and_layout_edits_keep_the_digest(tmp_path):
    d = _digest(tmp_path, SRC)
    assert _digest(tmp_path, SRC.replace("// sum", "// the sum of a and one")) == d
    assert _digest(tmp_path, SRC.replace("/* two\n lines */", "")) == d
    assert _digest(tmp_path, SRC.replace("  return", "\n\n      return")) == d


def test_code_edits_change_the_digest(tmp_path):
    d = _digest(tmp_path, SRC)
    assert _digest(tmp_path, SRC.replace("a + 1", "a + 2")) != d
    assert _digest(tmp_path, SRC.replace('"x // y"', '"x // z"')) != d    # inside a string literal
    assert _digest(tmp_path, SRC.replace("return a", "returna")) != d     # whitespace that separates tokens


def test_every_traffic_entry_names_existing_sources():
    csrc = os.path.join(os.path.dirname(bench.__file__), "weight_only_bit_w4_amd", "csrc")
    for name, (sources, digest, nbytes) in bench.TRAFFIC.items():
        assert all(os.path.isfile(os.path.join(csrc, s)) for s in sources), name
        assert len(digest) == 16 and nbytes > 0, name

"""Host-side tests of bench.py's bookkeeping (no GPU): the digest that ties a counter
summary under profiles/ to the kernel sources it was taken on (code only, so that an
edited comment does not void the summary, while any code change does)."""
import bench


def _digest_of(tmp_path, text):
    p = tmp_path / "k.hip"
    p.write_text(text)
    return bench.source_digest([str(p)])


def test_digest_ignores_comments_and_whitespace(tmp_path):
    code = "__global__ void k(int *p) {\n    p[0] = 1;  // store\n}\n"
    base = _digest_of(tmp_path, code)
    assert _digest_of(tmp_path, "// a header comment\n" + code) == base
    assert _digest_of(tmp_path, code.replace("// store", "// the only store")) == base
    assert _digest_of(tmp_path, code.replace("    p[0]", "p[0]")) == base
    assert _digest_of(tmp_path, "/* block\n comment */" + code) == base


def test_digest_follows_code(tmp_path):
    code = "__global__ void k(int *p) {\n    p[0] = 1;\n}\n"
    base = _digest_of(tmp_path, code)
    assert _digest_of(tmp_path, code.replace("p[0] = 1", "p[0] = 2")) != base
    assert _digest_of(tmp_path, code.replace("p[0]", "p[1]")) != base

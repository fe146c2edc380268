"""bench.py's kernel-source digest: it decides whether the committed rocprofv3
counter summary still describes the kernels, so a comment edit must keep it and
any change of code must change it."""
from __future__ import annotations

import bench


def _digest(tmp_path, text):
    p = tmp_path / "k.hip"
    p.write_text(text)
    return bench.source_digest([str(p)])


def test_comments_and_whitespace_do_not_count(tmp_path):
    base = 'int f(int x) {\n    return x + 1;   // one more\n}\n'
    assert _digest(tmp_path, base) == _digest(tmp_path, 'int f(int x) {\n  return x + 1; // a different note\n}\n')
    assert _digest(tmp_path, base) == _digest(tmp_path, '/* header\n   comment */ int f(int x) { return x + 1; }')


def test_code_changes_count(tmp_path):
    base = 'int f(int x) { return x + 1; }'
    assert _digest(tmp_path, base) != _digest(tmp_path, 'int f(int x) { return x + 2; }')
    assert _digest(tmp_path, base) != _digest(tmp_path, 'int f(int x) { return x - 1; }')


def test_string_literals_are_code(tmp_path):
    a = 'const char *s = "a // b"; int y;'
    b = 'const char *s = "a // c"; int y;'
    assert _digest(tmp_path, a) != _digest(tmp_path, b)
    assert bench._code_only(a) == a

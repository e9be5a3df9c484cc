"""The kernel-source digest that ties a stored counter summary (profiles/) to
a build: comments and layout do not change it, code does."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# build.py by path: importing the package would load the library
_spec = importlib.util.spec_from_file_location("_mbg_build", os.path.join(ROOT, "memory_bound_gemv_amd", "build.py"))
_build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(_build)
_code_tokens = _build._code_tokens


def test_comments_and_layout_are_ignored():
    a = "int a = 1; // note\n/* block\n comment */ int   b = a *  2;\n"
    b = "int a = 1;\nint b = a * 2;\n"
    assert _code_tokens(a) == _code_tokens(b)
    assert _code_tokens("x /* c */ y") == _code_tokens("x y")
    assert _code_tokens("x/**/y") == _code_tokens("x y")   # a comment still separates tokens


def test_literals_are_kept():
    s = 'const char* f = "a // not a comment /* nor this */";'
    assert "// not a comment /* nor this */" in _code_tokens(s)
    assert _code_tokens("c = '\\'';  // q") == _code_tokens("c = '\\'';")
    assert _code_tokens('s = "a  b";') != _code_tokens('s = "a b";')   # spaces inside a literal count


def test_code_changes_are_seen():
    assert _code_tokens("int a = 1;") != _code_tokens("int a = 2;")
    assert _code_tokens("ab") != _code_tokens("a b")
    # a preprocessor line ends at its newline
    assert _code_tokens("#define X 1\nint y;") != _code_tokens("#define X 1 int y;")

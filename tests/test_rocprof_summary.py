"""The source hash that ties committed rocprofv3 counters to a kernel's code: comments and
whitespace runs do not count, code does."""

from chunk_windowed_softmax_amd.rocprof_summary import SOURCES, _code_only, kernel_source_sha256


def test_comments_and_whitespace_do_not_count():
    a = "int f(int x) {\n  return x + 1;  // add one\n}\n"
    b = "// header\nint f(int x) { /* body */\n\n  return x + 1;\n}"
    assert _code_only(a) == _code_only(b) == "int f(int x) { return x + 1; }"


def test_code_changes_count():
    assert _code_only("return x + 1;") != _code_only("return x + 2;")
    assert _code_only("a /* c */ b") == "a b"  # a block comment still separates tokens
    assert _code_only("a//x\nb") == "a b"


def test_every_profiled_kernel_hashes():
    hashes = {k: kernel_source_sha256(k) for k in SOURCES}
    assert all(len(h) == 64 for h in hashes.values())
    assert len(set(hashes.values())) == len(hashes)
    assert kernel_source_sha256("attn_kernel") == hashes["attn_kernel"]  # stable

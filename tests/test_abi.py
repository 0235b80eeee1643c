"""The C ABI library loads without a GPU and exports what the header
declares; host-side validation paths (no device work) behave as documented."""
import ctypes
import os

import pytest

from sparse_mla_decode_indexer_amd import binding as B


def _lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail(f"{B.LIB_PATH} not built (run python -m sparse_mla_decode_indexer_amd.build)")
    return B.lib()


def test_exports_every_declared_function():
    L = _lib()
    names = B.header_functions()
    assert len(names) == 19
    for n in names:
        assert hasattr(L, n), n
    assert set(B._SIGS) == set(names)


def desc(**kw):
    d = dict(page_size=64, num_pool_pages=128, max_requests=2, max_context=8192, nope_dim=512,
             rope_dim=64, kv_dtype=B.HS_BF16, top_k=2048, hot_rows=0, max_batch=2, max_q_rows=128,
             select_q=0, host_rows=16384)
    d.update(kw)
    return B.HsPoolDesc(**d)


def test_requirements_sizes():
    _lib()
    s = B.pool_requirements(desc())
    assert s.row_bytes == 1152 and s.hot_rows == 4096 and s.pages_per_request == 128
    assert s.pool_bytes == 128 * 64 * 1152 and s.pool_scale_bytes == 0
    assert s.host_store_bytes == 16384 * 1152 and s.host_row_stride == 1152
    f8 = B.pool_requirements(desc(kv_dtype=B.HS_FP8_E4M3))
    assert f8.row_bytes == 576 and f8.pool_scale_bytes == 4 * 128 * 64
    # an fp8 host row carries its scale: 576 code bytes + 4 + 60 unused, so
    # that rows start on 128-byte boundaries
    assert f8.host_row_stride == 640 and f8.host_store_bytes == 16384 * 640
    assert B.pool_requirements(desc(kv_dtype=B.HS_F32)).row_bytes == 2304


def test_requirements_at_the_limits():
    _lib()
    s = B.pool_requirements(desc(max_context=4194304, top_k=4096, hot_rows=8192, select_q=8,
                                 kv_dtype=B.HS_FP8_E4M3))
    assert s.pages_per_request == 65536 and s.hot_rows == 8192


@pytest.mark.parametrize("kw,status", [
    (dict(hot_rows=1024), 2),          # S < K
    (dict(hot_rows=4100), 1),          # not a page multiple
    (dict(page_size=48), 1),           # not a power of two
    (dict(nope_dim=256), 3),
    (dict(kv_dtype=7), 3),
    (dict(top_k=0), 1),
    (dict(max_batch=3), 1),
    (dict(select_q=9), 1),
    (dict(select_q=-1), 1),
    (dict(top_k=4097, hot_rows=8192), 1),            # K above the largest top-K
    (dict(hot_rows=8256), 2),                       # above the largest hot buffer
    (dict(max_context=4194305), 2),                 # more than 2,048 filter chunks
    (dict(num_pool_pages=1 << 25, page_size=64), 2),  # more than 2^31 - 1 pool rows
])
def test_requirements_rejects(kw, status):
    _lib()
    with pytest.raises(B.HiSparseError) as e:
        B.pool_requirements(desc(**kw))
    assert e.value.status == status


def test_null_handles_rejected_without_device_work():
    L = _lib()
    assert L.hs_select_topk(None, None, 0, None, 1, None, None) == 1
    assert L.hs_resolve_rows(None, None, None, 1, None, None, None) == 1
    assert L.hs_sparse_mla_decode(None, None, 1, 1, 1, 1, None, 0.1, None, None, None) == 1
    assert L.hs_set_residency(None, 0, 0, 0, 0, 0, None, None, 0, None) == 1
    assert L.hs_update_residency(None, None, 1, None, 0, 0, None, None, None) == 1
    assert L.hs_indexer_scores(None, None, None, None, 0, 64, None, 1, None, 0, None) == 1
    assert L.hs_destroy_pool(None) == 0
    assert B.status_string(2) == "exceeds pool capacity"


def test_missing_library_raises_instead_of_falling_back(monkeypatch, tmp_path):
    # no CPU fallback: without the built library every entry point fails loudly
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "libhisparse.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()
    with pytest.raises(RuntimeError, match="missing"):
        B.pool_requirements(desc())


def _declared_params(header=B.HEADER, prefix="hs_"):
    """{function: [C parameter declarations]} parsed from a header."""
    import re
    text = open(header).read()
    out = {}
    for m in re.finditer(r"^(?:hs_status|int32_t|const char\*)\s+(" + prefix + r"\w+)\(([^)]*)\);", text, re.M):
        params = [p.strip() for p in " ".join(m.group(2).split()).split(",")]
        out[m.group(1)] = [] if params == ["void"] else params
    return out


def _ctype_for(decl: str):
    """The ctypes type a C parameter declaration must be marshalled as."""
    if "*" in decl or "[" in decl or decl.startswith("hipStream_t"):
        return "pointer"
    base = decl.rsplit(" ", 1)[0].replace("const ", "")
    return {"int32_t": ctypes.c_int32, "int64_t": ctypes.c_int64, "uint32_t": ctypes.c_uint32,
            "size_t": ctypes.c_size_t, "float": ctypes.c_float, "hs_status": ctypes.c_int32}[base]


def _probe_lib():
    from sparse_mla_decode_indexer_amd import probe as P
    if not os.path.exists(P.LIB_PATH):
        pytest.fail(f"{P.LIB_PATH} not built (run python -m sparse_mla_decode_indexer_amd.build)")
    return P


@pytest.mark.parametrize("which", ["hisparse", "hsprobe"])
def test_every_entry_point_has_matching_argtypes(which):
    """ctypes passes an undeclared argument as a C int, which truncates a
    64-bit pointer: every declared function is bound with argtypes whose
    count and kinds match the header's parameter list."""
    if which == "hisparse":
        L = _lib()
        decls = _declared_params()
        assert set(decls) == set(B.header_functions())
    else:
        P = _probe_lib()
        L = P.lib()
        decls = _declared_params(P.HEADER, "hsp_")
        assert set(decls) == set(P.header_functions()) == set(P._SIGS)
        assert len(decls) == 7
    for name, params in decls.items():
        f = getattr(L, name)
        assert f.argtypes is not None, name
        assert len(f.argtypes) == len(params), (name, f.argtypes, params)
        for decl, ct in zip(params, f.argtypes):
            want = _ctype_for(decl)
            if want == "pointer":
                assert ct is ctypes.c_void_p or hasattr(ct, "contents") or issubclass(ct, ctypes.Array), \
                    (name, decl, ct)
            else:
                assert ct is want, (name, decl, ct)

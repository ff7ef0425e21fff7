"""CPU checks of the C ABI: the library loads, exports every declared entry point, and rejects
bad arguments before touching a device (no GPU is needed for any of this)."""

import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(dsa_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_12_amd as pkg
    if not os.path.exists(pkg.LIB_PATH):
        from sparse_attention_12_amd import build
        build.build()
    return pkg.lib()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ["dsa_prepare_thd_metadata", "dsa_indexer_topk", "dsa_sparse_mla_fwd",
                     "dsa_sparse_mla_bwd", "dsa_last_error", "dsa_device_supported",
                     "dsa_thd_metadata_workspace_size", "dsa_indexer_topk_workspace_size",
                     "dsa_sparse_mla_bwd_workspace_size"]:
        assert required in names


def test_library_exports_every_declared_symbol(dsa):
    for name in _declared_functions():
        assert hasattr(dsa, name), f"libdsa.so does not export {name}"


def test_workspace_queries(dsa):
    assert dsa.dsa_thd_metadata_workspace_size(32768) >= 5 * 32768 * 4
    assert dsa.dsa_thd_metadata_workspace_size(-1) == 0
    one_pass = dsa.dsa_sparse_mla_bwd_workspace_size(1000, 1000, 64, 576, 2048, 0)
    assert one_pass >= 1000 * 64 * 4 + 1000 * 2048 * (576 * 2 + 16 + 4)
    one_row = dsa.dsa_sparse_mla_bwd_workspace_size(1000, 1000, 64, 576, 2048, 1)
    # passes of one row: two buffers, each staged contribution rows (576 16-bit mantissas and
    # 16 exponent bytes) + pair list + the counting-sort arrays of the 1000 latent rows
    per_buf = 2048 * (576 * 2 + 16 + 4) + 1001 * 4 + 1000 * 4
    assert 2 * per_buf <= one_row - 1000 * 64 * 4 < 2 * per_buf + 12 * 256 + 512
    assert dsa.dsa_sparse_mla_bwd_workspace_size(1000, 1000, 64, 576, 2048, 5000) == one_pass
    assert dsa.dsa_sparse_mla_bwd_workspace_size(1000, 1000, 64, 576, 0, 0) == 0
    assert dsa.dsa_indexer_topk_workspace_size(1000, 64, 128, 2048) == 0


def _err(dsa):
    return dsa.dsa_last_error().decode()


def test_argument_errors_without_device(dsa):
    import sparse_attention_12_amd as pkg
    md = pkg._Metadata()
    # metadata: bad B / K / missing workspace
    assert dsa.dsa_prepare_thd_metadata(None, 0, 10, 16, None, 0, C.byref(md), None) == \
        pkg.DSA_ERR_INVALID_VALUE
    assert "B=0" in _err(dsa)
    assert dsa.dsa_prepare_thd_metadata(C.c_void_p(16), 1, 10, 4096, None, 0, C.byref(md),
                                        None) == pkg.DSA_ERR_INVALID_VALUE
    assert dsa.dsa_prepare_thd_metadata(C.c_void_p(16), 1, 10, 16, None, 0, C.byref(md),
                                        None) == pkg.DSA_ERR_WORKSPACE
    # indexer: K above the fixed maximum, unsupported head dim, too many heads
    md.T = 8
    md.seq_start = 16
    md.groups = 16
    assert dsa.dsa_indexer_topk(16, 16, 16, C.byref(md), 64, 128, 2049, 16, 16, None, 0,
                                None) == pkg.DSA_ERR_INVALID_VALUE
    assert dsa.dsa_indexer_topk(16, 16, 16, C.byref(md), 64, 96, 16, 16, 16, None, 0,
                                None) == pkg.DSA_ERR_INVALID_VALUE
    assert dsa.dsa_indexer_topk(16, 16, 16, C.byref(md), 65, 128, 16, 16, 16, None, 0,
                                None) == pkg.DSA_ERR_INVALID_VALUE
    # key positions are 32-bit in the kernel: T is limited to INT32_MAX - 4096
    md.T = (1 << 31) - 1 - 4095
    assert dsa.dsa_indexer_topk(16, 16, 16, C.byref(md), 64, 128, 16, 16, 16, None, 0,
                                None) == pkg.DSA_ERR_INVALID_VALUE and "exceeds" in _err(dsa)
    md.T = 8
    # forward: width, value width, heads, K, scale, alignment
    args = dict(q=16, kv=16, idx=16, tl=None, Tq=4, Tkv=4, H=16, Dqk=576, Dv=512, K=8, sc=0.1,
                out=16, lse=16, s=None)

    def fwd(**kw):
        a = {**args, **kw}
        return dsa.dsa_sparse_mla_fwd(a["q"], a["kv"], a["idx"], a["tl"], a["Tq"], a["Tkv"],
                                      a["H"], a["Dqk"], a["Dv"], a["K"], a["sc"], a["out"],
                                      a["lse"], a["s"])
    assert fwd(Dqk=640) == pkg.DSA_ERR_INVALID_VALUE and "D_qk" in _err(dsa)
    assert fwd(Dv=256) == pkg.DSA_ERR_INVALID_VALUE
    assert fwd(H=0) == pkg.DSA_ERR_INVALID_VALUE
    assert fwd(H=65) == pkg.DSA_ERR_INVALID_VALUE
    assert fwd(K=4097) == pkg.DSA_ERR_INVALID_VALUE
    assert fwd(Tkv=(1 << 32) // 1152 + 1) == pkg.DSA_ERR_INVALID_VALUE and "4 GiB" in _err(dsa)
    assert fwd(K=0) == pkg.DSA_ERR_INVALID_VALUE
    assert fwd(sc=-1.0) == pkg.DSA_ERR_INVALID_VALUE
    assert fwd(sc=float("nan")) == pkg.DSA_ERR_INVALID_VALUE
    assert fwd(q=24) == pkg.DSA_ERR_INVALID_VALUE and "aligned" in _err(dsa)
    assert fwd(out=None) == pkg.DSA_ERR_INVALID_VALUE
    # backward: unknown flag, missing workspace, too many heads, K
    def bwd(flags=0, ws=16, ws_bytes=1 << 30, H=64, K=8):
        return dsa.dsa_sparse_mla_bwd(16, 16, 16, None, 16, 16, 16, 4, 4, H, 576, 512, K, 0.1,
                                      16, 16, flags, ws, ws_bytes, None)
    assert bwd(flags=0x8) == pkg.DSA_ERR_INVALID_VALUE
    assert bwd(ws=None) == pkg.DSA_ERR_WORKSPACE
    assert bwd(ws_bytes=4) == pkg.DSA_ERR_WORKSPACE
    assert bwd(H=65) == pkg.DSA_ERR_INVALID_VALUE
    assert bwd(K=4097) == pkg.DSA_ERR_INVALID_VALUE and "4096" in _err(dsa)


def test_local_metadata_argument_errors(dsa):
    import sparse_attention_12_amd as pkg
    md = pkg._Metadata()
    assert dsa.dsa_prepare_local_metadata(16, None, 16, None, 0, 8, 8, 16, None, 0, C.byref(md),
                                          None) == pkg.DSA_ERR_INVALID_VALUE
    assert "B=0" in _err(dsa)
    assert dsa.dsa_prepare_local_metadata(16, None, 16, None, 1, 8, 8, 2049, None, 0,
                                          C.byref(md), None) == pkg.DSA_ERR_INVALID_VALUE
    assert dsa.dsa_prepare_local_metadata(16, None, 16, None, 1, 8, 8, 16, None, 0, C.byref(md),
                                          None) == pkg.DSA_ERR_WORKSPACE
    assert dsa.dsa_local_metadata_workspace_size(8) >= 7 * 32


def test_sink_entry_points_reject_missing_sink(dsa):
    import sparse_attention_12_amd as pkg
    assert dsa.dsa_sparse_mla_fwd_sink(16, 16, 16, None, 4, 4, 16, 576, 512, 8, 0.1, None, 16,
                                       16, None) == pkg.DSA_ERR_INVALID_VALUE
    assert "sink" in _err(dsa)
    assert dsa.dsa_sparse_mla_bwd_sink(16, 16, 16, None, 16, 16, 16, 4, 4, 16, 576, 512, 8, 0.1,
                                       16, 16, 16, None, 0, None, 0, None) == \
        pkg.DSA_ERR_INVALID_VALUE
    assert "dsink" in _err(dsa)


def test_gather_probe_groups_and_argument_errors(dsa):
    assert [dsa.dsa_gather_probe_groups(n) for n in (-5, 0, 1, 2048, 2049, 4096)] == \
        [0, 0, 1, 1, 2, 2]
    fake = C.c_void_p(1 << 20)
    assert dsa.dsa_gather_probe(fake, 100, 500, fake, 10, fake, None) == 1
    assert "width" in _err(dsa)
    assert dsa.dsa_gather_probe(fake, 0, 576, fake, 10, fake, None) == 1
    assert "rows" in _err(dsa)
    assert dsa.dsa_gather_probe(fake, (4 << 30) // 1024, 512, fake, 10, fake, None) == 1
    assert "rows" in _err(dsa)
    assert dsa.dsa_gather_probe(fake, 100, 576, fake, -1, fake, None) == 1
    assert dsa.dsa_gather_probe(None, 100, 576, fake, 10, fake, None) == 1
    assert "NULL" in _err(dsa)
    assert dsa.dsa_gather_probe(C.c_void_p((1 << 20) + 8), 100, 576, fake, 10, fake, None) == 1
    assert "aligned" in _err(dsa)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import sparse_attention_12_amd as pkg
    monkeypatch.setattr(pkg, "_lib", None)
    monkeypatch.setattr(pkg, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not found"):
        pkg.lib()
    assert not pkg.is_available()


def test_noalloc_backward_rejects_sizes_beyond_its_scratch(dsa):
    """The allocation-free backward checks its sizes against the fixed scratch before it
    touches a device (the pointers below are never dereferenced)."""
    scratch = dsa.dsa_sparse_mla_bwd_noalloc_scratch_bytes()
    assert scratch == 256 << 20
    fake = C.c_void_p(1 << 20)
    T = (scratch // (64 * 4)) + 1  # Delta [T, 64] fp32 alone exceeds the scratch
    rc = dsa.dsa_sparse_mla_bwd_noalloc(fake, fake, fake, None, fake, fake, fake, T, T, 64, 576,
                                        512, 2048, C.c_float(0.04), fake, fake, 0, None)
    assert rc == 1  # DSA_ERR_INVALID_VALUE
    assert "scratch" in _err(dsa)

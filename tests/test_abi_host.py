"""Host-side checks of the C ABI (no GPU needed: no call here reaches a kernel).

The library must load and export every entry point include/gdn.h declares, and
every argument error checkable on the host must be reported before anything is
enqueued.  Pointers below are fake non-NULL addresses that are never dereferenced:
each call returns from host validation.
"""
import ctypes
import os
import re

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    import gated_deltanet_state_gdn_amd as gdn
    if not os.path.exists(gdn.LIB_PATH):
        pytest.skip("libgdn.so not built here")
    return gdn, gdn.load()


def test_header_declarations_are_exported():
    gdn, lib = _lib()
    hdr = open(os.path.join(ROOT, "include", "gdn.h")).read()
    declared = set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", hdr))
    assert declared == set(gdn._lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_status_and_replay_len():
    gdn, lib = _lib()
    assert gdn.gdn_abi_version() == 3
    for code in range(12):
        assert gdn.gdn_status_str(code) not in ("unknown status", "")
    for L in (0, 1, 7, 64, 100, 2048, 8192, 32768, 12345):
        for rho in (0.0, 0.01, 0.02, 0.05, 0.07, 0.1, 0.2, 0.5, 1.0, 1.5):
            assert gdn.gdn_replay_len(L, rho) == workloads.replay_len(L, rho), (L, rho)


def _desc(gdn, **kw):
    d = gdn._lib.GdnDesc()
    base = dict(n_seqs=1, h_qk=2, h_v=4, d_k=128, d_v=128, qkv_dtype=1, o_dtype=1, scale=1.0,
                total_tokens=100, total_out_tokens=10)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


P = ctypes.c_void_p(0x100000)      # 16-byte aligned fake address
PM = ctypes.c_void_p(0x100008)     # misaligned


def _replay(lib, d, q=P, o=None, ws=P, ws_bytes=256, r=P, cu=P, S=P):
    return lib.gdn_replay(ctypes.byref(d) if d is not None else None, q, P, P, P, P, cu, r, S, o,
                          None, ws, ws_bytes, None)


def test_host_validation_codes():
    gdn, lib = _lib()
    L = gdn._lib
    assert _replay(lib, None) == L.GDN_ERR_NULL
    assert _replay(lib, _desc(gdn, h_v=3)) == L.GDN_ERR_SHAPE
    assert _replay(lib, _desc(gdn, n_seqs=-1)) == L.GDN_ERR_SHAPE
    assert _replay(lib, _desc(gdn, total_out_tokens=101)) == L.GDN_ERR_SHAPE
    assert _replay(lib, _desc(gdn, d_k=96)) == L.GDN_ERR_UNSUPPORTED
    assert _replay(lib, _desc(gdn, d_v=256)) == L.GDN_ERR_UNSUPPORTED
    assert _replay(lib, _desc(gdn, d_k=32)) == L.GDN_ERR_UNSUPPORTED
    assert _replay(lib, _desc(gdn, qkv_dtype=7)) == L.GDN_ERR_DTYPE
    assert _replay(lib, _desc(gdn, qkv_dtype=0, o_dtype=1, d_k=64)) == L.GDN_ERR_DTYPE
    assert _replay(lib, _desc(gdn), q=PM) == L.GDN_ERR_ALIGN
    assert _replay(lib, _desc(gdn), o=PM) == L.GDN_ERR_ALIGN
    assert _replay(lib, _desc(gdn), ws_bytes=16) == L.GDN_ERR_WORKSPACE
    assert _replay(lib, _desc(gdn), ws=None) == L.GDN_ERR_NULL
    assert _replay(lib, _desc(gdn), r=None) == L.GDN_ERR_NULL
    assert _replay(lib, _desc(gdn), q=None) == L.GDN_ERR_NULL
    assert _replay(lib, _desc(gdn), cu=None) == L.GDN_ERR_NULL
    assert _replay(lib, _desc(gdn), S=None) == L.GDN_ERR_NULL
    # nothing to do: accepted without a launch
    assert _replay(lib, _desc(gdn, n_seqs=0)) == L.GDN_OK
    # prefill: one output row per token
    d = _desc(gdn)
    assert lib.gdn_prefill(ctypes.byref(d), P, P, P, P, P, P, None, P, None, P, 256, None) == L.GDN_ERR_SHAPE
    d = _desc(gdn, total_out_tokens=100, n_seqs=0)
    assert lib.gdn_prefill(ctypes.byref(d), P, P, P, P, P, P, None, P, None, P, 256, None) == L.GDN_OK


def test_relerr_and_status_validation():
    gdn, lib = _lib()
    L = gdn._lib
    assert lib.gdn_state_relerr(P, P, -1, 128, 128, P, None, None) == L.GDN_ERR_SHAPE
    assert lib.gdn_state_relerr(P, P, 0, 128, 128, P, None, None) == L.GDN_OK
    assert lib.gdn_state_relerr(None, P, 3, 128, 128, P, None, None) == L.GDN_ERR_NULL
    assert lib.gdn_state_relerr(PM, P, 3, 128, 128, P, None, None) == L.GDN_ERR_ALIGN
    out = ctypes.c_int32(0)
    assert lib.gdn_device_status(None, None, ctypes.byref(out)) == L.GDN_ERR_NULL
    assert lib.gdn_device_status(P, None, None) == L.GDN_ERR_NULL


def test_workspace_size():
    gdn, lib = _lib()
    assert gdn.gdn_workspace_bytes(_desc(gdn)) >= 256


def test_allocation_free_adaptive_rejects_oversized_requests():
    # n_seqs * h_v beyond the 65536 per-head slots of the static scratch is refused on the
    # host, before any device call
    gdn, lib = _lib()
    L = gdn._lib
    d = gdn._lib.GdnDesc()
    d.n_seqs, d.h_v, d.total_tokens = 2049, 32, 4096
    assert lib.gdn_adaptive_replay_len_static(ctypes.byref(d), P, P, 1e-3, 0, 100, P, None) == L.GDN_ERR_SCRATCH
    d.n_seqs, d.h_v = 1, 65537
    assert lib.gdn_adaptive_replay_len_static(ctypes.byref(d), P, P, 1e-3, 0, 100, P, None) == L.GDN_ERR_SCRATCH
    d.n_seqs, d.h_v = 2, 4
    assert lib.gdn_adaptive_replay_len_static(ctypes.byref(d), P, P, -1.0, 0, 100, P, None) == L.GDN_ERR_SHAPE
    assert lib.gdn_adaptive_replay_len_static(ctypes.byref(d), P, None, 1e-3, 0, 100, P, None) == L.GDN_ERR_NULL
    assert lib.gdn_adaptive_replay_len_static(ctypes.byref(d), PM, P, 1e-3, 0, 100, P, None) == L.GDN_ERR_ALIGN
    d.n_seqs = 0
    assert lib.gdn_adaptive_replay_len_static(ctypes.byref(d), P, P, 1e-3, 0, 100, P, None) == L.GDN_OK


def _seg(lib, d, n_segments=0, ws_bytes=1 << 40, o=None, r=P, cu=P, S=P, q=P, ws=P):
    return lib.gdn_replay_segmented(ctypes.byref(d) if d is not None else None, q, P, P, P, P, cu, r, S,
                                    o, None, n_segments, ws, ws_bytes, None)


def test_segmented_replay_host_validation():
    gdn, lib = _lib()
    L = gdn._lib
    assert _seg(lib, None) == L.GDN_ERR_NULL
    assert _seg(lib, _desc(gdn), n_segments=-1) == L.GDN_ERR_SHAPE
    assert _seg(lib, _desc(gdn), n_segments=65) == L.GDN_ERR_SHAPE
    assert _seg(lib, _desc(gdn, d_v=64)) == L.GDN_ERR_UNSUPPORTED        # square states only
    assert _seg(lib, _desc(gdn, h_v=3)) == L.GDN_ERR_SHAPE
    assert _seg(lib, _desc(gdn), r=None) == L.GDN_ERR_NULL
    assert _seg(lib, _desc(gdn), cu=None) == L.GDN_ERR_NULL
    assert _seg(lib, _desc(gdn), S=None) == L.GDN_ERR_NULL
    assert _seg(lib, _desc(gdn), ws=None) == L.GDN_ERR_NULL
    assert _seg(lib, _desc(gdn), q=PM) == L.GDN_ERR_ALIGN
    assert _seg(lib, _desc(gdn), o=PM) == L.GDN_ERR_ALIGN
    d = _desc(gdn)
    need = gdn.gdn_segmented_workspace_bytes(d, 8)
    assert _seg(lib, d, n_segments=8, ws_bytes=need - 1) == L.GDN_ERR_WORKSPACE
    assert _seg(lib, _desc(gdn, n_seqs=0), n_segments=8, ws_bytes=256) == L.GDN_OK


def test_segmented_workspace_bytes():
    gdn, lib = _lib()
    d = _desc(gdn, n_seqs=3, h_v=4, d_k=128, d_v=128)
    up = lambda b: (b + 255) // 256 * 256
    for P_ in (1, 5, 8):
        nv = 3 * P_
        st = nv * 4 * 128 * 128 * 4
        assert gdn.gdn_segmented_workspace_bytes(d, P_) == 256 + up(4 * (nv + 1)) + up(4 * nv) + 3 * st
    # 0 = the library's choice: clamp(min(128 / (n_seqs h_v), chunks / 6), 1, 16) segments,
    # chunks from the mean replay length total_out_tokens / n_seqs when it is given
    big = dict(total_tokens=200000)
    d0 = _desc(gdn, n_seqs=3, h_v=4, total_out_tokens=0, **big)
    assert gdn.gdn_segmented_workspace_bytes(d0, 0) == gdn.gdn_segmented_workspace_bytes(d0, 10)
    d1 = _desc(gdn, n_seqs=1, h_v=2, h_qk=2, total_out_tokens=0, **big)
    assert gdn.gdn_segmented_workspace_bytes(d1, 0) == gdn.gdn_segmented_workspace_bytes(d1, 16)
    d2 = _desc(gdn, n_seqs=1, h_v=16, h_qk=16, total_out_tokens=3277, **big)     # 52 chunks
    assert gdn.gdn_segmented_workspace_bytes(d2, 0) == gdn.gdn_segmented_workspace_bytes(d2, 8)
    d3 = _desc(gdn, n_seqs=1, h_v=16, h_qk=16, total_out_tokens=410, **big)      # 7 chunks
    assert gdn.gdn_segmented_workspace_bytes(d3, 0) == gdn.gdn_segmented_workspace_bytes(d3, 1)
    assert gdn.gdn_segmented_workspace_bytes(_desc(gdn, d_v=64), 4) == 0      # rejected descriptor
    assert gdn.gdn_segmented_workspace_bytes(d, 65) == 0


def test_missing_library_fails_loudly():
    # there is no fallback path: without the built library every call raises
    import subprocess
    import sys
    code = ("import gated_deltanet_state_gdn_amd as gdn\n"
            "try:\n"
            "    gdn.load()\n"
            "except ImportError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    raise SystemExit('loaded without a library')\n")
    env = dict(os.environ, GDN_LIB_PATH=os.path.join(ROOT, "no_such_dir", "libgdn.so"))
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0, out.stderr
    assert "raised:" in out.stdout and "not built" in out.stdout

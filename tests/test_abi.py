"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/lvtv.h declares, sizes its workspaces, and rejects
bad arguments with the documented codes before enqueueing anything."""

import ctypes
import os
import re

import pytest

import lossless_verify_tv_amd as lv
from lossless_verify_tv_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lvtv.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = "\n".join(l for l in text.splitlines() if not l.lstrip().startswith("#"))
    names = re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\([^;{]*\)\s*;", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_binding.LIB_PATH):
        from lossless_verify_tv_amd import build
        build.build()
    return lv.load_library()


def test_binding_constants_match_the_header():
    """The binding's objective and debug-path codes are the header's."""
    text = open(HEADER).read()
    defs = {k: int(v) for k, v in re.findall(r"#define\s+(LVTV_\w+)\s+\(?(-?\d+)\)?", text)}
    paths = {k[len("LVTV_PATH_"):].lower().replace("_", "-"): v
             for k, v in defs.items() if k.startswith("LVTV_PATH_")}
    assert paths == _binding.PATHS
    objs = {k[len("LVTV_OBJ_"):].lower(): v for k, v in defs.items() if k.startswith("LVTV_OBJ_")}
    assert objs == _binding.OBJECTIVES


def test_exports_every_declared_function(lib):
    declared = _declared_functions()
    assert set(declared) == set(lv.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_strerror(lib):
    assert lib.lvtv_version() >= 1
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        assert lv.strerror(code)
    assert "unknown" in lv.strerror(-99)


def test_workspace_queries(lib):
    assert lv.spec_verify_workspace_bytes(64, 7, 151936, lv.LVTV_BF16) > 0
    assert lv.spec_verify_workspace_bytes(1, 0, 1, lv.LVTV_F32) > 0
    assert lv.spec_verify_workspace_bytes(0, 7, 100) == 0
    assert lv.spec_verify_workspace_bytes(4, 17, 100) == 0
    assert lv.spec_verify_workspace_bytes(4, 4, 0) == 0
    assert lv.spec_verify_workspace_bytes(4, 4, 100, 7) == 0
    assert lv.e2e_tv_loss_workspace_bytes(512, 7, 151936) > 0
    assert lv.e2e_tv_loss_workspace_bytes(512, 17, 151936) == 0
    assert lv.e2e_tv_loss_workspace_bytes(0, 7, 100) == 0
    assert lv.draft_loss_workspace_bytes(512, 7, 151936) == lv.e2e_tv_loss_workspace_bytes(
        512, 7, 151936)
    assert lv.draft_loss_workspace_bytes(512, 17, 151936) == 0
    small = lv.spec_verify_workspace_bytes(8, 4, 1000)
    big = lv.spec_verify_workspace_bytes(8, 4, 100000)
    assert big > small


FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: every call below fails validation
NULL = ctypes.c_void_p(0)


def _verify(lib, **kw):
    args = dict(t=FAKE, d=FAKE, dtype=1, y=FAKE, k=FAKE, T=FAKE, seed=FAKE, B=4, K=3, V=100,
                acc=FAKE, tok=FAKE, alpha=FAKE, status=FAKE, ws=FAKE, ws_bytes=0, stream=NULL)
    args.update(kw)
    return lib.spec_verify(*args.values())


def test_spec_verify_host_errors(lib):
    need = lv.spec_verify_workspace_bytes(4, 3, 100, 1)
    assert _verify(lib, dtype=5, ws_bytes=need) == -3
    assert _verify(lib, B=0, ws_bytes=need) == -2
    assert _verify(lib, K=17, ws_bytes=need) == -2
    assert _verify(lib, V=0, ws_bytes=need) == -2
    assert _verify(lib, t=NULL, ws_bytes=need) == -1
    assert _verify(lib, d=NULL, ws_bytes=need) == -1
    assert _verify(lib, status=NULL, ws_bytes=need) == -1
    assert _verify(lib, ws_bytes=need - 1) == -4
    assert _verify(lib, ws=NULL, ws_bytes=need) == -4
    assert _verify(lib, ws=ctypes.c_void_p(0x1010), ws_bytes=need) == -4   # misaligned
    # Kmax = 0: draft pointers may be NULL, the workspace check still applies
    assert _verify(lib, K=0, d=NULL, y=NULL, alpha=NULL, ws_bytes=0) == -4


def test_loss_host_errors(lib):
    need = lv.e2e_tv_loss_workspace_bytes(4, 3, 100)
    call = lambda **kw: lib.e2e_tv_loss_fwd_bwd(*{**dict(
        z=FAKE, p=FAKE, N=4, W=3, V=100, loss=FAKE, alpha=FAKE, dz=FAKE, ws=FAKE,
        wsb=need, stream=NULL), **kw}.values())
    assert call(N=0) == -2
    assert call(W=17) == -2
    assert call(V=-5) == -2
    assert call(z=NULL) == -1
    assert call(dz=NULL) == -1
    assert call(wsb=need - 1) == -4


def test_draft_loss_host_errors(lib):
    need = lv.draft_loss_workspace_bytes(4, 3, 100)
    call = lambda **kw: lib.draft_loss_fwd_bwd(*{**dict(
        z=FAKE, p=FAKE, N=4, W=3, V=100, obj=2, loss=FAKE, alpha=FAKE, dz=FAKE, ws=FAKE,
        wsb=need, stream=NULL), **kw}.values())
    assert call(obj=4) == -6
    assert call(obj=-1) == -6
    assert call(N=0) == -2
    assert call(z=NULL) == -1
    assert call(wsb=need - 1) == -4


def test_draft_loss_logits_host_errors(lib):
    need = lv.draft_loss_logits_workspace_bytes(4, 3, 100)
    assert need == lv.draft_loss_workspace_bytes(4, 3, 100)
    call = lambda **kw: lib.draft_loss_logits_fwd_bwd(*{**dict(
        z=FAKE, t=FAKE, T=0.7, N=4, W=3, V=100, obj=0, loss=FAKE, alpha=FAKE, dz=FAKE,
        ws=FAKE, wsb=need, stream=NULL), **kw}.values())
    for bad in (0.0, -1.0, float("nan"), float("inf"), 1e-39):
        assert call(T=bad) == -7
    assert call(obj=4) == -6
    assert call(N=0) == -2
    assert call(W=17) == -2
    assert call(z=NULL) == -1
    assert call(t=NULL) == -1
    assert call(dz=NULL) == -1
    assert call(wsb=need - 1) == -4
    assert call(ws=ctypes.c_void_p(0x1010)) == -4


def test_debug_loss_host_errors(lib):
    need = lv.draft_loss_workspace_bytes(4, 3, 100)
    call = lambda **kw: lib.lvtv_debug_draft_loss(*{**dict(
        z=FAKE, p=FAKE, t=NULL, T=1.0, N=4, W=3, V=100, obj=0, path=0, spin=0, loss=FAKE,
        alpha=FAKE, dz=FAKE, dz32=NULL, ws=FAKE, wsb=need, stream=NULL), **kw}.values())
    assert call(path=1) == -8
    assert call(path=4) == -8
    assert call(path=7) == -8
    assert call(p=NULL) == -1              # neither target
    assert call(t=FAKE) == -1              # both targets
    assert call(p=NULL, t=FAKE, T=0.0) == -7
    assert call(obj=9) == -6
    assert call(N=0) == -2
    assert call(N=65536) == -2
    assert call(wsb=need - 1) == -4


def test_size_limits(lib):
    # B and N are limited to LVTV_MAX_B / LVTV_MAX_N = 65535
    assert lv.spec_verify_workspace_bytes(65535, 1, 8, 1) > 0
    assert lv.spec_verify_workspace_bytes(65536, 1, 8, 1) == 0
    assert lv.spec_verify_packed_workspace_bytes(65536, 65536, 8, 1) == 0
    assert lv.e2e_tv_loss_workspace_bytes(65535, 1, 8) > 0
    assert lv.e2e_tv_loss_workspace_bytes(65536, 1, 8) == 0


def test_packed_verify_host_errors(lib):
    need = lv.spec_verify_packed_workspace_bytes(4, 10, 100)
    assert need > 0
    assert lv.spec_verify_packed_workspace_bytes(4, 3, 100) == 0        # fewer rows than requests
    assert lv.spec_verify_packed_workspace_bytes(4, 4 * 17 + 1, 100) == 0
    call = lambda **kw: lib.spec_verify_packed(*{**dict(
        t=FAKE, d=FAKE, dtype=1, y=FAKE, off=FAKE, T=FAKE, seed=FAKE, B=4, rows=10, V=100,
        acc=FAKE, tok=FAKE, alpha=FAKE, status=FAKE, ws=FAKE, wsb=need, stream=NULL),
        **kw}.values())
    assert call(dtype=2) == -3
    assert call(rows=3) == -2
    assert call(off=NULL) == -1
    assert call(d=NULL) == -1
    assert call(rows=4, d=NULL, y=NULL, alpha=NULL, wsb=0) == -4   # K_b = 0 for all: drafts optional
    assert call(wsb=need - 1) == -4


def test_topkp_verify_host_errors(lib):
    need = lv.spec_verify_topkp_workspace_bytes(4, 3, 100, 1)
    assert need > lv.spec_verify_workspace_bytes(4, 3, 100, 1)    # the keep records
    assert lv.spec_verify_topkp_workspace_bytes(4, 17, 100, 1) == 0
    call = lambda **kw: lib.spec_verify_topkp(*{**dict(
        t=FAKE, d=FAKE, dtype=1, y=FAKE, k=FAKE, T=FAKE, seed=FAKE, tk=FAKE, tp=FAKE, B=4, K=3,
        V=100, acc=FAKE, tok=FAKE, alpha=FAKE, status=FAKE, ws=FAKE, wsb=need, stream=NULL),
        **kw}.values())
    assert call(tk=NULL) == -1
    assert call(tp=NULL) == -1
    assert call(dtype=2) == -3
    assert call(K=17) == -2
    assert call(wsb=need - 1) == -4
    # the plain verify's workspace is too small for the truncating one
    assert call(wsb=lv.spec_verify_workspace_bytes(4, 3, 100, 1)) == -4


def test_schedule_host_errors(lib):
    call = lambda **kw: lib.dspark_schedule(*{**dict(
        c=FAKE, sps=FAKE, R=4, L=3, lens=FAKE, best=FAKE, stream=NULL), **kw}.values())
    assert call(R=0) == -2
    assert call(L=0) == -2
    assert call(R=8193, L=1) == -2
    assert call(R=1024, L=9) == -2
    assert call(c=NULL) == -1
    assert call(best=NULL) == -1


def test_binding_rejects_cpu_tensors():
    import torch
    t = torch.zeros(2, 3, 10)
    with pytest.raises(ValueError):
        lv.spec_verify(t, t[:, :2], torch.zeros(2, 2, dtype=torch.int32),
                       torch.zeros(2, dtype=torch.int32), torch.ones(2),
                       torch.zeros(2, dtype=torch.int64))
    with pytest.raises(ValueError):
        lv.e2e_tv_loss_fwd_bwd(t.to(torch.bfloat16), t)
    with pytest.raises(ValueError):
        lv.draft_loss_fwd_bwd(t.to(torch.bfloat16), t, "ce")

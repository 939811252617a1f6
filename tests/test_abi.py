"""C-ABI conventions that can be checked without a GPU: the library loads, exports every
function declared in include/sss.h, and rejects bad arguments before touching a device."""
import ctypes
import os
import re
import subprocess

import pytest

import selective_state_space_20_amd as sss
from selective_state_space_20_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sss.h")

NULL_ARG, BAD_DIM, UNSUPPORTED, WORKSPACE, ALIAS, HIP = -1, -2, -3, -4, -5, -6


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = sss.load()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, flags=re.M), f"{n} not exported by libsss.so"


def test_library_is_built_for_gfx950_only():
    """The offload bundle of libsss.so names exactly one device target: gfx950."""
    blob = open(_lib.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx\w+)", blob))
    assert targets == {b"gfx950"}, targets


def test_status_strings():
    for code in (0, NULL_ARG, BAD_DIM, UNSUPPORTED, WORKSPACE, ALIAS, HIP):
        assert sss.status_string(code)
    assert "unknown" in sss.status_string(17)


P = 1 << 20  # a fake, 16-byte aligned address; never dereferenced: every call below is rejected first


def sel(**kw):
    a = dict(x=P, delta=2 * P, A=3 * P, B=4 * P, C=5 * P, D_skip=0, z=0, h0=0, y=64 * P, h_last=0, batch=2,
             seqlen=8, dim=4, dstate=4, io_dtype=0, workspace=0, workspace_bytes=0, stream=0)
    a.update(kw)
    return sss.selective_scan_fwd_raw(**a)


def ew(**kw):
    a = dict(x=P, A=2 * P, B=3 * P, C=4 * P, h0=0, y=64 * P, h_last=0, batch=2, seqlen=8, dim=4, workspace=0,
             workspace_bytes=0, stream=0)
    a.update(kw)
    return sss.elementwise_scan_raw(**a)


def selx(**kw):
    a = dict(x=P, delta=2 * P, A=3 * P, B=4 * P, C=5 * P, D_skip=0, z=0, h0=0, y=64 * P, h_last=0, delta_bias=0,
             flags=0, batch=2, seqlen=8, dim=4, dstate=4, io_dtype=0, workspace=0, workspace_bytes=0, stream=0)
    a.update(kw)
    return sss.selective_scan_fwd_ex_raw(**a)


def test_selective_ex_rejections():
    assert selx(x=0) == NULL_ARG
    assert selx(flags=8) == UNSUPPORTED                 # unknown option bit
    assert selx(flags=1 << 31) == UNSUPPORTED
    assert selx(flags=4, seqlen=1 << 23) == BAD_DIM     # channel-major rows past 32-bit offsets
    assert selx(delta_bias=6 * P + 4) == UNSUPPORTED    # misaligned bias
    assert selx(y=6 * P, delta_bias=6 * P) == ALIAS     # y over the bias
    assert selx(dim=0, flags=3) == BAD_DIM


def bwd(**kw):
    a = dict(x=P, delta=2 * P, A=3 * P, B=4 * P, C=5 * P, D_skip=0, z=0, h0=0, dy=6 * P, dh_last=0, dx=64 * P,
             ddelta=65 * P, dA=66 * P, dB=67 * P, dC=68 * P, dD=0, dz=0, dh0=0, batch=2, seqlen=8, dim=4, dstate=4,
             io_dtype=0, workspace=80 * P, workspace_bytes=1 << 30, stream=0)
    a.update(kw)
    return sss.selective_scan_bwd_raw(**a)


def bwdx(**kw):
    a = dict(x=P, delta=2 * P, A=3 * P, B=4 * P, C=5 * P, D_skip=0, z=0, h0=0, dy=6 * P, dh_last=0, delta_bias=7 * P,
             flags=2, dx=64 * P, ddelta=65 * P, dA=66 * P, dB=67 * P, dC=68 * P, dD=0, dz=0, dh0=0,
             ddelta_bias=69 * P, batch=2, seqlen=8, dim=4, dstate=4, io_dtype=0, workspace=80 * P,
             workspace_bytes=1 << 30, stream=0)
    a.update(kw)
    return sss.selective_scan_bwd_ex_raw(**a)


def test_backward_ex_rejections():
    assert bwdx(ddelta_bias=0) == NULL_ARG             # a bias without its gradient
    assert bwdx(flags=1) == UNSUPPORTED                # the exact hold has no gradients call
    assert bwdx(flags=4) == UNSUPPORTED                # nor the channel-major layout
    assert bwdx(flags=1 << 31) == UNSUPPORTED
    assert bwdx(delta_bias=7 * P + 4) == UNSUPPORTED   # misaligned bias
    assert bwdx(ddelta_bias=7 * P) == ALIAS            # the bias gradient over the bias
    assert bwdx(ddelta_bias=65 * P + 16) == ALIAS      # the bias gradient over ddelta
    assert bwdx(dx=7 * P) == ALIAS                     # dx over the bias
    assert bwdx(dim=0) == BAD_DIM


def test_backward_rejections():
    assert bwd(dy=0) == NULL_ARG
    assert bwd(dC=0) == NULL_ARG
    assert bwd(D_skip=7 * P) == NULL_ARG          # D given without dD
    assert bwd(z=7 * P) == NULL_ARG               # z given without dz
    assert bwd(dstate=3) == UNSUPPORTED
    assert bwd(dx=P) == ALIAS                     # dx over x
    assert bwd(dB=65 * P + 16) == ALIAS           # dB over ddelta
    assert bwd(dx=6 * P) == ALIAS                 # dx over dy
    assert bwd(seqlen=0) == BAD_DIM
    assert sss.selective_scan_bwd_workspace_size(1, 1000, 64, 16) > sss.selective_scan_fwd_workspace_size(1, 1000, 64, 16)


def upd(**kw):
    a = dict(x=P, delta=2 * P, A=3 * P, B=4 * P, C=5 * P, D_skip=0, z=0, state=32 * P, y=64 * P, batch=2, dim=4,
             dstate=4, io_dtype=0, stream=0)
    a.update(kw)
    return sss.selective_state_update_raw(**a)


@pytest.mark.parametrize("name", ["x", "delta", "A", "B", "C", "state", "y"])
def test_update_null_required(name):
    assert upd(**{name: 0}) == NULL_ARG


@pytest.mark.parametrize("kw", [dict(batch=0), dict(dim=0), dict(dstate=-1), dict(dim=(1 << 24) + 1),
                                dict(batch=1 << 20, dim=1 << 12, dstate=1 << 6)])
def test_update_bad_dims(kw):
    assert upd(**kw) == BAD_DIM


@pytest.mark.parametrize("kw", [dict(dstate=3), dict(dstate=128), dict(io_dtype=5), dict(state=32 * P + 4),
                                dict(z=7 * P + 8)])
def test_update_unsupported(kw):
    assert upd(**kw) == UNSUPPORTED


def test_update_alias():
    assert upd(state=P) == ALIAS            # state over x
    assert upd(y=5 * P) == ALIAS            # y over C
    assert upd(y=32 * P + 16) == ALIAS      # y over state
    assert upd(state=3 * P + 16) == ALIAS   # state over A


@pytest.mark.parametrize("name", ["x", "delta", "A", "B", "C", "y"])
def test_selective_null_required(name):
    assert sel(**{name: 0}) == NULL_ARG


@pytest.mark.parametrize("name", ["x", "A", "B", "C", "y"])
def test_elementwise_null_required(name):
    assert ew(**{name: 0}) == NULL_ARG


@pytest.mark.parametrize("kw", [dict(batch=0), dict(seqlen=0), dict(dim=-1), dict(dstate=0),
                                dict(batch=1 << 40, seqlen=1 << 30), dict(dim=(1 << 24) + 1, seqlen=4)])
def test_selective_bad_dims(kw):
    assert sel(**kw) == BAD_DIM


@pytest.mark.parametrize("kw", [dict(dstate=65), dict(io_dtype=2), dict(io_dtype=-1), dict(x=P + 4),
                                dict(B=4 * P + 8), dict(y=64 * P + 2), dict(z=7 * P + 4)])
def test_selective_unsupported(kw):
    assert sel(**kw) == UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(batch=0), dict(seqlen=-3), dict(dim=0)])
def test_elementwise_bad_dims(kw):
    assert ew(**kw) == BAD_DIM


def test_alias_detected_before_any_device_work():
    # y overlapping x, h_last overlapping B, y overlapping h_last
    assert sel(y=P) == ALIAS
    assert sel(h_last=4 * P) == ALIAS
    assert sel(h_last=64 * P + 16) == ALIAS
    assert ew(y=3 * P) == ALIAS
    assert ew(h_last=2 * P) == ALIAS


def test_workspace_query_is_sane():
    assert sss.selective_scan_fwd_workspace_size(0, 8, 4, 4) == 0
    # the channel-major layout adds time-major copies of B and C; unknown flags give 0
    plain = sss.selective_scan_fwd_ex_workspace_size(2, 4096, 4096, 16, 0)
    assert plain == sss.selective_scan_fwd_workspace_size(2, 4096, 4096, 16)
    assert sss.selective_scan_fwd_ex_workspace_size(2, 4096, 4096, 16, 4) >= plain + 2 * 2 * 4096 * 16 * 4
    assert sss.selective_scan_fwd_ex_workspace_size(2, 4096, 4096, 16, 8) == 0
    assert sss.selective_scan_fwd_ex_workspace_size(2, 1 << 23, 64, 16, 4) == 0
    a = sss.selective_scan_fwd_workspace_size(1, 1000, 64, 16)
    b = sss.selective_scan_fwd_workspace_size(1, 100000, 64, 16)
    assert 0 < a <= b and a % 256 == 0 and b % 256 == 0
    assert sss.elementwise_scan_workspace_size(1, 8, 0) == 0
    assert sss.elementwise_scan_workspace_size(8, 32768, 4096) == 0  # enough channels: single pass


def test_no_device_reports_hip_error():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; this checks the no-device path")
    assert sel() == HIP
    assert selx(flags=3, delta_bias=6 * P) == HIP
    assert selx(flags=4, workspace=80 * P, workspace_bytes=1 << 20) == HIP
    assert ew() == HIP
    assert upd() == HIP
    assert bwd() == HIP

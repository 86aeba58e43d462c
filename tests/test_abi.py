"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments on the host before any HIP
call.  Every call below carries at least one invalid argument, so none of
them can reach a kernel launch (the pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

import selective_state_space_selscan_amd as ss


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# The validation tests pass fake device addresses.  They are meant for hosts
# without a GPU: if a check ever regressed, a launch on a GPU would read them.
no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer tests run only without a GPU")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "selscan.h")

(OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_UNSUP, ERR_WS, ERR_ALIAS, ERR_HIP, ERR_TIMEOUT,
 ERR_TOO_LARGE) = range(10)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(selscan_\w+)\s*\(", text)))


def header_constant(name):
    m = re.search(r"#define\s+%s\s+(\d+)" % name, open(HEADER).read())
    return int(m.group(1))


def test_library_exports_every_declared_symbol():
    L = ss.lib()
    names = header_functions()
    assert {"selscan_fwd", "selscan_fwd_ex", "selscan_bwd", "selscan_bwd_ex", "selscan_state_update",
            "selscan_fwd_workspace_bytes", "selscan_bwd_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(L, n), "missing export " + n
    assert L.selscan_abi_version() == header_constant("SELSCAN_ABI_VERSION")


def test_every_registered_kernel_name_has_device_code():
    """The host side of the library launches a kernel by its mangled name,
    which must name a kernel descriptor (``<name>.kd``) in the device code.
    A name that mentions an unnamed type (``$_<n>``, numbered per compilation
    pass) can differ between the two and the launch then aborts."""
    blob = open(ss._abi._LIB_PATH, "rb").read()
    names = set(m.decode() for m in re.findall(rb"_ZN7selscan[A-Za-z0-9_$.]*", blob))
    descriptors = {n[:-3] for n in names if n.endswith(".kd")}
    kernels = {n for n in names if "." not in n and "kernel" in n and "__device_stub__" not in n}
    assert descriptors, "no device code found in the library"
    assert not [n for n in names if "$_" in n]
    assert kernels <= descriptors, sorted(kernels - descriptors)[:3]


def test_status_strings_and_supported_n():
    L = ss.lib()
    for s in range(10):
        assert len(L.selscan_status_string(s)) > 0
        assert L.selscan_status_string(s) != b"unknown status"
    assert L.selscan_status_string(99) == b"unknown status"
    for n in (4, 8, 16, 32, 64):
        assert L.selscan_supports_n(n) == 1
    for n in (0, 1, 5, 12, 128):
        assert L.selscan_supports_n(n) == 0


# Fake, 16-byte-aligned, well-separated addresses; never dereferenced.
BASE = 0x7F0000000000
STEP = 1 << 36


def fake(i):
    return ctypes.c_void_p(BASE + i * STEP)


def fwd_args(**kw):
    a = dict(u=fake(1), delta=fake(2), A=fake(3), Bm=fake(4), Cm=fake(5), D_skip=fake(6),
             z=fake(7), delta_bias=fake(8), delta_softplus=1, h0=fake(9), y=fake(10),
             h_last=fake(11), batch=2, L=64, dim=128, N=16, dtype=1, workspace=fake(12),
             workspace_bytes=1 << 30, stream=None)
    a.update(kw)
    order = ["u", "delta", "A", "Bm", "Cm", "D_skip", "z", "delta_bias", "delta_softplus", "h0",
             "y", "h_last", "batch", "L", "dim", "N", "dtype", "workspace", "workspace_bytes",
             "stream"]
    return [a[k] for k in order]


INVALID_FWD = [
    ("dtype", dict(dtype=2), ERR_DTYPE),
    ("dtype_neg", dict(dtype=-1), ERR_DTYPE),
    ("batch0", dict(batch=0), ERR_SHAPE),
    ("L0", dict(L=0), ERR_SHAPE),
    ("dim0", dict(dim=0), ERR_SHAPE),
    ("N0", dict(N=0), ERR_SHAPE),
    ("overflow", dict(batch=1 << 40, L=1 << 20, dim=1 << 10), ERR_SHAPE),
    ("u_null", dict(u=None), ERR_NULL),
    ("delta_null", dict(delta=None), ERR_NULL),
    ("A_null", dict(A=None), ERR_NULL),
    ("B_null", dict(Bm=None), ERR_NULL),
    ("C_null", dict(Cm=None), ERR_NULL),
    ("y_null", dict(y=None), ERR_NULL),
    ("N5", dict(N=5), ERR_UNSUP),
    ("N128", dict(N=128), ERR_UNSUP),
    ("dim_too_large", dict(dim=(1 << 24) + 64, batch=1, L=2), ERR_UNSUP),
    # 2^24 channel groups x 4096 sequence parts: a launch grid past 2^31 - 1
    ("grid_too_large", dict(batch=1 << 20, L=1 << 16, dim=1 << 10), ERR_UNSUP),
    ("misaligned_u", dict(u=ctypes.c_void_p(BASE + STEP + 2)), ERR_UNSUP),
    ("misaligned_hlast", dict(h_last=ctypes.c_void_p(BASE + 11 * STEP + 8)), ERR_UNSUP),
    ("y_aliases_u", dict(y=ctypes.c_void_p(BASE + STEP + 64)), ERR_ALIAS),
    ("hlast_aliases_h0", dict(h_last=fake(9)), ERR_ALIAS),
    ("y_aliases_hlast", dict(h_last=ctypes.c_void_p(BASE + 10 * STEP + 1024)), ERR_ALIAS),
]


@no_gpu_only
@pytest.mark.parametrize("name,kw,status", INVALID_FWD, ids=[c[0] for c in INVALID_FWD])
def test_fwd_rejects_invalid_arguments(name, kw, status):
    L = ss.lib()
    assert L.selscan_fwd(*fwd_args(**kw)) == status
    assert L.selscan_last_hip_error() == 0


@no_gpu_only
def test_fwd_workspace_checked_when_needed():
    L = ss.lib()
    need = L.selscan_fwd_workspace_bytes(1, 131072, 2048, 16, 1)
    assert need > 0
    assert L.selscan_fwd_workspace_bytes(1, 131072, 2048, 16, 9) == 0   # invalid dtype
    assert L.selscan_fwd_workspace_bytes(1, 131072, 2048, 5, 1) == 0    # unsupported N
    for ws, nbytes in ((None, 0), (fake(12), need - 1)):
        args = fwd_args(batch=1, L=131072, dim=2048, workspace=ws, workspace_bytes=nbytes)
        assert L.selscan_fwd(*args) == ERR_WS
    # misaligned workspace
    args = fwd_args(batch=1, L=131072, dim=2048, workspace=ctypes.c_void_p(BASE + 12 * STEP + 8))
    assert L.selscan_fwd(*args) == ERR_UNSUP


def fwd_ex_args(flags=0, conv_w=None, conv_b=None, conv_width=0, **kw):
    a = fwd_args(**kw)
    # flags, conv_weight, conv_bias, conv_width go between dtype and workspace
    return a[:17] + [flags, conv_w, conv_b, conv_width] + a[17:]


INVALID_FWD_EX = [
    ("unknown_flag", dict(flags=4), ERR_UNSUP),
    ("unknown_flag_16", dict(flags=16), ERR_UNSUP),
    # the plain forward or reverse alone keeps the backward's checkpoints
    ("keep_with_zoh", dict(flags=8 | 1), ERR_UNSUP),
    ("keep_with_zoh_reverse", dict(flags=8 | 2 | 1), ERR_UNSUP),
    ("keep_with_conv", dict(flags=8, conv_width=4, conv_w=fake(13)), ERR_UNSUP),
    ("negative_flag", dict(flags=-1), ERR_UNSUP),
    ("conv_width_5", dict(conv_width=5, conv_w=fake(13)), ERR_UNSUP),
    ("conv_width_neg", dict(conv_width=-1, conv_w=fake(13)), ERR_SHAPE),
    ("conv_w_null", dict(conv_width=4, conv_w=None), ERR_NULL),
    ("conv_w_misaligned", dict(conv_width=4, conv_w=ctypes.c_void_p(BASE + 13 * STEP + 4)),
     ERR_UNSUP),
    ("conv_b_misaligned", dict(conv_width=4, conv_w=fake(13),
                               conv_b=ctypes.c_void_p(BASE + 14 * STEP + 8)), ERR_UNSUP),
    ("y_aliases_conv_w", dict(conv_width=4, conv_w=ctypes.c_void_p(BASE + 10 * STEP + 512)),
     ERR_ALIAS),
    ("hlast_aliases_conv_b", dict(conv_width=2, conv_w=fake(13),
                                  conv_b=ctypes.c_void_p(BASE + 11 * STEP + 256)), ERR_ALIAS),
    # the checks of selscan_fwd apply as well
    ("dtype", dict(dtype=2, flags=1), ERR_DTYPE),
    ("L0", dict(L=0, flags=2), ERR_SHAPE),
    ("N5", dict(N=5, flags=3), ERR_UNSUP),
    ("u_null", dict(u=None, conv_width=4, conv_w=fake(13)), ERR_NULL),
    ("y_aliases_u", dict(y=ctypes.c_void_p(BASE + STEP + 64), flags=2), ERR_ALIAS),
]


@no_gpu_only
@pytest.mark.parametrize("name,kw,status", INVALID_FWD_EX, ids=[c[0] for c in INVALID_FWD_EX])
def test_fwd_ex_rejects_invalid_arguments(name, kw, status):
    L = ss.lib()
    assert L.selscan_fwd_ex(*fwd_ex_args(**kw)) == status
    assert L.selscan_last_hip_error() == 0


@no_gpu_only
def test_fwd_ex_workspace_checked_when_needed():
    L = ss.lib()
    need = L.selscan_fwd_workspace_bytes(1, 131072, 2048, 16, 1)
    for ws, nbytes in ((None, 0), (fake(12), need - 1)):
        args = fwd_ex_args(flags=3, conv_width=4, conv_w=fake(13), batch=1, L=131072, dim=2048,
                           workspace=ws, workspace_bytes=nbytes)
        assert L.selscan_fwd_ex(*args) == ERR_WS


def bwd_args(**kw):
    a = dict(u=fake(1), delta=fake(2), A=fake(3), Bm=fake(4), Cm=fake(5), D_skip=fake(6),
             z=fake(7), delta_bias=fake(8), delta_softplus=1, h0=fake(9), dy=fake(10),
             dh_last=fake(11), du=fake(12), ddelta=fake(13), dA=fake(14), dB=fake(15),
             dC=fake(16), dD=fake(17), dz=fake(18), ddelta_bias=fake(19), dh0=fake(20),
             batch=2, L=64, dim=128, N=16, dtype=1, workspace=fake(21),
             workspace_bytes=1 << 34, stream=None)
    a.update(kw)
    order = ["u", "delta", "A", "Bm", "Cm", "D_skip", "z", "delta_bias", "delta_softplus", "h0",
             "dy", "dh_last", "du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias", "dh0",
             "batch", "L", "dim", "N", "dtype", "workspace", "workspace_bytes", "stream"]
    return [a[k] for k in order]


INVALID_BWD = [
    ("dtype", dict(dtype=5), ERR_DTYPE),
    ("L0", dict(L=0), ERR_SHAPE),
    ("N0", dict(N=0), ERR_SHAPE),
    ("overflow", dict(batch=1 << 40, L=1 << 20, dim=1 << 10), ERR_SHAPE),
    ("dy_null", dict(dy=None), ERR_NULL),
    ("du_null", dict(du=None), ERR_NULL),
    ("ddelta_null", dict(ddelta=None), ERR_NULL),
    ("dA_null", dict(dA=None), ERR_NULL),
    ("dB_null", dict(dB=None), ERR_NULL),
    ("dC_null", dict(dC=None), ERR_NULL),
    ("dz_null_with_z", dict(dz=None), ERR_NULL),
    ("N12", dict(N=12), ERR_UNSUP),
    ("dim_too_large", dict(dim=(1 << 24) + 64, batch=1, L=2), ERR_UNSUP),
    ("grid_too_large", dict(batch=1 << 20, L=1 << 16, dim=1 << 10), ERR_UNSUP),
    ("misaligned_dy", dict(dy=ctypes.c_void_p(BASE + 10 * STEP + 4)), ERR_UNSUP),
    ("misaligned_dh0", dict(dh0=ctypes.c_void_p(BASE + 20 * STEP + 8)), ERR_UNSUP),
    ("no_workspace", dict(workspace=None), ERR_WS),
    ("small_workspace", dict(workspace_bytes=1024), ERR_WS),
    ("du_aliases_u", dict(du=ctypes.c_void_p(BASE + STEP + 128)), ERR_ALIAS),
    ("dB_aliases_Bm", dict(dB=ctypes.c_void_p(BASE + 4 * STEP + 64)), ERR_ALIAS),
    ("dA_aliases_dD", dict(dD=ctypes.c_void_p(BASE + 14 * STEP + 256)), ERR_ALIAS),
    ("dh0_aliases_workspace", dict(dh0=ctypes.c_void_p(BASE + 21 * STEP + 4096)), ERR_ALIAS),
    ("ddelta_aliases_dz", dict(dz=ctypes.c_void_p(BASE + 13 * STEP + 512)), ERR_ALIAS),
]


@no_gpu_only
@pytest.mark.parametrize("name,kw,status", INVALID_BWD, ids=[c[0] for c in INVALID_BWD])
def test_bwd_rejects_invalid_arguments(name, kw, status):
    L = ss.lib()
    assert L.selscan_bwd(*bwd_args(**kw)) == status
    assert L.selscan_last_hip_error() == 0


def bwd_ex_args(flags=0, conv_w=None, conv_b=None, conv_width=0, dconv_w=None, dconv_b=None,
                **kw):
    a = bwd_args(**kw)
    # flags, conv_weight, conv_bias, conv_width, dconv_weight, dconv_bias go
    # between dh0 and batch
    return a[:21] + [flags, conv_w, conv_b, conv_width, dconv_w, dconv_b] + a[21:]


INVALID_BWD_EX = [
    ("unknown_flag", dict(flags=16), ERR_UNSUP),
    # kept checkpoints are read with the forward's part state (plain or reverse)
    ("keep_without_reuse", dict(flags=8), ERR_UNSUP),
    ("keep_reverse_without_reuse", dict(flags=8 | 2), ERR_UNSUP),
    ("keep_with_zoh", dict(flags=8 | 4 | 1), ERR_UNSUP),
    ("keep_with_conv", dict(flags=8 | 4, conv_width=4, conv_w=fake(22), dconv_w=fake(24)),
     ERR_UNSUP),
    # the forward's part state is reusable only where both run the default plan
    ("reuse_with_zoh", dict(flags=4 | 1), ERR_UNSUP),
    ("reuse_with_conv", dict(flags=4, conv_width=4, conv_w=fake(22), dconv_w=fake(24)),
     ERR_UNSUP),
    ("conv_width_5", dict(conv_width=5, conv_w=fake(22), dconv_w=fake(24)), ERR_UNSUP),
    ("conv_width_neg", dict(conv_width=-2, conv_w=fake(22), dconv_w=fake(24)), ERR_SHAPE),
    ("conv_w_null", dict(conv_width=4, dconv_w=fake(24)), ERR_NULL),
    ("dconv_w_null", dict(conv_width=4, conv_w=fake(22)), ERR_NULL),
    ("dconv_b_misaligned", dict(conv_width=3, conv_w=fake(22), dconv_w=fake(24),
                                dconv_b=ctypes.c_void_p(BASE + 25 * STEP + 4)), ERR_UNSUP),
    ("dconv_w_aliases_conv_w", dict(conv_width=4, conv_w=fake(22),
                                    dconv_w=ctypes.c_void_p(BASE + 22 * STEP + 64)), ERR_ALIAS),
    ("dconv_b_aliases_du", dict(conv_width=4, conv_w=fake(22), dconv_w=fake(24),
                                dconv_b=ctypes.c_void_p(BASE + 12 * STEP + 256)), ERR_ALIAS),
    ("dconv_w_aliases_dconv_b", dict(conv_width=4, conv_w=fake(22), dconv_w=fake(24),
                                     dconv_b=ctypes.c_void_p(BASE + 24 * STEP + 128)), ERR_ALIAS),
    ("du_aliases_conv_b", dict(conv_width=2, conv_w=fake(22), conv_b=fake(23), dconv_w=fake(24),
                               du=ctypes.c_void_p(BASE + 23 * STEP)), ERR_ALIAS),
    # the checks of selscan_bwd apply as well
    ("dtype", dict(dtype=4, flags=1), ERR_DTYPE),
    ("N3", dict(N=3, flags=2), ERR_UNSUP),
    ("dy_null", dict(dy=None, flags=3), ERR_NULL),
    ("small_workspace", dict(workspace_bytes=4096, conv_width=4, conv_w=fake(22),
                             dconv_w=fake(24)), ERR_WS),
]


@no_gpu_only
@pytest.mark.parametrize("name,kw,status", INVALID_BWD_EX, ids=[c[0] for c in INVALID_BWD_EX])
def test_bwd_ex_rejects_invalid_arguments(name, kw, status):
    L = ss.lib()
    assert L.selscan_bwd_ex(*bwd_ex_args(**kw)) == status
    assert L.selscan_last_hip_error() == 0


@no_gpu_only
@pytest.mark.parametrize("plan", ["lookback", "chunked", "dpp"])
def test_bwd_ex_refuses_reuse_under_forced_plan(monkeypatch, plan):
    """A forward under another plan leaves another workspace layout, so the
    backward cannot read its part state from it."""
    monkeypatch.setenv("SELSCAN_FORCE_PLAN", plan)
    L = ss.lib()
    for flags in (4, 4 | 2, 8 | 4):
        assert L.selscan_bwd_ex(*bwd_ex_args(flags=flags)) == ERR_UNSUP
        assert L.selscan_last_hip_error() == 0


def test_fwd_status_without_lookback_plan_touches_nothing(monkeypatch):
    """Only the look-back plan has waits that can give up; under any other
    plan the status call returns OK without reading the workspace (a fake
    address here) or touching the stream."""
    L = ss.lib()
    for plan in (None, "chunked", "dpp"):
        if plan is None:
            monkeypatch.delenv("SELSCAN_FORCE_PLAN", raising=False)
        else:
            monkeypatch.setenv("SELSCAN_FORCE_PLAN", plan)
        assert L.selscan_fwd_status(fake(12), None) == OK
    monkeypatch.setenv("SELSCAN_FORCE_PLAN", "lookback")
    assert L.selscan_fwd_status(None, None) == ERR_NULL


def test_flag_constants_match_header():
    assert ss.SELSCAN_FLAG_ZOH_EXACT == header_constant("SELSCAN_FLAG_ZOH_EXACT")
    assert ss.SELSCAN_FLAG_REVERSE == header_constant("SELSCAN_FLAG_REVERSE")
    assert ss.SELSCAN_FLAG_REUSE_FWD_STATE == header_constant("SELSCAN_FLAG_REUSE_FWD_STATE")
    assert ss.SELSCAN_FLAG_KEEP_CHECKPOINTS == header_constant("SELSCAN_FLAG_KEEP_CHECKPOINTS")


@no_gpu_only
def test_fwd_ex_keep_checkpoints_needs_a_backward_workspace():
    """Keeping the checkpoints writes them where the backward's layout has
    them: a forward-sized workspace is refused before any launch."""
    L = ss.lib()
    fwd_bytes = L.selscan_fwd_workspace_bytes(2, 64, 128, 16, 1)
    bwd_bytes = L.selscan_bwd_workspace_bytes(2, 64, 128, 16, 1)
    assert 0 < fwd_bytes < bwd_bytes
    assert L.selscan_fwd_ex(*fwd_ex_args(flags=8, workspace_bytes=fwd_bytes)) == ERR_WS
    assert L.selscan_fwd_ex(*fwd_ex_args(flags=8, workspace_bytes=bwd_bytes - 1)) == ERR_WS
    assert L.selscan_fwd_ex(*fwd_ex_args(flags=8, workspace=None)) == ERR_WS
    assert L.selscan_fwd_ex(*fwd_ex_args(flags=8 | 2, workspace_bytes=fwd_bytes)) == ERR_WS
    assert L.selscan_last_hip_error() == 0


def test_workspace_size_zero_when_grids_do_not_fit():
    L = ss.lib()
    assert L.selscan_fwd_workspace_bytes(1 << 20, 1 << 16, 1 << 10, 16, 1) == 0
    assert L.selscan_bwd_workspace_bytes(1 << 20, 1 << 16, 1 << 10, 16, 1) == 0
    # the largest dim with a long sequence still fits
    assert L.selscan_fwd_workspace_bytes(1, 1 << 17, 1 << 14, 16, 1) > 0


def test_bwd_workspace_size():
    L = ss.lib()
    # checkpoints alone: batch * ceil(dim/64) * ceil(L/4) * N * 256 bytes
    need = L.selscan_bwd_workspace_bytes(2, 64, 128, 16, 1)
    assert need >= 2 * 2 * 16 * 16 * 256
    assert L.selscan_bwd_workspace_bytes(2, 64, 128, 16, 7) == 0
    assert L.selscan_bwd_workspace_bytes(2, 64, 128, 12, 1) == 0
    assert L.selscan_bwd_workspace_bytes(0, 64, 128, 16, 1) == 0


def step_args(**kw):
    a = dict(state=fake(1), u=fake(2), delta=fake(3), A=fake(4), Bm=fake(5), Cm=fake(6),
             D_skip=fake(7), z=fake(8), delta_bias=fake(9), delta_softplus=1, y=fake(10),
             batch=4, dim=256, N=16, dtype=1, stream=None)
    a.update(kw)
    order = ["state", "u", "delta", "A", "Bm", "Cm", "D_skip", "z", "delta_bias",
             "delta_softplus", "y", "batch", "dim", "N", "dtype", "stream"]
    return [a[k] for k in order]


INVALID_STEP = [
    ("dtype", dict(dtype=3), ERR_DTYPE),
    ("batch0", dict(batch=0), ERR_SHAPE),
    ("dim0", dict(dim=0), ERR_SHAPE),
    ("state_null", dict(state=None), ERR_NULL),
    ("y_null", dict(y=None), ERR_NULL),
    ("B_null", dict(Bm=None), ERR_NULL),
    ("N7", dict(N=7), ERR_UNSUP),
    ("misaligned_state", dict(state=ctypes.c_void_p(BASE + STEP + 4)), ERR_UNSUP),
    ("y_aliases_state", dict(y=ctypes.c_void_p(BASE + STEP + 4096)), ERR_ALIAS),
    ("state_aliases_u", dict(u=ctypes.c_void_p(BASE + STEP + 256)), ERR_ALIAS),
    # the state is indexed with 32 bits: batch * dim * N < 2^31
    ("state_too_large", dict(batch=1 << 15, dim=1 << 12, N=16), ERR_UNSUP),
]


@no_gpu_only
@pytest.mark.parametrize("name,kw,status", INVALID_STEP, ids=[c[0] for c in INVALID_STEP])
def test_state_update_rejects_invalid_arguments(name, kw, status):
    L = ss.lib()
    assert L.selscan_state_update(*step_args(**kw)) == status


def test_binding_fails_loudly_without_library(monkeypatch):
    from selective_state_space_selscan_amd import _abi
    monkeypatch.setattr(_abi, "_lib", None)
    monkeypatch.setattr(_abi, "_LIB_PATH", "/nonexistent/libselscan.so")
    with pytest.raises(RuntimeError, match="not built"):
        _abi.lib()


def noalloc_args(**kw):
    a = fwd_args(**kw)
    return a[:17] + [a[19]]   # no workspace, workspace_bytes


INVALID_NOALLOC = [
    # 64 x 4096 x 4096 at N = 64 needs about 1.2 GB of workspace, more than the
    # 128 MiB fixed scratch
    ("beyond_scratch", dict(batch=64, L=4096, dim=4096, N=64), ERR_TOO_LARGE),
    ("dtype", dict(dtype=2), ERR_DTYPE),
    ("L0", dict(L=0), ERR_SHAPE),
    ("u_null", dict(u=None), ERR_NULL),
    ("N5", dict(N=5), ERR_UNSUP),
    ("misaligned_u", dict(u=ctypes.c_void_p(BASE + STEP + 2)), ERR_UNSUP),
    ("y_aliases_u", dict(y=ctypes.c_void_p(BASE + STEP + 64)), ERR_ALIAS),
]


@no_gpu_only
@pytest.mark.parametrize("name,kw,status", INVALID_NOALLOC, ids=[c[0] for c in INVALID_NOALLOC])
def test_fwd_noalloc_rejects_invalid_arguments(name, kw, status):
    """Checked on the host before any HIP call, like selscan_fwd, and shapes
    whose workspace exceeds the fixed scratch are refused."""
    L = ss.lib()
    assert L.selscan_fwd_workspace_bytes(64, 4096, 4096, 64, 1) > header_constant_expr(
        "SELSCAN_NOALLOC_SCRATCH_BYTES")
    assert L.selscan_fwd_noalloc(*noalloc_args(**kw)) == status
    assert L.selscan_last_hip_error() == 0


def header_constant_expr(name):
    m = re.search(r"#define\s+%s\s+\((\d+)u\s*<<\s*(\d+)\)" % name, open(HEADER).read())
    return int(m.group(1)) << int(m.group(2))


def test_noalloc_scratch_holds_the_workloads():
    """The fixed scratch holds the forward workspace of every workload here."""
    L = ss.lib()
    limit = header_constant_expr("SELSCAN_NOALLOC_SCRATCH_BYTES")
    assert limit == 128 << 20
    for shape in ((1, 256, 64), (8, 2048, 1536), (1, 131072, 2048), (16, 2048, 5120)):
        need = L.selscan_fwd_workspace_bytes(*shape, 16, 1)
        assert 0 < need <= limit, (shape, need)

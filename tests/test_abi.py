"""The C-ABI library loads, exports what include/dspark.h declares, and rejects bad calls
on the host before any HIP call (these run without a GPU; no compute is launched)."""
import ctypes
import os
import re

import pytest

from draft_sampling_verification_head_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


cpu_only = pytest.mark.skipif(not _no_gpu(), reason="host error paths are exercised where no GPU exists")


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.dspark_version() == 10000
    for s in range(5):
        assert lib.dspark_status_string(s)
    assert lib.dspark_status_string(99) == b"unknown status"


def test_workspace_sizes(lib):
    B, V, r, G = 64, 151936, 256, 16
    ntiles = -(-V // 256)
    need = lib.dspark_markov_draft_workspace_bytes(B, V, r, G)
    assert need >= 2 * B * ntiles * 8 + 2 * B * V * 4
    assert lib.dspark_markov_draft_workspace_bytes(0, V, r, G) == 0
    assert lib.dspark_verify_workspace_bytes(256, V, 16) >= 256 * 33 * 4
    assert lib.dspark_tv_labels_workspace_bytes(256, V, 16) >= 256 * 33 * 4
    assert lib.dspark_schedule_workspace_bytes(512, 16, 4096) >= 512 * 16 * 8


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def test_draft_path_host_rules(lib):
    """Path choices that depend on sizes, dtype and alignment only (no device query)."""
    lib.dspark_markov_draft_path.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 2
    odd = ctypes.c_void_p(0x1002)                 # not 16-byte aligned
    assert lib.dspark_markov_draft_path(64, 151936, 256, 1, FAKE, FAKE) == 3     # bf16 slab
    assert lib.dspark_markov_draft_path(2048, 151936, 256, 1, FAKE, FAKE) == 3   # slab at its B cap
    assert lib.dspark_markov_draft_path(2049, 151936, 256, 1, FAKE, FAKE) == 1   # MFMA beyond it
    assert lib.dspark_markov_draft_path(8192, 129280, 256, 1, FAKE, FAKE) == 3
    assert lib.dspark_markov_draft_path(8193, 129280, 256, 1, FAKE, FAKE) == 1
    assert lib.dspark_markov_draft_path(64, 163848, 256, 1, FAKE, FAKE) == 1     # V past the slab cap
    assert lib.dspark_markov_draft_path(9, 2056, 16, 1, FAKE, FAKE) == 3
    assert lib.dspark_markov_draft_path(64, 151936, 256, 0, FAKE, FAKE) == 0     # fp32: sweep
    assert lib.dspark_markov_draft_path(8, 151936, 256, 1, FAKE, FAKE) == 0      # B <= 8
    assert lib.dspark_markov_draft_path(64, 151936, 256, 1, odd, FAKE) == 0      # misaligned
    assert lib.dspark_markov_draft_path(1, 151936, 256, 0, FAKE, FAKE) == 0      # fp32, B = 1
    assert lib.dspark_markov_draft_path(1, 151936, 260, 1, FAKE, FAKE) == 0      # r > 256
    assert lib.dspark_markov_draft_path(1, 151937, 256, 1, FAKE, FAKE) == 0      # V % 8 != 0
    # one launch for all positions: only on the resident / slab paths, and only where the
    # device holds every workgroup at once (no device here)
    f = lib.dspark_markov_draft_one_launch
    f.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 2 + [ctypes.c_int]
    assert f(64, 151936, 256, 1, FAKE, FAKE, 1) == 0
    assert f(64, 151936, 256, 0, FAKE, FAKE, 0) == 0
    assert f(2049, 151936, 256, 1, FAKE, FAKE, 0) == 0


def _draft(lib, B=2, V=64, r=4, G=3, wdt=0, ws=FAKE, wsb=1 << 30, U=FAKE, x_out=FAKE):
    return lib.dspark_markov_draft(B, V, r, G, U, FAKE, FAKE, wdt, FAKE, FAKE, x_out, None,
                                   None, None, ws, wsb, None)


@cpu_only
@pytest.mark.parametrize("kw,status", [
    (dict(B=0), binding.ERR_INVALID_ARG),
    (dict(V=0), binding.ERR_INVALID_ARG),
    (dict(r=0), binding.ERR_INVALID_ARG),
    (dict(G=0), binding.ERR_INVALID_ARG),
    (dict(G=65), binding.ERR_UNSUPPORTED),
    (dict(r=1025), binding.ERR_UNSUPPORTED),
    (dict(B=1 << 20, V=1 << 20, G=2), binding.ERR_UNSUPPORTED),
    (dict(wdt=7), binding.ERR_INVALID_ARG),
    (dict(U=None), binding.ERR_INVALID_ARG),
    (dict(x_out=None), binding.ERR_INVALID_ARG),
    (dict(ws=None), binding.ERR_WORKSPACE),
    (dict(wsb=100), binding.ERR_WORKSPACE),
])
def test_draft_rejects(lib, kw, status):
    assert _draft(lib, **kw) == status
    assert lib.dspark_last_error()


@cpu_only
@pytest.mark.parametrize("options,status", [
    (2, binding.ERR_INVALID_ARG),                     # unknown option bit
    (-1, binding.ERR_INVALID_ARG),
    (binding.DRAFT_PER_POSITION, binding.ERR_WORKSPACE),   # a known bit: validation goes on
])
def test_draft_ex_options(lib, options, status):
    f = lib.dspark_markov_draft_ex
    f.argtypes = ([ctypes.c_int] * 4 + [ctypes.c_void_p] * 3 + [ctypes.c_int] + [ctypes.c_void_p] * 7 +
                  [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int])
    assert f(2, 64, 4, 3, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, None, None, None, FAKE, 100, None,
             options) == status
    assert lib.dspark_last_error()


def _verify(lib, B=2, V=64, G=3, Ld=FAKE, Lt_rows=8, t_off=None, x=FAKE, y=FAKE, ws=FAKE,
            wsb=1 << 30):
    return lib.dspark_verify(B, V, G, Ld, FAKE, Lt_rows, t_off, None, x, None, FAKE, FAKE, FAKE,
                             y, None, None, ws, wsb, None)


@cpu_only
@pytest.mark.parametrize("kw,status", [
    (dict(B=0), binding.ERR_INVALID_ARG),
    (dict(G=65), binding.ERR_UNSUPPORTED),
    (dict(Ld=None), binding.ERR_INVALID_ARG),
    (dict(Lt_rows=0), binding.ERR_INVALID_ARG),
    (dict(Lt_rows=7), binding.ERR_INVALID_ARG),       # padded layout needs B*(G+1) = 8 rows
    (dict(x=None), binding.ERR_INVALID_ARG),
    (dict(y=None), binding.ERR_INVALID_ARG),
    (dict(ws=None), binding.ERR_WORKSPACE),
    (dict(wsb=4), binding.ERR_WORKSPACE),
])
def test_verify_rejects(lib, kw, status):
    assert _verify(lib, **kw) == status


@cpu_only
def test_tv_rejects(lib):
    assert lib.dspark_tv_labels(2, 64, 3, FAKE, FAKE, 8, None, None, None, None, None, FAKE,
                                1 << 20, None) == binding.ERR_INVALID_ARG
    assert lib.dspark_tv_labels(2, 64, 3, FAKE, FAKE, 8, None, None, None, None, FAKE, None,
                                0, None) == binding.ERR_WORKSPACE


@cpu_only
def test_verify_tv_rejects(lib):
    args = (2, 64, 3, FAKE, FAKE, 8, None, None, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None)
    assert lib.dspark_verify_tv(*args, None, FAKE, 1 << 30, None) == binding.ERR_INVALID_ARG
    assert lib.dspark_verify_tv(*args, FAKE, FAKE, 4, None) == binding.ERR_WORKSPACE
    need = lib.dspark_verify_tv_workspace_bytes(2, 64, 3)
    assert need > lib.dspark_verify_workspace_bytes(2, 64, 3)
    bad = (2, 64, 65) + args[3:]
    assert lib.dspark_verify_tv(*bad, FAKE, FAKE, 1 << 30, None) == binding.ERR_UNSUPPORTED


def _vm(lib, B=2, V=64, r=8, G=3, wdt=1, U=FAKE, ld_lse=FAKE, Lt=FAKE, ws=FAKE, wsb=1 << 30):
    return lib.dspark_verify_markov(B, V, r, G, U, FAKE, FAKE, wdt, FAKE, FAKE, ld_lse, Lt, 8, None,
                                    None, FAKE, FAKE, FAKE, FAKE, None, None, ws, wsb, None)


@cpu_only
@pytest.mark.parametrize("kw,status", [
    (dict(B=0), binding.ERR_INVALID_ARG),
    (dict(G=65), binding.ERR_UNSUPPORTED),
    (dict(wdt=0), binding.ERR_UNSUPPORTED),            # fp32 factors
    (dict(r=264), binding.ERR_UNSUPPORTED),            # rank past the register slabs
    (dict(r=12), binding.ERR_UNSUPPORTED),             # r % 8 != 0
    (dict(V=68), binding.ERR_UNSUPPORTED),             # V % 8 != 0
    (dict(V=163848), binding.ERR_UNSUPPORTED),         # more than 2048 wave tiles
    (dict(r=0), binding.ERR_INVALID_ARG),
    (dict(U=None), binding.ERR_INVALID_ARG),
    (dict(ld_lse=None), binding.ERR_INVALID_ARG),      # the draft's normalisers are required
    (dict(U=ctypes.c_void_p(0x1004)), binding.ERR_INVALID_ARG),   # not 16-byte aligned
    (dict(ws=None), binding.ERR_WORKSPACE),
    (dict(wsb=16), binding.ERR_WORKSPACE),
])
def test_verify_markov_rejects(lib, kw, status):
    assert _vm(lib, **kw) == status
    assert lib.dspark_last_error()


def test_verify_markov_workspace(lib):
    B, V, r, G = 512, 129280, 256, 16
    need = lib.dspark_verify_markov_workspace_bytes(B, V, r, G)
    tiles = -(-V // 512) * 8                       # 16-column tiles x 4 per wave, 8 waves
    assert need >= B * G * tiles * 8               # wave-tile partials of every verified row
    assert lib.dspark_verify_markov_workspace_bytes(0, V, r, G) == 0


@cpu_only
@pytest.mark.parametrize("args,status", [
    ((0, 4, 10, 0), binding.ERR_INVALID_ARG),
    ((4, 0, 10, 0), binding.ERR_INVALID_ARG),
    ((4, 65, 1000, 0), binding.ERR_UNSUPPORTED),
    ((2048, 16, 4096, 0), binding.ERR_UNSUPPORTED),   # 32768 candidates
    ((8, 4, 7, 0), binding.ERR_INVALID_ARG),          # Bmax < R
    ((8, 4, 40, 2), binding.ERR_INVALID_ARG),         # unknown mode
])
def test_schedule_rejects(lib, args, status):
    R, G, Bmax, mode = args
    assert lib.dspark_schedule(R, G, FAKE, None, FAKE, Bmax, mode, FAKE, None, None, None, None,
                               FAKE, 1 << 30, None) == status


@cpu_only
def test_schedule_null_required(lib):
    assert lib.dspark_schedule(4, 4, None, None, FAKE, 40, 0, FAKE, None, None, None, None, FAKE,
                               1 << 30, None) == binding.ERR_INVALID_ARG
    assert lib.dspark_schedule(4, 4, FAKE, None, FAKE, 40, 0, None, None, None, None, None, FAKE,
                               1 << 30, None) == binding.ERR_INVALID_ARG
    assert lib.dspark_schedule(4, 4, FAKE, None, FAKE, 40, 0, FAKE, None, None, None, None, FAKE,
                               8, None) == binding.ERR_WORKSPACE


def test_conf_ring_bytes(lib):
    """Counter header (256 bytes) plus three [R][gamma] fp32 slots."""
    assert lib.dspark_conf_ring_bytes(512, 16) == 256 + 3 * 512 * 16 * 4
    assert lib.dspark_conf_ring_bytes(0, 16) == 0
    assert lib.dspark_conf_ring_bytes(4, 0) == 0


@cpu_only
def test_conf_ring_rejects(lib):
    n = lib.dspark_conf_ring_bytes(4, 4)
    odd = ctypes.c_void_p(0x1004)
    assert lib.dspark_conf_ring_init(4, 4, None, n, None) == binding.ERR_INVALID_ARG
    assert lib.dspark_conf_ring_init(4, 4, odd, n, None) == binding.ERR_INVALID_ARG   # not 8-aligned
    assert lib.dspark_conf_ring_init(4, 4, FAKE, n - 1, None) == binding.ERR_WORKSPACE
    assert lib.dspark_conf_ring_init(0, 4, FAKE, n, None) == binding.ERR_INVALID_ARG
    assert lib.dspark_conf_ring_init(2048, 16, FAKE, 1 << 30, None) == binding.ERR_UNSUPPORTED
    assert lib.dspark_conf_ring_push(4, 4, FAKE, n, None, None) == binding.ERR_INVALID_ARG
    assert lib.dspark_conf_ring_push(4, 4, FAKE, n - 1, FAKE, None) == binding.ERR_WORKSPACE
    lag = lib.dspark_schedule_lagged
    assert lag(4, 4, None, n, None, FAKE, 40, 0, FAKE, None, None, None, None, FAKE, 1 << 30,
               None) == binding.ERR_INVALID_ARG
    assert lag(4, 4, FAKE, n - 1, None, FAKE, 40, 0, FAKE, None, None, None, None, FAKE, 1 << 30,
               None) == binding.ERR_WORKSPACE
    assert lag(4, 4, FAKE, n, None, FAKE, 3, 0, FAKE, None, None, None, None, FAKE, 1 << 30,
               None) == binding.ERR_INVALID_ARG                                  # Bmax < R
    assert lag(4, 4, FAKE, n, None, FAKE, 40, 0, FAKE, None, None, None, None, FAKE, 8,
               None) == binding.ERR_WORKSPACE                                    # schedule workspace


@cpu_only
@pytest.mark.parametrize("args,status", [
    ((0, 4, 8, 15, 0), binding.ERR_INVALID_ARG),
    ((16, 65, 8, 15, 0), binding.ERR_UNSUPPORTED),
    ((16, 4, 8, 17, 0), binding.ERR_UNSUPPORTED),     # more bins than the kernel keeps
    ((16, 4, 5000, 15, 0), binding.ERR_UNSUPPORTED),
    ((16, 4, 8, 15, 2), binding.ERR_INVALID_ARG),     # unknown objective
])
def test_sts_rejects(lib, args, status):
    N, G, nT, bins, obj = args
    assert lib.dspark_sts_fit(N, G, FAKE, FAKE, None, FAKE, nT, bins, obj, FAKE, FAKE, FAKE, None,
                              FAKE, 1 << 30, None) == status


@cpu_only
def test_sts_null_and_workspace(lib):
    assert lib.dspark_sts_fit(16, 4, None, FAKE, None, FAKE, 8, 15, 0, FAKE, FAKE, FAKE, None,
                              FAKE, 1 << 30, None) == binding.ERR_INVALID_ARG
    assert lib.dspark_sts_fit(16, 4, FAKE, FAKE, None, FAKE, 8, 15, 0, FAKE, FAKE, FAKE, None,
                              FAKE, 8, None) == binding.ERR_WORKSPACE
    assert lib.dspark_sts_fit_workspace_bytes(16, 4, 8) >= 16 * 4 * 5


def test_binding_refuses_missing_library(tmp_path, monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        binding.load(str(tmp_path / "nope.so"))


def _plan(lib, B, V, r, G, wdt, W1=FAKE, W2=FAKE, U=FAKE, Ld=None, options=0):
    path, one, nb = ctypes.c_int(-1), ctypes.c_int(-1), ctypes.c_size_t(0)
    st = lib.dspark_markov_draft_plan(B, V, r, G, wdt, W1, W2, U, Ld, options, ctypes.byref(path),
                                      ctypes.byref(one), ctypes.byref(nb))
    return st, path.value, one.value, nb.value


def test_draft_plan_host_rules(lib):
    """The plan of an exact call: its path (U and the logits output's alignment included),
    whether it runs in one launch, and the workspace it needs, which is never more than the
    all-path figure and drops the logits rows where the path does not use them."""
    B, V, r, G = 64, 151936, 256, 16
    full = lib.dspark_markov_draft_workspace_bytes(B, V, r, G)
    st, path, one, nb = _plan(lib, B, V, r, G, 1)
    assert st == binding.OK and path == 3 and one == 0 and nb <= full          # slab: no rows
    assert nb < full - 2 * B * V * 4 + 4096
    odd = ctypes.c_void_p(0x1004)
    st, path, _, nb_m = _plan(lib, B, V, r, G, 1, U=odd)                         # U misaligned
    assert st == binding.OK and path == 1 and nb_m == full                      # MFMA, rows in ws
    st, path, _, nb_ml = _plan(lib, B, V, r, G, 1, U=odd, Ld=FAKE)              # logits to the caller
    assert path == 1 and nb_ml == full - 2 * ((B * V * 4 + 255) // 256 * 256)
    st, path, _, nb_s = _plan(lib, B, V, r, G, 0)                                # fp32: sweep
    assert path == 0 and nb_s == full
    st, path, _, _ = _plan(lib, B, V, r, G, 1, options=binding.DRAFT_PER_POSITION)
    assert path == 3
    assert _plan(lib, 0, V, r, G, 1)[0] == binding.ERR_INVALID_ARG
    assert _plan(lib, B, V, r, 65, 1)[0] == binding.ERR_INVALID_ARG
    assert _plan(lib, B, V, r, G, 5)[0] == binding.ERR_INVALID_ARG
    assert _plan(lib, B, V, r, G, 1, options=2)[0] == binding.ERR_INVALID_ARG
    st = lib.dspark_markov_draft_plan(B, V, r, G, 1, FAKE, FAKE, FAKE, None, 0, None, None, None)
    assert st == binding.OK                                                      # outputs nullable


@cpu_only
def test_draft_accepts_the_planned_workspace(lib):
    """A call checks its workspace against its own plan: the planned bytes pass the check (the
    call then fails only at launch, here without a device), one byte less is refused."""
    B, V, r, G = 64, 151936, 256, 16
    _, _, _, nb = _plan(lib, B, V, r, G, 1)
    f = lib.dspark_markov_draft_ex
    f.argtypes = ([ctypes.c_int] * 4 + [ctypes.c_void_p] * 3 + [ctypes.c_int] + [ctypes.c_void_p] * 7 +
                  [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int])
    args = (B, V, r, G, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, None, None, FAKE)
    assert f(*args, nb - 1, None, 0) == binding.ERR_WORKSPACE
    assert f(*args, nb, None, 0) != binding.ERR_WORKSPACE


def _draft_schedule_fn(lib):
    f = lib.dspark_markov_draft_schedule
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    f.argtypes = ([I] * 4 + [P] * 3 + [I] + [P] * 6 + [I, P, P, Z, P, P, I, I] + [P] * 5 + [P, Z, P])
    return f


def test_draft_schedule_workspace_and_fusion_rules(lib):
    """The fused call's workspace is the draft's worst case, aligned, then the schedule's; the
    schedule rides in the draft's launch only for the single-request path and <= 64
    candidates (and never where no device answers the residency query)."""
    B, V, r, G, R, Bmax = 1, 151936, 256, 7, 1, 4096
    d = lib.dspark_markov_draft_workspace_bytes(B, V, r, G)
    s = lib.dspark_schedule_workspace_bytes(R, G, Bmax)
    got = lib.dspark_markov_draft_schedule_workspace_bytes(B, V, r, G, R, Bmax)
    assert got == -(-d // 256) * 256 + s
    assert lib.dspark_markov_draft_schedule_workspace_bytes(0, V, r, G, R, Bmax) == 0
    assert lib.dspark_markov_draft_schedule_workspace_bytes(B, V, r, G, 0, Bmax) == 0
    f = lib.dspark_markov_draft_schedule_fused
    f.argtypes = [ctypes.c_int] * 5 + [ctypes.c_void_p] * 2 + [ctypes.c_int]
    assert f(64, V, r, 16, 1, FAKE, FAKE, 64) == 0        # slab path
    assert f(1, V, r, 16, 1, FAKE, FAKE, 5) == 0          # 80 candidates
    assert f(1, V, r, 16, 1, FAKE, FAKE, 0) == 0
    if _no_gpu():
        assert f(1, V, r, 7, 1, FAKE, FAKE, 1) == 0       # no device: no residency answer


@cpu_only
@pytest.mark.parametrize("kw,status", [
    (dict(conf=None), binding.ERR_INVALID_ARG),            # neither conf nor ring
    (dict(R=0), binding.ERR_INVALID_ARG),
    (dict(mode=7), binding.ERR_INVALID_ARG),
    (dict(Bmax=0), binding.ERR_INVALID_ARG),               # Bmax < R
    (dict(len_out=None), binding.ERR_INVALID_ARG),
    (dict(ring=ctypes.c_void_p(0x1004), ring_bytes=1 << 20), binding.ERR_INVALID_ARG),   # misaligned
    (dict(ring=FAKE, ring_bytes=8), binding.ERR_WORKSPACE),    # ring too small
    (dict(ws=None), binding.ERR_WORKSPACE),
    (dict(wsb=100), binding.ERR_WORKSPACE),
])
def test_draft_schedule_rejects(lib, kw, status):
    a = dict(B=1, V=64, r=8, G=3, R=1, conf=FAKE, ring=None, ring_bytes=0, Bmax=64, mode=0,
             len_out=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    f = _draft_schedule_fn(lib)
    st = f(a["B"], a["V"], a["r"], a["G"], FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, None, None,
           a["R"], a["conf"], a["ring"], a["ring_bytes"], None, FAKE, a["Bmax"], a["mode"],
           a["len_out"], None, None, None, None, a["ws"], a["wsb"], None)
    assert st == status
    assert lib.dspark_last_error()

"""The C ABI library, without a GPU: it loads, exports every symbol declared
in include/dtree.h, and rejects bad arguments before enqueuing anything."""
import ctypes as C
import os
import re

import pytest

import conditional_draft_tree_amd as dtree
from conditional_draft_tree_amd._lib import dt_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dtree.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dt_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("dt_create", "dt_destroy", "dt_workspace_bytes", "dt_build", "dt_topm",
                 "dt_gru_step", "dt_correct", "dt_last_error", "dt_status_string",
                 "dt_timing_enable", "dt_timing_read"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = dtree.load_library()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_library_is_built_for_gfx950():
    with open(dtree.lib_path(), "rb") as f:
        blob = f.read()
    assert b"gfx950" in blob


def make(**kw):
    cfg = dict(B=2, L=4, V=100, E=32, H=32, M=8, n=6, temperature=0.0, dtype=dtree.DT_BF16,
               near_tie_eps=1e-5)
    cfg.update(kw)
    return dtree.dt_create(**cfg)


def test_create_accepts_the_limits():
    # the largest shapes each limit allows (L = 64, M = 64 or n = 64, H = 4096)
    for kw in (dict(L=64, M=32, n=32, V=1000), dict(M=64, n=64, V=1000), dict(H=4096), dict(L=64, V=1000)):
        dtree.dt_destroy(make(**kw))


def test_create_valid_and_workspace():
    h = make()
    assert dtree.dt_workspace_bytes(h) > 0
    dtree.dt_destroy(h)
    h = make(B=0)
    dtree.dt_destroy(h)


@pytest.mark.parametrize("kw,code", [
    (dict(L=0), "INVALID_ARG"), (dict(V=0), "INVALID_ARG"), (dict(M=0), "INVALID_ARG"),
    (dict(n=0), "INVALID_ARG"), (dict(B=-1), "INVALID_ARG"), (dict(M=101), "INVALID_ARG"),
    (dict(temperature=-1.0), "INVALID_ARG"), (dict(dtype=7), "INVALID_ARG"),
    (dict(M=65, V=1000), "UNSUPPORTED"), (dict(n=65), "UNSUPPORTED"), (dict(L=65), "UNSUPPORTED"),
    (dict(E=48), "UNSUPPORTED"), (dict(H=24), "UNSUPPORTED"), (dict(H=48), "UNSUPPORTED"), (dict(H=8192), "UNSUPPORTED"),
    (dict(dtype=dtree.DT_F32, E=6), "UNSUPPORTED"),
    # per-request state beyond 64 KiB of LDS: the L x M table and n x 64 child lists
    (dict(L=64, M=64, n=64, V=1000), "UNSUPPORTED"),
])
def test_create_rejects(kw, code):
    with pytest.raises(ValueError, match=code):
        make(**kw)
    assert dtree.dt_last_error(None)  # message available without a handle


def test_status_strings():
    for s in (0, -1, -2, -3, -4):
        assert dtree.dt_status_string(s)


def _raw_build(lib, h, ws, nbytes, ptr, **override):
    args = dict(base=ptr, emb=ptr, w_ih=ptr, w_hh=ptr, b_ih=None, b_hh=None, C=ptr, h0=None,
                tokens=ptr, parents=ptr, depths=ptr, scores=ptr, mask=ptr, count=ptr, flags=ptr)
    args.update(override)
    vals = [C.c_void_p(v) if v is not None else None for v in args.values()]
    return lib.dt_build(h, C.c_void_p(ws) if ws else None, nbytes, *vals, None)


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


@pytest.mark.skipif(not _no_gpu(), reason="uses fake device addresses; CPU-only machines")
def test_build_argument_errors_before_any_launch():
    lib = dtree.load_library()
    h = make()
    need = dtree.dt_workspace_bytes(h)
    fake = 0x10000  # never dereferenced: every call below fails validation
    assert _raw_build(lib, h, fake, need, fake, C=None) == -1
    assert "null" in dtree.dt_last_error(h)
    assert _raw_build(lib, h, fake, need, fake, emb=fake + 4) == -1
    assert "aligned" in dtree.dt_last_error(h)
    assert _raw_build(lib, h, None, need, fake) == -3
    assert _raw_build(lib, h, fake, need - 1, fake) == -3
    assert _raw_build(lib, h, fake + 16, need, fake) == -3  # workspace alignment
    dtree.dt_destroy(h)


@pytest.mark.skipif(not _no_gpu(), reason="uses fake device addresses; CPU-only machines")
def test_build_marginal_argument_errors_before_any_launch():
    lib = dtree.load_library()
    h = make()
    need = dtree.dt_workspace_bytes(h)
    fake = C.c_void_p(0x10000)  # never dereferenced: every call below fails validation
    outs = [fake] * 7
    # no GRU inputs are needed; the logits and the outputs are
    assert lib.dt_build_marginal(h, fake, need, None, *outs, None) == -1
    assert "null" in dtree.dt_last_error(h)
    assert lib.dt_build_marginal(h, fake, need, C.c_void_p(0x10004), *outs, None) == -1
    assert "aligned" in dtree.dt_last_error(h)
    assert lib.dt_build_marginal(h, None, need, fake, *outs, None) == -3
    dtree.dt_destroy(h)


def test_full_vocab_flag_is_validated():
    lib = dtree.load_library()
    bad = dt_config(1, 4, 100, 32, 32, 8, 4, 0.0, dtree.DT_F32, 1e-5, 2)
    out = C.c_void_p()
    assert lib.dt_create(C.byref(bad), C.byref(out)) == -1 and not out.value
    assert "full_vocab" in dtree.dt_last_error(None)
    h = dtree.dt_create(1, 4, 100, 32, 32, 8, 4, 0.0, dtree.DT_F32, 1e-5, full_vocab=True)
    fake = C.c_void_p(0x10000)
    need = dtree.dt_workspace_bytes(h)
    assert lib.dt_topm_tail(h, fake, need, fake, fake, fake, None, None) == -1
    assert lib.dt_topm_tail(h, fake, need, C.c_void_p(0x10004), fake, fake, fake, None) == -1
    assert lib.dt_topm_tail(h, None, need, fake, fake, fake, fake, None) == -3
    dtree.dt_destroy(h)


def test_folded_entry_points_validate_before_any_launch():
    lib = dtree.load_library()
    h = make()
    need = dtree.dt_workspace_bytes(h)
    fake = C.c_void_p(0x10000)  # never dereferenced: every call below fails validation
    assert lib.dt_fold_input(h, None, fake, None, fake, None) == -1
    assert lib.dt_fold_input(h, fake, fake, None, C.c_void_p(0x10004), None) == -1
    outs = [fake] * 7
    assert lib.dt_build_folded(h, fake, need, fake, None, fake, None, fake, None, *outs, None) == -1
    assert "table" in dtree.dt_last_error(h)
    assert lib.dt_build_folded(h, fake, need, fake, fake, None, None, fake, None, *outs, None) == -1
    assert lib.dt_build_folded(h, None, need, fake, fake, fake, None, fake, None, *outs, None) == -3
    dtree.dt_destroy(h)


def test_accept_greedy_null_pointer_before_any_launch():
    lib = dtree.load_library()
    h = make()
    fake = C.c_void_p(0x10000)  # never dereferenced: every call below fails validation
    for i in range(7):
        args = [fake] * 7
        args[i] = None
        assert lib.dt_accept_greedy(h, *args, None) == -1
        assert "null" in dtree.dt_last_error(h)
    assert lib.dt_accept_greedy(None, *([fake] * 7), None) == -1
    dtree.dt_destroy(h)


def test_empty_batch_is_a_noop():
    lib = dtree.load_library()
    h = make(B=0)
    # B = 0: nothing to do, every pointer may be NULL
    assert lib.dt_build(h, None, 0, *([None] * 15), None) == 0
    assert lib.dt_build_marginal(h, None, 0, *([None] * 8), None) == 0
    assert lib.dt_topm(h, None, 0, None, None, None, None) == 0
    assert lib.dt_accept_greedy(h, *([None] * 7), None) == 0
    assert lib.dt_topm_tail(h, None, 0, None, None, None, None, None) == 0
    assert lib.dt_build_folded(h, None, 0, None, fake_table(), *([None] * 11), None) == 0
    dtree.dt_destroy(h)


def fake_table():
    return C.c_void_p(0x10000)  # B = 0: never dereferenced


def test_timing_argument_checks():
    lib = dtree.load_library()
    h = make()
    assert lib.dt_timing_enable(h, 3, 10) == -1
    assert lib.dt_timing_enable(h, 1, -1) == -1
    assert lib.dt_timing_enable(h, 0, 0) == 0
    n = C.c_int(0)
    assert lib.dt_timing_read(h, 9, None, 0, C.byref(n)) == -1
    assert lib.dt_timing_read(h, 9, None, 0, C.byref(n)) == -1
    assert lib.dt_timing_read(h, -1, None, 0, C.byref(n)) == -1
    assert lib.dt_timing_read(h, 8, None, 0, C.byref(n)) == 0 and n.value == 0
    assert lib.dt_timing_read(h, 0, None, 0, C.byref(n)) == 0 and n.value == 0
    assert lib.dt_timing_read(h, 6, None, 0, C.byref(n)) == 0 and n.value == 0
    dtree.dt_destroy(h)


def test_expand_mode_is_validated():
    lib = dtree.load_library()
    out = C.c_void_p()
    for e in (5, -1):
        bad = dt_config(2, 4, 100, 32, 32, 8, 4, 0.0, dtree.DT_BF16, 1e-5, 0, e)
        assert lib.dt_create(C.byref(bad), C.byref(out)) == -1 and not out.value
        assert "expand" in dtree.dt_last_error(None)
    # the fused expansion (per-step launches or persistent) is bf16 with
    # H <= 1024; one launch per step holds at most 64 requests, the persistent
    # launch takes more in slices of 64
    for e in (dtree.DT_EXPAND_FUSED, dtree.DT_EXPAND_PERSISTENT, dtree.DT_EXPAND_RESIDENT):
        for kw in (dict(dtype=dtree.DT_F32), dict(H=2048)):
            with pytest.raises(ValueError, match="UNSUPPORTED"):
                make(expand=e, **kw)
    with pytest.raises(ValueError, match="UNSUPPORTED"):
        make(expand=dtree.DT_EXPAND_FUSED, B=65)
    # the mode dt_build runs, before any call: auto selects the persistent
    # launch where the fused expansion applies (a call may fall back to the
    # per-step launches)
    for e, want in ((dtree.DT_EXPAND_AUTO, dtree.DT_EXPAND_RESIDENT),
                    (dtree.DT_EXPAND_RESIDENT, dtree.DT_EXPAND_RESIDENT),
                    (dtree.DT_EXPAND_STEPPED, dtree.DT_EXPAND_STEPPED),
                    (dtree.DT_EXPAND_FUSED, dtree.DT_EXPAND_FUSED),
                    (dtree.DT_EXPAND_PERSISTENT, dtree.DT_EXPAND_PERSISTENT)):
        h = make(expand=e)
        assert dtree.dt_expand_mode(h) == want
        dtree.dt_destroy(h)
    for kw in (dict(dtype=dtree.DT_F32), dict(H=2048)):
        h = make(**kw)
        assert dtree.dt_expand_mode(h) == dtree.DT_EXPAND_STEPPED
        dtree.dt_destroy(h)
    # more than 64 requests: stepped unless the persistent launch (in slices
    # of 64) is asked for
    for e, want in ((dtree.DT_EXPAND_AUTO, dtree.DT_EXPAND_STEPPED),
                    (dtree.DT_EXPAND_PERSISTENT, dtree.DT_EXPAND_PERSISTENT),
                    (dtree.DT_EXPAND_RESIDENT, dtree.DT_EXPAND_RESIDENT)):
        h = make(expand=e, B=65)
        assert dtree.dt_expand_mode(h) == want
        dtree.dt_destroy(h)
    # the stress shape (B = 256, n = 64) fits the persistent plan: four launches
    h = dtree.dt_create(256, 16, 151936, 2560, 1024, 64, 64, 0.0, dtree.DT_BF16, 1e-5,
                        expand=dtree.DT_EXPAND_PERSISTENT)
    assert dtree.dt_expand_mode(h) == dtree.DT_EXPAND_PERSISTENT
    dtree.dt_destroy(h)
    assert lib.dt_expand_mode(None) == -1
    # the fused expansion's workspace holds its per-slot gate sums besides the stepped path's
    assert dtree.dt_workspace_bytes(make(expand=dtree.DT_EXPAND_FUSED)) > \
        dtree.dt_workspace_bytes(make(expand=dtree.DT_EXPAND_STEPPED))

"""ctypes binding of include/dtree.h.  Argument marshalling only."""
from __future__ import annotations

import ctypes as C
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libdtree.so")
_lock = threading.Lock()
_lib = None

DT_F32, DT_BF16 = 0, 1
DT_EXPAND_AUTO, DT_EXPAND_STEPPED, DT_EXPAND_FUSED, DT_EXPAND_PERSISTENT, DT_EXPAND_RESIDENT = 0, 1, 2, 3, 4
_STATUS = {0: "DT_OK", -1: "DT_ERR_INVALID_ARG", -2: "DT_ERR_UNSUPPORTED", -3: "DT_ERR_WORKSPACE",
           -4: "DT_ERR_HIP"}


class DtreeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class dt_config(C.Structure):
    _fields_ = [("B", C.c_int32), ("L", C.c_int32), ("V", C.c_int32), ("E", C.c_int32),
                ("H", C.c_int32), ("M", C.c_int32), ("n", C.c_int32), ("temperature", C.c_float),
                ("dtype", C.c_int), ("near_tie_eps", C.c_float), ("full_vocab", C.c_int32),
                ("expand", C.c_int32)]


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libdtree.so; raises if it has not been built (no fallback)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m conditional_draft_tree_amd.build`")
        lib = C.CDLL(_LIB_PATH)
        vp, i32p, f32p = C.c_void_p, C.c_void_p, C.c_void_p
        H = C.c_void_p
        lib.dt_create.argtypes = [C.POINTER(dt_config), C.POINTER(H)]
        lib.dt_destroy.argtypes = [H]
        lib.dt_destroy.restype = None
        lib.dt_workspace_bytes.argtypes = [H]
        lib.dt_workspace_bytes.restype = C.c_size_t
        lib.dt_expand_mode.argtypes = [H]
        lib.dt_expand_mode.restype = C.c_int32
        lib.dt_status_string.argtypes = [C.c_int]
        lib.dt_status_string.restype = C.c_char_p
        lib.dt_last_error.argtypes = [H]
        lib.dt_last_error.restype = C.c_char_p
        # handle, workspace, bytes, base, emb, W_ih, W_hh, b_ih, b_hh, C, h0,
        # tokens, parents, depths, scores, mask, count, flags, stream
        lib.dt_build.argtypes = [H, vp, C.c_size_t] + [vp] * 7 + [f32p] + [i32p] * 3 + [
            f32p, vp, i32p, vp, vp]
        # handle, base, emb, W_ih, W_hh, b_ih, b_hh, C, h0, tokens, parents, depths, scores, mask,
        # count, flags, stream
        lib.dt_build_noalloc.argtypes = [H] + [vp] * 7 + [f32p] + [i32p] * 3 + [f32p, vp, i32p, vp, vp]
        # handle, workspace, bytes, base, tokens, parents, depths, scores, mask, count, flags, stream
        lib.dt_build_marginal.argtypes = [H, vp, C.c_size_t, vp] + [i32p] * 3 + [f32p, vp, i32p, vp, vp]
        lib.dt_topm.argtypes = [H, vp, C.c_size_t, vp, i32p, f32p, vp]
        lib.dt_topm_tail.argtypes = [H, vp, C.c_size_t, vp, i32p, f32p, f32p, vp]
        lib.dt_gru_step.argtypes = [H, vp, C.c_size_t, vp, f32p, vp, vp, vp, vp, f32p, vp]
        lib.dt_correct.argtypes = [H, i32p, f32p, vp, f32p, i32p, i32p, f32p, vp]
        lib.dt_accept_greedy.argtypes = [H] + [i32p] * 7 + [vp]
        lib.dt_fold_input.argtypes = [H, vp, vp, vp, f32p, vp]
        # handle, workspace, bytes, base, table, W_hh, b_hh, C, h0, tokens, parents, depths,
        # scores, mask, count, flags, stream
        lib.dt_build_folded.argtypes = [H, vp, C.c_size_t, vp, f32p, vp, vp, vp, f32p] + [i32p] * 3 + [
            f32p, vp, i32p, vp, vp]
        lib.dt_timing_enable.argtypes = [H, C.c_int, C.c_int]
        lib.dt_timing_read.argtypes = [H, C.c_int, C.POINTER(C.c_float), C.c_int,
                                       C.POINTER(C.c_int)]
        for f in (lib.dt_create, lib.dt_build, lib.dt_build_noalloc, lib.dt_build_marginal, lib.dt_topm, lib.dt_topm_tail,
                  lib.dt_gru_step,
                  lib.dt_correct, lib.dt_accept_greedy, lib.dt_fold_input, lib.dt_build_folded,
                  lib.dt_timing_enable, lib.dt_timing_read):
            f.restype = C.c_int
        _lib = lib
        return lib


def _check(status: int, handle=None):
    if status != 0:
        lib = load_library()
        msg = lib.dt_last_error(handle).decode(errors="replace")
        if status in (-1, -2, -3):
            raise ValueError(f"{_STATUS.get(status, status)}: {msg}")
        raise DtreeError(status, msg)


# ---- C entry points with the same names ---------------------------------------

def dt_status_string(status: int) -> str:
    return load_library().dt_status_string(status).decode()


def dt_last_error(handle=None) -> str:
    return load_library().dt_last_error(handle).decode(errors="replace")


def dt_create(B, L, V, E, H, M, n, temperature=0.0, dtype=DT_BF16, near_tie_eps=1e-5, full_vocab=False,
              expand=DT_EXPAND_AUTO):
    """Returns an opaque handle (host only; no GPU needed)."""
    lib = load_library()
    cfg = dt_config(B, L, V, E, H, M, n, float(temperature), int(dtype), float(near_tie_eps),
                    int(bool(full_vocab)), int(expand))
    h = C.c_void_p()
    _check(lib.dt_create(C.byref(cfg), C.byref(h)), None)
    return h


def dt_destroy(handle):
    load_library().dt_destroy(handle)


def dt_workspace_bytes(handle) -> int:
    return int(load_library().dt_workspace_bytes(handle))


def dt_expand_mode(handle) -> int:
    return int(load_library().dt_expand_mode(handle))


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def dt_build(handle, workspace, base, emb, w_ih, w_hh, b_ih, b_hh, Cmat, h0, tokens, parents,
             depths, scores, mask, count, flags, stream=None):
    lib = load_library()
    _check(lib.dt_build(handle, _p(workspace), workspace.numel() if workspace is not None else 0,
                        _p(base), _p(emb), _p(w_ih), _p(w_hh), _p(b_ih), _p(b_hh), _p(Cmat), _p(h0),
                        _p(tokens), _p(parents), _p(depths), _p(scores), _p(mask), _p(count),
                        _p(flags), _stream(stream)), handle)


def dt_build_noalloc(handle, base, emb, w_ih, w_hh, b_ih, b_hh, Cmat, h0, tokens, parents, depths, scores, mask,
                     count, flags, stream=None):
    lib = load_library()
    _check(lib.dt_build_noalloc(handle, _p(base), _p(emb), _p(w_ih), _p(w_hh), _p(b_ih), _p(b_hh), _p(Cmat),
                                _p(h0), _p(tokens), _p(parents), _p(depths), _p(scores), _p(mask), _p(count),
                                _p(flags), _stream(stream)), handle)


def dt_fold_input(handle, emb, w_ih, b_ih, table, stream=None):
    _check(load_library().dt_fold_input(handle, _p(emb), _p(w_ih), _p(b_ih), _p(table), _stream(stream)), handle)


def dt_build_folded(handle, workspace, base, table, w_hh, b_hh, Cmat, h0, tokens, parents, depths, scores, mask,
                    count, flags, stream=None):
    lib = load_library()
    _check(lib.dt_build_folded(handle, _p(workspace), workspace.numel() if workspace is not None else 0,
                               _p(base), _p(table), _p(w_hh), _p(b_hh), _p(Cmat), _p(h0), _p(tokens),
                               _p(parents), _p(depths), _p(scores), _p(mask), _p(count), _p(flags),
                               _stream(stream)), handle)


def dt_build_marginal(handle, workspace, base, tokens, parents, depths, scores, mask, count, flags,
                      stream=None):
    lib = load_library()
    _check(lib.dt_build_marginal(handle, _p(workspace), workspace.numel() if workspace is not None else 0,
                                 _p(base), _p(tokens), _p(parents), _p(depths), _p(scores), _p(mask),
                                 _p(count), _p(flags), _stream(stream)), handle)


def dt_topm(handle, workspace, base, idx, val, stream=None):
    lib = load_library()
    _check(lib.dt_topm(handle, _p(workspace), workspace.numel() if workspace is not None else 0,
                       _p(base), _p(idx), _p(val), _stream(stream)), handle)


def dt_topm_tail(handle, workspace, base, idx, val, tail, stream=None):
    lib = load_library()
    _check(lib.dt_topm_tail(handle, _p(workspace), workspace.numel() if workspace is not None else 0,
                            _p(base), _p(idx), _p(val), _p(tail), _stream(stream)), handle)


def dt_gru_step(handle, workspace, x, h, w_ih, w_hh, b_ih, b_hh, h_out, stream=None):
    lib = load_library()
    _check(lib.dt_gru_step(handle, _p(workspace), workspace.numel() if workspace is not None else 0,
                           _p(x), _p(h), _p(w_ih), _p(w_hh), _p(b_ih), _p(b_hh), _p(h_out),
                           _stream(stream)), handle)


def dt_correct(handle, idx, val, Cmat, h, pos, tok_sorted, logp_sorted, stream=None):
    lib = load_library()
    _check(lib.dt_correct(handle, _p(idx), _p(val), _p(Cmat), _p(h), _p(pos), _p(tok_sorted),
                          _p(logp_sorted), _stream(stream)), handle)


def dt_accept_greedy(handle, tokens, parents, count, target, path, accepted, bonus, stream=None):
    lib = load_library()
    _check(lib.dt_accept_greedy(handle, _p(tokens), _p(parents), _p(count), _p(target), _p(path),
                                _p(accepted), _p(bonus), _stream(stream)), handle)


def dt_timing_enable(handle, level: int, capacity: int):
    _check(load_library().dt_timing_enable(handle, int(level), int(capacity)), handle)


def dt_timing_read(handle, stage: int, max_items: int = 4096):
    buf = (C.c_float * max(1, max_items))()
    n = C.c_int(0)
    _check(load_library().dt_timing_read(handle, int(stage), buf, max_items, C.byref(n)), handle)
    return [buf[i] for i in range(min(n.value, max_items))]


# ---- convenience wrapper over torch tensors --------------------------------------

class Builder:
    """Owns a handle and its workspace; validates tensors before each call.

    Tensors must be on one CUDA (HIP) device, contiguous, and of the handle's
    dtype (torch.float32 or torch.bfloat16) where the C ABI says "dtype".
    """

    def __init__(self, B, L, V, E, H, M, n, temperature=0.0, dtype="bf16", near_tie_eps=1e-5,
                 device=None, full_vocab=False, expand=DT_EXPAND_AUTO):
        import torch
        self.cfg = dict(B=B, L=L, V=V, E=E, H=H, M=M, n=n, temperature=float(temperature),
                        near_tie_eps=float(near_tie_eps), full_vocab=bool(full_vocab), expand=int(expand))
        self.dtype_name = dtype
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.handle = dt_create(B, L, V, E, H, M, n, temperature,
                                DT_BF16 if dtype == "bf16" else DT_F32, near_tie_eps, full_vocab, expand)
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else device
        nbytes = dt_workspace_bytes(self.handle)
        self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=self.device)

    @property
    def fused(self) -> bool:
        """True when dt_build runs the fused expansion (per-step launches or the
        persistent launch) for this configuration."""
        return dt_expand_mode(self.handle) in (DT_EXPAND_FUSED, DT_EXPAND_PERSISTENT, DT_EXPAND_RESIDENT)

    @property
    def expand_mode(self) -> int:
        """dt_expand_mode of the handle: what the last build ran (before any,
        what the configuration selects)."""
        return dt_expand_mode(self.handle)

    def close(self):
        if getattr(self, "handle", None) is not None:
            dt_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _chk(self, name, t, shape, dtype=None, optional=False):
        if t is None:
            if optional:
                return
            raise ValueError(f"{name} is required")
        dtype = self.tdtype if dtype is None else dtype
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)} != expected {tuple(shape)}")
        if t.dtype != dtype:
            raise ValueError(f"{name}: dtype {t.dtype} != expected {dtype}")
        if t.device != self.device:
            raise ValueError(f"{name}: on {t.device}, expected {self.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    def build(self, base, emb, w_ih, w_hh, b_ih, b_hh, Cmat, h0=None, out=None, stream=None):
        import torch
        c = self.cfg
        B, L, V, E, H, n = c["B"], c["L"], c["V"], c["E"], c["H"], c["n"]
        self._chk("base", base, (B, L, V))
        self._chk("emb", emb, (V, E))
        self._chk("w_ih", w_ih, (3 * H, E))
        self._chk("w_hh", w_hh, (3 * H, H))
        self._chk("b_ih", b_ih, (3 * H,), optional=True)
        self._chk("b_hh", b_hh, (3 * H,), optional=True)
        self._chk("C", Cmat, (V, H))
        self._chk("h0", h0, (B, H), dtype=torch.float32, optional=True)
        if out is None:
            out = self._outputs()
        dt_build(self.handle, self.workspace, base, emb, w_ih, w_hh, b_ih, b_hh, Cmat, h0,
                 out["tokens"], out["parents"], out["depths"], out["scores"], out["mask"],
                 out["count"], out["flags"], stream)
        return out

    def _outputs(self):
        import torch
        B, S = self.cfg["B"], self.cfg["n"] + 1
        dev = self.device
        return dict(tokens=torch.empty((B, S), dtype=torch.int32, device=dev),
                    parents=torch.empty((B, S), dtype=torch.int32, device=dev),
                    depths=torch.empty((B, S), dtype=torch.int32, device=dev),
                    scores=torch.empty((B, S), dtype=torch.float32, device=dev),
                    mask=torch.empty((B, S, S), dtype=torch.uint8, device=dev),
                    count=torch.empty((B,), dtype=torch.int32, device=dev),
                    flags=torch.empty((B,), dtype=torch.uint32, device=dev))  # uint32 [B], as declared

    def fold_input(self, emb, w_ih, b_ih=None, stream=None):
        """The folded input projection table [V, 3H] float32 (b_ih + W_ih . emb[v])."""
        import torch
        c = self.cfg
        self._chk("emb", emb, (c["V"], c["E"]))
        self._chk("w_ih", w_ih, (3 * c["H"], c["E"]))
        self._chk("b_ih", b_ih, (3 * c["H"],), optional=True)
        table = torch.empty((c["V"], 3 * c["H"]), dtype=torch.float32, device=self.device)
        dt_fold_input(self.handle, emb, w_ih, b_ih, table, stream)
        return table

    def build_folded(self, base, table, w_hh, b_hh, Cmat, h0=None, out=None, stream=None):
        """dt_build with the folded input projection ``table`` (from fold_input)."""
        import torch
        c = self.cfg
        B, L, V, H = c["B"], c["L"], c["V"], c["H"]
        self._chk("base", base, (B, L, V))
        self._chk("table", table, (V, 3 * H), dtype=torch.float32)
        self._chk("w_hh", w_hh, (3 * H, H))
        self._chk("b_hh", b_hh, (3 * H,), optional=True)
        self._chk("C", Cmat, (V, H))
        self._chk("h0", h0, (B, H), dtype=torch.float32, optional=True)
        if out is None:
            out = self._outputs()
        dt_build_folded(self.handle, self.workspace, base, table, w_hh, b_hh, Cmat, h0, out["tokens"],
                        out["parents"], out["depths"], out["scores"], out["mask"], out["count"], out["flags"],
                        stream)
        return out

    def build_marginal(self, base, out=None, stream=None):
        """The factorized (marginal) scoring mode: dt_build with no GRU and no
        correction."""
        c = self.cfg
        self._chk("base", base, (c["B"], c["L"], c["V"]))
        if out is None:
            out = self._outputs()
        dt_build_marginal(self.handle, self.workspace, base, out["tokens"], out["parents"], out["depths"],
                          out["scores"], out["mask"], out["count"], out["flags"], stream)
        return out

    def topm(self, base, stream=None):
        import torch
        c = self.cfg
        self._chk("base", base, (c["B"], c["L"], c["V"]))
        idx = torch.empty((c["B"], c["L"], c["M"]), dtype=torch.int32, device=self.device)
        val = torch.empty((c["B"], c["L"], c["M"]), dtype=torch.float32, device=self.device)
        dt_topm(self.handle, self.workspace, base, idx, val, stream)
        return idx, val

    def topm_tail(self, base, stream=None):
        """Top-M tables and each row's tail_lse [B, L] (log sum of exp(x / T)
        over the logits outside the row's top M)."""
        import torch
        c = self.cfg
        self._chk("base", base, (c["B"], c["L"], c["V"]))
        idx = torch.empty((c["B"], c["L"], c["M"]), dtype=torch.int32, device=self.device)
        val = torch.empty((c["B"], c["L"], c["M"]), dtype=torch.float32, device=self.device)
        tail = torch.empty((c["B"], c["L"]), dtype=torch.float32, device=self.device)
        dt_topm_tail(self.handle, self.workspace, base, idx, val, tail, stream)
        return idx, val, tail

    def gru_step(self, x, h, w_ih, w_hh, b_ih=None, b_hh=None, stream=None):
        import torch
        c = self.cfg
        B, E, H = c["B"], c["E"], c["H"]
        self._chk("x", x, (B, E))
        self._chk("h", h, (B, H), dtype=torch.float32)
        self._chk("w_ih", w_ih, (3 * H, E))
        self._chk("w_hh", w_hh, (3 * H, H))
        self._chk("b_ih", b_ih, (3 * H,), optional=True)
        self._chk("b_hh", b_hh, (3 * H,), optional=True)
        h_out = torch.empty((B, H), dtype=torch.float32, device=self.device)
        dt_gru_step(self.handle, self.workspace, x, h, w_ih, w_hh, b_ih, b_hh, h_out, stream)
        return h_out

    def correct(self, idx, val, Cmat, h, pos, stream=None):
        import torch
        c = self.cfg
        B, L, M, H, V = c["B"], c["L"], c["M"], c["H"], c["V"]
        self._chk("idx", idx, (B, L, M), dtype=torch.int32)
        self._chk("val", val, (B, L, M), dtype=torch.float32)
        self._chk("C", Cmat, (V, H))
        self._chk("h", h, (B, H), dtype=torch.float32)
        self._chk("pos", pos, (B,), dtype=torch.int32)
        tok = torch.empty((B, M), dtype=torch.int32, device=self.device)
        lp = torch.empty((B, M), dtype=torch.float32, device=self.device)
        dt_correct(self.handle, idx, val, Cmat, h, pos, tok, lp, stream)
        return tok, lp

    def accept_greedy(self, tree, target, out=None, stream=None):
        """Greedy acceptance walk of the trees in ``tree`` (dt_build's outputs:
        tokens, parents, count) against the target's greedy tokens ``target``
        [B, n+1] int32.  Returns dict(path [B, n+1], accepted [B], bonus [B])
        (``out``, if given, is filled and returned)."""
        import torch
        B, S = self.cfg["B"], self.cfg["n"] + 1
        self._chk("tokens", tree["tokens"], (B, S), dtype=torch.int32)
        self._chk("parents", tree["parents"], (B, S), dtype=torch.int32)
        self._chk("count", tree["count"], (B,), dtype=torch.int32)
        self._chk("target", target, (B, S), dtype=torch.int32)
        dev = self.device
        res = out if out is not None else dict(path=torch.empty((B, S), dtype=torch.int32, device=dev),
                                               accepted=torch.empty((B,), dtype=torch.int32, device=dev),
                                               bonus=torch.empty((B,), dtype=torch.int32, device=dev))
        dt_accept_greedy(self.handle, tree["tokens"], tree["parents"], tree["count"], target, res["path"],
                         res["accepted"], res["bonus"], stream)
        return res

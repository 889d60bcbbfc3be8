"""ctypes binding of libdspark.so: argument marshalling only.

Each wrapper takes torch tensors that already live on the current GPU,
checks their shapes, types and contiguity on the host, and passes raw device
pointers and torch's current HIP stream to the C entry point of the same
name.  No step of the round runs in Python: if the library is missing the
import fails, and a non-zero status raises DSparkError.
"""

from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdspark.so")

F32, BF16 = 0, 1
CHUNK = 16   # tokens per chunk of the two-level Gumbel draw
WS_SAMPLE, WS_SCHEDULE, WS_VERIFY, WS_VERIFY_GREEDY, WS_ACCEPTANCE, WS_RNN_SAMPLE, WS_STS = 0, 2, 3, 4, 5, 6, 7
SCHED_EARLY_STOP, SCHED_WHOLE_WALK, SCHED_CAPACITY = 0, 1, 2

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "dspark_markov_sample": [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "dspark_markov_sample_ex": [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                _P, _P, _P, _P, _SZ, _P],
    "dspark_confidence": [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "dspark_schedule": [_I, _I, _P, _P, _I, _P, _P, _P, _P, _SZ, _P],
    "dspark_schedule_ex": [_I, _I, _P, _P, _I, _I, _P, _P, _P, _P, _P, _SZ, _P],
    "dspark_schedule_noalloc": [_I, _I, _P, _P, _I, _I, _P, _P, _P, _P, _P],
    "dspark_verify": [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                      _P, _SZ, _P],
    "dspark_verify_greedy": [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "dspark_acceptance": [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P],
    "dspark_verify_ex": [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                         _SZ, _P],
    "dspark_rnn_sample": [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                          _SZ, _P],
    "dspark_rnn_sample_ex": [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                             _P, _SZ, _P],
    "dspark_rnn_prepare": [_I, _I, _I, _I, _P, _P, _P, _P],
    "dspark_sts_fit": [_I, _I, _P, _P, _P, _I, _I, _P, _P, _P, _P, _P, _SZ, _P],
    "dspark_workspace_size": [_I, _I, _I, _I, _I, _I],
    "dspark_status_string": [_I],
    "dspark_markov_sample_kernel": [_I, _I, _I, _I, _I],
    "dspark_rnn_sample_kernel": [_I, _I, _I, _I, _I],
}
EXPORTED = tuple(_SIGNATURES)


class DSparkError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({dspark_status_string(status)})")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdspark.so (built by semi_ar_draft_round_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: run `python -m semi_ar_draft_round_amd.build` first")
    lib = ctypes.CDLL(path)
    for name, args in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.dspark_workspace_size.restype = ctypes.c_size_t
    lib.dspark_status_string.restype = ctypes.c_char_p
    lib.dspark_markov_sample_kernel.restype = ctypes.c_char_p
    lib.dspark_rnn_sample_kernel.restype = ctypes.c_char_p
    _lib = lib
    return lib


def dspark_status_string(status: int) -> str:
    return load_library().dspark_status_string(int(status)).decode()


def dspark_markov_sample_kernel(dtype: torch.dtype, R: int, gamma: int, V: int, r: int):
    """Which kernel the sampling call runs for this shape on the current
    device (None when the call would reject the shape)."""
    name = load_library().dspark_markov_sample_kernel(BF16 if dtype == torch.bfloat16 else F32,
                                                      R, gamma, V, r)
    return None if name is None else name.decode()


def dspark_rnn_sample_kernel(dtype: torch.dtype, R: int, gamma: int, V: int, r: int):
    """Which kernels the RNN-head sampling call runs for this shape on the
    current device (None when the call would reject the shape)."""
    name = load_library().dspark_rnn_sample_kernel(BF16 if dtype == torch.bfloat16 else F32, R, gamma, V, r)
    return None if name is None else name.decode()


def dspark_workspace_size(kind: int, R: int, gamma: int, V: int, r: int = 0, n_sps: int = 0) -> int:
    return int(load_library().dspark_workspace_size(kind, R, gamma, V, r, n_sps))


def _ptr(t) -> int | None:
    if t is None:
        return None
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(t, name, shape, dtypes, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _dt(t) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported storage dtype {t.dtype}")


def _raise(fn, st):
    if st != 0:
        raise DSparkError(fn, st)


_ws_cache: dict = {}


def workspace(kind: int, R: int, gamma: int, V: int, r: int, device) -> torch.Tensor:
    """A cached device workspace of the size the library asks for.

    One buffer serves every call of the same kind and shape on a device, so
    calls that may overlap (on different streams) must each pass a workspace
    of their own."""
    n = max(1, dspark_workspace_size(kind, R, gamma, V, r, 0))
    key = (kind, R, gamma, V, r, str(device))
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < n:
        ws = torch.empty(n, dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def dspark_markov_sample(U, W1, W2t, x0, G, g, x=None, lse=None, logit=None, ws=None):
    """x, lse, logit = sampled tokens, log-normalisers and logits, [R][gamma]."""
    lib = load_library()
    R, gamma, V = U.shape
    r = W1.shape[1]
    dev = U.device
    sdt = (U.dtype,)
    _check(U, "U", (R, gamma, V), sdt, dev)
    _check(W1, "W1", (V, r), sdt, dev)
    _check(W2t, "W2t", (V, r), sdt, dev)
    _check(x0, "x0", (R,), (torch.int32,), dev)
    _check(G, "G", (gamma, (V + CHUNK - 1) // CHUNK, R), (torch.float32,), dev)
    _check(g, "g", (R, gamma, CHUNK), (torch.float32,), dev)
    x = torch.empty((R, gamma), dtype=torch.int32, device=dev) if x is None else x
    lse = torch.empty((R, gamma), dtype=torch.float32, device=dev) if lse is None else lse
    logit = torch.empty((R, gamma), dtype=torch.float32, device=dev) if logit is None else logit
    _check(x, "x", (R, gamma), (torch.int32,), dev)
    _check(lse, "lse", (R, gamma), (torch.float32,), dev)
    _check(logit, "logit", (R, gamma), (torch.float32,), dev)
    ws = workspace(WS_SAMPLE, R, gamma, V, r, dev) if ws is None else ws
    st = lib.dspark_markov_sample(_dt(U), R, gamma, V, r, _ptr(U), _ptr(W1), _ptr(W2t), _ptr(x0),
                                  _ptr(G), _ptr(g), _ptr(x), _ptr(lse), _ptr(logit), _ptr(ws),
                                  ws.numel(), _stream())
    _raise("dspark_markov_sample", st)
    return x, lse, logit


def dspark_markov_sample_ex(U, W1, W2t, x0, G, g, h=None, w=None, T=None, x=None, lse=None, logit=None,
                            c=None, z=None, cancel=None, status=None, ws=None, timer=None):
    """dspark_markov_sample plus, when h and w are given, the confidence head
    on the drafted tokens.  cancel: an optional uint32/int32 [1] device word
    (non-zero ends the grid-barrier waits); status: an int32 [1] device word
    out (0 = ok, 6 = the grid barrier gave up); timer: a SweepTimer whose
    events record the position sweep.  Returns x, lse, logit, c, z, status
    (c and z None without h)."""
    lib = load_library()
    R, gamma, V = U.shape
    r = W1.shape[1]
    dev = U.device
    sdt = (U.dtype,)
    _check(U, "U", (R, gamma, V), sdt, dev)
    _check(W1, "W1", (V, r), sdt, dev)
    _check(W2t, "W2t", (V, r), sdt, dev)
    _check(x0, "x0", (R,), (torch.int32,), dev)
    _check(G, "G", (gamma, (V + CHUNK - 1) // CHUNK, R), (torch.float32,), dev)
    _check(g, "g", (R, gamma, CHUNK), (torch.float32,), dev)
    x = torch.empty((R, gamma), dtype=torch.int32, device=dev) if x is None else x
    lse = torch.empty((R, gamma), dtype=torch.float32, device=dev) if lse is None else lse
    logit = torch.empty((R, gamma), dtype=torch.float32, device=dev) if logit is None else logit
    _check(x, "x", (R, gamma), (torch.int32,), dev)
    _check(lse, "lse", (R, gamma), (torch.float32,), dev)
    _check(logit, "logit", (R, gamma), (torch.float32,), dev)
    d = 0
    if h is not None:
        d = h.shape[2]
        _check(h, "h", (R, gamma, d), sdt, dev)
        _check(w, "w", (d + r,), sdt, dev)
        if T is not None:
            _check(T, "T", (gamma,), (torch.float32,), dev)
        c = torch.empty((R, gamma), dtype=torch.float32, device=dev) if c is None else c
        _check(c, "c", (R, gamma), (torch.float32,), dev)
        if z is not None:
            _check(z, "z", (R, gamma), (torch.float32,), dev)
    else:
        c = z = None
    if cancel is not None:
        _check(cancel, "cancel", (1,), (torch.int32,), dev)
    status = torch.empty(1, dtype=torch.int32, device=dev) if status is None else status
    _check(status, "status", (1,), (torch.int32,), dev)
    ws = workspace(WS_SAMPLE, R, gamma, V, r, dev) if ws is None else ws
    st = lib.dspark_markov_sample_ex(_dt(U), R, gamma, V, r, d, _ptr(U), _ptr(W1), _ptr(W2t), _ptr(x0), _ptr(G),
                                     _ptr(g), _ptr(h), _ptr(w), _ptr(T), _ptr(x), _ptr(lse), _ptr(logit), _ptr(c),
                                     _ptr(z), _ptr(cancel), _ptr(status), None if timer is None else timer.pair,
                                     _ptr(ws), ws.numel(), _stream())
    _raise("dspark_markov_sample_ex", st)
    return x, lse, logit, c, z, status


class SweepTimer:
    """Two HIP events with timing enabled, made by the HIP runtime this
    process already has loaded, for dspark_markov_sample_ex's `events`."""

    def __init__(self):
        self._hip = ctypes.CDLL("libamdhip64.so.7")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.pair = (ctypes.c_void_p * 2)()
        for i in range(2):
            ev = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.pair[i] = ev.value

    def elapsed_ms(self) -> float:
        """Milliseconds between the two events of the last call (waits for it)."""
        if self._hip.hipEventSynchronize(self.pair[1]) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.pair[0], self.pair[1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        try:
            for i in range(2):
                if self.pair[i]:
                    self._hip.hipEventDestroy(self.pair[i])
        except Exception:
            pass


def dspark_confidence(h, w, W1, x0, x, T=None, c=None, z=None, want_z=True):
    """c (and z) [R][gamma]: sigmoid(w . [h_k ; W1[x_{k-1}]] / T_k)."""
    lib = load_library()
    R, gamma, d = h.shape
    V, r = W1.shape
    dev = h.device
    sdt = (h.dtype,)
    _check(h, "h", (R, gamma, d), sdt, dev)
    _check(w, "w", (d + r,), sdt, dev)
    _check(W1, "W1", (V, r), sdt, dev)
    _check(x0, "x0", (R,), (torch.int32,), dev)
    _check(x, "x", (R, gamma), (torch.int32,), dev)
    if T is not None:
        _check(T, "T", (gamma,), (torch.float32,), dev)
    c = torch.empty((R, gamma), dtype=torch.float32, device=dev) if c is None else c
    if want_z and z is None:
        z = torch.empty((R, gamma), dtype=torch.float32, device=dev)
    st = lib.dspark_confidence(_dt(h), R, gamma, d, r, V, _ptr(h), _ptr(w), _ptr(W1), _ptr(x0),
                               _ptr(x), _ptr(T), _ptr(c), _ptr(z), _stream())
    _raise("dspark_confidence", st)
    return c, z


def dspark_schedule(c, sps, ell=None, admitted=None, theta_best=None, ws=None):
    """ell [R] int32, admitted [1] int32, theta_best [1] float64 (Algorithm 1).
    ws: uint8 workspace of dspark_workspace_size(WS_SCHEDULE, R, gamma, 0) bytes
    (a cached one when None)."""
    lib = load_library()
    R, gamma = c.shape
    dev = c.device
    _check(c, "c", (R, gamma), (torch.float32,), dev)
    _check(sps, "sps", (sps.shape[0],), (torch.float64,), dev)
    ell = torch.empty(R, dtype=torch.int32, device=dev) if ell is None else ell
    admitted = torch.empty(1, dtype=torch.int32, device=dev) if admitted is None else admitted
    theta_best = torch.empty(1, dtype=torch.float64, device=dev) if theta_best is None else theta_best
    ws = workspace(WS_SCHEDULE, R, gamma, 0, 0, dev) if ws is None else ws
    st = lib.dspark_schedule(R, gamma, _ptr(c), _ptr(sps), int(sps.shape[0]), _ptr(ell), _ptr(admitted),
                             _ptr(theta_best), _ptr(ws), ws.numel(), _stream())
    _raise("dspark_schedule", st)
    return ell, admitted, theta_best


def dspark_schedule_ex(c, sps, mode, cap=None, ell=None, admitted=None, theta_best=None, ws=None):
    """The scheduler with an admission rule (SCHED_EARLY_STOP, SCHED_WHOLE_WALK
    or SCHED_CAPACITY; the last reads the capacity from the int32 [1] device
    tensor `cap`).  Returns ell [R] int32, admitted [1] int32, theta_best [1]
    float64.  ws as for dspark_schedule."""
    lib = load_library()
    R, gamma = c.shape
    dev = c.device
    _check(c, "c", (R, gamma), (torch.float32,), dev)
    _check(sps, "sps", (sps.shape[0],), (torch.float64,), dev)
    if cap is not None:
        _check(cap, "cap", (1,), (torch.int32,), dev)
    ell = torch.empty(R, dtype=torch.int32, device=dev) if ell is None else ell
    admitted = torch.empty(1, dtype=torch.int32, device=dev) if admitted is None else admitted
    theta_best = torch.empty(1, dtype=torch.float64, device=dev) if theta_best is None else theta_best
    ws = workspace(WS_SCHEDULE, R, gamma, 0, 0, dev) if ws is None else ws
    st = lib.dspark_schedule_ex(R, gamma, _ptr(c), _ptr(sps), int(sps.shape[0]), int(mode), _ptr(cap), _ptr(ell),
                                _ptr(admitted), _ptr(theta_best), _ptr(ws), ws.numel(), _stream())
    _raise("dspark_schedule_ex", st)
    return ell, admitted, theta_best


def dspark_schedule_noalloc(c, sps, mode, cap=None, ell=None, admitted=None, theta_best=None):
    """dspark_schedule_ex with the library's static device scratch instead of
    a workspace (for callers that cannot allocate).  Calls on one device must
    not overlap.  Returns ell [R] int32, admitted [1] int32, theta_best [1]
    float64."""
    lib = load_library()
    R, gamma = c.shape
    dev = c.device
    _check(c, "c", (R, gamma), (torch.float32,), dev)
    _check(sps, "sps", (sps.shape[0],), (torch.float64,), dev)
    if cap is not None:
        _check(cap, "cap", (1,), (torch.int32,), dev)
    ell = torch.empty(R, dtype=torch.int32, device=dev) if ell is None else ell
    admitted = torch.empty(1, dtype=torch.int32, device=dev) if admitted is None else admitted
    theta_best = torch.empty(1, dtype=torch.float64, device=dev) if theta_best is None else theta_best
    st = lib.dspark_schedule_noalloc(R, gamma, _ptr(c), _ptr(sps), int(sps.shape[0]), int(mode), _ptr(cap),
                                     _ptr(ell), _ptr(admitted), _ptr(theta_best), _stream())
    _raise("dspark_schedule_noalloc", st)
    return ell, admitted, theta_best


def dspark_verify(target, U, W1, W2t, x0, x, lse, logit, ell, u_acc, u_res, row0=None,
                  n_acc=None, next_tok=None, ws=None, bvec=None):
    """n_acc [R], next_tok [R] int32: rejection sampling with residual draw.
    bvec: the RNN head's bias vectors [R][gamma][r] (dspark_verify_ex)."""
    lib = load_library()
    R, gamma, V = U.shape
    r = W1.shape[1]
    dev = U.device
    sdt = (U.dtype,)
    if row0 is None:
        _check(target, "target", (R, gamma + 1, V), sdt, dev)
    else:
        _check(target, "target", (target.shape[0], V), sdt, dev)
        _check(row0, "row0", (R,), (torch.int32,), dev)
    _check(U, "U", (R, gamma, V), sdt, dev)
    _check(W1, "W1", (V, r), sdt, dev)
    _check(W2t, "W2t", (V, r), sdt, dev)
    _check(x0, "x0", (R,), (torch.int32,), dev)
    _check(x, "x", (R, gamma), (torch.int32,), dev)
    _check(lse, "lse", (R, gamma), (torch.float32,), dev)
    _check(logit, "logit", (R, gamma), (torch.float32,), dev)
    _check(ell, "ell", (R,), (torch.int32,), dev)
    _check(u_acc, "u_acc", (R, gamma), (torch.float32,), dev)
    _check(u_res, "u_res", (R,), (torch.float32,), dev)
    n_acc = torch.empty(R, dtype=torch.int32, device=dev) if n_acc is None else n_acc
    next_tok = torch.empty(R, dtype=torch.int32, device=dev) if next_tok is None else next_tok
    ws = workspace(WS_VERIFY, R, gamma, V, r, dev) if ws is None else ws
    if bvec is None:
        st = lib.dspark_verify(_dt(U), R, gamma, V, r, _ptr(target), _ptr(row0), _ptr(U), _ptr(W1),
                               _ptr(W2t), _ptr(x0), _ptr(x), _ptr(lse), _ptr(logit), _ptr(ell),
                               _ptr(u_acc), _ptr(u_res), _ptr(n_acc), _ptr(next_tok), _ptr(ws),
                               ws.numel(), _stream())
        _raise("dspark_verify", st)
    else:
        _check(bvec, "bvec", (R, gamma, r), sdt, dev)
        st = lib.dspark_verify_ex(_dt(U), R, gamma, V, r, _ptr(target), _ptr(row0), _ptr(U), _ptr(W1),
                                  _ptr(W2t), _ptr(bvec), _ptr(x0), _ptr(x), _ptr(lse), _ptr(logit), _ptr(ell),
                                  _ptr(u_acc), _ptr(u_res), _ptr(n_acc), _ptr(next_tok), _ptr(ws),
                                  ws.numel(), _stream())
        _raise("dspark_verify_ex", st)
    return n_acc, next_tok


def _target_check(target, row0, R, gamma, V, sdt, dev):
    if row0 is None:
        _check(target, "target", (R, gamma + 1, V), sdt, dev)
    else:
        _check(target, "target", (target.shape[0], V), sdt, dev)
        _check(row0, "row0", (R,), (torch.int32,), dev)


def dspark_verify_greedy(target, x, ell, row0=None, n_acc=None, next_tok=None, ws=None):
    """n_acc [R], next_tok [R] int32: temperature-0 (exact-match) verification."""
    lib = load_library()
    R, gamma = x.shape
    V = target.shape[-1]
    dev = x.device
    _target_check(target, row0, R, gamma, V, (torch.bfloat16, torch.float32), dev)
    _check(x, "x", (R, gamma), (torch.int32,), dev)
    _check(ell, "ell", (R,), (torch.int32,), dev)
    n_acc = torch.empty(R, dtype=torch.int32, device=dev) if n_acc is None else n_acc
    next_tok = torch.empty(R, dtype=torch.int32, device=dev) if next_tok is None else next_tok
    ws = workspace(WS_VERIFY_GREEDY, R, gamma, V, 0, dev) if ws is None else ws
    st = lib.dspark_verify_greedy(_dt(target), R, gamma, V, _ptr(target), _ptr(row0), _ptr(x), _ptr(ell),
                                  _ptr(n_acc), _ptr(next_tok), _ptr(ws), ws.numel(), _stream())
    _raise("dspark_verify_greedy", st)
    return n_acc, next_tok


def dspark_acceptance(target, U, W1, W2t, x0, x, lse, row0=None, c_star=None, ws=None, bvec=None):
    """c_star [R][gamma] f32: sum_v min(p_d, p_t) at every drafted position."""
    lib = load_library()
    R, gamma, V = U.shape
    r = W1.shape[1]
    dev = U.device
    sdt = (U.dtype,)
    _target_check(target, row0, R, gamma, V, sdt, dev)
    _check(U, "U", (R, gamma, V), sdt, dev)
    _check(W1, "W1", (V, r), sdt, dev)
    _check(W2t, "W2t", (V, r), sdt, dev)
    _check(x0, "x0", (R,), (torch.int32,), dev)
    _check(x, "x", (R, gamma), (torch.int32,), dev)
    _check(lse, "lse", (R, gamma), (torch.float32,), dev)
    c_star = torch.empty((R, gamma), dtype=torch.float32, device=dev) if c_star is None else c_star
    ws = workspace(WS_ACCEPTANCE, R, gamma, V, r, dev) if ws is None else ws
    if bvec is not None:
        _check(bvec, "bvec", (R, gamma, r), sdt, dev)
    st = lib.dspark_acceptance(_dt(U), R, gamma, V, r, _ptr(target), _ptr(row0), _ptr(U), _ptr(W1), _ptr(W2t),
                               _ptr(bvec), _ptr(x0), _ptr(x), _ptr(lse), _ptr(c_star), _ptr(ws), ws.numel(),
                               _stream())
    _raise("dspark_acceptance", st)
    return c_star


def dspark_rnn_prepare(W1, Wrnn, d, P=None):
    """P [V][3r] f32: the W1-row part of the RNN head's projection for every
    token (bf16 weights)."""
    lib = load_library()
    V, r = W1.shape
    dev = W1.device
    _check(W1, "W1", (V, r), (torch.bfloat16,), dev)
    _check(Wrnn, "Wrnn", (3 * r, 2 * r + d), (torch.bfloat16,), dev)
    P = torch.empty((V, 3 * r), dtype=torch.float32, device=dev) if P is None else P
    _check(P, "P", (V, 3 * r), (torch.float32,), dev)
    _raise("dspark_rnn_prepare", lib.dspark_rnn_prepare(BF16, V, r, d, _ptr(W1), _ptr(Wrnn), _ptr(P), _stream()))
    return P


def dspark_rnn_sample(U, W1, W2t, Wrnn, h, x0, G, g, x=None, lse=None, logit=None, s=None, o=None, ws=None,
                      P=None):
    """x [R][gamma] int32, lse and logit [R][gamma] f32, s [R][gamma][r] f32 (the
    states) and o [R][gamma][r] (the bias vectors): sampling with the RNN head
    (with P from dspark_rnn_prepare: dspark_rnn_sample_ex)."""
    lib = load_library()
    R, gamma, V = U.shape
    r = W1.shape[1]
    d = h.shape[2]
    dev = U.device
    sdt = (U.dtype,)
    nC = (V + CHUNK - 1) // CHUNK
    _check(U, "U", (R, gamma, V), sdt, dev)
    _check(W1, "W1", (V, r), sdt, dev)
    _check(W2t, "W2t", (V, r), sdt, dev)
    _check(Wrnn, "Wrnn", (3 * r, 2 * r + d), sdt, dev)
    _check(h, "h", (R, gamma, d), sdt, dev)
    _check(x0, "x0", (R,), (torch.int32,), dev)
    _check(G, "G", (gamma, nC, R), (torch.float32,), dev)
    _check(g, "g", (R, gamma, CHUNK), (torch.float32,), dev)
    x = torch.empty((R, gamma), dtype=torch.int32, device=dev) if x is None else x
    lse = torch.empty((R, gamma), dtype=torch.float32, device=dev) if lse is None else lse
    logit = torch.empty((R, gamma), dtype=torch.float32, device=dev) if logit is None else logit
    s = torch.empty((R, gamma, r), dtype=torch.float32, device=dev) if s is None else s
    o = torch.empty((R, gamma, r), dtype=U.dtype, device=dev) if o is None else o
    ws = workspace(WS_RNN_SAMPLE, R, gamma, V, r, dev) if ws is None else ws
    if P is None:
        st = lib.dspark_rnn_sample(_dt(U), R, gamma, V, r, d, _ptr(U), _ptr(W1), _ptr(W2t), _ptr(Wrnn), _ptr(h),
                                   _ptr(x0), _ptr(G), _ptr(g), _ptr(x), _ptr(lse), _ptr(logit), _ptr(s), _ptr(o),
                                   _ptr(ws), ws.numel(), _stream())
        _raise("dspark_rnn_sample", st)
    else:
        _check(P, "P", (V, 3 * r), (torch.float32,), dev)
        st = lib.dspark_rnn_sample_ex(_dt(U), R, gamma, V, r, d, _ptr(U), _ptr(W1), _ptr(W2t), _ptr(Wrnn),
                                      _ptr(h), _ptr(x0), _ptr(G), _ptr(g), _ptr(P), _ptr(x), _ptr(lse),
                                      _ptr(logit), _ptr(s), _ptr(o), _ptr(ws), ws.numel(), _stream())
        _raise("dspark_rnn_sample_ex", st)
    return x, lse, logit, s, o


def dspark_sts_fit(z, n_acc, grid, n_bins=15, ws=None):
    """Sequential temperature scaling on a held-out set: T [gamma] f32 and
    ece_before, ece_after, auc [gamma] f64."""
    lib = load_library()
    N, gamma = z.shape
    dev = z.device
    G = grid.shape[0]
    _check(z, "z", (N, gamma), (torch.float32,), dev)
    _check(n_acc, "n_acc", (N,), (torch.int32,), dev)
    _check(grid, "grid", (G,), (torch.float32,), dev)
    T = torch.empty(gamma, dtype=torch.float32, device=dev)
    e0 = torch.empty(gamma, dtype=torch.float64, device=dev)
    e1 = torch.empty(gamma, dtype=torch.float64, device=dev)
    auc = torch.empty(gamma, dtype=torch.float64, device=dev)
    ws = workspace(WS_STS, N, gamma, G, n_bins, dev) if ws is None else ws
    st = lib.dspark_sts_fit(N, gamma, _ptr(z), _ptr(n_acc), _ptr(grid), G, int(n_bins), _ptr(T), _ptr(e0), _ptr(e1),
                            _ptr(auc), _ptr(ws), ws.numel(), _stream())
    _raise("dspark_sts_fit", st)
    return T, e0, e1, auc


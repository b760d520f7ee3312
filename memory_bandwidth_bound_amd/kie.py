"""Python binding of libkie.so (include/kie.h): argument marshalling only.

Every step of decode runs in the library's HIP kernels. PyTorch is used only
to allocate the device workspace and to name the stream the library enqueues
on. If the shared library is missing this module raises at import of the
library: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_float, c_int32, c_size_t, c_void_p
from typing import Optional, Sequence

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkie.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kie.h")

KIE_OK = 0
STATUS = {0: "KIE_OK", -1: "KIE_ERR_ARG", -2: "KIE_ERR_CONFIG", -3: "KIE_ERR_CAPACITY",
          -4: "KIE_ERR_WORKSPACE", -5: "KIE_ERR_DEVICE", -6: "KIE_ERR_HIP", -7: "KIE_ERR_TIMEOUT",
          -8: "KIE_ERR_STATE"}


class KieConfig(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("d_model", c_int32), ("n_heads", c_int32),
                ("n_kv_heads", c_int32), ("head_dim", c_int32), ("ffn_dim", c_int32),
                ("vocab", c_int32), ("n_experts", c_int32), ("top_k", c_int32),
                ("rms_eps", c_float), ("rope_theta", c_float), ("max_seq", c_int32),
                ("weight_format", c_int32)]

WEIGHT_FORMATS = {"fp16": 0, "fp8": 1, "fp4": 2}


class KieDebug(ctypes.Structure):
    _fields_ = [("force_ids", POINTER(c_int32)), ("logits", POINTER(c_float)),
                ("experts", POINTER(c_int32)), ("trace", POINTER(ctypes.c_int64)),
                ("router", POINTER(c_float))]


class KieError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkie.so once. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m memory_bandwidth_bound_amd.build`")
    # torch ships its own HIP runtime: load it first so that the library binds
    # to that same runtime instead of a second copy from /opt/rocm
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    sig = {
        "kie_workspace_bytes": (c_size_t, [POINTER(KieConfig)]),
        "kie_tensor_count": (c_int32, [POINTER(KieConfig)]),
        "kie_phases_per_pass": (c_int32, [POINTER(KieConfig)]),
        "kie_load": (c_int32, [POINTER(KieConfig), POINTER(c_void_p), c_int32, c_void_p, c_size_t,
                               c_void_p, POINTER(c_void_p)]),
        "kie_prefill": (c_int32, [c_void_p, POINTER(c_int32), c_int32, POINTER(c_int32), POINTER(KieDebug)]),
        "kie_set_kv": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_int32]),
        "kie_decode": (c_int32, [c_void_p, c_int32, POINTER(c_int32), POINTER(KieDebug)]),
        "kie_rewind": (c_int32, [c_void_p, c_int32, c_int32]),
        "kie_reset": (c_int32, [c_void_p]),
        "kie_state": (c_int32, [c_void_p, POINTER(c_int32), POINTER(c_int32)]),
        "kie_last_kernel_ms": (c_float, [c_void_p]),
        "kie_grid_size": (c_int32, [c_void_p]),
        "kie_free": (None, [c_void_p]),
        "kie_set_limits": (c_int32, [c_void_p, ctypes.c_uint32, c_int32]),
        "kie_last_error": (ctypes.c_char_p, [c_void_p]),
        "kie_status_str": (ctypes.c_char_p, [c_int32]),
        "kie_gemv_probe": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                     c_void_p, POINTER(c_float)]),
        "kie_barrier_probe_bytes": (c_size_t, []),
        "kie_barrier_probe": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, POINTER(c_float), POINTER(c_int32)]),
        "kie_launch_probe": (c_int32, [c_int32, c_void_p, POINTER(c_float)]),
        "kie_barrier_probe_noalloc": (c_int32, [c_int32, c_int32, c_void_p, POINTER(c_float), POINTER(c_int32)]),
        "kie_xcd_map": (c_int32, [POINTER(c_int32), c_void_p]),
        "kie_set_prefill_mode": (c_int32, [c_void_p, c_int32]),
        "kie_set_attention_mode": (c_int32, [c_void_p, c_int32]),
        "kie_gemm_probe": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                     POINTER(c_float)]),
        "kie_e4m3_table_probe": (c_int32, [POINTER(c_float), c_void_p]),
        "kie_quantize_e4m3_rows": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_void_p, POINTER(c_float)]),
        "kie_quantize_e2m1_rows": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_void_p, POINTER(c_float)]),
        "kie_e2m1_table_probe": (c_int32, [POINTER(c_float), c_void_p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def header_symbols(path: str = HEADER):
    """Function names declared in include/kie.h."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kie_\w+)\s*\(", text)))


def make_config(cfg) -> KieConfig:
    """kie_config from a synth.DecoderConfig (or anything with the same fields)."""
    return KieConfig(cfg.n_layers, cfg.d_model, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim,
                     cfg.ffn_dim, cfg.vocab, cfg.n_experts, cfg.top_k if cfg.n_experts else 0,
                     cfg.rms_eps, cfg.rope_theta, cfg.max_seq,
                     WEIGHT_FORMATS[getattr(cfg, "weight_format", "fp16")])


def expected_shapes(cfg):
    """Shapes of kie_load's tensors in the canonical order include/kie.h
    documents (row-major [out][in] matrices, [d] gains)."""
    d, q, kv, f = cfg.d_model, cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim, cfg.ffn_dim
    shapes = [(cfg.vocab, d)]
    for _ in range(cfg.n_layers):
        shapes += [(d,), (q, d), (kv, d), (kv, d), (d, q), (d,)]
        if cfg.n_experts:
            shapes.append((cfg.n_experts, d))
            shapes += [(f, d), (f, d), (d, f)] * cfg.n_experts
        else:
            shapes += [(f, d), (f, d), (d, f)]
    return shapes + [(d,), (cfg.vocab, d)]


def check_tensors(cfg, tensors) -> None:
    """Raise KieError(KIE_ERR_ARG) unless ``tensors`` are fp16 arrays of the
    canonical shapes: the library reads exactly that many bytes from each."""
    want = expected_shapes(cfg)
    if len(tensors) != len(want):
        raise KieError(-1, f"expected {len(want)} tensors, got {len(tensors)}")
    for i, (t, s) in enumerate(zip(tensors, want)):
        if getattr(t, "dtype", None) != np.float16:
            raise KieError(-1, f"tensor {i}: dtype {getattr(t, 'dtype', type(t))}, expected float16")
        if tuple(t.shape) != s:
            raise KieError(-1, f"tensor {i}: shape {tuple(t.shape)}, expected {s}")


def check_kv(cfg, K, V) -> int:
    """Raise KieError(KIE_ERR_ARG) unless K and V are fp16 [n_layers][n_pos]
    [n_kv_heads][head_dim] of the same shape; returns n_pos."""
    for name, a in (("K", K), ("V", V)):
        if getattr(a, "dtype", None) != np.float16:
            raise KieError(-1, f"{name}: dtype {getattr(a, 'dtype', type(a))}, expected float16")
        if a.ndim != 4 or a.shape[0] != cfg.n_layers or a.shape[2:] != (cfg.n_kv_heads, cfg.head_dim):
            raise KieError(-1, f"{name}: shape {a.shape}, expected ({cfg.n_layers}, n_pos, "
                               f"{cfg.n_kv_heads}, {cfg.head_dim})")
    if K.shape != V.shape:
        raise KieError(-1, f"K shape {K.shape} != V shape {V.shape}")
    return int(K.shape[1])


def check_tokens(tokens, n: int, name: str) -> np.ndarray:
    """A 1-D int32 copy of at least n token ids (raises KieError otherwise)."""
    t = np.asarray(tokens)
    if t.ndim != 1 or (t.size and not np.issubdtype(t.dtype, np.integer)):
        raise KieError(-1, f"{name} must be a 1-D array of integer token ids")
    if t.size < n:
        raise KieError(-1, f"{name} holds {t.size} tokens, {n} needed")
    return np.ascontiguousarray(t[:n] if n else t, dtype=np.int32)


def workspace_bytes(cfg) -> int:
    return int(load_library().kie_workspace_bytes(ctypes.byref(make_config(cfg))))


def _check(code: int, model_ptr=None):
    if code != KIE_OK:
        msg = load_library().kie_last_error(model_ptr)
        raise KieError(code, msg.decode() if msg else "")


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(POINTER(c_int32))


def _stream_handle(torch, device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return c_void_p(s.cuda_stream)


class Model:
    """One loaded decoder: a device workspace plus the library's model handle."""

    def __init__(self, cfg, tensors: Sequence[np.ndarray], device: str = "cuda:0", stream=None):
        import torch
        lib = load_library()
        self.cfg = cfg
        self.device = torch.device(device)
        self._torch = torch
        kc = make_config(cfg)
        self._kc = kc
        nbytes = int(lib.kie_workspace_bytes(ctypes.byref(kc)))
        if nbytes == 0:
            raise KieError(-2, lib.kie_last_error(None).decode())
        n = int(lib.kie_tensor_count(ctypes.byref(kc)))
        if n != len(tensors):
            raise KieError(-1, f"expected {n} tensors, got {len(tensors)}")
        check_tensors(cfg, tensors)
        host = [np.ascontiguousarray(t) for t in tensors]
        ptrs = (c_void_p * n)(*[t.ctypes.data for t in host])
        with torch.cuda.device(self.device):
            self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            self._stream = stream
            handle = c_void_p()
            rc = lib.kie_load(ctypes.byref(kc), ptrs, n, c_void_p(self.workspace.data_ptr()), nbytes,
                              _stream_handle(torch, self.device, stream), ctypes.byref(handle))
        _check(rc)
        self._h = handle
        self._lib = lib

    # ---- calls -------------------------------------------------------------
    def _dbg(self, n, force, logits, experts, router=False):
        dbg = KieDebug()
        keep = {}
        if force is not None:
            f = check_tokens(force, n, "force")
            keep["force"] = f
            dbg.force_ids = _i32p(f)
        if logits:
            lg = np.zeros((n, self.cfg.vocab), dtype=np.float32)
            keep["logits"] = lg
            dbg.logits = lg.ctypes.data_as(POINTER(c_float))
        if experts:
            ex = np.zeros((n, self.cfg.n_layers, self.cfg.top_k), dtype=np.int32)
            keep["experts"] = ex
            dbg.experts = _i32p(ex)
        if router:
            rt = np.zeros((n, self.cfg.n_layers, self.cfg.n_experts), dtype=np.float32)
            keep["router"] = rt
            dbg.router = rt.ctypes.data_as(POINTER(c_float))
        return dbg, keep

    def prefill(self, tokens, logits: bool = False, experts: bool = False, router: bool = False):
        """Returns (first token, logits [n][vocab] or None, experts or None).
        With router=True the router logits [n][n_layers][n_experts] of the
        passes are left in ``last_router``."""
        t = check_tokens(tokens, 0, "tokens")
        first = c_int32()
        dbg, keep = self._dbg(len(t), None, logits, experts, router)
        with self._torch.cuda.device(self.device):
            rc = self._lib.kie_prefill(self._h, _i32p(t), len(t), ctypes.byref(first),
                                       ctypes.byref(dbg) if keep else None)
        _check(rc, self._h)
        self.last_router = keep.get("router")
        return first.value, keep.get("logits"), keep.get("experts")

    def decode(self, n: int, force=None, logits: bool = False, experts: bool = False, router: bool = False):
        """Returns (ids [n], logits [n][vocab] or None, experts or None).
        force, if given, must hold at least n tokens (the first n are used).
        With router=True the router logits [n][n_layers][n_experts] of the
        passes are left in ``last_router``."""
        out = np.zeros(max(int(n), 0), dtype=np.int32)
        dbg, keep = self._dbg(n, force, logits, experts, router)
        with self._torch.cuda.device(self.device):
            rc = self._lib.kie_decode(self._h, n, _i32p(out), ctypes.byref(dbg) if keep else None)
        _check(rc, self._h)
        self.last_router = keep.get("router")
        return out, keep.get("logits"), keep.get("experts")

    def trace_decode(self, n: int):
        """Decode n tokens recording the phase timeline of the launch.

        Returns (ids [n], trace int64 [phases][256][4]) where phases =
        min(n * phases_per_pass, 2048) and the 4 events per workgroup are the
        device clock (100 MHz ticks) at phase begin, input gathered, compute
        waves done, output published."""
        out = np.zeros(n, dtype=np.int32)
        pp = int(self._lib.kie_phases_per_pass(ctypes.byref(self._kc)))
        tr = np.zeros((2048, 256, 4), dtype=np.int64)
        dbg = KieDebug()
        dbg.trace = tr.ctypes.data_as(POINTER(ctypes.c_int64))
        with self._torch.cuda.device(self.device):
            rc = self._lib.kie_decode(self._h, n, _i32p(out), ctypes.byref(dbg))
        _check(rc, self._h)
        return out, tr[:min(n * pp, 2048)]

    def set_kv(self, K: np.ndarray, V: np.ndarray, pending: int):
        n_pos = check_kv(self.cfg, K, V)
        K = np.ascontiguousarray(K)
        V = np.ascontiguousarray(V)
        with self._torch.cuda.device(self.device):
            rc = self._lib.kie_set_kv(self._h, c_void_p(K.ctypes.data), c_void_p(V.ctypes.data),
                                      n_pos, int(pending))
        _check(rc, self._h)

    def set_prefill_mode(self, mode: str):
        """"auto" (batched on the matrix cores where supported) or "passes"
        (one decode pass per prompt token in one persistent launch)."""
        code = {"auto": 0, "passes": 1}[mode]
        _check(self._lib.kie_set_prefill_mode(self._h, code), self._h)

    def set_attention_mode(self, mode: str):
        """"global" (one workgroup of the grid per head-mode work item) or
        "xcd_local" (every XCD recomputes the attention its output-projection
        rows read, while the items fit one XCD's workgroups)."""
        code = {"global": 0, "xcd_local": 1}[mode]
        _check(self._lib.kie_set_attention_mode(self._h, code), self._h)

    def set_limits(self, spin_limit: int = 0, watchdog_ms: int = 0):
        """Device wait limit (polls; 0 = default) and host watchdog per launch
        (ms; 0 = automatic, negative = none) for later calls."""
        _check(self._lib.kie_set_limits(self._h, int(spin_limit), int(watchdog_ms)), self._h)

    def rewind(self, pos: int, pending: int):
        _check(self._lib.kie_rewind(self._h, int(pos), int(pending)), self._h)

    def reset(self):
        with self._torch.cuda.device(self.device):
            _check(self._lib.kie_reset(self._h), self._h)

    def state(self):
        p, t = c_int32(), c_int32()
        _check(self._lib.kie_state(self._h, ctypes.byref(p), ctypes.byref(t)), self._h)
        return p.value, t.value

    @property
    def last_kernel_ms(self) -> float:
        return float(self._lib.kie_last_kernel_ms(self._h))

    @property
    def grid_size(self) -> int:
        return int(self._lib.kie_grid_size(self._h))

    def close(self):
        if getattr(self, "_h", None):
            self._lib.kie_free(self._h)
            self._h = None
            self.workspace = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---- probes -----------------------------------------------------------------

def gemv_probe(A, x, variant: int = 0, stream=None):
    """y[c] = A[c] @ x for a device fp16 tensor A [copies, M, K] and x [K].

    Returns (y float32 [copies, M], device milliseconds of the one launch).
    """
    import torch
    lib = load_library()
    assert A.dtype == torch.float16 and x.dtype == torch.float16 and A.is_cuda and x.is_cuda
    A = A.contiguous()
    x = x.contiguous()
    copies, M, K = A.shape
    y = torch.empty((copies, M), dtype=torch.float32, device=A.device)
    ms = c_float()
    with torch.cuda.device(A.device):
        rc = lib.kie_gemv_probe(c_void_p(A.data_ptr()), c_void_p(x.data_ptr()), c_void_p(y.data_ptr()),
                                M, K, copies, variant, _stream_handle(torch, A.device, stream),
                                ctypes.byref(ms))
    _check(rc)
    return y, float(ms.value)


def barrier_probe(rounds: int, variant: int = 1, device: str = "cuda:0"):
    """Mean microseconds per exchange round across the 256-workgroup grid
    (variant 0: fenced grid barrier; 1: flagged-word all-gather of 5 words per
    workgroup; 2: XCD-aware barrier), and the count of wrong values (0 when
    correct)."""
    import torch
    lib = load_library()
    scratch = torch.zeros(int(lib.kie_barrier_probe_bytes()), dtype=torch.uint8, device=device)
    us, err = c_float(), c_int32()
    with torch.cuda.device(scratch.device):
        rc = lib.kie_barrier_probe(c_void_p(scratch.data_ptr()), variant, rounds,
                                   _stream_handle(torch, scratch.device, None), ctypes.byref(us),
                                   ctypes.byref(err))
    _check(rc)
    return float(us.value), int(err.value)


def barrier_probe_noalloc(rounds: int, variant: int = 1, device: str = "cuda:0"):
    """kie_barrier_probe without a caller workspace: the library's own scratch
    array. Returns (host-timed microseconds per round, wrong values)."""
    import torch
    lib = load_library()
    us, err = c_float(), c_int32()
    dev = torch.device(device)
    with torch.cuda.device(dev):
        rc = lib.kie_barrier_probe_noalloc(variant, rounds, _stream_handle(torch, dev, None), ctypes.byref(us),
                                           ctypes.byref(err))
    _check(rc)
    return float(us.value), int(err.value)


def quantize_e4m3_rows(W: np.ndarray, gain: Optional[np.ndarray] = None):
    """The library's host FP8 quantizer (kie_quantize_e4m3_rows) on fp16 W
    [rows][K] with an optional fp16 gain [K]: returns (codes uint8, scales f32)."""
    lib = load_library()
    W = np.ascontiguousarray(W, dtype=np.float16)
    if W.ndim != 2:
        raise KieError(-1, "W must be [rows][K]")
    g = None if gain is None else np.ascontiguousarray(gain, dtype=np.float16)
    if g is not None and g.shape != (W.shape[1],):
        raise KieError(-1, "gain must be [K]")
    q = np.zeros(W.shape, dtype=np.uint8)
    s = np.zeros(W.shape[0], dtype=np.float32)
    _check(lib.kie_quantize_e4m3_rows(c_void_p(W.ctypes.data), None if g is None else c_void_p(g.ctypes.data),
                                      W.shape[0], W.shape[1], c_void_p(q.ctypes.data),
                                      s.ctypes.data_as(POINTER(c_float))))
    return q, s


def quantize_e2m1_rows(W: np.ndarray, gain: Optional[np.ndarray] = None):
    """The library's host FP4 quantizer (kie_quantize_e2m1_rows) on fp16 W
    [rows][K] with an optional fp16 gain [K]: returns (codes uint8 0..15, scales f32)."""
    lib = load_library()
    W = np.ascontiguousarray(W, dtype=np.float16)
    if W.ndim != 2:
        raise KieError(-1, "W must be [rows][K]")
    g = None if gain is None else np.ascontiguousarray(gain, dtype=np.float16)
    if g is not None and g.shape != (W.shape[1],):
        raise KieError(-1, "gain must be [K]")
    q = np.zeros(W.shape, dtype=np.uint8)
    s = np.zeros(W.shape[0], dtype=np.float32)
    _check(lib.kie_quantize_e2m1_rows(c_void_p(W.ctypes.data), None if g is None else c_void_p(g.ctypes.data),
                                      W.shape[0], W.shape[1], c_void_p(q.ctypes.data),
                                      s.ctypes.data_as(POINTER(c_float))))
    return q, s


def gemm_probe(A, W, stream=None):
    """Y = A @ W.T on the matrix cores for device tensors A float32 [n, K] and
    W float16 [M, K]; returns (Y float32 [n, M], device milliseconds)."""
    import torch
    lib = load_library()
    assert A.dtype == torch.float32 and W.dtype == torch.float16 and A.is_cuda and W.is_cuda
    A = A.contiguous()
    W = W.contiguous()
    n, K = A.shape
    M, K2 = W.shape
    if K2 != K:
        raise KieError(-1, "A and W must share K")
    Y = torch.empty((n, M), dtype=torch.float32, device=A.device)
    ms = c_float()
    with torch.cuda.device(A.device):
        rc = lib.kie_gemm_probe(c_void_p(A.data_ptr()), c_void_p(W.data_ptr()), c_void_p(Y.data_ptr()), n, M, K,
                                _stream_handle(torch, A.device, stream), ctypes.byref(ms))
    _check(rc)
    return Y, float(ms.value)


def e4m3_table_probe(device: str = "cuda:0"):
    """The fp32 values the device's E4M3 conversion gives codes 0..255."""
    import torch
    lib = load_library()
    out = np.zeros(256, dtype=np.float32)
    dev = torch.device(device)
    with torch.cuda.device(dev):
        rc = lib.kie_e4m3_table_probe(out.ctypes.data_as(POINTER(c_float)), _stream_handle(torch, dev, None))
    _check(rc)
    return out


def e2m1_table_probe(device: str = "cuda:0"):
    """What the device's E2M1 conversion gives for eight words: [8][4][2]
    values, word l's byte b holding the codes (2l + b) % 16 (low nibble) and
    (2l + b + 8) % 16 (high nibble)."""
    import torch
    lib = load_library()
    out = np.zeros(64, dtype=np.float32)
    dev = torch.device(device)
    with torch.cuda.device(dev):
        rc = lib.kie_e2m1_table_probe(out.ctypes.data_as(POINTER(c_float)), _stream_handle(torch, dev, None))
    _check(rc)
    return out.reshape(8, 4, 2)


def xcd_map(device: str = "cuda:0"):
    """The XCD each of the 256 workgroups of a cooperative launch runs on."""
    import torch
    lib = load_library()
    out = np.zeros(256, dtype=np.int32)
    dev = torch.device(device)
    with torch.cuda.device(dev):
        rc = lib.kie_xcd_map(_i32p(out), _stream_handle(torch, dev, None))
    _check(rc)
    return out


def launch_probe(launches: int, device: str = "cuda:0"):
    """Host wall-clock microseconds per back-to-back launch of an empty kernel."""
    import torch
    lib = load_library()
    us = c_float()
    dev = torch.device(device)
    with torch.cuda.device(dev):
        rc = lib.kie_launch_probe(launches, _stream_handle(torch, dev, None), ctypes.byref(us))
    _check(rc)
    return float(us.value)

"""Python binding of libtq.so, the TurboQuant packed-KV library for MI355X (gfx950).

Argument marshalling only: every step of quantization and decode attention runs
in the library's HIP kernels. PyTorch provides device memory and the stream.
The names follow the C ABI in include/tq.h:

    make_codebook(bits)                        -> (centroids, thresholds)   host
    make_rotation(seed, kind=HAAR, d=128)      -> float32 [d, d]            host
    quantize_kv(x, cache, t_offset=0)          x: [B, T, H_kv, d] on the GPU
    dequantize(cache, t0, t1)                  -> float32 [B, H_kv, t1-t0, d]
    decode_attention(k, v, q, ...)             -> float32 [B, H_q, d]

d (the head dimension) is 128, 64 or 256; QJL keys take d = 128 only.
    decode_workspace_bytes(...), decode_splits(...), status_string(code)

Cache bundles the device buffers of one packed cache (keys or values) with its
rotation, QJL projection and codebook.

If libtq.so is missing the import fails: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
# torch is loaded before libtq.so so that the process holds one HIP runtime:
# torch brings its own copy of libamdhip64, and libtq.so then binds to it. The
# other order loads a second runtime beside torch's, and the two do not share
# the device.
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python decode_attention_tq_amd/build.py` "
        "(hipcc for gfx950); this package has no CPU fallback")

_lib = ctypes.CDLL(LIB_PATH)

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_ALIGNMENT, ERR_WORKSPACE_TOO_SMALL, ERR_DEVICE = range(6)
F32, BF16 = 0, 1
HAAR, GAUSSIAN, HADAMARD = 0, 1, 2
KEYS, VALUES = 0, 1
D = 128
HEAD_DIMS = (64, 128, 256)
VALUE_BLOCK = 8

EXPORTS = ("tq_make_codebook", "tq_make_codebook_sphere", "tq_make_rotation", "tq_quantize_kv", "tq_append_kv",
           "tq_dequantize",
           "tq_decode_attention", "tq_decode_attention_noalloc", "tq_decode_attention_append", "tq_prefill_attention",
           "tq_decode_splits", "tq_decode_workspace_bytes",
           "tq_prefill_workspace_bytes", "tq_stream_read", "tq_status_string",
           "tq_last_hip_error")


class TQCache(ctypes.Structure):
    _fields_ = [
        ("role", ctypes.c_int32), ("bits", ctypes.c_int32), ("qjl", ctypes.c_int32), ("d", ctypes.c_int32),
        ("B", ctypes.c_int64), ("H_kv", ctypes.c_int64), ("T_cap", ctypes.c_int64),
        ("codes", ctypes.c_void_p), ("norms", ctypes.c_void_p),
        ("qjl_signs", ctypes.c_void_p), ("qjl_gamma", ctypes.c_void_p),
        ("rot", ctypes.c_void_p), ("qjl_proj", ctypes.c_void_p),
        ("centroids", ctypes.c_float * 16),
        ("block_table", ctypes.c_void_p), ("block_tokens", ctypes.c_int64), ("n_blocks", ctypes.c_int64),
    ]


_P = ctypes.c_void_p
_I32, _I64, _U64, _F = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float


def _bind(lib):
    """Declare the C-ABI signatures on a loaded libtq."""
    lib.tq_make_codebook.argtypes = [_I32, _I32, _P, _P]
    lib.tq_make_codebook_sphere.argtypes = [_I32, _I32, _P, _P]
    lib.tq_make_rotation.argtypes = [_U64, _I32, _I32, _P]
    lib.tq_quantize_kv.argtypes = [_P, _I32, _I64, _I64, _I64, _I64, _I64, _I64, ctypes.POINTER(TQCache), _I64, _P]
    lib.tq_append_kv.argtypes = [_P, _P, _I32, _I64, _I64, _I64, _I64, _I64, _I64, ctypes.POINTER(TQCache),
                                 ctypes.POINTER(TQCache), _I64, _P]
    lib.tq_dequantize.argtypes = [ctypes.POINTER(TQCache), _I64, _I64, _P, _P]
    lib.tq_decode_attention.argtypes = [ctypes.POINTER(TQCache), ctypes.POINTER(TQCache), _P, _I32, _I64, _P,
                                        _I64, _F, _I32, _P, _P, ctypes.c_size_t, _P]
    lib.tq_decode_attention_noalloc.argtypes = [ctypes.POINTER(TQCache), ctypes.POINTER(TQCache), _P, _I32, _I64,
                                                _P, _I64, _F, _I32, _P, _P]
    lib.tq_decode_attention_append.argtypes = [ctypes.POINTER(TQCache), ctypes.POINTER(TQCache), _P, _P, _I32, _I64,
                                               _I64, _I64, _I64, _P, _I32, _I64, _P, _I64, _F, _I32, _P, _P,
                                               ctypes.c_size_t, _P]
    lib.tq_prefill_attention.argtypes = [ctypes.POINTER(TQCache), ctypes.POINTER(TQCache), _P, _I32, _I64, _I64,
                                         _P, _I64, _F, _I32, _P, _P, ctypes.c_size_t, _P]
    lib.tq_prefill_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, _I64, _I32, _I32]
    lib.tq_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.tq_decode_splits.argtypes = [_I64, _I64, _I64, _I32]
    lib.tq_decode_splits.restype = _I32
    lib.tq_decode_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, _I32, _I32]
    lib.tq_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.tq_stream_read.argtypes = [_P, ctypes.c_size_t, _P, _I32, _P]
    lib.tq_stream_read.restype = ctypes.c_int
    lib.tq_status_string.argtypes = [ctypes.c_int]
    lib.tq_status_string.restype = ctypes.c_char_p
    lib.tq_last_hip_error.argtypes = []
    lib.tq_last_hip_error.restype = ctypes.c_char_p
    for name in ("tq_make_codebook", "tq_make_codebook_sphere", "tq_make_rotation", "tq_quantize_kv", "tq_append_kv",
                 "tq_dequantize", "tq_decode_attention", "tq_decode_attention_noalloc", "tq_decode_attention_append",
                 "tq_prefill_attention"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


_bind(_lib)


class TQError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


def lib():
    """The loaded ctypes library (for tests that call the C ABI directly)."""
    return _lib


def status_string(status: int) -> str:
    return _lib.tq_status_string(status).decode()


def _check(status: int, what: str):
    if status != OK:
        if status == ERR_DEVICE:
            what = f"{what} [{_lib.tq_last_hip_error().decode()}]"
        raise TQError(status, what)


# ------------------------------------------------------------------ host ----

def make_codebook(bits: int, d: int = D):
    """Gaussian Lloyd-Max codebook: (centroids float32 [2^bits], thresholds float32 [2^bits - 1])."""
    L = 1 << bits
    c = np.zeros(L, dtype=np.float32)
    t = np.zeros(max(L - 1, 1), dtype=np.float32)
    _check(_lib.tq_make_codebook(bits, d, c.ctypes.data, t.ctypes.data), "tq_make_codebook")
    return c, t[:L - 1]


def make_codebook_sphere(bits: int, d: int = D):
    """Sphere-exact Lloyd-Max codebook (law of one coordinate of a uniform unit
    vector in d dimensions): (centroids float32 [2^bits], thresholds float32 [2^bits - 1])."""
    L = 1 << bits
    c = np.zeros(L, dtype=np.float32)
    t = np.zeros(max(L - 1, 1), dtype=np.float32)
    _check(_lib.tq_make_codebook_sphere(bits, d, c.ctypes.data, t.ctypes.data), "tq_make_codebook_sphere")
    return c, t[:L - 1]


def make_rotation(seed: int, kind: int = HAAR, d: int = D) -> np.ndarray:
    """Seeded d x d float32 matrix (HAAR rotation Pi, HADAMARD randomized Hadamard
    rotation, or GAUSSIAN projection S)."""
    out = np.zeros((d, d), dtype=np.float32)
    _check(_lib.tq_make_rotation(seed & 0xFFFFFFFFFFFFFFFF, d, kind, out.ctypes.data), "tq_make_rotation")
    return out


def decode_splits(B: int, H_kv: int, T: int, n_split: int = 0) -> int:
    return int(_lib.tq_decode_splits(B, H_kv, T, n_split))


def decode_workspace_bytes(B: int, H_q: int, H_kv: int, T: int, n_split: int = 0, k_qjl: int = 0) -> int:
    return int(_lib.tq_decode_workspace_bytes(B, H_q, H_kv, T, n_split, k_qjl))


def prefill_workspace_bytes(B: int, H_q: int, H_kv: int, M: int, T: int, n_split: int = 0, k_qjl: int = 0) -> int:
    return int(_lib.tq_prefill_workspace_bytes(B, H_q, H_kv, M, T, n_split, k_qjl))


# ---------------------------------------------------------------- device ----

def _torch():
    import torch
    return torch


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


class Cache:
    """Device buffers of one packed cache (keys or values of one layer).

    Contiguous layout (block_table None):
      codes  int32 words [B, H_kv, T_cap * d * bits / 32] (layout set by `role`)
      norms  float32 [B, H_kv, T_cap]
      signs  int32 [B, H_kv, T_cap, d/32] and gamma float32 [B, H_kv, T_cap] for QJL keys
    Paged layout (block_table int32 [B, T_cap / block_tokens] on the device,
    entries in [0, n_blocks)): the same arrays with [n_blocks, H_kv, block_tokens ...]
    in place of [B, H_kv, T_cap ...].
    rot    float32 [d, d] (Pi), proj float32 [d, d] (S, QJL keys), centroids (host)
    """

    def __init__(self, role: int, bits: int, B: int, H_kv: int, T_cap: int, device="cuda",
                 rot=None, proj=None, qjl: bool = False, centroids=None, rot_seed: int = 42,
                 qjl_seed: int = 4242, block_table=None, block_tokens: int = 0, n_blocks: int = 0,
                 d: int = D):
        torch = _torch()
        if d not in HEAD_DIMS:
            raise ValueError(f"head dimension d must be one of {HEAD_DIMS}")
        self.role, self.bits, self.qjl = role, bits, int(bool(qjl))
        self.B, self.H_kv, self.T_cap, self.d = B, H_kv, T_cap, d
        self.device = torch.device(device)
        self.block_table = block_table
        self.block_tokens, self.n_blocks = int(block_tokens), int(n_blocks)
        if block_table is not None:
            if block_table.dtype != torch.int32 or tuple(block_table.shape) != (B, T_cap // max(block_tokens, 1)):
                raise ValueError("block_table must be int32 [B, T_cap / block_tokens]")
            lead, per = (n_blocks, H_kv), block_tokens
        else:
            lead, per = (B, H_kv), T_cap
        W = d * bits // 32
        self.codes = torch.zeros((*lead, per * W), dtype=torch.int32, device=self.device)
        self.norms = torch.zeros((*lead, per), dtype=torch.float32, device=self.device)
        if rot is None:
            rot = make_rotation(rot_seed, HAAR, d)
        self.rot = torch.as_tensor(np.asarray(rot, dtype=np.float32)).to(self.device).contiguous()
        if self.qjl:
            if proj is None:
                proj = make_rotation(qjl_seed, GAUSSIAN, d)
            self.proj = torch.as_tensor(np.asarray(proj, dtype=np.float32)).to(self.device).contiguous()
            self.signs = torch.zeros((*lead, per, d // 32), dtype=torch.int32, device=self.device)
            self.gamma = torch.zeros((*lead, per), dtype=torch.float32, device=self.device)
        else:
            self.proj = self.signs = self.gamma = None
        if centroids is None:
            centroids, _ = make_codebook(bits, d)
        self.centroids = np.asarray(centroids, dtype=np.float32)

    def __setattr__(self, name, value):
        # any change of an attribute drops the cached C struct
        object.__setattr__(self, name, value)
        if name != "_struct":
            object.__setattr__(self, "_struct", None)

    def struct(self) -> TQCache:
        """The tq_cache struct of this cache (built once, rebuilt after an
        attribute is reassigned; in-place edits of the centroids array need a
        reassignment to be seen)."""
        s = self.__dict__.get("_struct")
        if s is None:
            s = self._make_struct()
            object.__setattr__(self, "_struct", s)
        return s

    def _make_struct(self) -> TQCache:
        s = TQCache()
        s.role, s.bits, s.qjl, s.d = self.role, self.bits, self.qjl, self.d
        s.B, s.H_kv, s.T_cap = self.B, self.H_kv, self.T_cap
        s.codes = self.codes.data_ptr()
        s.norms = self.norms.data_ptr()
        s.qjl_signs = self.signs.data_ptr() if self.qjl else None
        s.qjl_gamma = self.gamma.data_ptr() if self.qjl else None
        s.rot = self.rot.data_ptr()
        s.qjl_proj = self.proj.data_ptr() if self.qjl else None
        for i, c in enumerate(self.centroids):
            s.centroids[i] = float(c)
        if self.block_table is not None:
            s.block_table = self.block_table.data_ptr()
            s.block_tokens, s.n_blocks = self.block_tokens, self.n_blocks
        return s

    @property
    def nbytes(self) -> int:
        n = self.codes.numel() * 4 + self.norms.numel() * 4
        if self.qjl:
            n += self.signs.numel() * 4 + self.gamma.numel() * 4
        return n


def quantize_kv(x, cache: Cache, t_offset: int = 0):
    """Quantize x [B, T, H_kv, d] (float32 or bfloat16, last dim contiguous, on the
    cache's device) into tokens t_offset .. t_offset+T-1 of `cache`."""
    if x.dim() != 4 or x.shape[-1] != cache.d or x.stride(-1) != 1:
        raise ValueError(f"x must be [B, T, H_kv, {cache.d}] with a contiguous last dimension")
    B, T, H, _ = x.shape
    s = cache.struct()
    _check(_lib.tq_quantize_kv(x.data_ptr(), _dtype_code(x), B, T, H, x.stride(0), x.stride(1), x.stride(2),
                               ctypes.byref(s), t_offset, _stream_handle(x.device)), "tq_quantize_kv")


def append_kv(k, v, kcache: Cache, vcache: Cache, t_offset: int):
    """The key and value of one new token per (row, head): k, v [B, H_kv, d]
    (or [B, 1, H_kv, d]), float32 or bfloat16, last dim contiguous, into token
    t_offset of kcache and vcache in one call (tq_append_kv)."""
    if k.dim() == 4:
        k = k[:, 0]
    if v.dim() == 4:
        v = v[:, 0]
    if (k.dim() != 3 or v.dim() != 3 or k.shape != v.shape or k.shape[-1] != kcache.d or k.stride(-1) != 1
            or v.stride(-1) != 1):
        raise ValueError(f"k and v must be [B, H_kv, {kcache.d}] with a contiguous last dimension")
    if k.dtype != v.dtype:
        raise ValueError("k and v must have the same dtype")
    B, H, _ = k.shape
    sk, sv = kcache.struct(), vcache.struct()
    _check(_lib.tq_append_kv(k.data_ptr(), v.data_ptr(), _dtype_code(k), B, H, k.stride(0), k.stride(1), v.stride(0),
                             v.stride(1), ctypes.byref(sk), ctypes.byref(sv), t_offset, _stream_handle(k.device)),
           "tq_append_kv")


def dequantize(cache: Cache, t0: int = 0, t1: int | None = None, out=None):
    torch = _torch()
    t1 = cache.T_cap if t1 is None else t1
    if out is None:
        out = torch.empty((cache.B, cache.H_kv, t1 - t0, cache.d), dtype=torch.float32, device=cache.device)
    s = cache.struct()
    _check(_lib.tq_dequantize(ctypes.byref(s), t0, t1, out.data_ptr(), _stream_handle(cache.device)),
           "tq_dequantize")
    return out


def stream_read(buf, workgroups: int = 0, sink=None):
    """Read the device tensor `buf` once with the library's plain streaming-read
    kernel (a measurement reference, not part of the method); returns the sink
    tensor of one XOR-folded word per workgroup (0 workgroups: 8 per compute unit)."""
    torch = _torch()
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    if workgroups <= 0:
        workgroups = 8 * torch.cuda.get_device_properties(buf.device).multi_processor_count
    if sink is None or sink.numel() < workgroups:
        sink = torch.empty(workgroups, dtype=torch.int32, device=buf.device)
    _check(_lib.tq_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), workgroups,
                               _stream_handle(buf.device)), "tq_stream_read")
    return sink


class Workspace:
    """Reusable device workspace for decode_attention."""

    def __init__(self, nbytes: int, device="cuda"):
        torch = _torch()
        self.buf = torch.empty(max(nbytes, 256) + 256, dtype=torch.uint8, device=device)
        base = self.buf.data_ptr()
        self.ptr = (base + 255) & ~255
        self.nbytes = self.buf.numel() - (self.ptr - base)


def decode_attention(k: Cache, v: Cache, q, ctx_lens=None, T: int | None = None, scale: float = 0.0,
                     n_split: int = 0, out=None, workspace: Workspace | None = None):
    """Decode attention of q [B, H_q, d] over the packed caches -> float32 [B, H_q, d]."""
    torch = _torch()
    if q.dim() != 3 or q.shape[-1] != k.d or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous [B, H_q, {k.d}] tensor")
    B, H_q, _ = q.shape
    T = k.T_cap if T is None else T
    if out is None:
        out = torch.empty((B, H_q, k.d), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, H_q, k.H_kv, T, n_split, k.qjl)
    if workspace is None or workspace.nbytes < need:
        workspace = Workspace(need, q.device)
    sk, sv = k.struct(), v.struct()
    cl = 0
    if ctx_lens is not None:
        if ctx_lens.dtype != torch.int32 or not ctx_lens.is_contiguous() or ctx_lens.numel() != B:
            raise ValueError("ctx_lens must be a contiguous int32 tensor of B entries")
        cl = ctx_lens.data_ptr()
    _check(_lib.tq_decode_attention(ctypes.byref(sk), ctypes.byref(sv), q.data_ptr(), _dtype_code(q), H_q,
                                    cl or None, T, scale, n_split, out.data_ptr(), workspace.ptr,
                                    workspace.nbytes, _stream_handle(q.device)), "tq_decode_attention")
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20


def decode_attention_noalloc(k: Cache, v: Cache, q, ctx_lens=None, T: int | None = None, scale: float = 0.0,
                             n_split: int = 0, out=None):
    """decode_attention without a workspace: the chunk partials live in the
    library's static per-GPU scratch (tq_decode_attention_noalloc). Pass `out`
    to allocate nothing at all; calls that overlap on one GPU race."""
    torch = _torch()
    if q.dim() != 3 or q.shape[-1] != k.d or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous [B, H_q, {k.d}] tensor")
    B, H_q, _ = q.shape
    T = k.T_cap if T is None else T
    if out is None:
        out = torch.empty((B, H_q, k.d), dtype=torch.float32, device=q.device)
    sk, sv = k.struct(), v.struct()
    cl = 0
    if ctx_lens is not None:
        if ctx_lens.dtype != torch.int32 or not ctx_lens.is_contiguous() or ctx_lens.numel() != B:
            raise ValueError("ctx_lens must be a contiguous int32 tensor of B entries")
        cl = ctx_lens.data_ptr()
    _check(_lib.tq_decode_attention_noalloc(ctypes.byref(sk), ctypes.byref(sv), q.data_ptr(), _dtype_code(q), H_q,
                                            cl or None, T, scale, n_split, out.data_ptr(), _stream_handle(q.device)),
           "tq_decode_attention_noalloc")
    return out


def decode_attention_append(k: Cache, v: Cache, k_new, v_new, q, ctx_lens=None, T: int | None = None,
                            scale: float = 0.0, n_split: int = 0, out=None, workspace: Workspace | None = None):
    """One decode step in one launch: k_new, v_new [B, H_kv, d] (or [B, 1, H_kv, d])
    go to token ctx_len[b] - 1 of the caches (ctx_len = T without ctx_lens), then
    decode attention of q [B, H_q, d] over tokens 0 .. ctx_len[b] - 1."""
    torch = _torch()
    if q.dim() != 3 or q.shape[-1] != k.d or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous [B, H_q, {k.d}] tensor")
    if k_new.dim() == 4:
        k_new = k_new[:, 0]
    if v_new.dim() == 4:
        v_new = v_new[:, 0]
    if (k_new.dim() != 3 or k_new.shape != v_new.shape or k_new.shape[-1] != k.d or k_new.stride(-1) != 1
            or v_new.stride(-1) != 1 or k_new.dtype != v_new.dtype):
        raise ValueError(f"k_new and v_new must be [B, H_kv, {k.d}] of one dtype with a contiguous last dimension")
    B, H_q, _ = q.shape
    T = k.T_cap if T is None else T
    if out is None:
        out = torch.empty((B, H_q, k.d), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, H_q, k.H_kv, T, n_split, k.qjl)
    if workspace is None or workspace.nbytes < need:
        workspace = Workspace(need, q.device)
    sk, sv = k.struct(), v.struct()
    cl = 0
    if ctx_lens is not None:
        if ctx_lens.dtype != torch.int32 or not ctx_lens.is_contiguous() or ctx_lens.numel() != B:
            raise ValueError("ctx_lens must be a contiguous int32 tensor of B entries")
        cl = ctx_lens.data_ptr()
    _check(_lib.tq_decode_attention_append(ctypes.byref(sk), ctypes.byref(sv), k_new.data_ptr(), v_new.data_ptr(),
                                           _dtype_code(k_new), k_new.stride(0), k_new.stride(1), v_new.stride(0),
                                           v_new.stride(1), q.data_ptr(), _dtype_code(q), H_q, cl or None, T, scale,
                                           n_split, out.data_ptr(), workspace.ptr, workspace.nbytes,
                                           _stream_handle(q.device)), "tq_decode_attention_append")
    return out


def prefill_attention(k: Cache, v: Cache, q, ctx_lens=None, T: int | None = None, scale: float = 0.0,
                      n_split: int = 0, out=None, workspace: Workspace | None = None):
    """Chunked causal attention of the M newest tokens of each row, q [B, M, H_q, d]
    (their keys and values already in the caches), over the packed caches ->
    float32 [B, M, H_q, d]; token i of row b attends to cache tokens
    0 .. ctx_len[b] - M + i. (d = 256: at most 8 (token, head) columns per KV head.)"""
    torch = _torch()
    if q.dim() != 4 or q.shape[-1] != k.d or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous [B, M, H_q, {k.d}] tensor")
    B, M, H_q, _ = q.shape
    T = k.T_cap if T is None else T
    if out is None:
        out = torch.empty((B, M, H_q, k.d), dtype=torch.float32, device=q.device)
    need = prefill_workspace_bytes(B, H_q, k.H_kv, M, T, n_split, k.qjl)
    if workspace is None or workspace.nbytes < need:
        workspace = Workspace(need, q.device)
    sk, sv = k.struct(), v.struct()
    cl = 0
    if ctx_lens is not None:
        if ctx_lens.dtype != torch.int32 or not ctx_lens.is_contiguous() or ctx_lens.numel() != B:
            raise ValueError("ctx_lens must be a contiguous int32 tensor of B entries")
        cl = ctx_lens.data_ptr()
    _check(_lib.tq_prefill_attention(ctypes.byref(sk), ctypes.byref(sv), q.data_ptr(), _dtype_code(q), H_q, M,
                                     cl or None, T, scale, n_split, out.data_ptr(), workspace.ptr,
                                     workspace.nbytes, _stream_handle(q.device)), "tq_prefill_attention")
    return out

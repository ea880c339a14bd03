"""Thin Python binding of libqk4v8 (include/qk4v8.h): argument marshalling only.

Every step of the QK4V8 path runs in the library's HIP kernels; torch is used
here for device memory and the current stream.  Loading fails loudly when the
library has not been built - there is no CPU fallback.
"""

import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqk4v8.so")
_lib = None

QK4V8_OK = 0
# probability formats of the prefill P·V product (QK4V8_P_* of include/qk4v8.h)
P_DEFAULT, P_FP8_SINGLE, P_FP8_TWO_TERM, P_BF16 = 0, 1, 2, 3
P_DEFAULT_MODE = P_BF16          # what P_DEFAULT selects (QK4V8_P_DEFAULT_MODE)
STATUS_NAMES = {0: "QK4V8_OK", 1: "QK4V8_ERR_NULL", 2: "QK4V8_ERR_SHAPE", 3: "QK4V8_ERR_STRIDE",
                4: "QK4V8_ERR_UNSUPPORTED", 5: "QK4V8_ERR_WORKSPACE", 6: "QK4V8_ERR_HIP"}

EXPORTED = ["qk4v8_abi_version", "qk4v8_status_string", "qk4v8_quantize_qk", "qk4v8_quantize_v",
            "qk4v8_prefill_workspace_bytes", "qk4v8_attn_prefill", "qk4v8_prefill_pack_kv",
            "qk4v8_attn_prefill_packed", "qk4v8_decode_workspace_bytes", "qk4v8_attn_decode",
            "qk4v8_attn_decode_noalloc", "qk4v8_kv_append"]

# Size of the fixed per-GPU array qk4v8_attn_decode_noalloc keeps its split
# partials in (QK4V8_NOALLOC_SCRATCH_BYTES of include/qk4v8.h).
NOALLOC_SCRATCH_BYTES = 32 << 20


class PrefillArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
                ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
                ("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("seq_q", ctypes.c_int32), ("seq_k", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("v_tile_rows", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("p_mode", ctypes.c_int32), ("hadamard", ctypes.c_int32), ("window", ctypes.c_int32)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
                ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p), ("kv_lens", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("q_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
                ("batch", ctypes.c_int32), ("q_len", ctypes.c_int32), ("q_heads", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("kv_len", ctypes.c_int32), ("cap", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("v_tile_rows", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("hadamard", ctypes.c_int32), ("window", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("page_size", ctypes.c_int32), ("pages_per_seq", ctypes.c_int32)]


class AppendArgs(ctypes.Structure):
    _fields_ = [("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
                ("k_stride", ctypes.c_int64 * 3), ("v_stride", ctypes.c_int64 * 3),
                ("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("v_scales", ctypes.c_void_p), ("v_tail", ctypes.c_void_p), ("kv_lens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("kv_heads", ctypes.c_int32), ("n_new", ctypes.c_int32),
                ("kv_len", ctypes.c_int32), ("cap", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("v_tile_rows", ctypes.c_int32), ("hadamard", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("page_size", ctypes.c_int32), ("pages_per_seq", ctypes.c_int32)]


class QK4V8Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({lib().qk4v8_status_string(status).decode()})")


def lib():
    """Load libqk4v8.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m bit_quantized_attention_online_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        L.qk4v8_abi_version.restype = ctypes.c_int
        L.qk4v8_status_string.restype = ctypes.c_char_p
        L.qk4v8_status_string.argtypes = [ctypes.c_int]
        L.qk4v8_quantize_qk.restype = ctypes.c_int
        L.qk4v8_quantize_qk.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.qk4v8_quantize_v.restype = ctypes.c_int
        L.qk4v8_quantize_v.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
        L.qk4v8_prefill_workspace_bytes.restype = ctypes.c_size_t
        L.qk4v8_prefill_workspace_bytes.argtypes = [ctypes.POINTER(PrefillArgs)]
        for fn in ("qk4v8_attn_prefill", "qk4v8_prefill_pack_kv", "qk4v8_attn_prefill_packed"):
            getattr(L, fn).restype = ctypes.c_int
            getattr(L, fn).argtypes = [ctypes.POINTER(PrefillArgs), ctypes.c_void_p]
        L.qk4v8_decode_workspace_bytes.restype = ctypes.c_size_t
        L.qk4v8_decode_workspace_bytes.argtypes = [ctypes.POINTER(DecodeArgs)]
        for fn in ("qk4v8_attn_decode", "qk4v8_attn_decode_noalloc"):
            getattr(L, fn).restype = ctypes.c_int
            getattr(L, fn).argtypes = [ctypes.POINTER(DecodeArgs), ctypes.c_void_p]
        L.qk4v8_kv_append.restype = ctypes.c_int
        L.qk4v8_kv_append.argtypes = [ctypes.POINTER(AppendArgs), ctypes.c_void_p]
        _lib = L
    return _lib


def _check(status, where):
    if status != QK4V8_OK:
        raise QK4V8Error(status, where)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _bits16(t):
    if t.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise TypeError(f"expected bf16 (or its uint16 bit patterns), got {t.dtype}")
    return t


def quantize_qk(x, stream=None):
    """MXFP4 along the last dim of a bf16 tensor [..., d] whose rows have a
    common stride.  Returns (codes uint8 [..., d/2], scales uint8 [..., d/32])."""
    _bits16(x)
    d = x.shape[-1]
    x2 = x.reshape(-1, d) if x.dim() != 2 else x
    if x2.stride(-1) != 1:
        raise ValueError("innermost stride must be 1")
    rows = x2.shape[0]
    codes = torch.empty(x.shape[:-1] + (d // 2,), dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1] + (d // 32,), dtype=torch.uint8, device=x.device)
    ld = x2.stride(0) if rows > 1 else d
    _check(lib().qk4v8_quantize_qk(_ptr(x2), rows, d, ld, _ptr(codes), _ptr(scales), _stream(stream)),
           "qk4v8_quantize_qk")
    return codes, scales


def quantize_v(v, tile_rows, stream=None):
    """FP8 E4M3FN with one E8M0 scale per tile of rows.  v: bf16 [groups, n, d]
    (any strides with unit innermost).  Returns (codes [groups, n, d],
    scales [groups, ceil(n / tile_rows)])."""
    _bits16(v)
    g, n, d = v.shape
    codes = torch.empty((g, n, d), dtype=torch.uint8, device=v.device)
    scales = torch.empty((g, -(-n // tile_rows)), dtype=torch.uint8, device=v.device)
    gs = v.stride(0) if g > 1 else n * v.stride(1)
    rs = v.stride(1) if n > 1 else d
    _check(lib().qk4v8_quantize_v(_ptr(v), g, n, d, gs, rs, tile_rows, _ptr(codes), _ptr(scales), _stream(stream)),
           "qk4v8_quantize_v")
    return codes, scales


class PreparedQuantizeQK:
    """``quantize_qk`` with its output tensors allocated and its arguments
    marshalled once; ``__call__`` only enqueues qk4v8_quantize_qk.  The
    outputs are ``codes`` and ``scales``."""

    def __init__(self, x):
        _bits16(x)
        d = x.shape[-1]
        x2 = x.reshape(-1, d) if x.dim() != 2 else x
        if x2.stride(-1) != 1:
            raise ValueError("innermost stride must be 1")
        rows = x2.shape[0]
        self.codes = torch.empty(x.shape[:-1] + (d // 2,), dtype=torch.uint8, device=x.device)
        self.scales = torch.empty(x.shape[:-1] + (d // 32,), dtype=torch.uint8, device=x.device)
        ld = x2.stride(0) if rows > 1 else d
        self._args = (_ptr(x2), ctypes.c_int64(rows), ctypes.c_int32(d), ctypes.c_int64(ld), _ptr(self.codes),
                      _ptr(self.scales))
        self._keep = (x, x2)

    def __call__(self, stream=None):
        _check(lib().qk4v8_quantize_qk(*self._args, _stream(stream)), "qk4v8_quantize_qk")
        return self.codes, self.scales


class PreparedQuantizeV:
    """``quantize_v`` with its output tensors allocated and its arguments
    marshalled once; ``__call__`` only enqueues qk4v8_quantize_v."""

    def __init__(self, v, tile_rows):
        _bits16(v)
        g, n, d = v.shape
        self.codes = torch.empty((g, n, d), dtype=torch.uint8, device=v.device)
        self.scales = torch.empty((g, -(-n // tile_rows)), dtype=torch.uint8, device=v.device)
        gs = v.stride(0) if g > 1 else n * v.stride(1)
        rs = v.stride(1) if n > 1 else d
        self._args = (_ptr(v), ctypes.c_int64(g), ctypes.c_int64(n), ctypes.c_int32(d), ctypes.c_int64(gs),
                      ctypes.c_int64(rs), ctypes.c_int32(tile_rows), _ptr(self.codes), _ptr(self.scales))
        self._keep = v

    def __call__(self, stream=None):
        _check(lib().qk4v8_quantize_v(*self._args, _stream(stream)), "qk4v8_quantize_v")
        return self.codes, self.scales


def _prefill_args(q, k, v, o, lse, causal, softmax_scale, v_tile_rows, p_mode=P_DEFAULT, hadamard=False, window=0):
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    a = PrefillArgs()
    a.q, a.k, a.v, a.o = q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()
    a.lse = lse.data_ptr() if lse is not None else None
    for name, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", o)):
        if t.stride(3) != 1:
            raise ValueError("innermost stride must be 1")
        getattr(a, name)[:] = [t.stride(0), t.stride(1), t.stride(2)]
    a.batch, a.q_heads, a.kv_heads, a.seq_q, a.seq_k, a.head_dim = B, Hq, Hkv, Nq, Nk, d
    a.v_tile_rows, a.causal = v_tile_rows, int(bool(causal))
    a.softmax_scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(d)
    a.p_mode = p_mode
    a.hadamard = int(bool(hadamard))
    a.window = window
    return a


def prefill_workspace_bytes(q, k, v, causal=False, softmax_scale=None, v_tile_rows=64):
    o = q  # sizes only
    return lib().qk4v8_prefill_workspace_bytes(ctypes.byref(_prefill_args(q, k, v, o, None, causal, softmax_scale,
                                                                          v_tile_rows)))


def attn_prefill(q, k, v, causal=False, softmax_scale=None, v_tile_rows=64, return_lse=False, out=None,
                 workspace=None, stream=None, p_mode=P_DEFAULT, hadamard=False, window=0):
    """QK4V8 prefill.  q [B, Hq, Nq, d], k/v [B, Hkv, Nk, d] bf16 (any strides
    with unit innermost).  Returns o [B, Hq, Nq, d] bf16 (and lse fp32
    [B, Hq, Nq] when return_lse).  p_mode selects the probability format of
    P·V (P_FP8_TWO_TERM, P_BF16, P_FP8_SINGLE = fast mode; P_DEFAULT);
    hadamard=True rotates Q and K by H_d before quantization; window=W > 0
    (causal only) keeps the W most recent keys of each row."""
    for t in (q, k, v):
        _bits16(t)
    o = out if out is not None else torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    a = _prefill_args(q, k, v, o, lse, causal, softmax_scale, v_tile_rows, p_mode, hadamard, window)
    need = lib().qk4v8_prefill_workspace_bytes(ctypes.byref(a))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    _check(lib().qk4v8_attn_prefill(ctypes.byref(a), _stream(stream)), "qk4v8_attn_prefill")
    return (o, lse) if return_lse else o


class PackedPrefill:
    """A prefill split in its two library calls with one reusable workspace:
    ``pack()`` quantizes K/V into the workspace, ``attend()`` runs the
    attention kernel from it (used to time the two halves separately)."""

    def __init__(self, q, k, v, causal=False, softmax_scale=None, v_tile_rows=64, return_lse=False, p_mode=P_DEFAULT,
                 hadamard=False, window=0):
        for t in (q, k, v):
            _bits16(t)
        self.o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
        self.lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
        self.args = _prefill_args(q, k, v, self.o, self.lse, causal, softmax_scale, v_tile_rows, p_mode,
                                  hadamard, window)
        need = lib().qk4v8_prefill_workspace_bytes(ctypes.byref(self.args))
        self.workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        self.args.workspace, self.args.workspace_bytes = self.workspace.data_ptr(), self.workspace.numel()
        self._keep = (q, k, v)

    def pack(self, stream=None):
        _check(lib().qk4v8_prefill_pack_kv(ctypes.byref(self.args), _stream(stream)), "qk4v8_prefill_pack_kv")

    def attend(self, stream=None):
        _check(lib().qk4v8_attn_prefill_packed(ctypes.byref(self.args), _stream(stream)),
               "qk4v8_attn_prefill_packed")
        return self.o


def _paging(a, block_table, page_size):
    """Fill the paged-cache fields; returns the per-sequence capacity."""
    if block_table is None:
        return None
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
        raise TypeError("block_table must be a contiguous int32 [batch, pages_per_seq] tensor")
    a.block_table, a.page_size, a.pages_per_seq = block_table.data_ptr(), page_size, block_table.shape[1]
    return page_size * block_table.shape[1]


def _decode_args(q, k_codes, k_scales, v_codes, v_scales, o, lse, kv_len, v_tile_rows, kv_lens, num_splits,
                 softmax_scale, block_table=None, page_size=0):
    B, q_len, Hq, d = q.shape
    _, Hkv, cap, _ = k_codes.shape
    for t in (k_codes, k_scales, v_codes, v_scales):
        if not t.is_contiguous():
            raise ValueError("cache tensors must be contiguous")
    a = DecodeArgs()
    a.q, a.k_codes, a.k_scales = q.data_ptr(), k_codes.data_ptr(), k_scales.data_ptr()
    a.v_codes, a.v_scales = v_codes.data_ptr(), v_scales.data_ptr()
    a.kv_lens = kv_lens.data_ptr() if kv_lens is not None else None
    a.o = o.data_ptr()
    a.lse = lse.data_ptr() if lse is not None else None
    if q.stride(3) != 1 or o.stride(3) != 1:
        raise ValueError("innermost stride must be 1")
    a.q_stride[:] = [q.stride(0), q.stride(1), q.stride(2)]
    a.o_stride[:] = [o.stride(0), o.stride(1), o.stride(2)]
    a.batch, a.q_len, a.q_heads, a.kv_heads, a.kv_len, a.cap = B, q_len, Hq, Hkv, kv_len, cap
    a.head_dim, a.v_tile_rows, a.num_splits = d, v_tile_rows, num_splits
    a.softmax_scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(d)
    paged_cap = _paging(a, block_table, page_size)
    if paged_cap is not None:
        a.cap = paged_cap
    return a


def decode_workspace_bytes(q, k_codes, kv_len, v_tile_rows=256, num_splits=0, window=0, block_table=None,
                           page_size=0):
    a = _decode_args(q, k_codes, k_codes, k_codes, k_codes, q, None, kv_len, v_tile_rows, None, num_splits, None,
                     block_table, page_size)
    a.window = window
    return lib().qk4v8_decode_workspace_bytes(ctypes.byref(a))


def attn_decode(q, k_codes, k_scales, v_codes, v_scales, kv_len, v_tile_rows=256, kv_lens=None, num_splits=0,
                softmax_scale=None, return_lse=False, out=None, workspace=None, stream=None, hadamard=False,
                window=0, block_table=None, page_size=0):
    """QK4V8 decode / block verify over a quantized cache.
    q [B, q_len, Hq, d] bf16; k_codes [B, Hkv, cap, d/2], k_scales [B, Hkv, cap, d/32],
    v_codes [B, Hkv, cap, d], v_scales [B, Hkv, ceil(cap/v_tile_rows)] uint8.
    window=W > 0 keeps the W most recent keys of each query.
    Paged cache: block_table int32 [B, pages_per_seq] and page_size; the cache
    tensors are then page pools [pages, Hkv, page_size, ...] (v_scales
    [pages, Hkv, page_size / v_tile_rows]).
    Returns o [B, q_len, Hq, d] bf16 (and lse fp32 [B, q_len, Hq])."""
    _bits16(q)
    o = out if out is not None else torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    if kv_lens is not None and kv_lens.dtype != torch.int32:
        raise TypeError("kv_lens must be int32")
    a = _decode_args(q, k_codes, k_scales, v_codes, v_scales, o, lse, kv_len, v_tile_rows, kv_lens, num_splits,
                     softmax_scale, block_table, page_size)
    a.hadamard = int(bool(hadamard))
    a.window = window
    need = lib().qk4v8_decode_workspace_bytes(ctypes.byref(a))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
    _check(lib().qk4v8_attn_decode(ctypes.byref(a), _stream(stream)), "qk4v8_attn_decode")
    return (o, lse) if return_lse else o


class PreparedDecode:
    """A decode / block-verify call whose arguments are marshalled once:
    ``__call__`` only enqueues qk4v8_attn_decode on the stream (for loops that
    call the same shapes and buffers repeatedly).  Same arguments as
    ``attn_decode``; the output (and lse) tensors are ``self.o`` / ``self.lse``."""

    def __init__(self, q, k_codes, k_scales, v_codes, v_scales, kv_len, v_tile_rows=256, kv_lens=None, num_splits=0,
                 softmax_scale=None, return_lse=False, out=None, workspace=None, hadamard=False, window=0,
                 block_table=None, page_size=0):
        _bits16(q)
        if kv_lens is not None and kv_lens.dtype != torch.int32:
            raise TypeError("kv_lens must be int32")
        self.o = out if out is not None else torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
        self.lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
        a = _decode_args(q, k_codes, k_scales, v_codes, v_scales, self.o, self.lse, kv_len, v_tile_rows, kv_lens,
                         num_splits, softmax_scale, block_table, page_size)
        a.hadamard = int(bool(hadamard))
        a.window = window
        need = lib().qk4v8_decode_workspace_bytes(ctypes.byref(a))
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel()
        self.args, self.workspace = a, workspace
        self._ref = ctypes.byref(a)
        self._keep = (q, k_codes, k_scales, v_codes, v_scales, kv_lens, block_table)

    def __call__(self, stream=None):
        _check(lib().qk4v8_attn_decode(self._ref, _stream(stream)), "qk4v8_attn_decode")
        return self.o


def attn_decode_noalloc(q, k_codes, k_scales, v_codes, v_scales, kv_len, out, lse=None, v_tile_rows=256,
                        kv_lens=None, num_splits=0, softmax_scale=None, stream=None, hadamard=False, window=0,
                        block_table=None, page_size=0):
    """``attn_decode`` through qk4v8_attn_decode_noalloc: the caller passes the
    output (and optionally an fp32 lse [B, q_len, Hq]) and the library keeps
    the split partials in its fixed per-GPU array, allocating nothing.  Calls
    that overlap on one GPU race (they share the array)."""
    _bits16(q)
    if kv_lens is not None and kv_lens.dtype != torch.int32:
        raise TypeError("kv_lens must be int32")
    a = _decode_args(q, k_codes, k_scales, v_codes, v_scales, out, lse, kv_len, v_tile_rows, kv_lens, num_splits,
                     softmax_scale, block_table, page_size)
    a.hadamard = int(bool(hadamard))
    a.window = window
    _check(lib().qk4v8_attn_decode_noalloc(ctypes.byref(a), _stream(stream)), "qk4v8_attn_decode_noalloc")
    return out


def _append_args(k_new, v_new, k_codes, k_scales, v_codes, v_scales, v_tail, kv_len, v_tile_rows, kv_lens, hadamard,
                 block_table, page_size):
    """Checked AppendArgs for qk4v8_kv_append, or None for an empty append."""
    _bits16(k_new)
    _bits16(v_new)
    if kv_lens is not None and kv_lens.dtype != torch.int32:
        raise TypeError("kv_lens must be int32")
    B, n_new, Hkv, d = k_new.shape
    if B == 0 or n_new == 0:
        return None
    for t in (k_new, v_new):
        if t.stride(-1) != 1:
            raise ValueError("innermost stride must be 1")
    if tuple(v_new.shape) != (B, n_new, Hkv, d):
        raise ValueError("k_new and v_new shapes differ")
    for t in (k_codes, k_scales, v_codes, v_scales, v_tail):
        if not t.is_contiguous():
            raise ValueError("cache tensors and v_tail must be contiguous")
    if tuple(v_tail.shape) != (B, Hkv, v_tile_rows, d):
        raise ValueError("v_tail must be [B, Hkv, v_tile_rows, d]")
    a = AppendArgs()
    a.k_new, a.v_new = k_new.data_ptr(), v_new.data_ptr()
    for i, ax in enumerate((0, 1, 2)):
        a.k_stride[i] = k_new.stride(ax)
        a.v_stride[i] = v_new.stride(ax)
    a.k_codes, a.k_scales, a.v_codes, a.v_scales = (k_codes.data_ptr(), k_scales.data_ptr(), v_codes.data_ptr(),
                                                    v_scales.data_ptr())
    a.v_tail = v_tail.data_ptr()
    a.kv_lens = kv_lens.data_ptr() if kv_lens is not None else None
    a.batch, a.kv_heads, a.n_new, a.kv_len = B, Hkv, n_new, int(kv_len)
    a.cap, a.head_dim, a.v_tile_rows = k_codes.shape[2], d, v_tile_rows
    a.hadamard = int(bool(hadamard))
    paged_cap = _paging(a, block_table, page_size)
    if paged_cap is not None:
        a.cap = paged_cap
    return a


def kv_append(k_new, v_new, k_codes, k_scales, v_codes, v_scales, v_tail, kv_len, v_tile_rows=256,
              kv_lens=None, stream=None, hadamard=False, block_table=None, page_size=0):
    """Quantize n_new tokens per sequence into a decode cache (in place).
    k_new, v_new [B, n_new, Hkv, d] bf16 (token-major, strided); cache tensors as
    for attn_decode with capacity cap = k_codes.shape[2] (paged: page pools and
    block_table / page_size as for attn_decode); v_tail [B, Hkv, R, d] bf16
    keeps the source rows of each sequence's partial V tile.  kv_lens (device
    int32 [B]) or kv_len: tokens already cached; not modified."""
    a = _append_args(k_new, v_new, k_codes, k_scales, v_codes, v_scales, v_tail, kv_len, v_tile_rows, kv_lens,
                     hadamard, block_table, page_size)
    if a is not None:
        _check(lib().qk4v8_kv_append(ctypes.byref(a), _stream(stream)), "qk4v8_kv_append")


class PreparedAppend:
    """A cache append whose arguments are marshalled once (same arguments as
    ``kv_append``); ``__call__`` only enqueues qk4v8_kv_append."""

    def __init__(self, k_new, v_new, k_codes, k_scales, v_codes, v_scales, v_tail, kv_len, v_tile_rows=256,
                 kv_lens=None, hadamard=False, block_table=None, page_size=0):
        self.args = _append_args(k_new, v_new, k_codes, k_scales, v_codes, v_scales, v_tail, kv_len, v_tile_rows,
                                 kv_lens, hadamard, block_table, page_size)
        self._ref = ctypes.byref(self.args) if self.args is not None else None
        self._keep = (k_new, v_new, k_codes, k_scales, v_codes, v_scales, v_tail, kv_lens, block_table)

    def __call__(self, stream=None):
        if self._ref is not None:
            _check(lib().qk4v8_kv_append(self._ref, _stream(stream)), "qk4v8_kv_append")

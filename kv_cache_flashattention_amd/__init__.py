"""Python binding of libkvfa: paged KV cache + exact causal attention on MI355X.

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the computation runs in the HIP kernels
of libkvfa.so behind the C ABI declared in include/kvfa.h.  There is no
fallback: if the library is missing or fails to load, importing the
binding's entry points raises.

Low level: ``lib()`` returns the ctypes handle whose functions carry the C
names (kvc_create, kvc_append, kvc_attn_decode, ...).  High level:
``KvCache`` owns the device buffers (torch tensors) of one cache and exposes
the same calls as methods named after the C functions without the prefix.
"""
import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvfa.so")
_lib = None

KVC_OK, KVC_E_INVAL, KVC_E_UNSUPPORTED, KVC_E_NO_BLOCKS = 0, -1, -2, -3
KVC_E_STATE, KVC_E_WORKSPACE, KVC_E_HIP = -4, -5, -6
KVC_F32, KVC_F16, KVC_BF16, KVC_FP8_E4M3FN, KVC_INT4 = 0, 1, 2, 3, 4

DTYPES = {"f32": KVC_F32, "f16": KVC_F16, "bf16": KVC_BF16, "fp8": KVC_FP8_E4M3FN,
          "int4": KVC_INT4}
STORAGE_TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
                 "fp8": torch.uint8, "int4": torch.uint8}
IO_TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
            "fp8": torch.bfloat16, "int4": torch.bfloat16}
SCALED = ("fp8", "int4")
BLOCK = 16


class KvcError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"kvc error {code}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "n_q_heads", "n_kv_heads", "d_head", "block_size", "n_blocks", "max_seqs",
        "max_blocks_per_seq", "kv_dtype")]


class Sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "k_pool", "v_pool", "k_scale", "v_scale", "block_table", "seq_len")]


class Buffers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "k_pool", "v_pool", "k_scale", "v_scale", "block_table", "seq_len")]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGS = {
    "kvc_bytes_per_token": [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_uint64)],
    "kvc_required_sizes": [ctypes.POINTER(Config), ctypes.POINTER(Sizes)],
    "kvc_create": [ctypes.POINTER(Config), ctypes.POINTER(Buffers), _P, ctypes.POINTER(_P)],
    "kvc_destroy": [_P],
    "kvc_seq_alloc": [_P, _I, _I, _P],
    "kvc_seq_grow": [_P, _I, ctypes.POINTER(_I), _P],
    "kvc_seq_grow_by": [_P, _I, _I, _P],
    "kvc_seq_share_prefix": [_P, _I, _I, _I, _P],
    "kvc_block_refs": [_P, _I, ctypes.POINTER(_I)],
    "kvc_seq_release": [_P, _I, _P],
    "kvc_set_block_table": [_P, _I, ctypes.POINTER(_I), _I, _I, _P],
    "kvc_seq_len": [_P, _I, ctypes.POINTER(_I)],
    "kvc_seq_blocks": [_P, _I, ctypes.POINTER(_I), _I, ctypes.POINTER(_I)],
    "kvc_free_blocks": [_P, ctypes.POINTER(_I)],
    "kvc_append": [_P, _I, _I, _P, _P, _P, _P],
    "kvc_seq_grow_append": [_P, _I, _I, ctypes.POINTER(_I), _P, _P, _P],
    "kvc_write": [_P, _I, _I, _P, _I, _I, _P, _P, _P],
    "kvc_attn_prefill": [_P, _I, _I, _P, _I, _P, _P, _P, _P, ctypes.c_float, _P],
    "kvc_attn_extend": [_P, _I, _I, _P, _I, _P, _P, ctypes.c_float, _P],
    "kvc_decode_workspace_bytes": [_P, _I, _I, ctypes.POINTER(ctypes.c_uint64)],
    "kvc_attn_decode": [_P, _I, _I, _P, _P, _P, ctypes.c_float, _I, _P, ctypes.c_uint64, _P],
    "kvc_attn_decode_window": [_P, _I, _I, _P, _P, _P, ctypes.c_float, _I, _I, _I, _P,
                               ctypes.c_uint64, _P],
    "kvc_attn_prefill_window": [_P, _I, _I, _P, _I, _P, _P, _P, _P, ctypes.c_float, _I, _I, _P],
    "kvc_attn_extend_window": [_P, _I, _I, _P, _I, _P, _P, ctypes.c_float, _I, _I, _P],
    "kvc_attn_decode_append": [_P, _I, _I, _P, _P, _P, _P, _P, ctypes.c_float, _I, _I, _I, _P,
                               ctypes.c_uint64, _P],
    "kvc_attn_decode_noalloc": [_P, _I, _I, _P, _P, _P, ctypes.c_float, _I, _P],
    "kvc_gather": [_P, _I, _I, _I, _I, _P, _P, _P],
    "kvc_set_dispatch_events": [_P, _P, _P, _I],
    "kvc_last_error": [],
}


def lib():
    """Load libkvfa.so (built in-tree by build.py); raises if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m kv_cache_flashattention_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_char_p if name == "kvc_last_error" else ctypes.c_int
        _lib = L
    return _lib


def _check(rc):
    if rc != KVC_OK:
        raise KvcError(rc, lib().kvc_last_error().decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def make_config(n_layers, n_q_heads, n_kv_heads, d_head, n_blocks, max_seqs,
                max_blocks_per_seq, kv_dtype):
    return Config(n_layers, n_q_heads, n_kv_heads, d_head, BLOCK, n_blocks, max_seqs,
                  max_blocks_per_seq, DTYPES[kv_dtype])


def bytes_per_token(cfg):
    out = ctypes.c_uint64()
    _check(lib().kvc_bytes_per_token(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def required_sizes(cfg):
    s = Sizes()
    _check(lib().kvc_required_sizes(ctypes.byref(cfg), ctypes.byref(s)))
    return {n: getattr(s, n) for n, _ in Sizes._fields_}


class KvCache:
    """One paged cache: device pools and tables as torch tensors + the handle.

    kv_dtype: 'f32' | 'f16' | 'bf16' | 'fp8' | 'int4'.  device=None makes a
    host-only handle (allocator only).  `poison` fills the pools with 0xFF
    bytes (NaN in every floating storage format, code -1 in int4) so that
    reads of unwritten slots would show.  int4 pools are uint8 tensors
    [L][B][h][16][d/2] (K) and [L][B][h][d][8] (V), two codes per byte.
    """

    def __init__(self, n_layers, n_q_heads, n_kv_heads, d_head, n_blocks, max_seqs,
                 max_blocks_per_seq, kv_dtype="bf16", device="cuda", poison=False):
        self.cfg = make_config(n_layers, n_q_heads, n_kv_heads, d_head, n_blocks, max_seqs,
                               max_blocks_per_seq, kv_dtype)
        self.kv_dtype, self.device = kv_dtype, device
        self.n_layers, self.n_q, self.n_kv, self.d = n_layers, n_q_heads, n_kv_heads, d_head
        self.io_dtype = IO_TORCH[kv_dtype]
        self._h = ctypes.c_void_p()
        if device is None:
            _check(lib().kvc_create(ctypes.byref(self.cfg), None, None, ctypes.byref(self._h)))
            return
        sizes = required_sizes(self.cfg)
        st = STORAGE_TORCH[kv_dtype]
        fill = 0xFF if poison else 0
        half = 2 if kv_dtype == "int4" else 1
        self.k_pool = torch.full((n_layers, n_blocks, n_kv_heads, BLOCK, d_head // half), 0,
                                 dtype=st, device=device)
        self.v_pool = torch.full((n_layers, n_blocks, n_kv_heads, d_head, BLOCK // half), 0,
                                 dtype=st, device=device)
        if poison:
            self.k_pool.view(torch.uint8).fill_(fill)
            self.v_pool.view(torch.uint8).fill_(fill)
        if kv_dtype in SCALED:
            self.k_scale = torch.zeros((n_layers, n_blocks, n_kv_heads), dtype=torch.float32,
                                       device=device)
            self.v_scale = torch.zeros_like(self.k_scale)
            if poison:
                self.k_scale.view(torch.int32).fill_(-1)
                self.v_scale.view(torch.int32).fill_(-1)
        else:
            self.k_scale = self.v_scale = None
        self.block_table = torch.empty((max_seqs, max_blocks_per_seq), dtype=torch.int32,
                                       device=device)
        self.seq_len_dev = torch.empty((max_seqs,), dtype=torch.int32, device=device)
        assert self.k_pool.numel() * self.k_pool.element_size() == sizes["k_pool"]
        bufs = Buffers(self.k_pool.data_ptr(), self.v_pool.data_ptr(),
                       self.k_scale.data_ptr() if self.k_scale is not None else None,
                       self.v_scale.data_ptr() if self.v_scale is not None else None,
                       self.block_table.data_ptr(), self.seq_len_dev.data_ptr())
        _check(lib().kvc_create(ctypes.byref(self.cfg), ctypes.byref(bufs), _stream(),
                                ctypes.byref(self._h)))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.kvc_destroy(h)
            self._h = None

    # ------------------------------------------------------------ allocator
    def seq_alloc(self, seq, n_tokens):
        _check(lib().kvc_seq_alloc(self._h, seq, n_tokens, self._s()))

    def seq_grow(self, seqs):
        arr = (_I * len(seqs))(*[int(s) for s in seqs])
        _check(lib().kvc_seq_grow(self._h, len(seqs), arr, self._s()))

    def seq_release(self, seq):
        _check(lib().kvc_seq_release(self._h, seq, self._s()))

    def seq_share_prefix(self, src, dst, prefix_len):
        _check(lib().kvc_seq_share_prefix(self._h, src, dst, prefix_len, self._s()))

    def block_refs(self, block):
        out = _I()
        _check(lib().kvc_block_refs(self._h, block, ctypes.byref(out)))
        return out.value

    def seq_grow_by(self, seq, n_tokens):
        _check(lib().kvc_seq_grow_by(self._h, seq, n_tokens, self._s()))

    def set_block_table(self, seq, blocks, length):
        arr = (_I * len(blocks))(*[int(b) for b in blocks])
        _check(lib().kvc_set_block_table(self._h, seq, arr, len(blocks), length, self._s()))

    def seq_len(self, seq):
        out = _I()
        _check(lib().kvc_seq_len(self._h, seq, ctypes.byref(out)))
        return out.value

    def seq_blocks(self, seq):
        n = _I()
        _check(lib().kvc_seq_blocks(self._h, seq, None, 0, ctypes.byref(n)))
        arr = (_I * max(n.value, 1))()
        _check(lib().kvc_seq_blocks(self._h, seq, arr, n.value, ctypes.byref(n)))
        return list(arr[:n.value])

    def free_blocks(self):
        out = _I()
        _check(lib().kvc_free_blocks(self._h, ctypes.byref(out)))
        return out.value

    def _s(self):
        return _stream() if self.device is not None else ctypes.c_void_p(0)

    # ------------------------------------------------------------ device calls
    def _io(self, t, shape, name):
        if t.dtype != self.io_dtype or not t.is_cuda or not t.is_contiguous() \
                or tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: need a contiguous {self.io_dtype} CUDA tensor of shape "
                             f"{tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
        return _ptr(t)

    @staticmethod
    def _seqs(seqs):
        if seqs.dtype != torch.int32 or not seqs.is_cuda or not seqs.is_contiguous():
            raise ValueError("seqs must be a contiguous int32 CUDA tensor")
        return _ptr(seqs)

    def append(self, layer, seqs, k, v):
        n = seqs.numel()
        shape = (n, self.n_kv, self.d)
        _check(lib().kvc_append(self._h, layer, n, self._seqs(seqs), self._io(k, shape, "k"),
                                self._io(v, shape, "v"), _stream()))

    def seq_grow_append(self, layer, seqs, k, v):
        """seq_grow of the host ids `seqs`, then append of their new rows
        k, v [n, n_kv, d] to `layer`, in one launch."""
        n = len(seqs)
        arr = (_I * n)(*[int(s) for s in seqs])
        shape = (n, self.n_kv, self.d)
        _check(lib().kvc_seq_grow_append(self._h, layer, n, arr, self._io(k, shape, "k"),
                                         self._io(v, shape, "v"), _stream()))

    def write(self, layer, seqs, start, k, v):
        n, T = seqs.numel(), k.shape[1]
        shape = (n, T, self.n_kv, self.d)
        _check(lib().kvc_write(self._h, layer, n, self._seqs(seqs), start, T,
                               self._io(k, shape, "k"), self._io(v, shape, "v"), _stream()))

    def attn_prefill(self, layer, q, k, v, seqs=None, scale=None, out=None, window=0, sinks=0):
        n, T = q.shape[0], q.shape[1]
        scale = 1.0 / math.sqrt(self.d) if scale is None else scale
        if out is None:
            out = torch.empty((n, T, self.n_q, self.d), dtype=self.io_dtype, device=q.device)
        sp = self._seqs(seqs) if seqs is not None else ctypes.c_void_p(0)
        if seqs is not None and seqs.numel() != n:
            raise ValueError("seqs must have one entry per prompt")
        args = (self._h, layer, n, sp, T, self._io(q, (n, T, self.n_q, self.d), "q"),
                self._io(k, (n, T, self.n_kv, self.d), "k"),
                self._io(v, (n, T, self.n_kv, self.d), "v"),
                self._io(out, (n, T, self.n_q, self.d), "out"), ctypes.c_float(scale))
        if window or sinks:
            _check(lib().kvc_attn_prefill_window(*args, window, sinks, _stream()))
        else:
            _check(lib().kvc_attn_prefill(*args, _stream()))
        return out

    def attn_extend(self, layer, seqs, q, scale=None, out=None, window=0, sinks=0):
        """T new query rows per sequence (q [n, T, n_q, d]) against the whole
        cached context, whose last T rows are the new tokens' own K/V."""
        n, T = q.shape[0], q.shape[1]
        scale = 1.0 / math.sqrt(self.d) if scale is None else scale
        if seqs.numel() != n:
            raise ValueError("seqs must have one entry per query block")
        if out is None:
            out = torch.empty((n, T, self.n_q, self.d), dtype=self.io_dtype, device=q.device)
        args = (self._h, layer, n, self._seqs(seqs), T, self._io(q, (n, T, self.n_q, self.d), "q"),
                self._io(out, (n, T, self.n_q, self.d), "out"), ctypes.c_float(scale))
        if window or sinks:
            _check(lib().kvc_attn_extend_window(*args, window, sinks, _stream()))
        else:
            _check(lib().kvc_attn_extend(*args, _stream()))
        return out

    def decode_workspace_bytes(self, n, num_splits=0):
        out = ctypes.c_uint64()
        _check(lib().kvc_decode_workspace_bytes(self._h, n, num_splits, ctypes.byref(out)))
        return out.value

    def attn_decode(self, layer, seqs, q, scale=None, num_splits=0, out=None, ws=None,
                    window=0, sinks=0):
        """One query row per sequence against its whole cache; window > 0
        restricts it to the last `window` rows plus the first `sinks`."""
        n = seqs.numel()
        scale = 1.0 / math.sqrt(self.d) if scale is None else scale
        if out is None:
            out = torch.empty((n, self.n_q, self.d), dtype=self.io_dtype, device=q.device)
        if ws is None:
            nb = self.decode_workspace_bytes(n, num_splits)
            ws = torch.empty((max(nb, 16),), dtype=torch.uint8, device=q.device)
        qp, op = self._io(q, (n, self.n_q, self.d), "q"), self._io(out, (n, self.n_q, self.d), "out")
        wsp, wsb = _ptr(ws), ws.numel() * ws.element_size()
        if window or sinks:
            _check(lib().kvc_attn_decode_window(
                self._h, layer, n, self._seqs(seqs), qp, op, ctypes.c_float(scale), window, sinks,
                num_splits, wsp, wsb, _stream()))
        else:
            _check(lib().kvc_attn_decode(
                self._h, layer, n, self._seqs(seqs), qp, op, ctypes.c_float(scale), num_splits,
                wsp, wsb, _stream()))
        return out

    def attn_decode_append(self, layer, seqs, k, v, q, scale=None, num_splits=0, out=None,
                           ws=None, window=0, sinks=0):
        """kv_append of the newest rows k, v [n, n_kv, d] (after seq_grow),
        then attn_decode, in one library call."""
        n = seqs.numel()
        scale = 1.0 / math.sqrt(self.d) if scale is None else scale
        if out is None:
            out = torch.empty((n, self.n_q, self.d), dtype=self.io_dtype, device=q.device)
        if ws is None:
            nb = self.decode_workspace_bytes(n, num_splits)
            ws = torch.empty((max(nb, 16),), dtype=torch.uint8, device=q.device)
        kp = self._io(k, (n, self.n_kv, self.d), "k")
        vp = self._io(v, (n, self.n_kv, self.d), "v")
        qp, op = self._io(q, (n, self.n_q, self.d), "q"), self._io(out, (n, self.n_q, self.d), "out")
        _check(lib().kvc_attn_decode_append(
            self._h, layer, n, self._seqs(seqs), kp, vp, qp, op, ctypes.c_float(scale), window,
            sinks, num_splits, _ptr(ws), ws.numel() * ws.element_size(), _stream()))
        return out

    def attn_decode_noalloc(self, layer, seqs, q, scale=None, num_splits=0, out=None):
        """attn_decode with the partials in the library's own device scratch
        (no workspace argument; the call allocates nothing)."""
        n = seqs.numel()
        scale = 1.0 / math.sqrt(self.d) if scale is None else scale
        if out is None:
            out = torch.empty((n, self.n_q, self.d), dtype=self.io_dtype, device=q.device)
        qp, op = self._io(q, (n, self.n_q, self.d), "q"), self._io(out, (n, self.n_q, self.d), "out")
        _check(lib().kvc_attn_decode_noalloc(self._h, layer, n, self._seqs(seqs), qp, op,
                                             ctypes.c_float(scale), num_splits, _stream()))
        return out

    def set_dispatch_events(self, start=None, stop=None, main_kernel=False):
        """Timing hook: the next attention call on this cache records `start`
        as its first kernel begins and `stop` as its last kernel ends, or,
        with main_kernel, both on its main kernel (events attached to the
        kernels' own dispatches).  Each is a torch.cuda.Event made with
        enable_timing=True and recorded once already (torch creates the
        underlying event at its first record), or None."""
        def handle(e):
            if e is None:
                return None
            if not e.cuda_event:
                raise ValueError("record the event once before using it as a dispatch event")
            return e.cuda_event
        _check(lib().kvc_set_dispatch_events(self._h, handle(start), handle(stop),
                                             1 if main_kernel else 0))

    def gather(self, layer, seq, start, count):
        st = STORAGE_TORCH[self.kv_dtype]
        d = self.d // 2 if self.kv_dtype == "int4" else self.d
        k = torch.empty((count, self.n_kv, d), dtype=st, device=self.k_pool.device)
        v = torch.empty_like(k)
        _check(lib().kvc_gather(self._h, layer, seq, start, count, _ptr(k), _ptr(v), _stream()))
        return k, v

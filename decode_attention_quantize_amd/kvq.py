"""ctypes binding of libkvq.so (include/kvq.h), same entry-point names.

Argument marshalling only: every step of quantization and decode runs in the
HIP kernels of libkvq.so.  ``KVQCache`` adds torch plumbing (device buffers,
the current stream) around the raw calls.  There is no fallback: without the
built library every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkvq.so")

KVQ_OK, KVQ_ERR_ARG, KVQ_ERR_CAPACITY, KVQ_ERR_UNSUPPORTED, KVQ_ERR_STATE, KVQ_ERR_DEVICE = range(6)
KVQ_K_PER_CHANNEL, KVQ_K_INNER = 0, 1
KVQ_V_PER_TOKEN, KVQ_V_HADAMARD, KVQ_V_TERNARY = 0, 1, 2
KVQ_NBUF = 2
KVQ_BUF_BODY, KVQ_BUF_FP16 = 0, 1

EXPORTS = ("kvq_create", "kvq_destroy", "kvq_layer_buffer_sizes", "kvq_block_layout",
           "kvq_bind_layer", "kvq_unbind_layer", "kvq_workspace_size", "kvq_quantize_prefill",
           "kvq_append_token", "kvq_decode_attn", "kvq_append_decode_attn", "kvq_decode_attn_static",
           "kvq_decode_nonfinite_rows", "kvq_layer_state",
           "kvq_average_bits", "kvq_status_str", "kvq_fit_rate_distortion", "kvq_waterfill_bits",
           "kvq_allocate_bits", "kvq_stream_read")


class kvq_config(C.Structure):
    _fields_ = [
        ("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
        ("head_dim", C.c_int32), ("n_layers", C.c_int32), ("max_tokens", C.c_int32),
        ("sink_tokens", C.c_int32), ("recent_window", C.c_int32),
        ("k_mode", C.c_int32), ("k_group", C.c_int32), ("v_mode", C.c_int32), ("v_group", C.c_int32),
        ("k_hybrid", C.c_int32), ("sym_ratio_num", C.c_int32), ("sym_ratio_den", C.c_int32),
        ("k_pre_rope", C.c_int32), ("rope_base", C.c_float), ("nuq", C.c_int32),
        ("outliers_per_vector", C.c_int32), ("k_norm", C.c_int32), ("k_hi_groups", C.c_int32),
    ]


class kvq_bitpair(C.Structure):
    _fields_ = [("k_bits", C.c_uint8), ("v_bits", C.c_uint8)]


class kvq_block_layout_t(C.Structure):
    _fields_ = [(n, C.c_int32) for n in (
        "record_bytes", "k_codes", "k_meta", "v_codes", "v_meta", "k_out", "v_out",
        "k_row_bytes", "sink_cap", "window_cap", "flush_tokens", "k_ext", "k_sel")]


class KVQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


_lib = None


def lib():
    """Load libkvq.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        vp, i32, pcache = C.c_void_p, C.c_int32, C.c_void_p
        L.kvq_status_str.restype = C.c_char_p
        L.kvq_status_str.argtypes = [C.c_int]
        L.kvq_create.argtypes = [C.POINTER(kvq_config), C.POINTER(kvq_bitpair), C.POINTER(C.c_uint16),
                                 C.POINTER(C.c_void_p)]
        L.kvq_destroy.argtypes = [pcache]
        L.kvq_layer_buffer_sizes.argtypes = [pcache, i32, C.POINTER(C.c_size_t)]
        L.kvq_block_layout.argtypes = [pcache, i32, C.POINTER(kvq_block_layout_t)]
        L.kvq_bind_layer.argtypes = [pcache, i32, C.POINTER(C.c_void_p)]
        L.kvq_unbind_layer.argtypes = [pcache, i32]
        L.kvq_decode_nonfinite_rows.argtypes = [pcache, vp, vp, C.POINTER(C.c_uint32)]
        L.kvq_workspace_size.argtypes = [pcache, C.POINTER(C.c_size_t)]
        L.kvq_quantize_prefill.argtypes = [pcache, i32, vp, vp, i32, vp, vp]
        L.kvq_append_token.argtypes = [pcache, i32, vp, vp, vp]
        L.kvq_decode_attn.argtypes = [pcache, i32, vp, vp, vp, vp]
        L.kvq_append_decode_attn.argtypes = [pcache, i32, vp, vp, vp, vp, vp, vp]
        L.kvq_decode_attn_static.argtypes = [pcache, i32, vp, vp, vp]
        L.kvq_layer_state.argtypes = [pcache, i32] + [C.POINTER(C.c_int32)] * 4
        dp, ip = C.POINTER(C.c_double), C.POINTER(C.c_int32)
        L.kvq_average_bits.argtypes = [pcache, dp, dp]
        L.kvq_fit_rate_distortion.argtypes = [i32, dp, dp, dp, dp]
        L.kvq_waterfill_bits.argtypes = [i32, dp, dp, dp, C.c_double, dp]
        L.kvq_allocate_bits.argtypes = [i32, dp, dp, dp, ip, i32, i32, ip]
        L.kvq_stream_read.argtypes = [vp, C.c_size_t, i32, vp, vp]
        for name in EXPORTS:
            if name != "kvq_status_str":
                getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().kvq_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != KVQ_OK:
        raise KVQError(status, where)


# ---------------------------------------------------------------- raw entry points
def kvq_create(cfg: kvq_config, layer_bits, codebooks=None) -> int:
    pairs = (kvq_bitpair * len(layer_bits))(*[kvq_bitpair(kb, vb) for kb, vb in layer_bits])
    cb = None
    if codebooks is not None:
        import numpy as np
        arr = np.ascontiguousarray(codebooks, dtype=np.uint16).ravel()
        cb = (C.c_uint16 * arr.size)(*arr.tolist())
    h = C.c_void_p()
    _check(lib().kvq_create(C.byref(cfg), pairs, cb, C.byref(h)), "kvq_create")
    return h.value


def kvq_destroy(handle: int):
    _check(lib().kvq_destroy(handle), "kvq_destroy")


def kvq_layer_buffer_sizes(handle: int, layer: int):
    sizes = (C.c_size_t * KVQ_NBUF)()
    _check(lib().kvq_layer_buffer_sizes(handle, layer, sizes), "kvq_layer_buffer_sizes")
    return list(sizes)


def kvq_block_layout(handle: int, layer: int) -> dict:
    o = kvq_block_layout_t()
    _check(lib().kvq_block_layout(handle, layer, C.byref(o)), "kvq_block_layout")
    return {n: getattr(o, n) for n, _ in kvq_block_layout_t._fields_}


def kvq_bind_layer(handle: int, layer: int, ptrs):
    arr = (C.c_void_p * KVQ_NBUF)(*ptrs)
    _check(lib().kvq_bind_layer(handle, layer, arr), "kvq_bind_layer")


def kvq_unbind_layer(handle: int, layer: int):
    _check(lib().kvq_unbind_layer(handle, layer), "kvq_unbind_layer")


def kvq_decode_nonfinite_rows(handle: int, ws_ptr, stream) -> int:
    n = C.c_uint32()
    _check(lib().kvq_decode_nonfinite_rows(handle, ws_ptr, stream, C.byref(n)),
           "kvq_decode_nonfinite_rows")
    return n.value


def kvq_workspace_size(handle: int) -> int:
    n = C.c_size_t()
    _check(lib().kvq_workspace_size(handle, C.byref(n)), "kvq_workspace_size")
    return n.value


def kvq_quantize_prefill(handle, layer, k_ptr, v_ptr, T, ws_ptr, stream):
    _check(lib().kvq_quantize_prefill(handle, layer, k_ptr, v_ptr, T, ws_ptr, stream),
           "kvq_quantize_prefill")


def kvq_append_token(handle, layer, k_ptr, v_ptr, stream):
    _check(lib().kvq_append_token(handle, layer, k_ptr, v_ptr, stream), "kvq_append_token")


def kvq_decode_attn(handle, layer, q_ptr, out_ptr, ws_ptr, stream):
    _check(lib().kvq_decode_attn(handle, layer, q_ptr, out_ptr, ws_ptr, stream), "kvq_decode_attn")


def kvq_append_decode_attn(handle, layer, k_ptr, v_ptr, q_ptr, out_ptr, ws_ptr, stream):
    _check(lib().kvq_append_decode_attn(handle, layer, k_ptr, v_ptr, q_ptr, out_ptr, ws_ptr, stream),
           "kvq_append_decode_attn")


def kvq_decode_attn_static(handle, layer, q_ptr, out_ptr, stream):
    _check(lib().kvq_decode_attn_static(handle, layer, q_ptr, out_ptr, stream), "kvq_decode_attn_static")


def kvq_layer_state(handle, layer):
    v = [C.c_int32() for _ in range(4)]
    _check(lib().kvq_layer_state(handle, layer, *[C.byref(x) for x in v]), "kvq_layer_state")
    return tuple(x.value for x in v)


def kvq_average_bits(handle):
    """(code_bits, stored_bits): the memory objective f_m and the stored bits per element."""
    a, b = C.c_double(), C.c_double()
    _check(lib().kvq_average_bits(handle, C.byref(a), C.byref(b)), "kvq_average_bits")
    return a.value, b.value


def kvq_stream_read(src_ptr, nbytes, splits, sink_ptr, stream):
    """Read-ceiling kernel of the decode's access pattern (measurement helper)."""
    _check(lib().kvq_stream_read(src_ptr, nbytes, splits, sink_ptr, stream), "kvq_stream_read")


# ---------------------------------------------------------------- offline bit allocation
def _darr(x):
    x = [float(v) for v in x]
    return (C.c_double * len(x))(*x)


def kvq_fit_rate_distortion(bits, mse):
    a, b = C.c_double(), C.c_double()
    _check(lib().kvq_fit_rate_distortion(len(bits), _darr(bits), _darr(mse), C.byref(a), C.byref(b)),
           "kvq_fit_rate_distortion")
    return a.value, b.value


def kvq_waterfill_bits(alpha, beta, w, total_bits):
    n = len(w)
    out = (C.c_double * n)()
    _check(lib().kvq_waterfill_bits(n, _darr(alpha), _darr(beta), _darr(w), float(total_bits), out),
           "kvq_waterfill_bits")
    return list(out)


def kvq_allocate_bits(alpha, beta, w, allowed, total_bits):
    n = len(w)
    al = (C.c_int32 * len(allowed))(*[int(a) for a in allowed])
    out = (C.c_int32 * n)()
    _check(lib().kvq_allocate_bits(n, _darr(alpha), _darr(beta), _darr(w), al, len(allowed),
                                   int(total_bits), out), "kvq_allocate_bits")
    return list(out)


# ---------------------------------------------------------------- configuration helpers
def make_config(B, Hq, Hkv, L, max_tokens, D=128, sinks=0, window=0, k_mode=KVQ_K_PER_CHANNEL,
                k_group=32, v_mode=KVQ_V_PER_TOKEN, v_group=32, k_hybrid=0, sym_ratio=(1, 10),
                k_pre_rope=0, rope_base=10000.0, nuq=0, outliers=0, k_norm=0,
                k_hi_groups=0) -> kvq_config:
    c = kvq_config()
    c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim = B, Hq, Hkv, D
    c.n_layers, c.max_tokens, c.sink_tokens, c.recent_window = L, max_tokens, sinks, window
    c.k_mode, c.k_group, c.v_mode, c.v_group = k_mode, k_group, v_mode, v_group
    c.k_hybrid, c.sym_ratio_num, c.sym_ratio_den = k_hybrid, sym_ratio[0], sym_ratio[1]
    c.k_pre_rope, c.rope_base, c.nuq, c.outliers_per_vector = k_pre_rope, rope_base, nuq, outliers
    c.k_norm = k_norm
    c.k_hi_groups = k_hi_groups
    return c


def config_from_workload(wl, max_tokens=None) -> kvq_config:
    from fractions import Fraction
    f = Fraction(wl.sym_ratio).limit_denominator(1000)
    return make_config(
        wl.B, wl.Hq, wl.Hkv, wl.L,
        max_tokens if max_tokens is not None else wl.T + (wl.steps if wl.append else 0),
        D=wl.D, sinks=wl.sinks, window=wl.window,
        k_mode=KVQ_K_PER_CHANNEL if wl.k_mode == "channel" else KVQ_K_INNER, k_group=wl.k_group,
        v_mode=(KVQ_V_HADAMARD if wl.v_hadamard else
                KVQ_V_TERNARY if getattr(wl, "v_ternary", False) else KVQ_V_PER_TOKEN),
        v_group=wl.v_group,
        k_hybrid=int(wl.k_hybrid), sym_ratio=(f.numerator, f.denominator),
        k_pre_rope=int(wl.pre_rope), rope_base=wl.rope_base, nuq=int(wl.nuq), outliers=wl.outliers,
        k_norm=int(getattr(wl, "k_norm", False)), k_hi_groups=int(getattr(wl, "k_hi_groups", 0)))


# ---------------------------------------------------------------- torch plumbing
class KVQCache:
    """A libkvq cache whose device buffers are torch tensors on one GPU.

    Every device call checks that its tensors live on the cache's device and
    have the dtype and the exact shape the C entry point reads or writes, so
    a wrong tensor raises here instead of letting a kernel run past it.
    ``fill`` (tests) fills the layer buffers with that byte instead of zeros.
    """

    def __init__(self, cfg: kvq_config, layer_bits, codebooks=None, device="cuda", layers=None,
                 fill=None):
        import torch
        self.torch = torch
        self.device = torch.device(device)
        if self.device.type != "cuda":
            raise ValueError(f"KVQCache needs a GPU device, got {self.device}")
        if self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.cfg = cfg
        self.fill = fill
        self.handle = kvq_create(cfg, layer_bits, codebooks)
        self.buffers = {}
        for l in (range(cfg.n_layers) if layers is None else layers):
            self.bind(l)
        ws = kvq_workspace_size(self.handle)
        self.workspace = torch.zeros(ws, dtype=torch.uint8, device=self.device)

    def bind(self, layer):
        torch = self.torch
        sizes = kvq_layer_buffer_sizes(self.handle, layer)
        bufs = []
        for sz in sizes:
            b = torch.empty(max(sz, 256) + 256, dtype=torch.uint8, device=self.device)
            b.fill_(0 if self.fill is None else int(self.fill))
            bufs.append(b)
        ptrs = []
        for b in bufs:
            p = b.data_ptr()
            ptrs.append(p + (-p) % 256)
        kvq_bind_layer(self.handle, layer, ptrs)
        self.buffers[layer] = (bufs, ptrs, sizes)

    def unbind(self, layer):
        """Detach a layer in the C handle, then release its buffers (after
        the work already queued on the current stream has completed)."""
        kvq_unbind_layer(self.handle, layer)
        if layer in self.buffers:
            self.torch.cuda.current_stream(self.device).synchronize()
            del self.buffers[layer]

    def layout(self, layer):
        return kvq_block_layout(self.handle, layer)

    def raw(self, layer, which):
        """uint8 view of a bound buffer (exact size, aligned)."""
        bufs, ptrs, sizes = self.buffers[layer]
        b = bufs[which]
        off = ptrs[which] - b.data_ptr()
        return b[off:off + sizes[which]]

    def _stream(self):
        return self.torch.cuda.current_stream(self.device).cuda_stream

    def _check(self, x, name, dtype, shape):
        torch = self.torch
        if not isinstance(x, torch.Tensor):
            raise TypeError(f"{name}: expected a torch tensor")
        if x.device != self.device:
            raise ValueError(f"{name}: tensor on {x.device}, cache on {self.device}")
        if x.dtype != dtype:
            raise TypeError(f"{name}: dtype {x.dtype}, expected {dtype}")
        if tuple(x.shape) != tuple(shape):
            raise ValueError(f"{name}: shape {tuple(x.shape)}, expected {tuple(shape)}")
        if not x.is_contiguous():
            raise ValueError(f"{name}: tensor must be contiguous")

    def prefill(self, layer, k, v):
        """k, v: fp16 [B][Hkv][T][D] on the cache's device."""
        c = self.cfg
        if k.dim() != 4:
            raise ValueError(f"k: expected [B, Hkv, T, D], got shape {tuple(k.shape)}")
        shape = (c.batch, c.n_kv_heads, k.shape[2], c.head_dim)
        self._check(k, "k", self.torch.float16, shape)
        self._check(v, "v", self.torch.float16, shape)
        kvq_quantize_prefill(self.handle, layer, k.data_ptr(), v.data_ptr(), shape[2],
                             self.workspace.data_ptr(), self._stream())

    def append(self, layer, k, v):
        """k, v: fp16 [B][Hkv][D] (one token per unit)."""
        c = self.cfg
        shape = (c.batch, c.n_kv_heads, c.head_dim)
        self._check(k, "k", self.torch.float16, shape)
        self._check(v, "v", self.torch.float16, shape)
        kvq_append_token(self.handle, layer, k.data_ptr(), v.data_ptr(), self._stream())

    def decode(self, layer, q, out=None):
        """q: fp16 [B][Hq][D]; out: fp32 [B][Hq][D] (allocated when None)."""
        torch = self.torch
        c = self.cfg
        shape = (c.batch, c.n_q_heads, c.head_dim)
        self._check(q, "q", torch.float16, shape)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        self._check(out, "out", torch.float32, shape)
        kvq_decode_attn(self.handle, layer, q.data_ptr(), out.data_ptr(), self.workspace.data_ptr(),
                        self._stream())
        return out

    def append_decode(self, layer, k, v, q, out=None):
        """kvq_append_decode_attn: append(k, v), then decode(q) -- one launch
        where the library can.  Shapes as for append and decode."""
        torch = self.torch
        c = self.cfg
        kv_shape = (c.batch, c.n_kv_heads, c.head_dim)
        shape = (c.batch, c.n_q_heads, c.head_dim)
        self._check(k, "k", torch.float16, kv_shape)
        self._check(v, "v", torch.float16, kv_shape)
        self._check(q, "q", torch.float16, shape)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        self._check(out, "out", torch.float32, shape)
        kvq_append_decode_attn(self.handle, layer, k.data_ptr(), v.data_ptr(), q.data_ptr(), out.data_ptr(),
                               self.workspace.data_ptr(), self._stream())
        return out

    def decode_static(self, layer, q, out):
        """kvq_decode_attn_static: the library's static scratch instead of
        the workspace (out must be given: the call allocates nothing)."""
        c = self.cfg
        shape = (c.batch, c.n_q_heads, c.head_dim)
        self._check(q, "q", self.torch.float16, shape)
        self._check(out, "out", self.torch.float32, shape)
        kvq_decode_attn_static(self.handle, layer, q.data_ptr(), out.data_ptr(), self._stream())
        return out

    def nonfinite_rows(self):
        """Output rows with a non-finite element since the last call (waits
        for the current stream; resets the count)."""
        return kvq_decode_nonfinite_rows(self.handle, self.workspace.data_ptr(), self._stream())

    def state(self, layer):
        return kvq_layer_state(self.handle, layer)

    def close(self):
        if self.handle:
            kvq_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

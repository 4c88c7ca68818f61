"""ctypes binding of libjolt (include/jolt.h), one Python function per C
entry point, same names.  Argument marshalling only: every step of the decode
path runs in the library's HIP kernels.  torch is used for device memory and
streams; the library must have been built (``build.build()``), otherwise
every call raises.
"""
import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libjolt.so")

JOLT_OK, JOLT_E_INVALID, JOLT_E_UNSUPPORTED, JOLT_E_OOM, JOLT_E_HIP, JOLT_E_WORKSPACE = \
    0, -1, -2, -3, -4, -5
JOLT_F32, JOLT_BF16 = 0, 1
KERNEL_AUTO, KERNEL_GENERIC, KERNEL_MFMA = 0, 1, 2


class JoltError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"jolt status {status}: {msg}")
        self.status = status


class jolt_cell(C.Structure):
    _fields_ = [("r_T", C.c_int32), ("r_F", C.c_int32), ("bits", C.c_int32),
                ("A", C.c_void_p), ("B", C.c_void_p), ("G", C.c_void_p),
                ("codes", C.c_void_p), ("scales", C.c_void_p)]


class jolt_cache_desc(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("n_groups", C.c_int32), ("n_kv_heads", C.c_int32),
                ("n_q_heads", C.c_int32), ("head_dim", C.c_int32), ("T", C.c_int32),
                ("group_start", C.POINTER(C.c_int32)), ("factor_dtype", C.c_int),
                ("rotation_seed", C.c_uint64), ("cells", C.POINTER(jolt_cell))]


class jolt_launch(C.Structure):
    _fields_ = [("kernel", C.c_int32), ("split_tokens", C.c_int32),
                ("ev_begin", C.c_void_p), ("ev_end", C.c_void_p)]


_lib = None

EXPORTS = {
    "jolt_load_cache": (C.c_int, [C.POINTER(jolt_cache_desc), C.c_void_p, C.POINTER(C.c_void_p)]),
    "jolt_free_cache": (C.c_int, [C.c_void_p]),
    "jolt_cache_info": (C.c_int, [C.c_void_p] + [C.POINTER(C.c_int32)] * 5 + [C.POINTER(C.c_size_t)]),
    "jolt_decode_workspace_size": (C.c_int, [C.POINTER(C.c_void_p), C.c_int32, C.c_int32,
                                             C.POINTER(jolt_launch), C.POINTER(C.c_size_t)]),
    "jolt_decode_attention": (C.c_int, [C.POINTER(C.c_void_p), C.c_int32, C.c_int32, C.c_void_p,
                                        C.c_int, C.POINTER(C.c_int32), C.POINTER(C.c_float),
                                        C.c_float, C.c_void_p, C.c_void_p, C.c_size_t,
                                        C.POINTER(jolt_launch), C.c_void_p]),
    "jolt_dense_workspace_size": (C.c_int, [C.c_int32] * 5 + [C.POINTER(jolt_launch),
                                                              C.POINTER(C.c_size_t)]),
    "jolt_dense_attention": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int] + [C.c_int32] * 5 +
                             [C.c_void_p, C.c_int, C.POINTER(C.c_int32), C.POINTER(C.c_float),
                              C.c_float, C.c_void_p, C.c_void_p, C.c_size_t,
                              C.POINTER(jolt_launch), C.c_void_p]),
    "jolt_last_error": (C.c_char_p, []),
    "jolt_make_rotation": (C.c_int, [C.c_uint64, C.c_int32, C.POINTER(C.c_double)]),
    "jolt_debug_unpack": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]),
    "jolt_debug_sincos": (C.c_int, [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_int32]),
}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m compressed_cache_decode_jolt_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def jolt_last_error():
    return lib().jolt_last_error().decode()


def _check(st):
    if st != JOLT_OK:
        raise JoltError(st, jolt_last_error())


def _stream(stream):
    if stream is None:
        import torch
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def _launch(kernel=None, split_tokens=0, events=None):
    if kernel is None and not split_tokens and events is None:
        return None
    ev = events or (None, None)
    return jolt_launch(int(kernel or 0), int(split_tokens), ev[0], ev[1])


def _factor_bytes(x, dtype):
    """float32 values -> contiguous host buffer in the factor dtype."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("factor values are not exactly representable in bf16")
    return (u >> 16).astype(np.uint16)


class Cache:
    """A loaded device cache (owns the library handle)."""

    def __init__(self, handle, meta):
        self.handle = handle
        self.meta = meta

    def free(self):
        if self.handle:
            _check(lib().jolt_free_cache(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    def info(self):
        vals = [C.c_int32() for _ in range(5)]
        nb = C.c_size_t()
        _check(lib().jolt_cache_info(self.handle, *[C.byref(v) for v in vals], C.byref(nb)))
        keys = ("n_layers", "n_kv_heads", "n_q_heads", "head_dim", "T")
        out = {k: v.value for k, v in zip(keys, vals)}
        out["device_bytes"] = nb.value
        return out


def jolt_load_cache(cache, stream=None):
    """Upload a compressed cache dict (T, H, H_q, d, n_layers, group_start,
    factor_dtype, rotation_seed, cells[g] = (K cell, V cell))."""
    dt = cache["factor_dtype"]
    keep = []
    n_groups = len(cache["cells"])
    cells = (jolt_cell * (2 * n_groups))()
    for g, pair in enumerate(cache["cells"]):
        for tau, cell in enumerate(pair):
            c = cells[2 * g + tau]
            c.r_T, c.r_F, c.bits = int(cell["r_T"]), int(cell["r_F"]), int(cell["bits"])
            for name in ("A", "B", "G"):
                arr = cell.get(name)
                if arr is not None and arr.size:
                    buf = _factor_bytes(arr, dt)
                    keep.append(buf)
                    setattr(c, name, buf.ctypes.data)
            if cell.get("codes") is not None:
                codes = np.ascontiguousarray(cell["codes"], dtype=np.uint8)
                keep.append(codes)
                c.codes = codes.ctypes.data
            if cell.get("scales") is not None:
                scales = np.ascontiguousarray(cell["scales"], dtype=np.float32)
                keep.append(scales)
                c.scales = scales.ctypes.data
    gs = (C.c_int32 * (n_groups + 1))(*cache["group_start"])
    desc = jolt_cache_desc(cache["n_layers"], n_groups, cache["H"], cache["H_q"], cache["d"],
                           cache["T"], gs, JOLT_F32 if dt == "f32" else JOLT_BF16,
                           int(cache["rotation_seed"]), cells)
    h = C.c_void_p()
    _check(lib().jolt_load_cache(C.byref(desc), _stream(stream), C.byref(h)))
    return Cache(h, {k: cache[k] for k in ("T", "H", "H_q", "d", "n_layers", "factor_dtype")})


def _handles(caches):
    return (C.c_void_p * max(1, len(caches)))(*[c.handle for c in caches])


def jolt_decode_workspace_size(caches, layer, kernel=None, split_tokens=0):
    n = C.c_size_t()
    L = _launch(kernel, split_tokens)
    _check(lib().jolt_decode_workspace_size(_handles(caches), len(caches), layer,
                                            C.byref(L) if L else None, C.byref(n)))
    return n.value


def _ptr(t):
    return C.c_void_p(t.data_ptr() if t is not None else 0)


def _nbytes(t):
    return t.numel() * t.element_size() if t is not None else 0


def _dtype_code(t):
    import torch
    if t is None:
        return JOLT_F32
    if t.dtype == torch.float32:
        return JOLT_F32
    if t.dtype == torch.bfloat16:
        return JOLT_BF16
    raise TypeError(t.dtype)


def jolt_decode_attention(caches, layer, q, q_pos, inv_freq, softmax_scale, out, workspace,
                          kernel=None, split_tokens=0, stream=None, events=None):
    """q: device tensor [B, H_q, d] (f32/bf16); out: device f32 [B, H_q, d];
    workspace: device tensor of at least jolt_decode_workspace_size bytes;
    events: optional (begin, end) raw hipEvent_t handles recorded around the
    split-T kernel."""
    B = len(caches)
    qp = (C.c_int32 * max(1, B))(*[int(x) for x in q_pos])
    inv = np.ascontiguousarray(inv_freq, dtype=np.float32)
    L = _launch(kernel, split_tokens, events)
    _check(lib().jolt_decode_attention(
        _handles(caches), B, layer, _ptr(q), _dtype_code(q), qp,
        inv.ctypes.data_as(C.POINTER(C.c_float)), C.c_float(softmax_scale), _ptr(out),
        _ptr(workspace), _nbytes(workspace), C.byref(L) if L else None, _stream(stream)))


def jolt_dense_workspace_size(batch, n_kv, n_q, d, T, kernel=None, split_tokens=0):
    n = C.c_size_t()
    L = _launch(kernel, split_tokens)
    _check(lib().jolt_dense_workspace_size(batch, n_kv, n_q, d, T, C.byref(L) if L else None,
                                           C.byref(n)))
    return n.value


def jolt_dense_attention(k_rope, v, q, q_pos, inv_freq, softmax_scale, out, workspace,
                         split_tokens=0, stream=None):
    """k_rope, v: device [B, H, T, d] (f32/bf16); q: [B, H_q, d]; out f32."""
    B, H, T, d = k_rope.shape
    qp = (C.c_int32 * max(1, B))(*[int(x) for x in q_pos])
    inv = np.ascontiguousarray(inv_freq, dtype=np.float32)
    L = _launch(None, split_tokens)
    _check(lib().jolt_dense_attention(
        _ptr(k_rope), _ptr(v), _dtype_code(k_rope), B, H, q.shape[1], d, T, _ptr(q),
        _dtype_code(q), qp, inv.ctypes.data_as(C.POINTER(C.c_float)), C.c_float(softmax_scale),
        _ptr(out), _ptr(workspace), _nbytes(workspace), C.byref(L) if L else None,
        _stream(stream)))


def jolt_make_rotation(seed, d):
    out = np.empty((d, d), dtype=np.float64)
    _check(lib().jolt_make_rotation(C.c_uint64(seed), d, out.ctypes.data_as(C.POINTER(C.c_double))))
    return out


def jolt_debug_unpack(cache, layer, tau, stream=None):
    m = cache.meta
    out = np.empty((m["H"], m["T"], m["d"]), dtype=np.uint8)
    _check(lib().jolt_debug_unpack(cache.handle, layer, tau, out.ctypes.data, _stream(stream)))
    return out


def jolt_debug_sincos(angles, variant=0):
    x = np.ascontiguousarray(angles, dtype=np.float32)
    sn, cs = np.empty_like(x), np.empty_like(x)
    _check(lib().jolt_debug_sincos(x.ctypes.data, x.size, sn.ctypes.data, cs.ctypes.data,
                                   int(variant)))
    return sn, cs

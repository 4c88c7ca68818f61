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


class jolt_flash_params(C.Structure):
    _fields_ = [("q_cap", C.c_int32), ("oversample", C.c_int32), ("power_iters", C.c_int32),
                ("sketch_seed", C.c_uint64)]


class jolt_alloc_cell(C.Structure):
    _fields_ = [("T", C.c_int32), ("d", C.c_int32), ("group_size", C.c_int32),
                ("n_kv_heads", C.c_int32), ("factor_bytes", C.c_int32),
                ("n_sT2", C.c_int32), ("sT2", C.POINTER(C.c_double)),
                ("n_sF2", C.c_int32), ("sF2", C.POINTER(C.c_double)),
                ("norm2", C.c_double), ("cap", C.c_int32)]


class jolt_launch(C.Structure):
    _fields_ = [("kernel", C.c_int32), ("split_tokens", C.c_int32),
                ("ev_begin", C.c_void_p), ("ev_end", C.c_void_p),
                ("deterministic", C.c_int32)]


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
    "jolt_decode_tail_workspace_size": (C.c_int, [C.POINTER(C.c_void_p), C.c_int32, C.c_int32,
                                                  C.c_int32, C.POINTER(jolt_launch),
                                                  C.POINTER(C.c_size_t)]),
    "jolt_decode_attention_tail": (C.c_int, [C.POINTER(C.c_void_p), C.c_int32, C.c_int32,
                                             C.c_void_p, C.c_int, C.POINTER(C.c_int32),
                                             C.POINTER(C.c_float), C.c_float, C.c_void_p,
                                             C.c_void_p, C.c_int, C.c_int32,
                                             C.POINTER(C.c_int32), C.c_void_p, C.c_void_p,
                                             C.c_size_t, C.POINTER(jolt_launch), C.c_void_p]),
    "jolt_dense_workspace_size": (C.c_int, [C.c_int32] * 5 + [C.POINTER(jolt_launch),
                                                              C.POINTER(C.c_size_t)]),
    "jolt_dense_attention": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int] + [C.c_int32] * 5 +
                             [C.c_void_p, C.c_int, C.POINTER(C.c_int32), C.POINTER(C.c_float),
                              C.c_float, C.c_void_p, C.c_void_p, C.c_size_t,
                              C.POINTER(jolt_launch), C.c_void_p]),
    "jolt_flash_spectra": (C.c_int, [C.c_void_p, C.c_int, C.c_int32, C.c_int32, C.c_int32,
                                     C.c_int32, C.POINTER(jolt_flash_params), C.c_void_p,
                                     C.c_void_p, C.c_void_p, C.c_void_p]),
    "jolt_flash_compress_cell": (C.c_int, [C.c_void_p, C.c_int, C.c_int32, C.c_int32, C.c_int32,
                                           C.c_int32, C.POINTER(jolt_flash_params), C.c_int32,
                                           C.c_int32, C.c_int32, C.c_uint64, C.c_int, C.c_void_p,
                                           C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                           C.c_void_p]),
    "jolt_quantize_rows": (C.c_int, [C.c_void_p, C.c_int64, C.c_int32, C.c_int32, C.c_void_p,
                                     C.c_void_p, C.c_void_p]),
    "jolt_noalloc_scratch_bytes": (C.c_size_t, []),
    "jolt_decode_attention_noalloc": (C.c_int, [C.POINTER(C.c_void_p), C.c_int32, C.c_int32,
                                                C.c_void_p, C.c_int, C.POINTER(C.c_int32),
                                                C.POINTER(C.c_float), C.c_float, C.c_void_p,
                                                C.POINTER(jolt_launch), C.c_void_p]),
    "jolt_allocate": (C.c_int, [C.POINTER(jolt_alloc_cell), C.c_int32, C.c_double,
                                C.POINTER(C.c_int32), C.POINTER(C.c_double)]),
    "jolt_flash_layer_groups": (C.c_int, [C.POINTER(C.c_void_p), C.POINTER(C.c_void_p), C.c_int,
                                          C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                          C.POINTER(jolt_flash_params), C.c_double, C.c_int32,
                                          C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                          C.POINTER(C.c_double), C.c_void_p]),
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


def _launch(kernel=None, split_tokens=0, events=None, deterministic=False):
    if kernel is None and not split_tokens and events is None and not deterministic:
        return None
    ev = events or (None, None)
    return jolt_launch(int(kernel or 0), int(split_tokens), ev[0], ev[1], int(bool(deterministic)))


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


def _check_tensor(name, t, dtypes, shape):
    """Shape, dtype, device and layout rules of a device tensor argument (the
    library takes raw pointers and cannot check them itself)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _inv_freq(inv_freq, d):
    inv = np.ascontiguousarray(inv_freq, dtype=np.float32).ravel()
    if inv.size < d // 2:
        raise ValueError(f"inv_freq has {inv.size} values, needs d/2 = {d // 2}")
    return inv


def _workspace(ws):
    import torch
    if ws is None:
        return ws
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return ws


def jolt_decode_attention(caches, layer, q, q_pos, inv_freq, softmax_scale, out, workspace,
                          kernel=None, split_tokens=0, stream=None, events=None,
                          deterministic=False):
    """q: device tensor [B, H_q, d] (f32/bf16); out: device f32 [B, H_q, d];
    workspace: device tensor of at least jolt_decode_workspace_size bytes;
    events: optional (begin, end) raw hipEvent_t handles recorded around the
    split-T kernel; deterministic: fixed block schedule (bitwise repeatable)."""
    import torch
    B = len(caches)
    if B:
        m = caches[0].meta
        shape = (B, m["H_q"], m["d"])
        _check_tensor("q", q, (torch.float32, torch.bfloat16), shape)
        _check_tensor("out", out, (torch.float32,), shape)
        if len(q_pos) != B:
            raise ValueError(f"q_pos has {len(q_pos)} entries for {B} sequences")
        inv = _inv_freq(inv_freq, m["d"])
    else:
        inv = np.zeros(1, dtype=np.float32)
    qp = (C.c_int32 * max(1, B))(*[int(x) for x in q_pos])
    L = _launch(kernel, split_tokens, events, deterministic)
    _check(lib().jolt_decode_attention(
        _handles(caches), B, layer, _ptr(q), _dtype_code(q), qp,
        inv.ctypes.data_as(C.POINTER(C.c_float)), C.c_float(softmax_scale), _ptr(out),
        _ptr(_workspace(workspace)), _nbytes(workspace), C.byref(L) if L else None,
        _stream(stream)))


def jolt_noalloc_scratch_bytes():
    return int(lib().jolt_noalloc_scratch_bytes())


def jolt_decode_attention_noalloc(caches, layer, q, q_pos, inv_freq, softmax_scale, out,
                                  kernel=None, split_tokens=0, stream=None, deterministic=False):
    """jolt_decode_attention with the split partials in the library's own
    static device buffer (no workspace argument, no allocation)."""
    import torch
    B = len(caches)
    if B:
        m = caches[0].meta
        shape = (B, m["H_q"], m["d"])
        _check_tensor("q", q, (torch.float32, torch.bfloat16), shape)
        _check_tensor("out", out, (torch.float32,), shape)
        if len(q_pos) != B:
            raise ValueError(f"q_pos has {len(q_pos)} entries for {B} sequences")
        inv = _inv_freq(inv_freq, m["d"])
    else:
        inv = np.zeros(1, dtype=np.float32)
    qp = (C.c_int32 * max(1, B))(*[int(x) for x in q_pos])
    L = _launch(kernel, split_tokens, None, deterministic)
    _check(lib().jolt_decode_attention_noalloc(
        _handles(caches), B, layer, _ptr(q), _dtype_code(q), qp,
        inv.ctypes.data_as(C.POINTER(C.c_float)), C.c_float(softmax_scale), _ptr(out),
        C.byref(L) if L else None, _stream(stream)))


def jolt_decode_tail_workspace_size(caches, layer, tail_cap, kernel=None, split_tokens=0):
    n = C.c_size_t()
    L = _launch(kernel, split_tokens)
    _check(lib().jolt_decode_tail_workspace_size(_handles(caches), len(caches), layer,
                                                 int(tail_cap), C.byref(L) if L else None,
                                                 C.byref(n)))
    return n.value


def jolt_decode_attention_tail(caches, layer, q, q_pos, inv_freq, softmax_scale, k_tail, v_tail,
                               tail_len, out, workspace, kernel=None, split_tokens=0,
                               stream=None, deterministic=False):
    """As jolt_decode_attention, plus an uncompressed tail: k_tail / v_tail
    device [B, H, tail_cap, d] (f32/bf16, keys already rotated to their
    positions), tail_len [B] valid rows per sequence."""
    import torch
    B = len(caches)
    if B == 0:
        return
    m = caches[0].meta
    shape = (B, m["H_q"], m["d"])
    _check_tensor("q", q, (torch.float32, torch.bfloat16), shape)
    _check_tensor("out", out, (torch.float32,), shape)
    cap = k_tail.shape[2]
    _check_tensor("k_tail", k_tail, (torch.float32, torch.bfloat16), (B, m["H"], cap, m["d"]))
    _check_tensor("v_tail", v_tail, (k_tail.dtype,), (B, m["H"], cap, m["d"]))
    if len(q_pos) != B or len(tail_len) != B:
        raise ValueError("q_pos and tail_len need one entry per sequence")
    inv = _inv_freq(inv_freq, m["d"])
    qp = (C.c_int32 * B)(*[int(x) for x in q_pos])
    tl = (C.c_int32 * B)(*[int(x) for x in tail_len])
    L = _launch(kernel, split_tokens, None, deterministic)
    _check(lib().jolt_decode_attention_tail(
        _handles(caches), B, layer, _ptr(q), _dtype_code(q), qp,
        inv.ctypes.data_as(C.POINTER(C.c_float)), C.c_float(softmax_scale), _ptr(k_tail),
        _ptr(v_tail), _dtype_code(k_tail), int(cap), tl, _ptr(out), _ptr(_workspace(workspace)),
        _nbytes(workspace), C.byref(L) if L else None, _stream(stream)))


def jolt_dense_workspace_size(batch, n_kv, n_q, d, T, kernel=None, split_tokens=0):
    n = C.c_size_t()
    L = _launch(kernel, split_tokens)
    _check(lib().jolt_dense_workspace_size(batch, n_kv, n_q, d, T, C.byref(L) if L else None,
                                           C.byref(n)))
    return n.value


def jolt_dense_attention(k_rope, v, q, q_pos, inv_freq, softmax_scale, out, workspace,
                         split_tokens=0, stream=None):
    """k_rope, v: device [B, H, T, d] (f32/bf16); q: [B, H_q, d]; out f32."""
    import torch
    B, H, T, d = k_rope.shape
    Hq = q.shape[1]
    _check_tensor("k_rope", k_rope, (torch.float32, torch.bfloat16), (B, H, T, d))
    _check_tensor("v", v, (k_rope.dtype,), (B, H, T, d))
    _check_tensor("q", q, (torch.float32, torch.bfloat16), (B, Hq, d))
    _check_tensor("out", out, (torch.float32,), (B, Hq, d))
    if len(q_pos) != B:
        raise ValueError(f"q_pos has {len(q_pos)} entries for {B} sequences")
    qp = (C.c_int32 * max(1, B))(*[int(x) for x in q_pos])
    inv = _inv_freq(inv_freq, d)
    L = _launch(None, split_tokens)
    _check(lib().jolt_dense_attention(
        _ptr(k_rope), _ptr(v), _dtype_code(k_rope), B, H, Hq, d, T, _ptr(q),
        _dtype_code(q), qp, inv.ctypes.data_as(C.POINTER(C.c_float)), C.c_float(softmax_scale),
        _ptr(out), _ptr(_workspace(workspace)), _nbytes(workspace), C.byref(L) if L else None,
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
    """variant 0/1: angles [n]; variant 2: (position, inv_freq) pairs [n, 2]."""
    x = np.ascontiguousarray(angles, dtype=np.float32)
    if variant == 2:
        if x.ndim != 2 or x.shape[1] != 2:
            raise ValueError("variant 2 takes (position, inv_freq) pairs of shape [n, 2]")
        n = x.shape[0]
    else:
        n = x.size
    sn, cs = np.empty(n, np.float32), np.empty(n, np.float32)
    _check(lib().jolt_debug_sincos(x.ctypes.data, n, sn.ctypes.data, cs.ctypes.data, int(variant)))
    return sn, cs


# ------------------------------------------------------------- compressor --
def _flash_params(q_cap, oversample, power_iters, sketch_seed):
    return jolt_flash_params(int(q_cap), int(oversample), int(power_iters), int(sketch_seed))


def _cell_tensor(X):
    import torch
    if not isinstance(X, torch.Tensor) or X.dim() != 4 or not X.is_cuda or not X.is_contiguous():
        raise ValueError("X must be a contiguous GPU tensor [group_size, H, T, d]")
    if X.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(X.dtype)
    return X


def jolt_flash_spectra(X, q_cap, oversample=16, power_iters=2, sketch_seed=0, stream=None):
    """FlashJoLT allocator inputs of one cell X (device [group_size, H, T, d]):
    (sT2 [q_cap + 1] with the synthetic tail entry last, sF2 [d], norm2)."""
    X = _cell_tensor(X)
    gs, H, T, d = X.shape
    sT2 = np.empty(q_cap + 1, dtype=np.float64)
    sF2 = np.empty(d, dtype=np.float64)
    n2 = C.c_double()
    P = _flash_params(q_cap, oversample, power_iters, sketch_seed)
    _check(lib().jolt_flash_spectra(_ptr(X), _dtype_code(X), gs, H, T, d, C.byref(P),
                                    sT2.ctypes.data, sF2.ctypes.data, C.addressof(n2),
                                    _stream(stream)))
    return sT2, sF2, n2.value


def jolt_flash_compress_cell(X, r_T, r_F, bits, q_cap, rotation_seed, factor_dtype="bf16",
                             oversample=16, power_iters=2, sketch_seed=0, stream=None):
    """Compress one cell X (device [group_size, H, T, d]) on the GPU.  Returns a
    cell dict as jolt_load_cache takes it: r_T, r_F, bits, A, B, G (float32
    arrays holding the stored factor values), codes (uint8) and scales."""
    X = _cell_tensor(X)
    gs, H, T, d = X.shape
    fdt = JOLT_F32 if factor_dtype == "f32" else JOLT_BF16
    sto = np.float32 if factor_dtype == "f32" else np.uint16
    A = np.zeros((T, r_T), dtype=sto)
    B = np.zeros((d, r_F), dtype=sto)
    G = np.zeros((gs, H, r_T, r_F), dtype=sto)
    codes = np.zeros((gs, H, T, d * bits // 8), dtype=np.uint8) if bits else None
    scales = np.zeros((gs, H, T), dtype=np.float32) if bits else None
    P = _flash_params(q_cap, oversample, power_iters, sketch_seed)
    _check(lib().jolt_flash_compress_cell(
        _ptr(X), _dtype_code(X), gs, H, T, d, C.byref(P), int(r_T), int(r_F), int(bits),
        C.c_uint64(int(rotation_seed)), fdt, A.ctypes.data, B.ctypes.data, G.ctypes.data,
        codes.ctypes.data if bits else None, scales.ctypes.data if bits else None,
        _stream(stream)))

    def vals(a):
        if factor_dtype == "f32":
            return a
        return (a.astype(np.uint32) << 16).view(np.float32)
    return {"r_T": int(r_T), "r_F": int(r_F), "bits": int(bits), "A": vals(A), "B": vals(B),
            "G": vals(G), "codes": codes, "scales": scales}


def jolt_quantize_rows(rows, bits, stream=None):
    """rows: device float64 [n, d] (rotated residual rows) -> (codes uint8
    [n, d*bits/8], scales float32 [n]) device tensors."""
    import torch
    if rows.dtype != torch.float64 or not rows.is_cuda or not rows.is_contiguous() or rows.dim() != 2:
        raise ValueError("rows must be a contiguous float64 GPU tensor [n, d]")
    n, d = rows.shape
    codes = torch.empty((n, d * bits // 8), dtype=torch.uint8, device=rows.device)
    scales = torch.empty((n,), dtype=torch.float32, device=rows.device)
    _check(lib().jolt_quantize_rows(_ptr(rows), n, d, int(bits), _ptr(codes), _ptr(scales),
                                    _stream(stream)))
    return codes, scales


def jolt_allocate(cells, budget):
    """cells: list of dicts with T, d, group_size, H, factor_bytes, sT2, sF2,
    norm2 and optional cap.  Returns ([(r_T, r_F, bits)], lambda)."""
    n = len(cells)
    arr = (jolt_alloc_cell * max(1, n))()
    keep = []
    for i, c in enumerate(cells):
        sT2 = np.ascontiguousarray(c["sT2"], dtype=np.float64)
        sF2 = np.ascontiguousarray(c["sF2"], dtype=np.float64)
        keep += [sT2, sF2]
        arr[i] = jolt_alloc_cell(int(c["T"]), int(c["d"]), int(c["group_size"]), int(c["H"]),
                                 int(c["factor_bytes"]), sT2.size,
                                 sT2.ctypes.data_as(C.POINTER(C.c_double)), sF2.size,
                                 sF2.ctypes.data_as(C.POINTER(C.c_double)), float(c["norm2"]),
                                 int(c.get("cap") or 0))
    out = (C.c_int32 * max(1, 3 * n))()
    lam = C.c_double()
    _check(lib().jolt_allocate(arr, n, C.c_double(float(budget)), out, C.byref(lam)))
    return [tuple(out[3 * i:3 * i + 3]) for i in range(n)], lam.value


def jolt_flash_layer_groups(k_layers, v_layers, r, tau, max_group=0, oversample=16,
                            power_iters=2, sketch_seed=0, stream=None):
    """Alignment-based grouping of consecutive layers: k_layers[l], v_layers[l]
    device tensors [H, T, d].  Returns (group_start, alignments)."""
    import torch
    n = len(k_layers)
    if n < 1 or len(v_layers) != n:
        raise ValueError("one key and one value tensor per layer")
    H, T, d = k_layers[0].shape
    for t in list(k_layers) + list(v_layers):
        _check_tensor("layer", t, (k_layers[0].dtype,), (H, T, d))
    ks = (C.c_void_p * n)(*[t.data_ptr() for t in k_layers])
    vs = (C.c_void_p * n)(*[t.data_ptr() for t in v_layers])
    starts = (C.c_int32 * (n + 1))()
    ng = C.c_int32()
    al = (C.c_double * max(1, n - 1))()
    P = _flash_params(r, oversample, power_iters, sketch_seed)
    _check(lib().jolt_flash_layer_groups(ks, vs, _dtype_code(k_layers[0]), n, H, T, d,
                                         C.byref(P), C.c_double(tau), int(max_group), starts,
                                         C.byref(ng), al, _stream(stream)))
    return list(starts[:ng.value + 1]), list(al[:n - 1])

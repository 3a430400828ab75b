"""Python binding of libcacheblend.so (C ABI in include/cacheblend.h).

Argument marshalling only: every step of the fusion path runs in the HIP
kernels of the library.  PyTorch tensors are accepted for device memory and
`torch.cuda` streams; they are passed to the library as raw pointers.  There
is no fallback: importing this package fails when the library is not built.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# CACHEBLEND_LIB selects another build of the same library (e.g. the
# host-sanitized one the CPU tests load)
LIB_PATH = os.environ.get("CACHEBLEND_LIB") or os.path.join(_HERE, "libcacheblend.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python non_prefix_kv_amd/build.py` (hipcc, gfx950)")
_lib = ctypes.CDLL(LIB_PATH)

# ------------------------------------------------------------------ constants
CB_ABI_VERSION = 6
CB_OK, CB_E_INVALID, CB_E_SHAPE, CB_E_NOT_PINNED, CB_E_SCHEDULE = 0, -1, -2, -3, -4
CB_E_OOM, CB_E_HIP, CB_E_BAD_STATE, CB_E_UNSUPPORTED = -5, -6, -7, -8
CB_F32, CB_BF16 = 0, 1
CB_SCHED_GRADUAL, CB_SCHED_FIXED = 0, 1
CB_DEV_KV, CB_DEV_K, CB_DEV_V, CB_DEV_GIVEN, CB_DEV_ATTN = 0, 1, 2, 3, 4
CB_KV_PLAIN, CB_KV_U8, CB_KV_U4 = 0, 1, 2

_c_i32, _c_i64, _c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p


class cb_model_cfg(ctypes.Structure):
    _fields_ = [("n_layers", _c_i32), ("d_model", _c_i32), ("n_q_heads", _c_i32),
                ("n_kv_heads", _c_i32), ("head_dim", _c_i32), ("ffn_dim", _c_i32),
                ("rope_base", ctypes.c_double), ("rms_eps", ctypes.c_float),
                ("dtype", _c_i32)]


class cb_layer_weights(ctypes.Structure):
    _fields_ = [(n, _c_p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm",
                                     "w_gate", "w_up", "w_down")]


class cb_chunk_kv(ctypes.Structure):
    _fields_ = [("k", _c_p), ("v", _c_p), ("n_tokens", _c_i32), ("on_host", _c_i32),
                ("layer_stride", _c_i64), ("kv_format", _c_i32), ("reserved", _c_i32),
                ("qparams", _c_p), ("stage_k", _c_p), ("stage_v", _c_p),
                ("stage_qparams", _c_p)]


class cb_request(ctypes.Structure):
    _fields_ = [("n_chunks", _c_i32), ("chunks", ctypes.POINTER(cb_chunk_kv)),
                ("chunk_offsets", ctypes.POINTER(_c_i32)), ("n_suffix", _c_i32),
                ("x0", _c_p), ("schedule", ctypes.POINTER(_c_i32)),
                ("recompute_bp", _c_i32), ("schedule_kind", _c_i32), ("dev_mode", _c_i32),
                ("min_tokens", _c_i32), ("given_scores", _c_p)]


class cb_outputs(ctypes.Structure):
    _fields_ = [("fused_k", _c_p), ("fused_v", _c_p), ("sel_idx", _c_p),
                ("sel_count", ctypes.POINTER(_c_i32)), ("hidden_out", _c_p),
                ("deviation", _c_p)]


class cb_batch_item(ctypes.Structure):
    _fields_ = [("n_chunks", _c_i32), ("chunk_ids", ctypes.POINTER(_c_i32)),
                ("n_suffix", _c_i32), ("schedule", ctypes.POINTER(_c_i32))]


class cb_batch_request(ctypes.Structure):
    _fields_ = [("n_pool", _c_i32), ("pool", ctypes.POINTER(cb_chunk_kv)),
                ("n_requests", _c_i32), ("items", ctypes.POINTER(cb_batch_item)),
                ("x0", _c_p), ("recompute_bp", _c_i32), ("schedule_kind", _c_i32),
                ("dev_mode", _c_i32), ("min_tokens", _c_i32), ("given_scores", _c_p)]


class cb_batch_outputs(ctypes.Structure):
    _fields_ = [("fused_k", _c_p), ("fused_v", _c_p), ("sel_idx", _c_p),
                ("sel_count", ctypes.POINTER(_c_i32)), ("hidden_out", _c_p),
                ("deviation", _c_p)]


class cb_kernel_stat(ctypes.Structure):
    _fields_ = [("launches", _c_i64), ("total_ms", ctypes.c_double), ("flops", ctypes.c_double),
                ("bytes", ctypes.c_double)]


class cb_cache_stat(ctypes.Structure):
    _fields_ = [(n, _c_i64) for n in ("lookups", "hits", "admitted", "evicted",
                                       "resident_entries", "resident_bytes", "copied_bytes")]


KERNEL_CLASSES = ("rotate", "rmsnorm", "gemm_qkv", "deviation", "select", "scatter",
                  "attention", "gemm_o", "gemm_gateup", "gemm_down", "decode_gemv",
                  "decode_attention")


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_P = ctypes.POINTER
_fn = {
    "cb_abi_version": (ctypes.c_int,),
    "cb_last_error": (ctypes.c_char_p,),
    "cb_schedule": (ctypes.c_int, _c_i32, _c_i32, _c_i32, _c_i32, _P(_c_i32)),
    "cb_model_create": (ctypes.c_int, _P(cb_model_cfg), _P(cb_layer_weights), _c_p, _P(_c_p)),
    "cb_model_set_workspace": (ctypes.c_int, _c_p, _c_p, _c_i64),
    "cb_workspace_size": (ctypes.c_int, _c_p, _P(cb_request), _P(_c_i64)),
    "cb_model_destroy": (None, _c_p),
    "cb_blend": (ctypes.c_int, _c_p, _P(cb_request), _P(cb_outputs), _c_p),
    "cb_plan_create": (ctypes.c_int, _c_p, _P(cb_request), _P(cb_outputs), _c_p, _P(_c_p)),
    "cb_fetch_kv": (ctypes.c_int, _c_p, _c_i32),
    "cb_prefill_layer": (ctypes.c_int, _c_p, _c_i32),
    "cb_synchronize": (ctypes.c_int, _c_p),
    "cb_plan_destroy": (None, _c_p),
    "cb_blend_batch": (ctypes.c_int, _c_p, _P(cb_batch_request), _P(cb_batch_outputs), _c_p),
    "cb_prefill": (ctypes.c_int, _c_p, _c_p, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p),
    "cb_controller_ratio": (ctypes.c_int, ctypes.c_double, ctypes.c_double, _c_i64,
                            ctypes.c_double, _c_i32, _P(_c_i32)),
    "cb_cache_create": (ctypes.c_int, _c_i32, _c_i32, _c_i32, _c_i64, _P(_c_p)),
    "cb_cache_destroy": (None, _c_p),
    "cb_cache_resolve": (ctypes.c_int, _c_p, _c_i32, _P(ctypes.c_uint64), _P(cb_chunk_kv),
                         _P(cb_chunk_kv), _P(_c_i32), _c_p),
    "cb_cache_commit": (ctypes.c_int, _c_p, _c_i32, _P(ctypes.c_uint64)),
    "cb_cache_stats": (ctypes.c_int, _c_p, _P(cb_cache_stat)),
    "cb_cache_replay": (ctypes.c_int, _c_i64, _c_i32, _P(_c_i32), _P(ctypes.c_uint64),
                        _P(_c_i64), _P(_c_i32), _P(ctypes.c_uint64), _P(_c_i32)),
    "cb_lm_head": (ctypes.c_int, _c_p, _c_p, _c_i32, _c_p, _c_p, _c_i32, _c_p, _c_p, _c_p),
    "cb_decode_step": (ctypes.c_int, _c_p, _c_p, _c_i32, _c_p, _c_p, _c_i64, _c_p, _c_p, _c_p,
                       _c_p),
    "cb_profile_enable": (ctypes.c_int, _c_p, _c_i32),
    "cb_profile_read": (ctypes.c_int, _c_p, _P(cb_kernel_stat)),
    "cb_rope_rerotate": (ctypes.c_int, _c_i32, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32,
                         _c_i32, ctypes.c_double, _c_p),
    "cb_quantize_kv": (ctypes.c_int, _c_i32, _c_p, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _c_p,
                       _c_p, _c_p, _c_i64, _c_p),
    "cb_dequant_rerotate": (ctypes.c_int, _c_i32, _c_i32, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i32,
                            _c_i32, _c_i32, _c_i32, ctypes.c_double, _c_p),
    "cb_deviation": (ctypes.c_int, _c_i32, _c_p, _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_p,
                     _c_p),
    "cb_attention_deviation": (ctypes.c_int, _c_i32, _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32,
                               _c_i32, _c_p, _c_p),
    "cb_topk_select": (ctypes.c_int, _c_p, _c_i32, _c_i32, _c_p, _c_p),
    "cb_gather_rows": (ctypes.c_int, _c_p, _c_p, _c_p, _c_i32, _c_i64, _c_p),
    "cb_scatter_rows": (ctypes.c_int, _c_p, _c_p, _c_p, _c_i32, _c_i64, _c_p),
    "cb_rmsnorm": (ctypes.c_int, _c_i32, _c_p, _c_i32, _c_p, _c_p, _c_i32, _c_i32,
                   ctypes.c_float, _c_p),
    "cb_gemm": (ctypes.c_int, _c_i32, _c_p, _c_p, _c_p, _c_i32, _c_i32, _c_i32, _c_p),
    "cb_attention": (ctypes.c_int, _c_i32, _c_p, _c_p, _c_i32, _c_p, _c_p, _c_i32, _c_i32,
                     _c_i32, _c_i32, _c_p, _c_p),
    "cb_attention_noalloc": (ctypes.c_int, _c_i32, _c_p, _c_p, _c_i32, _c_p, _c_p, _c_i32,
                             _c_i32, _c_i32, _c_i32, _c_p, _c_p),
}
CB_NOALLOC_SCRATCH_BYTES = 80 << 20
RAW = {name: _sig(name, spec[0], *spec[1:]) for name, spec in _fn.items()}
EXPORTED = tuple(_fn)


class CBError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"cacheblend status {status}: {msg}")
        self.status = status


def _check(st):
    if st != CB_OK:
        raise CBError(st, RAW["cb_last_error"]().decode())
    return st


def _ptr(t):
    """Raw address of a tensor / int / None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _need(t, name, dtype=None, numel=0, device=True):
    """Argument checks before a raw pointer crosses the ABI: the library
    cannot see the size behind a pointer, so a tensor that is too small, of
    the wrong element type, not contiguous or on the wrong side would be
    written past instead of rejected.  Failures raise CBError with the
    library's codes (CB_E_INVALID for the kind of buffer, CB_E_SHAPE for its
    size).  Plain integers are addresses the caller vouches for and are
    passed as they are."""
    if t is None or isinstance(t, int):
        return
    import torch
    if not isinstance(t, torch.Tensor):
        raise CBError(CB_E_INVALID, f"{name}: expected a tensor or an address, "
                                    f"got {type(t).__name__}")
    if device and not t.is_cuda:
        raise CBError(CB_E_INVALID, f"{name} must be a device tensor")
    if not device and t.is_cuda:
        raise CBError(CB_E_INVALID, f"{name} must be a host tensor")
    if not t.is_contiguous():
        raise CBError(CB_E_INVALID, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise CBError(CB_E_INVALID, f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() < numel:
        raise CBError(CB_E_SHAPE, f"{name} holds {t.numel()} elements, needs at least {numel}")


def _torch_dtype(code):
    import torch
    return torch.float32 if code == CB_F32 else torch.bfloat16


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return CB_F32
    if t.dtype == torch.bfloat16:
        return CB_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------------------ basics
def cb_abi_version():
    return RAW["cb_abi_version"]()


def cb_last_error():
    return RAW["cb_last_error"]().decode()


def cb_schedule(n_chunk_tokens, recompute_bp, kind, n_layers):
    out = (_c_i32 * (n_layers + 1))()
    _check(RAW["cb_schedule"](n_chunk_tokens, recompute_bp, kind, n_layers, out))
    return list(out)


# ------------------------------------------------------------------ model
class Model:
    """cb_model over torch weight tensors (kept referenced for its lifetime).

    layers: list of dicts with attn_norm, wq, wk, wv, wo, mlp_norm, w_gate,
    w_up, w_down as contiguous device tensors of one dtype.
    """

    def __init__(self, n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim,
                 layers, rope_base=10000.0, rms_eps=1e-5, dtype=None, final_norm=None):
        if dtype is None:
            dtype = _dtype_code(layers[0]["wq"])
        self.cfg = cb_model_cfg(n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim,
                                rope_base, rms_eps, dtype)
        self._keep = layers
        arr = (cb_layer_weights * n_layers)()
        for i, w in enumerate(layers):
            for f, _ in cb_layer_weights._fields_:
                t = w[f]
                if not t.is_contiguous():
                    raise ValueError(f"layer {i} {f} is not contiguous")
                setattr(arr[i], f, t.data_ptr())
        h = _c_p()
        if final_norm is not None:
            _need(final_norm, "final_norm", _torch_dtype(dtype), d_model)
        self._final_norm = final_norm
        _check(RAW["cb_model_create"](ctypes.byref(self.cfg), arr, _ptr(final_norm),
                                      ctypes.byref(h)))
        self.handle = h
        self._ws = None

    def set_workspace(self, ws=None, nbytes=0):
        """Plans carve their workspace from the device buffer ws (a tensor
        kept referenced here, or an address) of nbytes bytes; ws None with
        nbytes > 0 limits pool allocations to nbytes; (None, 0) restores the
        default."""
        if ws is not None and not isinstance(ws, int):
            _need(ws, "workspace")
            nbytes = nbytes or ws.numel() * ws.element_size()
        self._ws = ws
        _check(RAW["cb_model_set_workspace"](self.handle, _ptr(ws), int(nbytes)))

    def workspace_size(self, chunks, offsets, n_suffix, x0, schedule=None, recompute_bp=1500,
                       schedule_kind=CB_SCHED_GRADUAL, dev_mode=CB_DEV_KV, min_tokens=0,
                       given_scores=None):
        """Bytes of workspace cb_blend needs for this request."""
        req, keep = _request(chunks, offsets, n_suffix, x0, schedule, recompute_bp,
                             schedule_kind, dev_mode, min_tokens, given_scores)
        out = _c_i64()
        _check(RAW["cb_workspace_size"](self.handle, ctypes.byref(req), ctypes.byref(out)))
        del keep
        return out.value

    def close(self):
        if getattr(self, "handle", None):
            RAW["cb_model_destroy"](self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _chunk_array(chunks):
    """chunks: list of dicts {k, v, n_tokens, on_host, layer_stride} with
    tensors or ints, plus kv_format (CB_KV_U8 / CB_KV_U4) and qparams for
    quantized chunks."""
    if isinstance(chunks, ctypes.Array):
        return chunks
    arr = (cb_chunk_kv * max(1, len(chunks)))()
    for i, c in enumerate(chunks):
        arr[i].k = _ptr(c["k"])
        arr[i].v = _ptr(c["v"])
        arr[i].n_tokens = c["n_tokens"]
        arr[i].on_host = int(c.get("on_host", 0))
        arr[i].layer_stride = c["layer_stride"]
        arr[i].kv_format = int(c.get("kv_format", CB_KV_PLAIN))
        arr[i].qparams = _ptr(c.get("qparams"))
        arr[i].stage_k = _ptr(c.get("stage_k"))
        arr[i].stage_v = _ptr(c.get("stage_v"))
        arr[i].stage_qparams = _ptr(c.get("stage_qparams"))
    return arr


def _check_chunks(model, chunks, what="chunk"):
    """Element type, memory side and extent of chunk descriptors given as
    dicts of tensors (a resolved descriptor array is passed unchecked)."""
    import torch
    if isinstance(chunks, ctypes.Array):
        return
    L = model.cfg.n_layers
    row = model.cfg.n_kv_heads * model.cfg.head_dim
    for i, c in enumerate(chunks):
        fmt = int(c.get("kv_format", CB_KV_PLAIN))
        n, stride = int(c["n_tokens"]), int(c["layer_stride"])
        on_host = bool(c.get("on_host", 0))
        if fmt == CB_KV_PLAIN:
            dt, need = _torch_dtype(model.cfg.dtype), (L - 1) * stride + n * row
        else:
            per = 1 if fmt == CB_KV_U8 else 2
            dt, need = torch.uint8, ((L - 1) * stride + n * row) // per
            _need(c.get("qparams"), f"{what} {i} qparams", torch.float32, L * 4 * row,
                  device=not on_host)
        for key in ("k", "v"):
            _need(c[key], f"{what} {i} {key}", dt, need, device=not on_host)


def _schedule_last(model, n_chunk, n_tokens, schedule, recompute_bp, schedule_kind, min_tokens):
    """s[L] of a request (the schedule the library derives, or the caller's)."""
    L = model.cfg.n_layers
    if min_tokens > 0 and n_tokens < min_tokens:
        return n_chunk
    if schedule is not None:
        if len(schedule) != L + 1:
            raise CBError(CB_E_SCHEDULE,
                          f"schedule has {len(schedule)} entries, needs n_layers + 1 = {L + 1}")
        return int(schedule[-1])
    return cb_schedule(n_chunk, recompute_bp, schedule_kind, L)[-1]


def _check_blend_args(model, chunks, n_suffix, x0, fused_k, fused_v, sel_idx, hidden_out,
                      deviation, schedule, recompute_bp, schedule_kind, min_tokens, given_scores):
    import torch
    cfg = model.cfg
    L, d, row = cfg.n_layers, cfg.d_model, cfg.n_kv_heads * cfg.head_dim
    nc = sum(int(c["n_tokens"]) for c in chunks) if not isinstance(chunks, ctypes.Array) \
        else sum(chunks[i].n_tokens for i in range(len(chunks)))
    n = nc + n_suffix
    mdt = _torch_dtype(cfg.dtype)
    _check_chunks(model, chunks)
    _need(x0, "x0", mdt, n * d)
    _need(fused_k, "fused_k", mdt, L * n * row)
    _need(fused_v, "fused_v", mdt, L * n * row)
    _need(sel_idx, "sel_idx", torch.int32, L * nc)
    _need(deviation, "deviation", torch.float32, L * nc)
    _need(given_scores, "given_scores", torch.float32, nc)
    last = _schedule_last(model, nc, n, schedule, recompute_bp, schedule_kind, min_tokens)
    _need(hidden_out, "hidden_out", torch.float32, (last + n_suffix) * d)


def _request(chunks, offsets, n_suffix, x0, schedule, recompute_bp, schedule_kind, dev_mode,
             min_tokens, given_scores=None):
    arr = _chunk_array(chunks)
    offs = (_c_i32 * max(1, len(offsets)))(*offsets)
    sched = None
    if schedule is not None:
        sched = (_c_i32 * len(schedule))(*schedule)
    req = cb_request(len(chunks), arr, offs, n_suffix, _ptr(x0),
                     sched if sched is not None else ctypes.POINTER(_c_i32)(),
                     recompute_bp, schedule_kind, dev_mode, min_tokens, _ptr(given_scores))
    return req, (arr, offs, sched)


def _outputs(fused_k, fused_v, sel_idx, sel_count, hidden_out, deviation):
    return cb_outputs(_ptr(fused_k), _ptr(fused_v), _ptr(sel_idx),
                      sel_count if sel_count is not None else ctypes.POINTER(_c_i32)(),
                      _ptr(hidden_out), _ptr(deviation))


def cb_blend(model, chunks, offsets, n_suffix, x0, fused_k, fused_v, sel_idx=None,
             hidden_out=None, deviation=None, schedule=None, recompute_bp=1500,
             schedule_kind=CB_SCHED_GRADUAL, dev_mode=CB_DEV_KV, min_tokens=0, stream=None,
             given_scores=None):
    """Queues one fusion; returns the host list sel_count[l] = s[l+1]."""
    _check_blend_args(model, chunks, n_suffix, x0, fused_k, fused_v, sel_idx, hidden_out,
                      deviation, schedule, recompute_bp, schedule_kind, min_tokens, given_scores)
    req, keep = _request(chunks, offsets, n_suffix, x0, schedule, recompute_bp, schedule_kind,
                         dev_mode, min_tokens, given_scores)
    L = model.cfg.n_layers
    cnt = (_c_i32 * L)()
    out = _outputs(fused_k, fused_v, sel_idx, cnt, hidden_out, deviation)
    _check(RAW["cb_blend"](model.handle, ctypes.byref(req), ctypes.byref(out), _stream(stream)))
    del keep
    return list(cnt)


def cb_blend_batch(model, pool, requests, x0, fused_k, fused_v, sel_idx=None, hidden_out=None,
                   deviation=None, recompute_bp=1500, schedule_kind=CB_SCHED_GRADUAL,
                   dev_mode=CB_DEV_KV, min_tokens=0, stream=None, given_scores=None):
    """Queues the fusion of a batch.  pool: chunk dicts as for cb_blend;
    requests: list of dicts {chunk_ids: [...], n_suffix, schedule (optional)}.
    Returns sel_count as a list per request of s_b[l+1]."""
    import torch
    cfg = model.cfg
    L, d, row = cfg.n_layers, cfg.d_model, cfg.n_kv_heads * cfg.head_dim
    if not isinstance(pool, ctypes.Array):
        _check_chunks(model, pool, "pool chunk")
        lens = [int(c["n_tokens"]) for c in pool]
    else:
        lens = [pool[i].n_tokens for i in range(len(pool))]
    nc_tot = n_tot = last_tot = 0
    ids_ok = all(0 <= i < len(lens) for r in requests for i in r["chunk_ids"])
    for r in requests if ids_ok else ():      # ids outside the pool: the library rejects them
        nc = sum(lens[i] for i in r["chunk_ids"])
        nc_tot += nc
        n_tot += nc + r["n_suffix"]
        last_tot += _schedule_last(model, nc, nc + r["n_suffix"], r.get("schedule"),
                                   recompute_bp, schedule_kind, min_tokens) + r["n_suffix"]
    mdt = _torch_dtype(cfg.dtype)
    if not ids_ok:
        n_tot = nc_tot = last_tot = 0
    _need(x0, "x0", mdt, n_tot * d)
    _need(fused_k, "fused_k", mdt, L * n_tot * row)
    _need(fused_v, "fused_v", mdt, L * n_tot * row)
    _need(sel_idx, "sel_idx", torch.int32, L * nc_tot)
    _need(deviation, "deviation", torch.float32, L * nc_tot)
    _need(given_scores, "given_scores", torch.float32, nc_tot)
    _need(hidden_out, "hidden_out", torch.float32, last_tot * d)
    parr = _chunk_array(pool)
    items = (cb_batch_item * len(requests))()
    keep = []
    for i, r in enumerate(requests):
        ids = (_c_i32 * max(1, len(r["chunk_ids"])))(*r["chunk_ids"])
        keep.append(ids)
        items[i].n_chunks = len(r["chunk_ids"])
        items[i].chunk_ids = ids
        items[i].n_suffix = r["n_suffix"]
        sch = r.get("schedule")
        if sch is not None:
            sa = (_c_i32 * len(sch))(*sch)
            keep.append(sa)
            items[i].schedule = sa
    req = cb_batch_request(len(pool), parr, len(requests), items, _ptr(x0), recompute_bp,
                           schedule_kind, dev_mode, min_tokens, _ptr(given_scores))
    L = model.cfg.n_layers
    cnt = (_c_i32 * (L * len(requests)))()
    out = cb_batch_outputs(_ptr(fused_k), _ptr(fused_v), _ptr(sel_idx), cnt, _ptr(hidden_out),
                           _ptr(deviation))
    _check(RAW["cb_blend_batch"](model.handle, ctypes.byref(req), ctypes.byref(out),
                                 _stream(stream)))
    del keep
    return [list(cnt[b * L:(b + 1) * L]) for b in range(len(requests))]


class Plan:
    """Layer-stepped fusion: cb_plan_create / cb_fetch_kv / cb_prefill_layer /
    cb_synchronize / cb_plan_destroy."""

    def __init__(self, model, chunks, offsets, n_suffix, x0, fused_k, fused_v, sel_idx=None,
                 hidden_out=None, deviation=None, schedule=None, recompute_bp=1500,
                 schedule_kind=CB_SCHED_GRADUAL, dev_mode=CB_DEV_KV, min_tokens=0,
                 stream=None, given_scores=None):
        self.handle = None
        _check_blend_args(model, chunks, n_suffix, x0, fused_k, fused_v, sel_idx, hidden_out,
                          deviation, schedule, recompute_bp, schedule_kind, min_tokens,
                          given_scores)
        req, self._keep = _request(chunks, offsets, n_suffix, x0, schedule, recompute_bp,
                                   schedule_kind, dev_mode, min_tokens, given_scores)
        self._cnt = (_c_i32 * model.cfg.n_layers)()
        out = _outputs(fused_k, fused_v, sel_idx, self._cnt, hidden_out, deviation)
        h = _c_p()
        _check(RAW["cb_plan_create"](model.handle, ctypes.byref(req), ctypes.byref(out),
                                     _stream(stream), ctypes.byref(h)))
        self.handle = h
        self.sel_count = list(self._cnt)

    def fetch_kv(self, layer):
        _check(RAW["cb_fetch_kv"](self.handle, layer))

    def prefill_layer(self, layer):
        _check(RAW["cb_prefill_layer"](self.handle, layer))

    def synchronize(self):
        _check(RAW["cb_synchronize"](self.handle))

    def destroy(self):
        if self.handle:
            RAW["cb_plan_destroy"](self.handle)
            self.handle = None


def cb_prefill(model, x0, n_tokens, pos0, k_out, v_out, hidden_out=None, stream=None):
    import torch
    cfg = model.cfg
    mdt = _torch_dtype(cfg.dtype)
    kv = cfg.n_layers * n_tokens * cfg.n_kv_heads * cfg.head_dim
    _need(x0, "x0", mdt, n_tokens * cfg.d_model)
    _need(k_out, "k_out", mdt, kv)
    _need(v_out, "v_out", mdt, kv)
    _need(hidden_out, "hidden_out", torch.float32, n_tokens * cfg.d_model)
    _check(RAW["cb_prefill"](model.handle, _ptr(x0), n_tokens, pos0, _ptr(k_out), _ptr(v_out),
                             _ptr(hidden_out), _stream(stream)))


# ------------------------------------------------------------------ first token
def cb_lm_head(model, x, rows, final_norm, w_lm, vocab, logits, argmax=None, stream=None):
    """logits [rows][vocab] = W_lm rmsnorm(x); argmax (int32 [rows]) optional."""
    _check(RAW["cb_lm_head"](model.handle, _ptr(x), rows, _ptr(final_norm), _ptr(w_lm), vocab,
                             _ptr(logits), _ptr(argmax), _stream(stream)))


def cb_decode_step(model, x, n_ctx, fused_k, fused_v, layer_rows, k_new, v_new, hidden_out,
                   stream=None):
    """One token (embedding x) at position n_ctx through every layer over the
    fused cache; writes its K/V per layer and the last layer's row."""
    _check(RAW["cb_decode_step"](model.handle, _ptr(x), n_ctx, _ptr(fused_k), _ptr(fused_v),
                                 layer_rows, _ptr(k_new), _ptr(v_new), _ptr(hidden_out),
                                 _stream(stream)))


# ------------------------------------------------------------------ chunk store
def cb_controller_ratio(t_prefill_s, per_token_kv_bytes, n_tokens, throughput_bytes_per_s,
                        r_min_bp=1500):
    """r* = max(r_min, T_load / T_prefill) in basis points."""
    out = _c_i32()
    _check(RAW["cb_controller_ratio"](t_prefill_s, per_token_kv_bytes, n_tokens,
                                      throughput_bytes_per_s, r_min_bp, ctypes.byref(out)))
    return out.value


def cb_cache_replay(capacity_bytes, batches):
    """batches: list of lists of (key, bytes).  Returns [(hit flags, evicted
    keys)] per batch, as the tier's policy decides them."""
    sizes = [len(b) for b in batches]
    total = sum(sizes)
    keys = (ctypes.c_uint64 * max(1, total))(*[k for b in batches for k, _ in b])
    nbytes = (_c_i64 * max(1, total))(*[n for b in batches for _, n in b])
    hits = (_c_i32 * max(1, total))()
    ev = (ctypes.c_uint64 * max(1, total))()
    per = (_c_i32 * max(1, len(batches)))()
    bs = (_c_i32 * max(1, len(batches)))(*sizes)
    _check(RAW["cb_cache_replay"](capacity_bytes, len(batches), bs, keys, nbytes, hits, ev, per))
    out, at, e = [], 0, 0
    for b, n in enumerate(sizes):
        out.append(([bool(hits[at + i]) for i in range(n)], [ev[e + j] for j in range(per[b])]))
        at += n
        e += per[b]
    return out


class ChunkCache:
    """cb_chunk_cache: HBM tier for pinned-host chunk caches.  Per request or
    batch: resolve, queue the fusion with the resolved descriptors, commit."""

    def __init__(self, n_layers, row, dtype, capacity_bytes):
        h = _c_p()
        _check(RAW["cb_cache_create"](n_layers, row, dtype, int(capacity_bytes), ctypes.byref(h)))
        self.handle = h

    def resolve(self, keys, chunks, stream=None):
        """Returns (resolved chunk array, hit flags) for cb_blend /
        cb_blend_batch (the array replaces the chunk dicts)."""
        n = len(chunks)
        arr = _chunk_array(chunks)
        out = (cb_chunk_kv * max(1, n))()
        hits = (_c_i32 * max(1, n))()
        ka = (ctypes.c_uint64 * max(1, n))(*keys)
        _check(RAW["cb_cache_resolve"](self.handle, n, ka, arr, out, hits, _stream(stream)))
        return out, [bool(hits[i]) for i in range(n)]

    def commit(self, keys):
        """After the fusion that reads the resolved descriptors is queued."""
        ka = (ctypes.c_uint64 * max(1, len(keys)))(*keys)
        _check(RAW["cb_cache_commit"](self.handle, len(keys), ka))

    def stats(self):
        st = cb_cache_stat()
        _check(RAW["cb_cache_stats"](self.handle, ctypes.byref(st)))
        return {n: getattr(st, n) for n, _ in cb_cache_stat._fields_}

    def close(self):
        if getattr(self, "handle", None):
            RAW["cb_cache_destroy"](self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def cb_profile_enable(model, enable=True):
    _check(RAW["cb_profile_enable"](model.handle, 1 if enable else 0))


def cb_profile_read(model):
    """{class name: {launches, total_ms, flops, bytes}} of the timed launches."""
    arr = (cb_kernel_stat * len(KERNEL_CLASSES))()
    _check(RAW["cb_profile_read"](model.handle, arr))
    return {n: {"launches": a.launches, "total_ms": a.total_ms, "flops": a.flops,
                "bytes": a.bytes} for n, a in zip(KERNEL_CLASSES, arr)}


# ------------------------------------------------------------------ kernel level
def cb_rope_rerotate(k_in, k_out, v_in, v_out, n_tokens, n_heads, head_dim, delta,
                     rope_base=10000.0, stream=None):
    _check(RAW["cb_rope_rerotate"](_dtype_code(k_in), _ptr(k_in), _ptr(k_out), _ptr(v_in),
                                   _ptr(v_out), n_tokens, n_heads, head_dim, delta, rope_base,
                                   _stream(stream)))


def cb_quantize_kv(x, n_layers, n_tokens, row, x_layer_stride, bits, codes, scale, zero,
                   param_stride, stream=None):
    _check(RAW["cb_quantize_kv"](_dtype_code(x), _ptr(x), n_layers, n_tokens, row,
                                 x_layer_stride, bits, _ptr(codes), _ptr(scale), _ptr(zero),
                                 param_stride, _stream(stream)))


def cb_dequant_rerotate(kv_format, k_codes, v_codes, qparams, k_out, v_out, n_tokens, n_heads,
                        head_dim, delta, rope_base=10000.0, stream=None):
    _check(RAW["cb_dequant_rerotate"](_dtype_code(k_out), kv_format, _ptr(k_codes),
                                      _ptr(v_codes), _ptr(qparams), _ptr(k_out), _ptr(v_out),
                                      n_tokens, n_heads, head_dim, delta, rope_base,
                                      _stream(stream)))


def quantize_chunk(k, v, bits, stream=None):
    """Device codes of a chunk cache k, v [L][n][H_kv][d_head] (model dtype):
    returns {k, v, qparams, kv_format, n_tokens, layer_stride} ready for
    cb_blend / cb_blend_batch (device-resident)."""
    import torch
    L, n = k.shape[0], k.shape[1]
    row = k.shape[2] * k.shape[3]
    kc = torch.empty((L, n, row * bits // 8), dtype=torch.uint8, device=k.device)
    vc = torch.empty_like(kc)
    qp = torch.empty((L, 4, row), dtype=torch.float32, device=k.device)
    for x, codes, j in ((k, kc, 0), (v, vc, 2)):
        cb_quantize_kv(x, L, n, row, n * row, bits, codes, qp[:, j], qp[:, j + 1], 4 * row,
                       stream)
    return {"k": kc, "v": vc, "qparams": qp, "n_tokens": n, "layer_stride": n * row,
            "kv_format": CB_KV_U8 if bits == 8 else CB_KV_U4}


def cb_deviation(k_new, v_new, k_cached, v_cached, n_rows, row_elems, dev_mode, dev_out,
                 stream=None):
    _check(RAW["cb_deviation"](_dtype_code(k_new), _ptr(k_new), _ptr(v_new), _ptr(k_cached),
                               _ptr(v_cached), n_rows, row_elems, dev_mode, _ptr(dev_out),
                               _stream(stream)))


def cb_attention_deviation(q, k_new, k_cached, n, n_q_heads, n_kv_heads, head_dim, dev_out,
                           stream=None):
    """Per-token attention deviation of n rows at positions 0..n-1 (bf16)."""
    import torch
    _need(dev_out, "dev_out", torch.float32, n)
    _check(RAW["cb_attention_deviation"](_dtype_code(q), _ptr(q), _ptr(k_new), _ptr(k_cached), n,
                                         n_q_heads, n_kv_heads, head_dim, _ptr(dev_out),
                                         _stream(stream)))


def cb_topk_select(dev, n, k, idx_out, stream=None):
    _check(RAW["cb_topk_select"](_ptr(dev), n, k, _ptr(idx_out), _stream(stream)))


def cb_gather_rows(src, dst, idx, n_rows, row_bytes, stream=None):
    _check(RAW["cb_gather_rows"](_ptr(src), _ptr(dst), _ptr(idx), n_rows, row_bytes,
                                 _stream(stream)))


def cb_scatter_rows(src, dst, idx, n_rows, row_bytes, stream=None):
    _check(RAW["cb_scatter_rows"](_ptr(src), _ptr(dst), _ptr(idx), n_rows, row_bytes,
                                  _stream(stream)))


def cb_rmsnorm(x, g, y, rows, d, eps=1e-5, stream=None):
    _check(RAW["cb_rmsnorm"](_dtype_code(x), _ptr(x), _dtype_code(y), _ptr(g), _ptr(y), rows, d,
                             eps, _stream(stream)))


def cb_gemm(a, b, c, m, n, k, stream=None):
    _check(RAW["cb_gemm"](_dtype_code(a), _ptr(a), _ptr(b), _ptr(c), m, n, k, _stream(stream)))


def cb_attention(q, q_pos, n_q, k, v, n_kv, n_q_heads, n_kv_heads, head_dim, out, stream=None):
    _check(RAW["cb_attention"](_dtype_code(q), _ptr(q), _ptr(q_pos), n_q, _ptr(k), _ptr(v), n_kv,
                               n_q_heads, n_kv_heads, head_dim, _ptr(out), _stream(stream)))


def cb_attention_noalloc(q, q_pos, n_q, k, v, n_kv, n_q_heads, n_kv_heads, head_dim, out,
                         stream=None):
    """cb_attention without any device allocation (fixed library scratch)."""
    _check(RAW["cb_attention_noalloc"](_dtype_code(q), _ptr(q), _ptr(q_pos), n_q, _ptr(k),
                                       _ptr(v), n_kv, n_q_heads, n_kv_heads, head_dim, _ptr(out),
                                       _stream(stream)))

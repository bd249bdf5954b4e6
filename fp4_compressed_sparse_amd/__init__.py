"""Python binding of the CSA2 FP4 decode-path library (libcsa2.so, gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in include/csa2.h.  PyTorch supplies device memory
and the stream.  There is no fallback: if the library is missing, importing
the binding's entry points raises.

Names follow the C ABI: fp4_quantize_kv, append_kv, fp8_quantize_kv,
swa_append, index_topk, sparse_attend, prefill_attend, decode_step,
decode_step_noalloc, block_scores, device_error, workspace_bytes,
workspace_init.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# CSA2_LIB_PATH: another build of the same library (the tests' host-sanitizer
# build, or libcsa2_checked.so)
LIB_PATH = os.environ.get("CSA2_LIB_PATH") or os.path.join(HERE, "libcsa2.so")
CHECKED_LIB_PATH = os.path.join(HERE, "libcsa2_checked.so")

FULL, REINDEX, REUSE = 0, 1, 2
SCORE_SUM, SCORE_HEADMAX = 0, 1     # indexer score rules: heads summed / best head
MODE_HEADMAX = 0x100                # OR-ed into an index_topk mode: the per-head rule
D, BLOCK, CODE_BYTES, SCALE_BYTES = 512, 8, 256, 32
MAX_POOL, MAX_TOPK, MAX_CACHES = 8192, 2048, 16
FLAG_NONFINITE_KV, FLAG_CAPACITY, FLAG_NONFINITE_Q, FLAG_BAD_INDEX, FLAG_SWA_RANGE, FLAG_Q_RANGE = 1, 2, 4, 8, 16, 32
FLAG_CHECK = 64                     # checked build (libcsa2_checked.so) only
MAX_WINDOW, MAX_SWA_LAYERS, MAX_SWA_SLOTS = 1024, 64, 1 << 22

EXPORTED = ("fp4_quantize_kv", "csa2_append_kv", "fp8_quantize_kv", "csa2_swa_append",
            "csa2_workspace_bytes", "csa2_workspace_init",
            "csa2_index_topk", "csa2_sparse_attend", "csa2_prefill_workspace_bytes",
            "csa2_prefill_attend", "csa2_decode_step", "csa2_decode_step_noalloc", "csa2_block_scores",
            "csa2_device_error", "csa2_set_scan_events", "csa2_read_probe", "csa2_status_string",
            "csa2_last_error")


class Csa2Error(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"csa2 status {status}: {message}")
        self.status = status


class _Kv(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("seq_len", ctypes.c_void_p),
                ("capacity", ctypes.c_int64), ("max_len", ctypes.c_int64), ("batch", ctypes.c_int32)]


class _Swa(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("seq_len", ctypes.c_void_p),
                ("window", ctypes.c_int32), ("batch", ctypes.c_int32), ("slots", ctypes.c_int32)]


class _Layer(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("cache", ctypes.c_int32), ("q", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("idx", ctypes.c_void_p), ("swa", ctypes.POINTER(_Swa)),
                ("swa_row", ctypes.c_void_p)]


class _Step(ctypes.Structure):
    _fields_ = [("caches", ctypes.POINTER(_Kv)), ("n_caches", ctypes.c_int32),
                ("layers", ctypes.POINTER(_Layer)), ("n_layers", ctypes.c_int32),
                ("new_rows", ctypes.c_void_p), ("heads", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("pool", ctypes.c_int32), ("scale", ctypes.c_float), ("pool_out", ctypes.c_void_p),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t), ("score_rule", ctypes.c_int32)]


_lib = None


def load():
    """Load libcsa2.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run python -c 'import __graft_entry__ as g; g.build()' "
                          "or python fp4_compressed_sparse_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "fp4_quantize_kv": (i32, [vp, i64, vp, i64, vp, vp, vp]),
        "csa2_append_kv": (i32, [ctypes.POINTER(_Kv), vp, vp]),
        "fp8_quantize_kv": (i32, [vp, i64, vp, i64, vp, vp, vp]),
        "csa2_swa_append": (i32, [ctypes.POINTER(_Swa), vp, vp]),
        "csa2_workspace_bytes": (sz, [i32, i32, i64, i32, i32]),
        "csa2_workspace_init": (i32, [vp, sz, vp]),
        "csa2_index_topk": (i32, [i32, ctypes.POINTER(_Kv), vp, i32, vp, i32, i32, vp, i32, vp, vp, vp, sz, vp]),
        "csa2_sparse_attend": (i32, [ctypes.POINTER(_Kv), vp, i32, vp, i32, ctypes.c_float,
                                     ctypes.POINTER(_Swa), vp, vp, sz, vp]),
        "csa2_prefill_workspace_bytes": (sz, [i32, i32, i32]),
        "csa2_prefill_attend": (i32, [ctypes.POINTER(_Kv), i32, vp, i32, i32, vp, vp, i32, ctypes.c_float,
                                      ctypes.POINTER(_Swa), vp, vp, sz, vp]),
        "csa2_decode_step": (i32, [ctypes.POINTER(_Step), vp]),
        "csa2_decode_step_noalloc": (i32, [ctypes.POINTER(_Step), vp]),
        "csa2_block_scores": (i32, [ctypes.POINTER(_Kv), vp, i32, vp, i32, vp, i32, vp]),
        "csa2_device_error": (i32, [ctypes.POINTER(ctypes.c_int32), vp]),
        "csa2_set_scan_events": (i32, [vp, vp]),
        "csa2_read_probe": (i32, [vp, i64, vp, vp]),
        "csa2_status_string": (ctypes.c_char_p, [i32]),
        "csa2_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status):
    if status != 0:
        lib = load()
        raise Csa2Error(status, f"{lib.csa2_status_string(status).decode()}: {lib.csa2_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class KVCache:
    """One Full layer's FP4 cache: torch uint8 codes [B][cap][256], scales
    [B][cap][32] and int64 seq_len [B] on the GPU."""

    def __init__(self, batch, capacity, device="cuda"):
        import torch
        if capacity % BLOCK:
            raise ValueError("capacity must be a multiple of 8")
        self.codes = torch.zeros((batch, capacity, CODE_BYTES), dtype=torch.uint8, device=device)
        self.scales = torch.zeros((batch, capacity, SCALE_BYTES), dtype=torch.uint8, device=device)
        self.seq_len = torch.zeros(batch, dtype=torch.int64, device=device)
        self.batch, self.capacity = batch, capacity
        self.max_len = 0            # host bound on seq_len, kept by the caller

    def view(self, max_len=None):
        return _Kv(self.codes.data_ptr(), self.scales.data_ptr(), self.seq_len.data_ptr(),
                   self.capacity, self.max_len if max_len is None else max_len, self.batch)


def fp4_quantize_kv(x, codes, scales, dst_row=None, stream=None):
    """x float32 [rows, 512] -> codes [*, 256] / scales [*, 32] rows dst_row (or 0..rows-1)."""
    lib = load()
    rows = x.shape[0]
    dst_rows = codes.numel() // CODE_BYTES
    if scales.numel() // SCALE_BYTES != dst_rows:
        raise ValueError("codes and scales hold different row counts")
    _check(lib.fp4_quantize_kv(_ptr(x), rows, _ptr(dst_row), dst_rows, _ptr(codes), _ptr(scales),
                               _stream(stream)))


def append_kv(cache: KVCache, x, stream=None):
    """Append x float32 [B, 512] at seq_len; the caller bumps cache.max_len."""
    lib = load()
    kv = cache.view()
    _check(lib.csa2_append_kv(ctypes.byref(kv), _ptr(x), _stream(stream)))


class SwaCache:
    """One layer's FP8 sliding-window ring: torch uint8 codes [B][slots][512],
    float32 scales [B][slots] and int64 seq_len [B] (positions written) on
    the GPU; position p lives in slot p % slots.  A decode step attends to
    the last `window` positions; slots (default: window) may be larger so a
    prefill chunk's queries find their own windows."""

    def __init__(self, batch, window, device="cuda", slots=None):
        import torch
        if not 1 <= window <= MAX_WINDOW:
            raise ValueError(f"window must be in [1, {MAX_WINDOW}]")
        slots = window if slots is None else int(slots)
        if slots < window:
            raise ValueError("slots must be >= window")
        self.codes = torch.zeros((batch, slots, D), dtype=torch.uint8, device=device)
        self.scales = torch.zeros((batch, slots), dtype=torch.float32, device=device)
        self.seq_len = torch.zeros(batch, dtype=torch.int64, device=device)
        self.batch, self.window, self.slots = batch, window, slots

    def view(self):
        return _Swa(self.codes.data_ptr(), self.scales.data_ptr(), self.seq_len.data_ptr(),
                    self.window, self.batch, self.slots)


def fp8_quantize_kv(x, codes, scales, dst_row=None, stream=None):
    """x float32 [rows, 512] -> codes [*, 512] uint8 / scales [*] float32 rows
    dst_row (or 0..rows-1)."""
    lib = load()
    rows = x.shape[0]
    dst_rows = codes.numel() // D
    if scales.numel() != dst_rows:
        raise ValueError("codes and scales hold different row counts")
    _check(lib.fp8_quantize_kv(_ptr(x), rows, _ptr(dst_row), dst_rows, _ptr(codes), _ptr(scales),
                               _stream(stream)))


def swa_append(swa: SwaCache, x, stream=None):
    """Append x float32 [B, 512] at each sequence's seq_len (slot seq_len % window)."""
    v = swa.view()
    _check(load().csa2_swa_append(ctypes.byref(v), _ptr(x), _stream(stream)))


def workspace_bytes(batch, heads, max_len, pool, topk):
    n = load().csa2_workspace_bytes(batch, heads, max_len, pool, topk)
    if n == 0:
        raise ValueError("unsupported workspace bounds")
    return n


def workspace(batch, heads, max_len, pool, topk, device="cuda"):
    """A zeroed workspace tensor sized for these bounds."""
    import torch
    n = workspace_bytes(batch, heads, max_len, pool, topk)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def workspace_init(ws, stream=None):
    _check(load().csa2_workspace_init(_ptr(ws), ws.numel(), _stream(stream)))


def index_topk(mode, cache, q, topk, idx_out, ws, cand=None, pool=0, pool_out=None, prior_idx=None,
               max_len=None, stream=None, score=SCORE_SUM):
    """score: SCORE_SUM or SCORE_HEADMAX (Full/Reindex only)."""
    lib = load()
    if score == SCORE_HEADMAX and mode != REUSE:
        mode |= MODE_HEADMAX
    elif score not in (SCORE_SUM, SCORE_HEADMAX):
        raise ValueError(f"unknown score rule {score}")
    kv = cache.view(max_len) if cache is not None else _Kv(None, None, None, 8, 0, idx_out.shape[0])
    heads = q.shape[1] if q is not None else 0
    n_cand = cand.shape[1] if cand is not None else 0
    _check(lib.csa2_index_topk(mode, ctypes.byref(kv), _ptr(q), heads, _ptr(cand), n_cand, topk,
                               _ptr(idx_out), pool, _ptr(pool_out), _ptr(prior_idx), _ptr(ws),
                               ws.numel() if ws is not None else 0, _stream(stream)))


def sparse_attend(cache, q, idx, scale, out, ws, max_len=None, stream=None, swa=None):
    """swa: None or the layer's SwaCache (its window joins the softmax)."""
    lib = load()
    kv = cache.view(max_len)
    sv = ctypes.byref(swa.view()) if swa is not None else None
    _check(lib.csa2_sparse_attend(ctypes.byref(kv), _ptr(q), q.shape[1], _ptr(idx), idx.shape[1],
                                  float(scale), sv, _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))


def prefill_attend(cache, seq, q, qpos, idx, scale, out, ws=None, max_len=None, stream=None, swa=None):
    """n_q queries of sequence `seq`: q float32 [n_q, H, 512], qpos int64
    [n_q], idx int32 [n_q, topk] -> out float32 [n_q, H, 512] (causal:
    positions <= qpos).  ws: None or a tensor of prefill_workspace_bytes.
    swa: None or the layer's SwaCache (each query's window joins its softmax)."""
    lib = load()
    kv = cache.view(max_len)
    nbytes = ws.numel() if ws is not None else 0
    sv = ctypes.byref(swa.view()) if swa is not None else None
    _check(lib.csa2_prefill_attend(ctypes.byref(kv), int(seq), _ptr(q), q.shape[0], q.shape[1], _ptr(qpos),
                                   _ptr(idx), idx.shape[1], float(scale), sv, _ptr(out), _ptr(ws), nbytes,
                                   _stream(stream)))


def prefill_workspace(n_q, heads, topk, device="cuda"):
    """Workspace tensor for prefill_attend (None when none is needed)."""
    import torch
    n = load().csa2_prefill_workspace_bytes(n_q, heads, topk)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def block_scores(cache, q, scores, cand=None, max_len=None, stream=None, score=SCORE_SUM):
    lib = load()
    kv = cache.view(max_len)
    n_cand = cand.shape[1] if cand is not None else 0
    _check(lib.csa2_block_scores(ctypes.byref(kv), _ptr(q), q.shape[1], _ptr(cand), n_cand,
                                 _ptr(scores), int(score), _stream(stream)))


class StepPlan:
    """A decode step's C structures, built once and reusable (e.g. for
    repeated launches or graph capture).  layers: list of (mode, cache, q,
    out, idx) or (mode, cache, q, out, idx, swa, swa_row) with torch tensors
    (swa: the layer's SwaCache or None; swa_row float32 [B, 512] or None).
    score: SCORE_SUM or SCORE_HEADMAX for every selecting layer."""

    def __init__(self, caches, layers, heads, topk, pool, scale, ws, pool_out=None, new_rows=None,
                 score=SCORE_SUM):
        self.caches = caches
        self._kv = (_Kv * len(caches))(*[c.view() for c in caches])
        self._swa = [ly[5].view() if len(ly) > 5 and ly[5] is not None else None for ly in layers]
        built = []
        for ly, sv in zip(layers, self._swa):
            m, ci, q, out, idx = ly[:5]
            row = ly[6] if len(ly) > 6 else None
            built.append(_Layer(m, ci, q.data_ptr(), out.data_ptr(), idx.data_ptr(),
                                ctypes.pointer(sv) if sv is not None else None,
                                row.data_ptr() if row is not None else None))
        self._layers = (_Layer * len(layers))(*built)
        self._keep = (layers, ws, pool_out, new_rows)
        self._step = _Step(self._kv, len(caches), self._layers, len(layers),
                           new_rows.data_ptr() if new_rows is not None else None, heads, topk, pool,
                           float(scale), pool_out.data_ptr() if pool_out is not None else None,
                           ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
                           int(score))

    def refresh_lengths(self):
        """Copy each cache's host max_len bound into the C views."""
        for i, c in enumerate(self.caches):
            self._kv[i].max_len = c.max_len

    def run(self, stream=None):
        _check(load().csa2_decode_step(ctypes.byref(self._step), _stream(stream)))

    def run_noalloc(self, stream=None):
        """The same step through csa2_decode_step_noalloc (the library's own
        per-device workspace; this plan's ws is ignored)."""
        _check(load().csa2_decode_step_noalloc(ctypes.byref(self._step), _stream(stream)))


def decode_step(caches, layers, heads, topk, pool, scale, ws, pool_out=None, new_rows=None, stream=None,
                score=SCORE_SUM):
    StepPlan(caches, layers, heads, topk, pool, scale, ws, pool_out, new_rows, score).run(stream)


def decode_step_noalloc(caches, layers, heads, topk, pool, scale, pool_out=None, new_rows=None, stream=None,
                        score=SCORE_SUM):
    """decode_step on the library's own per-device workspace (no allocation)."""
    StepPlan(caches, layers, heads, topk, pool, scale, None, pool_out, new_rows, score).run_noalloc(stream)


def set_scan_events(before=None, after=None):
    """Record hipEvent_t handles `before`/`after` (ctypes c_void_p) around
    every full-scan kernel launched from this thread (None, None clears)."""
    _check(load().csa2_set_scan_events(before, after))


def read_probe(buf, sink, stream=None):
    """csa2_read_probe: read every byte of the device tensor `buf` once (the
    read-rate yardstick for the full scan); `sink` is a device int32 tensor
    of at least 512 * 256 entries."""
    assert buf.is_cuda and sink.is_cuda and sink.numel() >= 512 * 256 and sink.element_size() == 4
    _check(load().csa2_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


def device_error(stream=None):
    flags = ctypes.c_int32(0)
    _check(load().csa2_device_error(ctypes.byref(flags), _stream(stream)))
    return flags.value

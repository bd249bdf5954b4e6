"""The C-ABI library loads, exports every entry point include/csa2.h
declares, and rejects malformed arguments on the host before any launch.
Runs without a GPU: nothing here reaches a kernel."""
import ctypes
import os
import re

import pytest

import fp4_compressed_sparse_amd as csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "csa2.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(?:csa2_status|size_t|const char \*)\s*\*?\s*(\w+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(csa2.LIB_PATH):
        pytest.fail("libcsa2.so is not built; run __graft_entry__.build()")
    return csa2.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(csa2.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_checked_build_exports_the_same_symbols():
    # the checked build (workgroup order scrambled, device index checks) is
    # the same ABI: the GPU comparison loads it in place of libcsa2.so
    if not os.path.exists(csa2.CHECKED_LIB_PATH):
        pytest.fail("libcsa2_checked.so is not built; run __graft_entry__.build()")
    chk = ctypes.CDLL(csa2.CHECKED_LIB_PATH)
    for n in _declared():
        assert hasattr(chk, n), n


def test_status_strings(lib):
    assert lib.csa2_status_string(0) == b"ok"
    assert lib.csa2_status_string(3) == b"workspace too small"
    assert lib.csa2_status_string(99) == b"unknown status"


def test_workspace_bytes_host_only(lib):
    n3 = lib.csa2_workspace_bytes(1, 64, (1 << 20) + 64, 2048, 256)
    assert n3 > 0 and n3 % 256 == 0
    # bigger bounds never need less
    assert lib.csa2_workspace_bytes(2, 64, (1 << 20) + 64, 2048, 256) > n3
    assert lib.csa2_workspace_bytes(1, 64, 4096, 0, 64) < n3
    # unsupported bounds give 0
    assert lib.csa2_workspace_bytes(0, 64, 4096, 0, 64) == 0
    assert lib.csa2_workspace_bytes(1, 65, 4096, 0, 64) == 0
    assert lib.csa2_workspace_bytes(1, 16, 4096, 0, 4096) == 0
    assert lib.csa2_workspace_bytes(1, 16, 4096, 9000, 64) == 0


def _err(lib):
    return lib.csa2_last_error().decode()


def test_quantize_argument_errors(lib):
    assert lib.fp4_quantize_kv(None, 0, None, 0, None, None, None) == 0     # no-op
    assert lib.fp4_quantize_kv(None, -1, None, 0, None, None, None) == 1
    assert lib.fp4_quantize_kv(None, 4, None, 4, None, None, None) == 1
    assert "NULL" in _err(lib)
    assert lib.fp4_quantize_kv(ctypes.c_void_p(0x1004), 4, None, 4, ctypes.c_void_p(0x2000),
                               ctypes.c_void_p(0x3000), None) == 1          # x misaligned
    assert lib.fp4_quantize_kv(ctypes.c_void_p(0x1000), 4, None, 4, ctypes.c_void_p(0x2004),
                               ctypes.c_void_p(0x3000), None) == 1          # codes not 8-byte aligned
    assert "8-byte" in _err(lib)
    assert lib.fp4_quantize_kv(ctypes.c_void_p(0x1000), 4, None, 3, ctypes.c_void_p(0x2000),
                               ctypes.c_void_p(0x3000), None) == 4          # too few rows


def _kv(**kw):
    base = dict(codes=0x10000, scales=0x20000, seq_len=0x30000, capacity=4096, max_len=4096, batch=1)
    base.update(kw)
    return csa2._Kv(base["codes"], base["scales"], base["seq_len"], base["capacity"],
                    base["max_len"], base["batch"])


def _swa(**kw):
    base = dict(codes=0x20000, scales=0x60000, seq_len=0x30000, window=128, batch=1, slots=0)
    base.update(kw)
    return csa2._Swa(base["codes"], base["scales"], base["seq_len"] or None, base["window"], base["batch"],
                     base["slots"])


def test_index_and_attend_argument_errors(lib):
    idx = ctypes.c_void_p(0x40000)
    q = ctypes.c_void_p(0x50000)
    ws = ctypes.c_void_p(0x60000)
    need = lib.csa2_workspace_bytes(1, 16, 4096, 0, 64)
    call = lambda mode, kv, heads=16, topk=64, pool=0, wsb=need, cand=None, n_cand=0: lib.csa2_index_topk(
        mode, ctypes.byref(kv), q, heads, cand, n_cand, topk, idx, pool, None, None, ws, wsb, None)
    assert call(7, _kv()) == 1                                   # bad mode
    assert call(0, _kv(codes=0x10010)) == 1                      # misaligned codes
    assert call(0, _kv(capacity=4092)) == 2                      # capacity not a multiple of 8
    assert call(0, _kv(max_len=5000)) == 4                       # max_len > capacity
    assert call(0, _kv(), heads=0) == 2
    assert call(0, _kv(), topk=0) == 2
    assert call(0, _kv(), topk=128, pool=64) == 1                # pool < topk
    assert call(0, _kv(), wsb=need - 1) == 3                     # workspace too small
    assert "workspace" in _err(lib)
    assert call(2, _kv()) == 1                                   # Reuse without prior_idx
    out = ctypes.c_void_p(0x70000)
    assert lib.csa2_sparse_attend(ctypes.byref(_kv()), q, 24, idx, 64, ctypes.c_float(0.04), None, out,
                                  ws, need, None) == 2           # 24 heads unsupported
    assert lib.csa2_sparse_attend(ctypes.byref(_kv()), q, 16, idx, 64, ctypes.c_float(float("nan")),
                                  None, out, ws, need, None) == 1
    # local branch: window outside [1, 1024], batch mismatch, misaligned ring
    for bad, code in ((_swa(window=0), 2), (_swa(window=1025), 2), (_swa(batch=2), 1),
                      (_swa(codes=0x20008), 1), (_swa(seq_len=0), 1), (_swa(slots=100), 2),
                      (_swa(slots=(1 << 22) + 1), 2)):
        assert lib.csa2_sparse_attend(ctypes.byref(_kv()), q, 16, idx, 64, ctypes.c_float(0.04),
                                      ctypes.byref(bad), out, ws, need, None) == code


def test_decode_step_pattern_errors(lib):
    kv = (csa2._Kv * 2)(_kv(), _kv())
    q, out, idx = 0x50000, 0x70000, 0x40000
    ws = 0x100000
    need = lib.csa2_workspace_bytes(1, 16, 4096, 0, 64)

    def step(layers, heads=16, pool=0):
        arr = (csa2._Layer * len(layers))(*[csa2._Layer(m, c, q, out, idx, None, None) for m, c in layers])
        st = csa2._Step(kv, 2, arr, len(layers), None, heads, 64, pool, 0.04, None, ws, need)
        return lib.csa2_decode_step(ctypes.byref(st), None)

    assert step([(1, 0)]) == 1                  # Reindex first
    assert step([(2, 0)]) == 1                  # Reuse first
    assert step([(0, 0), (1, 1)]) == 1          # Reindex on a stale cache
    assert step([(0, 0), (0, 1), (1, 0)]) == 1  # Reindex must use the latest Full cache
    assert step([(0, 0)], heads=48) == 2
    assert step([(0, 0)], pool=64) == 1         # pool > 0 without pool_out


def test_noalloc_step_rejects_oversize_workspace(lib):
    # the batch-64 workload needs about 87 MiB, more than the library's scratch
    need = lib.csa2_workspace_bytes(64, 16, 131072 + 64, 2048, 128)
    assert need > (16 << 20)
    kv = (csa2._Kv * 1)(_kv(batch=64, capacity=131136, max_len=131072 + 64))
    arr = (csa2._Layer * 1)(csa2._Layer(0, 0, 0x50000, 0x70000, 0x40000, None, None))
    st = csa2._Step(kv, 1, arr, 1, None, 16, 128, 2048, 0.04, 0x80000, None, 0)
    assert lib.csa2_decode_step_noalloc(ctypes.byref(st), None) == 3
    assert "scratch" in _err(lib)


def test_swa_argument_errors(lib):
    x = ctypes.c_void_p(0x50000)
    assert lib.fp8_quantize_kv(None, 0, None, 0, None, None, None) == 0     # no-op
    assert lib.fp8_quantize_kv(x, -1, None, 0, None, None, None) == 1
    assert lib.fp8_quantize_kv(x, 4, None, 4, None, ctypes.c_void_p(0x60000), None) == 1
    assert lib.fp8_quantize_kv(ctypes.c_void_p(0x50004), 4, None, 4, ctypes.c_void_p(0x70000),
                               ctypes.c_void_p(0x60000), None) == 1       # x misaligned
    assert lib.fp8_quantize_kv(x, 4, None, 3, ctypes.c_void_p(0x70000), ctypes.c_void_p(0x60000),
                               None) == 4                                 # too few rows
    assert lib.csa2_swa_append(None, x, None) == 1
    assert lib.csa2_swa_append(ctypes.byref(_swa(window=2000)), x, None) == 2
    assert lib.csa2_swa_append(ctypes.byref(_swa(batch=0)), x, None) == 1
    assert lib.csa2_swa_append(ctypes.byref(_swa()), ctypes.c_void_p(0x50008), None) == 1
    # a decode-step layer with a bad ring
    kv = (csa2._Kv * 1)(_kv())
    bad = _swa(window=0)
    arr = (csa2._Layer * 1)(csa2._Layer(0, 0, 0x50000, 0x70000, 0x40000, ctypes.pointer(bad), 0x58000))
    need = lib.csa2_workspace_bytes(1, 16, 4096, 0, 64)
    st = csa2._Step(kv, 1, arr, 1, None, 16, 64, 0, 0.04, None, 0x100000, need)
    assert lib.csa2_decode_step(ctypes.byref(st), None) == 2
    assert "window" in _err(lib)
    # two layers appending into one ring (same length word) would race: rejected
    ring = _swa()
    arr2 = (csa2._Layer * 2)(csa2._Layer(0, 0, 0x50000, 0x70000, 0x40000, ctypes.pointer(ring), 0x58000),
                             csa2._Layer(2, 0, 0x50000, 0x74000, 0x40000, ctypes.pointer(ring), 0x5c000))
    st2 = csa2._Step(kv, 1, arr2, 2, None, 16, 64, 0, 0.04, None, 0x100000, need)
    assert lib.csa2_decode_step(ctypes.byref(st2), None) == 1
    assert "same SWA ring" in _err(lib)


def test_prefill_attend_argument_errors(lib):
    q, qpos, idx, out = (ctypes.c_void_p(a) for a in (0x50000, 0x58000, 0x40000, 0x70000))
    # the workspace holds partials only when one split per head tile is not enough
    assert lib.csa2_prefill_workspace_bytes(1024, 64, 256) == 0
    assert lib.csa2_prefill_workspace_bytes(4, 16, 256) > 0
    assert lib.csa2_prefill_workspace_bytes(0, 16, 64) == 0
    assert lib.csa2_prefill_workspace_bytes(4, 24, 64) == 0
    call = lambda seq=0, n_q=8, heads=16, topk=64, scale=0.04, qp=qpos, kv=None, sw=None: lib.csa2_prefill_attend(
        ctypes.byref(kv or _kv()), seq, q, n_q, heads, qp, idx, topk, ctypes.c_float(scale),
        ctypes.byref(sw) if sw is not None else None, out, None, 0, None)
    assert call(seq=1) == 1                                      # sequence outside the batch
    assert call(seq=-1) == 1
    assert call(heads=24) == 2
    assert call(topk=0) == 2
    assert call(n_q=0) == 2
    assert call(n_q=70000) == 2
    assert call(scale=float("inf")) == 1
    assert call(qp=None) == 1
    assert call(n_q=4) == 1                                      # partials needed, workspace NULL
    assert "workspace" in _err(lib)
    assert call(kv=_kv(capacity=4092)) == 2
    assert call(sw=_swa(window=0)) == 2                          # bad local branch
    assert call(sw=_swa(batch=3)) == 1


def test_read_probe_argument_errors(lib):
    buf, sink = ctypes.c_void_p(0x50000), ctypes.c_void_p(0x60000)
    assert lib.csa2_read_probe(None, 16, sink, None) == 1
    assert lib.csa2_read_probe(buf, 16, None, None) == 1
    assert lib.csa2_read_probe(ctypes.c_void_p(0x50008), 16, sink, None) == 1   # buf not 16-byte aligned
    assert lib.csa2_read_probe(buf, 16, ctypes.c_void_p(0x60002), None) == 1    # sink misaligned
    assert lib.csa2_read_probe(buf, 0, sink, None) == 1
    assert lib.csa2_read_probe(buf, 24, sink, None) == 1                       # not a multiple of 16
    assert "read probe" in _err(lib)

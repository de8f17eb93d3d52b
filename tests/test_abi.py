"""CPU-side checks of the C ABI: the library loads, exports every function
include/sf_kv.h declares, and rejects bad arguments before touching a GPU.
No compute call is made here (there is no GPU in this test tier)."""
import ctypes
import os
import re

import pytest

from selective_kv_cache_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sf_kv.h")


def _lib():
    if not os.path.exists(B.LIB_PATH):
        from selective_kv_cache_amd import build
        build.build()
    return B.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sf_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_three_method_calls():
    names = declared_functions()
    for n in ("sf_kv_quantize", "sf_refine_store", "sf_decode_step"):
        assert n in names
    assert set(names) == set(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = _lib()
    for st in (B.SF_OK, B.SF_ERR_INVALID_ARG, B.SF_ERR_UNSUPPORTED, B.SF_ERR_HIP, B.SF_ERR_OOM, B.SF_ERR_TIMEOUT,
               B.SF_ERR_STATE):
        assert lib.sf_status_string(st)


def _g(**kw):
    base = dict(head_dim=128, n_q_heads=32, n_kv_heads=8, base_bits=2, refine_bits=4)
    base.update(kw)
    return B.sf_geom(**base)


def _ws(g, batch=1, total=131072, max_seq=131072, t=2048):
    n = ctypes.c_size_t()
    st = _lib().sf_decode_workspace_size(ctypes.byref(g), batch, total, max_seq, t, ctypes.byref(n))
    return st, n.value


def test_workspace_size_host_logic():
    st, n = _ws(_g())
    assert st == B.SF_OK
    # at least the score scratch (4 B per token-head) and candidate lists
    assert n >= 8 * 131072 * 4 + 8 * 131072 * 8
    assert n < 64 << 20
    st2, n2 = _ws(_g(), batch=16, total=163840, max_seq=16384, t=256)
    assert st2 == B.SF_OK and n2 > 0


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), B.SF_ERR_UNSUPPORTED),
    (dict(n_q_heads=30), B.SF_ERR_INVALID_ARG),
    (dict(n_q_heads=24), B.SF_ERR_UNSUPPORTED),      # group of 3
    (dict(base_bits=5), B.SF_ERR_UNSUPPORTED),
    (dict(base_bits=1), B.SF_ERR_UNSUPPORTED),
    (dict(refine_bits=9), B.SF_ERR_UNSUPPORTED),
    (dict(refine_bits=-1), B.SF_ERR_INVALID_ARG),
])
def test_geometry_validation(kw, status):
    st, _ = _ws(_g(**kw))
    assert st == status


def test_workspace_bad_sizes():
    assert _ws(_g(), batch=0)[0] == B.SF_ERR_INVALID_ARG
    assert _ws(_g(), max_seq=200000)[0] == B.SF_ERR_INVALID_ARG
    assert _ws(_g(), t=-1)[0] == B.SF_ERR_INVALID_ARG


def test_quantize_rejects_before_launch():
    lib = _lib()
    g = _g()
    fake = 1 << 20   # never dereferenced: every call below fails validation
    # tok_begin + n_tok > cap
    assert lib.sf_kv_quantize(ctypes.byref(g), fake, 10, 95, 100, fake, fake, fake, None) == B.SF_ERR_INVALID_ARG
    # r > 0 but no refinement buffer
    assert lib.sf_kv_quantize(ctypes.byref(g), fake, 10, 0, 100, fake, fake, None, None) == B.SF_ERR_INVALID_ARG
    # misaligned pointer
    assert lib.sf_kv_quantize(ctypes.byref(g), fake + 4, 10, 0, 100, fake, fake, fake, None) == B.SF_ERR_INVALID_ARG
    # nothing to do
    assert lib.sf_kv_quantize(ctypes.byref(g), fake, 0, 0, 100, fake, fake, fake, None) == B.SF_OK


def test_decode_rejects_before_launch():
    import numpy as np
    lib = _lib()
    g = _g()
    fake = 1 << 20
    a = B.sf_decode_args()
    off = np.asarray([0, 100, 100], dtype=np.int64)          # second sequence empty
    a.batch = 2
    a.seq_off_host = off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    a.seq_off_dev = a.q = a.k_codes = a.k_scales = a.v_codes = a.v_scales = a.out = a.workspace = fake
    a.cap, a.top_t, a.workspace_bytes = 1000, 8, 1 << 30
    assert lib.sf_decode_step(ctypes.byref(g), ctypes.byref(a), None) == B.SF_ERR_INVALID_ARG
    off[2] = 200
    a.store = None                                           # r > 0 and T > 0 need a store
    assert lib.sf_decode_step(ctypes.byref(g), ctypes.byref(a), None) == B.SF_ERR_INVALID_ARG
    a.cap = 150                                              # tokens beyond capacity
    assert lib.sf_decode_step(ctypes.byref(g), ctypes.byref(a), None) == B.SF_ERR_INVALID_ARG
    a.cap, a.top_t = 1000, 0
    a.workspace_bytes = 16                                   # workspace too small
    assert lib.sf_decode_step(ctypes.byref(g), ctypes.byref(a), None) == B.SF_ERR_INVALID_ARG
    a.workspace_bytes, a.flags = 1 << 30, 8                  # reserved flags
    assert lib.sf_decode_step(ctypes.byref(g), ctypes.byref(a), None) == B.SF_ERR_INVALID_ARG


def test_store_rejects_before_allocation():
    lib = _lib()
    h = ctypes.c_void_p()
    g = _g()
    assert lib.sf_store_create(ctypes.byref(g), 0, 1, 0, 0, ctypes.byref(h)) == B.SF_ERR_INVALID_ARG
    assert lib.sf_store_create(ctypes.byref(g), 100, 1, 7, 0, ctypes.byref(h)) == B.SF_ERR_INVALID_ARG
    assert lib.sf_store_create(ctypes.byref(g), 100, 1, 1, 0, ctypes.byref(h)) == B.SF_ERR_INVALID_ARG
    assert lib.sf_store_create(ctypes.byref(g), 100, 1, 1, 1 << 20, ctypes.byref(h)) == B.SF_ERR_INVALID_ARG
    # global cache slot ids must fit in int32: max_seqs x Hkv x slots < 2^31
    assert lib.sf_store_create(ctypes.byref(g), 100, 1 << 17, 1, 4096, ctypes.byref(h)) == B.SF_ERR_INVALID_ARG
    g0 = _g(refine_bits=0)
    assert lib.sf_store_create(ctypes.byref(g0), 100, 1, 0, 0, ctypes.byref(h)) == B.SF_ERR_INVALID_ARG
    assert lib.sf_refine_store(None, 0, None, 0, 1, None) == B.SF_ERR_INVALID_ARG
    assert lib.sf_store_destroy(None) == B.SF_ERR_INVALID_ARG
    assert lib.sf_store_check(None, None) == B.SF_ERR_INVALID_ARG


def test_decoder_follows_a_growing_context():
    """Decoder.set_offsets (the multi-step run's growing context): offsets and
    sizes follow, the workspace is reallocated only when the new shape needs
    more (with a quarter to spare), and a reallocated one starts uncleared.
    Host logic only: buffers on the CPU, no step is run."""
    import numpy as np
    from selective_kv_cache_amd.kvcache import Decoder
    _lib()
    g = B.geom(128, 32, 8, 3, 2)
    dec = Decoder(g, [0, 8193], 512, device="cpu")
    size0 = dec.workspace.numel()
    assert size0 == B.sf_decode_workspace_size(g, 1, 8193, 8193, 512)
    dec._hist_clean = True
    dec.set_offsets([0, 8194])
    need = B.sf_decode_workspace_size(g, 1, 8194, 8194, 512)
    assert (dec.total, dec.max_seq, dec.batch) == (8194, 8194, 1)
    assert dec.seq_off_dev.tolist() == [0, 8194]
    if need <= size0:
        assert dec.workspace.numel() == size0 and dec._hist_clean
    else:
        assert dec.workspace.numel() == need + need // 4 and not dec._hist_clean
    dec._hist_clean = True
    dec.set_offsets([0, 40000])                              # well beyond: must grow
    need = B.sf_decode_workspace_size(g, 1, 40000, 40000, 512)
    assert dec.workspace.numel() == need + need // 4 and not dec._hist_clean
    dec._hist_clean = True
    dec.set_offsets([0, 30000])                              # smaller again: kept
    assert dec.workspace.numel() == need + need // 4 and dec._hist_clean
    dec.set_offsets(np.array([0, 100, 300]))                 # another batch size: not clean
    assert dec.batch == 2 and not dec._hist_clean and dec.seq_off_dev.tolist() == [0, 100, 300]


@pytest.mark.parametrize("geom,status", [
    ((33, 256, 2, 2, 4, 128), B.SF_ERR_INVALID_ARG),       # rows not a multiple of 32
    ((32, 200, 2, 2, 4, 128), B.SF_ERR_INVALID_ARG),       # channels not a multiple of 128
    ((32, 256, 1, 2, 4, 128), B.SF_ERR_INVALID_ARG),
    ((32, 256, 5, 2, 4, 128), B.SF_ERR_INVALID_ARG),
    ((32, 256, 2, 0, 4, 128), B.SF_ERR_INVALID_ARG),
    ((32, 256, 2, 9, 4, 128), B.SF_ERR_INVALID_ARG),
    ((32, 256, 2, 2, 129, 128), B.SF_ERR_INVALID_ARG),     # more channels than the chunk holds
    ((32, 256, 2, 2, 4, 0), B.SF_ERR_INVALID_ARG),
    ((32, 256, 2, 2, 4, 4097), B.SF_ERR_INVALID_ARG),
    ((32, 15488, 2, 2, 4, 128), B.SF_ERR_UNSUPPORTED),     # x no longer fits the work-group's LDS
])
def test_weight_gemv_rejects_before_launch(geom, status):
    lib = _lib()
    g = B.wgeom(*geom)
    fake = 1 << 20
    assert lib.sf_w_gemv(ctypes.byref(g), fake, fake, fake, fake, fake, fake, fake, None) == status
    n = ctypes.c_int32()
    assert lib.sf_w_gemv_workspace_words(ctypes.byref(g), ctypes.byref(n)) == status
    assert lib.sf_w_quantize(ctypes.byref(g), fake, fake, fake, fake, fake, None) == status


def test_weight_gemv_rejects_null_buffers():
    lib = _lib()
    g = B.wgeom(64, 1024, 3, 4, 32, 1024)
    fake = 1 << 20
    assert lib.sf_w_gemv(ctypes.byref(g), fake, fake, fake, fake, fake, None, fake, None) == B.SF_ERR_INVALID_ARG
    assert lib.sf_w_gemv(ctypes.byref(g), fake, fake, fake, fake, fake, fake, None, None) == B.SF_ERR_INVALID_ARG
    assert lib.sf_w_gemv(ctypes.byref(g), fake, fake, fake, fake + 4, fake, fake, fake, None) == B.SF_ERR_INVALID_ARG
    n = ctypes.c_int32()
    assert lib.sf_w_gemv_workspace_words(ctypes.byref(g), ctypes.byref(n)) == B.SF_OK and n.value == 512 + 2 * 32 + 2
    g2 = B.wgeom(64, 2688, 3, 4, 32, 1000)
    assert lib.sf_w_gemv_workspace_words(ctypes.byref(g2), ctypes.byref(n)) == B.SF_OK and n.value == 512 + 2 * 3 * 32 + 2
    assert lib.sf_w_quantize(ctypes.byref(g), fake, fake, fake, None, fake, None) == B.SF_ERR_INVALID_ARG


def test_noalloc_scratch_holds_every_workload_step():
    """sf_decode_step_noalloc's fixed device buffer holds the workspace of a
    step of every workload the benchmark and the tests run at full size (the
    16-sequence batch is the largest)."""
    from selective_kv_cache_amd import workloads as W
    cap = B.sf_decode_noalloc_max_bytes()
    for name, w in W.WORKLOADS.items():
        lens = w.seq_lengths()
        off = W.seq_offsets(lens)
        g = B.geom(w.head_dim, w.n_q_heads, w.n_kv_heads, w.base_bits, w.refine_bits)
        need = B.sf_decode_workspace_size(g, w.batch, int(off[-1]), int(max(lens)), w.top_t)
        assert need <= cap, (name, need, cap)

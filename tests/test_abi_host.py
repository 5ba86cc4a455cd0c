"""Host-side contract of libadakv.so (no GPU needed): every symbol the header
declares is exported, the ctypes structs match the C layout, and invalid
arguments return their status code before anything is launched."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from adaptive_head_budget_amd import configs, lib, pipeline

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "adakv.h")
FAKE = 0x100000     # an aligned address that is never dereferenced: each call below fails validation first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lib.LIB_PATH):
        from adaptive_head_budget_amd import build
        build.build()
    return lib.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:size_t|adakv_status|const char\*|int32_t)\s+(adakv_\w+)\s*\(", text, re.M)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for f in ("adakv_score", "adakv_allocate", "adakv_compact", "adakv_decode_attn"):
        assert f in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", lib.LIB_PATH], capture_output=True, text=True).stdout
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, re.M), name
    assert set(lib.EXPORTS) == set(declared_functions())


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "probe.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "adakv.h"\n'
        "int main(void){printf(\"%zu %zu %zu %zu %zu %zu\\n\", sizeof(adakv_shape), sizeof(adakv_alloc),"
        " offsetof(adakv_shape, eps), offsetof(adakv_alloc, budget), offsetof(adakv_shape, hidden),"
        " offsetof(adakv_alloc, inst_budget));return 0;}\n")
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got == [ctypes.sizeof(lib.AdakvShape), ctypes.sizeof(lib.AdakvAlloc), lib.AdakvShape.eps.offset,
                   lib.AdakvAlloc.budget.offset, lib.AdakvShape.hidden.offset, lib.AdakvAlloc.inst_budget.offset]


def test_strerror_and_version(L):
    assert lib.adakv_version() >= 100
    for s in range(6):
        assert isinstance(lib.strerror(s), str) and lib.strerror(s)
    assert lib.strerror(99) == "unknown status"


def test_workspace_bytes(L):
    for c in configs.ALL:
        assert lib.adakv_workspace_bytes(pipeline.make_shape(c), pipeline.make_alloc(c), c.reserve) > 0
    bad = pipeline.make_shape(configs.LLAMA8B_LAYER)
    bad.hq = 33
    assert lib.adakv_workspace_bytes(bad, None, 0) == 0


def _shape(**kw):
    s = pipeline.make_shape(configs.LLAMA8B_LAYER)
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def _alloc(**kw):
    a = pipeline.make_alloc(configs.LLAMA8B_LAYER)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def score_status(L, shape, ws_bytes=1 << 40, ptrs=FAKE):
    return L.adakv_score(ctypes.byref(shape), ptrs, ptrs, ptrs, ptrs, ptrs, ptrs, ptrs, ws_bytes, None)


def score_lse_status(L, shape, lse=FAKE, ws_bytes=1 << 40, ptrs=FAKE):
    return L.adakv_score_lse(ctypes.byref(shape), ptrs, ptrs, ptrs, ptrs, lse, ptrs, ptrs, ptrs, ws_bytes, None)


def test_score_lse_validates_like_score(L):
    s = _shape()
    assert score_lse_status(L, s, lse=None) == lib.ADAKV_EINVAL       # the normaliser is required
    assert score_lse_status(L, s, lse=FAKE + 4) == lib.ADAKV_EINVAL
    assert score_lse_status(L, s, ptrs=None) == lib.ADAKV_EINVAL
    assert score_lse_status(L, s, ws_bytes=16) == lib.ADAKV_EWORKSPACE
    assert score_lse_status(L, _shape(hq=33)) == lib.ADAKV_EINVAL
    assert score_lse_status(L, _shape(w=65)) == lib.ADAKV_EUNSUPPORTED


def causal_status(L, shape, q=FAKE, k=FAKE, lse=FAKE, out=FAKE, flag=None):
    return L.adakv_lse_from_causal(ctypes.byref(shape), q, k, lse, out, flag, None)


def test_lse_from_causal_rejects(L):
    s = _shape()
    assert causal_status(L, s, lse=None) == lib.ADAKV_EINVAL
    assert causal_status(L, s, out=None) == lib.ADAKV_EINVAL
    assert causal_status(L, s, q=None) == lib.ADAKV_EINVAL
    assert causal_status(L, s, k=FAKE + 8) == lib.ADAKV_EINVAL
    assert causal_status(L, s, flag=FAKE + 4) == lib.ADAKV_EINVAL       # the flags are optional, but aligned
    assert causal_status(L, _shape(hq=33)) == lib.ADAKV_EINVAL
    assert causal_status(L, _shape(n=32)) == lib.ADAKV_EINVAL
    assert causal_status(L, _shape(w=65)) == lib.ADAKV_EUNSUPPORTED
    assert causal_status(L, _shape(hq=80, hkv=8)) == lib.ADAKV_EUNSUPPORTED
    assert causal_status(L, _shape(d=96)) == lib.ADAKV_EUNSUPPORTED


@pytest.mark.parametrize("kw,status", [
    (dict(hq=33), lib.ADAKV_EINVAL),            # hq not a multiple of hkv
    (dict(n=32), lib.ADAKV_EINVAL),             # no prefix: n <= w
    (dict(pool=4), lib.ADAKV_EINVAL),           # even pool kernel
    (dict(pool=0), lib.ADAKV_EINVAL),
    (dict(n_inst=0), lib.ADAKV_EINVAL),
    (dict(dtype=7), lib.ADAKV_EINVAL),
    (dict(scorer=5), lib.ADAKV_EINVAL),
    (dict(d=96), lib.ADAKV_EUNSUPPORTED),       # head dim not built
    (dict(w=65), lib.ADAKV_EUNSUPPORTED),       # window wider than 64
    (dict(pool=9), lib.ADAKV_EUNSUPPORTED),
    (dict(hq=80, hkv=8), lib.ADAKV_EUNSUPPORTED),   # group of 10
])
def test_score_rejects(L, kw, status):
    assert score_status(L, _shape(**kw)) == status


def test_score_rejects_null_misaligned_and_small_workspace(L):
    s = _shape()
    assert score_status(L, s, ptrs=None) == lib.ADAKV_EINVAL
    assert score_status(L, s, ptrs=FAKE + 4) == lib.ADAKV_EINVAL
    assert score_status(L, s, ws_bytes=16) == lib.ADAKV_EWORKSPACE
    ck = _shape(scorer=lib.ADAKV_SCORE_CRITICALKV, hidden=100)
    assert score_status(L, ck) == lib.ADAKV_EUNSUPPORTED      # hidden not a multiple of 64


@pytest.mark.parametrize("kw,status", [
    (dict(budget=8 * 32 - 1), lib.ADAKV_EINVAL),            # budget smaller than the windows
    (dict(budget=8 * 16384 + 1), lib.ADAKV_EINVAL),         # budget larger than the cache
    (dict(alpha_num=6, alpha_den=5), lib.ADAKV_EINVAL),
    (dict(alpha_den=0), lib.ADAKV_EINVAL),
    (dict(mode=9), lib.ADAKV_EINVAL),
    (dict(mode=lib.ADAKV_ALLOC_ADA_CRITICALKV, ck_num=3, ck_den=2), lib.ADAKV_EINVAL),
])
def test_allocate_rejects(L, kw, status):
    s, a = _shape(), _alloc(**kw)
    st = L.adakv_allocate(ctypes.byref(s), ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == status


def test_allocate_small_workspace(L):
    s, a = _shape(), _alloc()
    st = L.adakv_allocate(ctypes.byref(s), ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, None)
    assert st == lib.ADAKV_EWORKSPACE


def test_lava_budget_range(L):
    s = _shape(n_inst=4, scorer=lib.ADAKV_SCORE_LAVA)
    a = _alloc(mode=lib.ADAKV_ALLOC_LAVA_LAYERS, budget=4 * 32 * 8 - 1)
    st = L.adakv_allocate(ctypes.byref(s), ctypes.byref(a), FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == lib.ADAKV_EINVAL


def test_preset_budgets_checked(L):
    """Per-instance budgets (preset layer budgets): each within [w*hkv, n*hkv],
    Ada-KV mode only; the workspace and the selection size follow them."""
    cfg = configs.LLAMA8B_LAYER
    s = _shape(n_inst=3)
    good = [8 * 32 + 900, 8 * 32 + 500, 8 * 32 + 100]
    a = pipeline.make_alloc(cfg, inst_budget=good)
    assert L.adakv_workspace_bytes(ctypes.byref(s), ctypes.byref(a), 2) > 0
    assert pipeline.selected_rows(s, a) == 1500
    for bad in ([8 * 32 - 1, 900, 900], [900, 8 * 16384 + 1, 900]):
        a = pipeline.make_alloc(cfg, inst_budget=bad)
        st = L.adakv_allocate(ctypes.byref(s), ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
        assert st == lib.ADAKV_EINVAL
    for mode in (lib.ADAKV_ALLOC_ADA_CRITICALKV, lib.ADAKV_ALLOC_ADA_FLOOR, lib.ADAKV_ALLOC_STREAMING,
                 lib.ADAKV_ALLOC_GLOBAL, lib.ADAKV_ALLOC_LAVA_LAYERS):
        a = pipeline.make_alloc(cfg, inst_budget=good)
        a.mode = mode
        a.budget = 3 * 8 * 32 + 10
        st = L.adakv_allocate(ctypes.byref(s), ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
        assert st == lib.ADAKV_EUNSUPPORTED, mode


def test_compact_rejects(L):
    s, a = _shape(), _alloc()
    assert L.adakv_compact(ctypes.byref(s), ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, -1, FAKE, FAKE, FAKE,
                           FAKE, None) == lib.ADAKV_EINVAL
    assert L.adakv_compact(ctypes.byref(s), ctypes.byref(a), None, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE,
                           FAKE, None) == lib.ADAKV_EINVAL


def test_decode_rejects(L):
    s, a = _shape(), _alloc()

    def dec(k_new, v_new, reserve, step, ws_bytes=1 << 40, shape=s):
        return L.adakv_decode_attn(ctypes.byref(shape), ctypes.byref(a), FAKE, k_new, v_new, FAKE, FAKE, FAKE,
                                   FAKE, reserve, step, FAKE, FAKE, ws_bytes, None)
    assert dec(FAKE, FAKE, 2, 2) == lib.ADAKV_ECAPACITY          # append past the reserve
    assert dec(FAKE, FAKE, 0, 0) == lib.ADAKV_ECAPACITY
    assert dec(FAKE, None, 2, 0) == lib.ADAKV_EINVAL             # k_new without v_new
    assert dec(None, None, 2, 3) == lib.ADAKV_EINVAL             # more appends than rows reserved
    assert dec(FAKE, FAKE, 2, 0, ws_bytes=8) == lib.ADAKV_EWORKSPACE
    assert dec(FAKE, FAKE, 2, 0, shape=_shape(hq=80, hkv=8)) == lib.ADAKV_EUNSUPPORTED


def test_decode_noalloc_rejects(L):
    """The allocation-free decode validates exactly as adakv_decode_attn
    (before it touches the device)."""
    s, a = _shape(), _alloc()

    def dec(k_new, v_new, reserve, step, shape=s):
        return L.adakv_decode_attn_noalloc(ctypes.byref(shape), ctypes.byref(a), FAKE, k_new, v_new, FAKE, FAKE,
                                           FAKE, FAKE, reserve, step, FAKE, None)
    assert dec(FAKE, FAKE, 2, 2) == lib.ADAKV_ECAPACITY
    assert dec(FAKE, None, 2, 0) == lib.ADAKV_EINVAL
    assert dec(None, None, 2, 3) == lib.ADAKV_EINVAL
    assert dec(FAKE, FAKE, 2, 0, shape=_shape(hq=80, hkv=8)) == lib.ADAKV_EUNSUPPORTED
    assert L.adakv_decode_attn_noalloc(None, ctypes.byref(a), FAKE, None, None, FAKE, FAKE, FAKE, FAKE, 2, 0, FAKE,
                                       None) == lib.ADAKV_EINVAL
    assert L.adakv_decode_attn_noalloc(ctypes.byref(s), ctypes.byref(a), FAKE + 4, None, None, FAKE, FAKE, FAKE,
                                       FAKE, 2, 0, FAKE, None) == lib.ADAKV_EINVAL


def test_no_undefined_kernel_stubs(L):
    """Every kernel launched from host code has its host-side stub in the
    library (a stub can silently go missing when a device-only construct is
    rejected by the host compilation pass)."""
    out = subprocess.run(["nm", "-D", "--undefined-only", lib.LIB_PATH], capture_output=True, text=True).stdout
    assert "device_stub" not in out


def test_laprox_score_rejects(L):
    lp = dict(scorer=lib.ADAKV_SCORE_LAPROX, hidden=4096, pool=1)
    assert score_status(L, _shape(**{**lp, "pool": 7})) == lib.ADAKV_EINVAL       # no pooling in LaProx
    assert score_status(L, _shape(**{**lp, "hidden": 0})) == lib.ADAKV_EINVAL
    assert score_status(L, _shape(**{**lp, "hidden": 100})) == lib.ADAKV_EUNSUPPORTED
    assert score_status(L, _shape(**{**lp, "d": 64})) == lib.ADAKV_EUNSUPPORTED
    assert score_status(L, _shape(**lp), ptrs=FAKE + 4) == lib.ADAKV_EINVAL
    assert score_status(L, _shape(**lp), ws_bytes=16) == lib.ADAKV_EWORKSPACE
    assert score_status(L, _shape(scorer=4)) == lib.ADAKV_EINVAL


def test_global_budget_range(L):
    s = _shape(n_inst=4, scorer=lib.ADAKV_SCORE_LAPROX, hidden=4096, pool=1)
    p = s.n - s.w
    for budget in (4 * 32 * 8 - 1, 4 * 32 * 8 + 4 * 8 * p + 1):
        a = _alloc(mode=lib.ADAKV_ALLOC_GLOBAL, budget=budget)
        st = L.adakv_allocate(ctypes.byref(s), ctypes.byref(a), FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
        assert st == lib.ADAKV_EINVAL
    big = _shape(n_inst=2048, n=200000)        # 2048 * 8 * 199968 scores: past 32-bit counts
    a = _alloc(mode=lib.ADAKV_ALLOC_GLOBAL, budget=2048 * 32 * 8)
    st = L.adakv_allocate(ctypes.byref(big), ctypes.byref(a), FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == lib.ADAKV_EUNSUPPORTED
    assert lib.adakv_workspace_bytes(s, _alloc(mode=lib.ADAKV_ALLOC_GLOBAL, budget=4 * 32 * 8 + 100), 0) > 0


def test_floor_and_streaming_rejects(L):
    s = _shape()
    for kw in (dict(mode=lib.ADAKV_ALLOC_STREAMING, sinks=-1), dict(mode=6),
               dict(mode=lib.ADAKV_ALLOC_ADA_FLOOR, alpha_num=2, alpha_den=1),
               dict(mode=lib.ADAKV_ALLOC_ADA_FLOOR, budget=8 * 32 - 1)):
        a = _alloc(**kw)
        st = L.adakv_allocate(ctypes.byref(s), ctypes.byref(a), FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
        assert st == lib.ADAKV_EINVAL, kw
    # StreamingLLM needs no scores, every other mode does
    a = _alloc(mode=lib.ADAKV_ALLOC_ADA_FLOOR)
    st = L.adakv_allocate(ctypes.byref(s), ctypes.byref(a), None, None, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == lib.ADAKV_EINVAL
    assert lib.adakv_workspace_bytes(s, _alloc(mode=lib.ADAKV_ALLOC_ADA_FLOOR), 0) > \
        lib.adakv_workspace_bytes(s, _alloc(mode=lib.ADAKV_ALLOC_ADA), 0) - 1


def online_status(L, shape, total, layer_ent=FAKE, prev_budgets=FAKE, prev_sel=FAKE, prev_off=FAKE,
                  ws_bytes=1 << 40):
    return L.adakv_lava_online_allocate(ctypes.byref(shape), total, FAKE, prev_off, prev_budgets, prev_sel,
                                        layer_ent, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)


def test_lava_online_allocate_rejects(L):
    """The online allocation's own arguments: the per-layer entropy array is
    required and 8-byte aligned, the previous budgets and selection come
    together and aligned, the previous offsets are aligned, the windows fit
    the total, and the workspace is large enough (every case is refused before
    anything is launched)."""
    s = _shape(n_inst=2, scorer=lib.ADAKV_SCORE_LAVA)
    total = 2 * s.w * s.hkv + 500
    assert online_status(L, s, total, layer_ent=None) == lib.ADAKV_EINVAL
    assert online_status(L, s, total, layer_ent=FAKE + 4) == lib.ADAKV_EINVAL
    assert online_status(L, s, total, prev_sel=None) == lib.ADAKV_EINVAL
    assert online_status(L, s, total, prev_budgets=None) == lib.ADAKV_EINVAL
    assert online_status(L, s, total, prev_sel=FAKE + 4) == lib.ADAKV_EINVAL
    assert online_status(L, s, total, prev_budgets=FAKE + 8) == lib.ADAKV_EINVAL
    assert online_status(L, s, total, prev_off=FAKE + 8) == lib.ADAKV_EINVAL
    assert online_status(L, s, 2 * s.w * s.hkv - 1) == lib.ADAKV_EINVAL
    assert online_status(L, s, total, ws_bytes=16) == lib.ADAKV_EWORKSPACE

"""The C ABI without a GPU: exports, version, status strings, workspace sizes
and host-side argument checks (every call here fails validation before any
HIP call, so nothing is launched)."""

import ctypes
import os
import re

import pytest

from mixture_experts_routing_moe_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import mixture_experts_routing_moe_amd.build as b
        b.build()
    return _lib.lib()


def test_header_declares_the_expected_calls():
    names = declared_functions()
    for n in ("moe_route", "moe_align", "moe_indices_to_multihot", "moe_multihot_to_indices",
              "moe_expert_ffn", "moe_expert_ffn_decode"):
        assert n in names
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings(lib):
    assert lib.moe_version() == 6
    for s in range(5):
        assert lib.moe_status_string(s)
    assert lib.moe_status_string(99) == b"unknown status"


def test_workspace_sizes(lib):
    assert lib.moe_align_workspace_size(16384, 8, 64) >= 64 * 4
    assert lib.moe_align_workspace_size(-1, 8, 64) == 0
    assert lib.moe_align_workspace_size(0, 8, 64) > 0
    n = lib.moe_expert_ffn_workspace_size(_lib.MOE_BF16, 4096, 4096, 14336, 8, 2)
    assert n >= 8192 * (14336 + 4096) * 2
    assert lib.moe_expert_ffn_workspace_size(_lib.MOE_F32, 4, 64, 128, 8, 2) >= 8 * (128 + 64) * 4


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def status(lib, fn, *args):
    return getattr(lib, fn)(*args)


def test_route_validation(lib):
    I = _lib.MOE_ERR_INVALID_ARG
    assert status(lib, "moe_route", FAKE, 4, 8, 9, 1, FAKE, FAKE, None) == I  # k > E
    assert b"k = 9 > E = 8" in lib.moe_last_error()
    assert status(lib, "moe_route", FAKE, 4, 0, 1, 1, FAKE, FAKE, None) == I  # E < 1
    assert status(lib, "moe_route", FAKE, 4, 2000, 8, 1, FAKE, FAKE, None) == I  # E too big
    assert status(lib, "moe_route", FAKE, 4, 128, 65, 1, FAKE, FAKE, None) == I  # k > 64
    assert status(lib, "moe_route", FAKE, -1, 8, 2, 1, FAKE, FAKE, None) == I
    assert status(lib, "moe_route", None, 4, 8, 2, 1, FAKE, FAKE, None) == I  # null
    assert status(lib, "moe_route", None, 0, 8, 2, 1, None, None, None) == _lib.MOE_OK  # T=0


def test_router_route_validation(lib):
    I, U = _lib.MOE_ERR_INVALID_ARG, _lib.MOE_ERR_UNSUPPORTED
    B = _lib.MOE_BF16

    def rr(dt, T, H, E, k, x=FAKE, w=FAKE, lg=FAKE, tw=FAKE, ti=FAKE):
        return lib.moe_router_route(dt, x, w, T, H, E, k, 1, lg, tw, ti, None)

    assert rr(_lib.MOE_F32, 4, 64, 8, 2) == U  # bf16 only
    assert rr(B, 4, 96, 8, 2) == U  # H % 64
    assert b"multiple of 64" in lib.moe_last_error()
    assert rr(B, 4, 64, 8, 9) == I  # k > E
    assert rr(7, 4, 64, 8, 2) == I  # unknown dtype
    assert rr(B, 4, 64, 8, 2, lg=None) == I  # logits are an output, required
    assert rr(B, 4, 64, 8, 2, x=ctypes.c_void_p(0x1008)) == I  # hidden not 16-byte aligned
    assert rr(B, 0, 64, 8, 2, x=None, w=None, lg=None, tw=None, ti=None) == _lib.MOE_OK


def test_route_align_validation(lib):
    I, W = _lib.MOE_ERR_INVALID_ARG, _lib.MOE_ERR_WORKSPACE
    ws_need = lib.moe_align_workspace_size(100, 8, 64)

    def ra(T=100, E=64, k=8, mh=(None, None, None), ws=FAKE, wsb=None, logits=FAKE):
        return lib.moe_route_align(logits, T, E, k, 1, FAKE, FAKE, *mh, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, ws, ws_need if wsb is None else wsb, None)

    assert ra(k=65) == I
    assert ra(E=4, k=5) == I  # k > E
    assert ra(mh=(FAKE, None, None)) == I  # some multihot outputs but not all
    assert b"all three" in lib.moe_last_error()
    assert ra(wsb=ws_need - 1) == W
    assert ra(ws=None) == W
    assert ra(logits=None) == I
    # fused-path predicate: E <= 64, k <= 16, chunks of whole rows
    assert lib.moe_route_align_fused(1, 64, 8) == 1
    assert lib.moe_route_align_fused(16384, 64, 8) == 1
    assert lib.moe_route_align_fused(16384, 64, 6) == 0  # 512-slot chunks hold no whole rows
    assert lib.moe_route_align_fused(4096, 8, 2) == 0  # 16 chunks of 256 rows: separate launches
    assert lib.moe_route_align_fused(100, 128, 8) == 0
    assert lib.moe_route_align_fused(100, 64, 20) == 0


def test_align_inverse_validation(lib):
    I, W = _lib.MOE_ERR_INVALID_ARG, _lib.MOE_ERR_WORKSPACE
    ws_need = lib.moe_align_workspace_size(100, 8, 64)

    def ai(k=8, pim=FAKE, pos=FAKE, probs=FAKE, ws=FAKE, wsb=None):
        return lib.moe_align_inverse(FAKE, 100, k, 64, FAKE, FAKE, FAKE, FAKE, FAKE, pim, pos,
                                     probs, FAKE, ws, ws_need if wsb is None else wsb, None)

    assert ai(k=65) == I
    assert ai(pim=None) == I
    assert ai(pos=None) == I
    assert ai(probs=None) == I
    assert ai(wsb=ws_need - 1) == W


def test_tile_schedule_validation(lib):
    I, U = _lib.MOE_ERR_INVALID_ARG, _lib.MOE_ERR_UNSUPPORTED
    assert lib.moe_tile_schedule_max(4096, 2, 8) == 26 + 8  # ceil(8192 / 320) + E
    assert lib.moe_tile_schedule_max(1, 8, 64) == 1 + 8  # min(E, T k) experts can hold a row
    assert lib.moe_tile_schedule_max(0, 8, 64) == 0

    def ts(E=8, mx=10, off=FAKE, out=FAKE, num=FAKE):
        return lib.moe_tile_schedule(off, E, mx, out, out, out, num, None)

    assert ts(E=0) == U
    assert ts(E=1025) == U
    assert ts(mx=-1) == I
    assert ts(off=None) == I
    assert ts(num=None) == I
    assert ts(out=None) == I
    assert b"null pointer" in lib.moe_last_error()


def test_route_align_inverse_validation(lib):
    I, W = _lib.MOE_ERR_INVALID_ARG, _lib.MOE_ERR_WORKSPACE
    ws_need = lib.moe_align_workspace_size(100, 8, 64)
    M3 = (FAKE, FAKE, FAKE)

    def rai(T=100, mh=M3, probs=FAKE, ids=FAKE, ws=FAKE, wsb=None):
        return lib.moe_route_align_inverse(FAKE, T, 64, 8, 1, FAKE, FAKE, *mh, FAKE, FAKE, FAKE,
                                           FAKE, FAKE, probs, ids, ws,
                                           ws_need if wsb is None else wsb, None)

    assert rai(mh=(None, None, None)) == I  # the multihot outputs are required
    assert rai(mh=(FAKE, None, FAKE)) == I
    assert rai(probs=None) == I
    assert rai(wsb=ws_need - 1) == W
    assert rai(ws=None) == W


def test_route_align_gate_up_validation(lib):
    I, W, U = _lib.MOE_ERR_INVALID_ARG, _lib.MOE_ERR_WORKSPACE, _lib.MOE_ERR_UNSUPPORTED
    bf, f32 = _lib.MOE_BF16, _lib.MOE_F32
    f = lib.moe_route_align_gate_up_fused
    # one launch: bf16 decode, T k <= 16, E <= 64, k <= 16
    assert f(1, 64, 8, bf, 1, 2048, 1408) == 1
    assert f(2, 64, 8, bf, 1, 2048, 1408) == 1
    assert f(16, 8, 1, bf, 1, 128, 128) == 1
    assert f(3, 64, 8, bf, 1, 2048, 1408) == 0  # 24 slots
    assert f(32, 64, 8, bf, 1, 2048, 1408) == 0
    assert f(2, 128, 4, bf, 1, 128, 128) == 0  # E > 64
    assert f(1, 64, 8, bf, 0, 2048, 1408) == 0  # prefill
    assert f(1, 64, 8, f32, 1, 2048, 1408) == 0
    assert f(0, 64, 8, bf, 1, 2048, 1408) == 0
    ws_need = lib.moe_align_workspace_size(4, 8, 64)
    M3 = (FAKE, FAKE, FAKE)

    def rag(T=4, mh=M3, probs=FAKE, ids=FAKE, dt=bf, decode=1, hidden=FAKE, w13=FAKE, H=128,
            I_=128, act=FAKE, ws=FAKE, wsb=None):
        return lib.moe_route_align_gate_up(FAKE, T, 64, 8, 1, FAKE, FAKE, *mh, FAKE, FAKE, FAKE,
                                           FAKE, FAKE, probs, ids, dt, decode, hidden, w13, H,
                                           I_, act, ws, ws_need if wsb is None else wsb, None)

    assert rag(mh=(FAKE, None, FAKE)) == I  # all three maps or none
    assert rag(mh=(None, None, None)) == I  # the inverse needs the maps
    assert rag(wsb=ws_need - 1) == W
    assert rag(H=100) == U  # H % 64
    assert rag(dt=7) == I
    assert rag(hidden=None) == I
    assert rag(act=ctypes.c_void_p(0x1008)) == I  # 16-byte alignment
    assert rag(T=65, wsb=1 << 40) == U  # decode T limit
    assert b"decode" in lib.moe_last_error()


def test_route_grouped_validation(lib):
    I = _lib.MOE_ERR_INVALID_ARG
    G, N = _lib.MOE_GROUP_LIMITED_GREEDY, _lib.MOE_NOAUX_TC

    def rg(T, E, k, ng, tg, m, scores=FAKE, bias=FAKE, w=FAKE, ids=FAKE, mh=(None, None, None)):
        return lib.moe_route_grouped(scores, bias, T, E, k, ng, tg, m, 0, w, ids, *mh, None)

    assert rg(4, 250, 8, 8, 4, N) == I  # E % n_group != 0
    assert b"not a multiple" in lib.moe_last_error()
    assert rg(4, 256, 8, 8, 9, N) == I  # topk_group > n_group
    assert rg(4, 256, 8, 8, 0, N) == I  # topk_group < 1
    assert rg(4, 256, 8, 128, 4, G) == I  # n_group > 64
    assert rg(4, 64, 9, 8, 1, G) == I  # k > topk_group * group size
    assert b"group size" in lib.moe_last_error()
    assert rg(4, 64, 2, 64, 4, N) == I  # noaux_tc with groups of one
    assert rg(4, 64, 2, 8, 2, 7) == I  # unknown method
    assert rg(4, 64, 2, 8, 2, N, bias=None) == I  # noaux_tc without the bias
    assert rg(4, 64, 2, 8, 2, G, scores=None) == I
    assert rg(4, 64, 2, 8, 2, G, scores=ctypes.c_void_p(0x1002)) == I  # misaligned
    assert rg(0, 64, 2, 8, 2, N, scores=None, bias=None, w=None, ids=None) == _lib.MOE_OK
    assert rg(4, 64, 2, 8, 2, G, mh=(FAKE, FAKE, None)) == I  # multihot outputs: all or none


def test_route_multihot_validation(lib):
    I = _lib.MOE_ERR_INVALID_ARG
    f = "moe_route_multihot"
    assert status(lib, f, FAKE, 4, 8, 9, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == I  # k > E
    assert status(lib, f, FAKE, 4, 8, 2, 1, FAKE, FAKE, None, FAKE, FAKE, None) == I  # null
    assert status(lib, f, FAKE, 4, 2000, 8, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == I
    assert status(lib, f, None, 0, 8, 2, 1, None, None, None, None, None, None) == _lib.MOE_OK
    fused = lib.moe_route_multihot_fused
    assert fused(64, 8) == 1 and fused(8, 2) == 1 and fused(4, 4) == 1
    assert fused(6, 2) == 0 and fused(128, 8) == 0 and fused(64, 17) == 0 and fused(8, 9) == 0


def test_align_validation(lib):
    ws = lib.moe_align_workspace_size(100, 2, 8)
    assert status(lib, "moe_align", FAKE, 100, 2, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1,
                  None) == _lib.MOE_ERR_WORKSPACE
    assert status(lib, "moe_align", FAKE, 100, 2, 8, FAKE, FAKE, FAKE, FAKE, FAKE, None, ws,
                  None) == _lib.MOE_ERR_WORKSPACE
    assert status(lib, "moe_align", FAKE, 100, 2, 8, None, FAKE, FAKE, FAKE, FAKE, FAKE, ws,
                  None) == _lib.MOE_ERR_INVALID_ARG
    assert status(lib, "moe_align", FAKE, 1 << 30, 4, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws,
                  None) == _lib.MOE_ERR_INVALID_ARG  # T*k overflows int32


def test_converter_validation(lib):
    I = _lib.MOE_ERR_INVALID_ARG
    assert status(lib, "moe_indices_to_multihot", FAKE, FAKE, 4, 2, 8, None, FAKE, FAKE,
                  None) == I
    assert status(lib, "moe_indices_to_multihot", FAKE, FAKE, 4, 0, 8, FAKE, FAKE, FAKE,
                  None) == I
    assert status(lib, "moe_multihot_to_indices", FAKE, None, 4, 8, 2, FAKE, None, None) == I
    assert status(lib, "moe_multihot_to_indices", None, None, 0, 8, 2, None, None,
                  None) == _lib.MOE_OK


def test_ffn_validation(lib):
    bf = _lib.MOE_BF16
    ws = lib.moe_expert_ffn_workspace_size(bf, 16, 128, 128, 8, 2)
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    # H not a multiple of 64
    assert status(lib, "moe_expert_ffn", bf, *args, 16, 96, 128, 8, 2, FAKE, FAKE, ws,
                  None) == _lib.MOE_ERR_UNSUPPORTED
    # workspace too small
    assert status(lib, "moe_expert_ffn", bf, *args, 16, 128, 128, 8, 2, FAKE, FAKE, ws - 1,
                  None) == _lib.MOE_ERR_WORKSPACE
    # decode beyond its token limit
    assert status(lib, "moe_expert_ffn_decode", bf, *args, 65, 128, 128, 8, 2, FAKE, FAKE,
                  1 << 40, None) == _lib.MOE_ERR_UNSUPPORTED
    # misaligned workspace
    assert status(lib, "moe_expert_ffn", bf, *args, 16, 128, 128, 8, 2, FAKE,
                  ctypes.c_void_p(0x1008), ws, None) == _lib.MOE_ERR_INVALID_ARG
    # unknown dtype
    assert status(lib, "moe_expert_ffn", 7, *args, 16, 128, 128, 8, 2, FAKE, FAKE, ws,
                  None) == _lib.MOE_ERR_INVALID_ARG
    # misaligned act for a phase call
    assert status(lib, "moe_ffn_gate_up", bf, 0, FAKE, FAKE, FAKE, FAKE, 16, 128, 128, 8, 2,
                  ctypes.c_void_p(0x1002), None) == _lib.MOE_ERR_INVALID_ARG
    assert status(lib, "moe_combine", bf, FAKE, 1, FAKE, FAKE, 4, 100, 2, FAKE,
                  None) == _lib.MOE_ERR_UNSUPPORTED
    assert status(lib, "moe_expert_ffn", bf, None, None, None, None, None, None, None, 0, 128,
                  128, 8, 2, None, None, 0, None) == _lib.MOE_OK  # T = 0


def test_down_splits(lib):
    bf, f32 = _lib.MOE_BF16, _lib.MOE_F32
    f = lib.moe_ffn_down_splits
    # Mixtral-shaped FC2: 30 x 16 = 480 expected tiles fill 1.9 rounds of
    # 256 CUs; two K slices of 7168 make 3.75 rounds, which does not pay for
    # the extra y plane.
    assert f(bf, 0, 4096, 4096, 14336, 8, 2) == 1
    # 4 experts of ~4096 rows: 54 x 16 = 864 expected tiles leave the last of
    # 3.4 rounds 40 % full; two slices make 6.75 rounds.
    assert f(bf, 0, 8192, 4096, 14336, 4, 2) == 2
    # Fine-grained FC2: ~2300 tiles already fill the chip; K = 1408 is too
    # short to cut.
    assert f(bf, 0, 8192, 2048, 1408, 64, 8) == 1
    assert f(f32, 0, 4096, 4096, 14336, 8, 2) == 1
    assert f(bf, 1, 32, 2048, 1408, 64, 8) == 1
    for T in (1, 7, 100, 1000, 5000, 20000):
        for I in (1408, 4096, 14336):
            sp = f(bf, 0, T, 4096, I, 8, 2)
            assert 1 <= sp <= _lib.MOE_MAX_SPLITS and I % (64 * sp) == 0
    # the one-call workspace holds act plus every y plane
    n1 = lib.moe_expert_ffn_workspace_size(bf, 8192, 2048, 1408, 64, 8)
    assert n1 >= 65536 * (1408 * 2 + 2048 * 4)
    n2 = lib.moe_expert_ffn_workspace_size(bf, 4096, 4096, 14336, 8, 2)
    sp = f(bf, 0, 4096, 4096, 14336, 8, 2)
    assert n2 >= 8192 * 14336 * 2 + sp * 8192 * 4096 * 4


def test_down_split_validation(lib):
    bf, f32 = _lib.MOE_BF16, _lib.MOE_F32
    a = (FAKE, FAKE, FAKE, 16, 128, 256, 8, 2)
    assert status(lib, "moe_ffn_down", bf, 0, *a, 0, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert status(lib, "moe_ffn_down", bf, 0, *a, _lib.MOE_MAX_SPLITS + 1, FAKE,
                  None) == _lib.MOE_ERR_INVALID_ARG
    # I = 256 cuts into at most 4 slices of 64
    assert status(lib, "moe_ffn_down", bf, 0, *a, 8, FAKE, None) == _lib.MOE_ERR_UNSUPPORTED
    assert status(lib, "moe_ffn_down", bf, 1, *a, 2, FAKE, None) == _lib.MOE_ERR_UNSUPPORTED
    assert status(lib, "moe_ffn_down", f32, 0, *a, 2, FAKE, None) == _lib.MOE_ERR_UNSUPPORTED
    assert status(lib, "moe_combine", bf, FAKE, 0, FAKE, FAKE, 4, 128, 2, FAKE,
                  None) == _lib.MOE_ERR_INVALID_ARG


def test_down_combine_validation(lib):
    bf, f32 = _lib.MOE_BF16, _lib.MOE_F32
    f = lib.moe_ffn_down_combine_fused
    # one launch for bf16 decode with at most 32 slots and I <= 1536
    assert f(bf, 1, 1, 2048, 1408, 64, 8) == 1
    assert f(bf, 1, 4, 2048, 1408, 64, 8) == 1
    assert f(bf, 1, 8, 128, 1536, 8, 4) == 1
    assert f(bf, 1, 32, 2048, 1408, 64, 8) == 0  # 256 slots
    assert f(bf, 1, 1, 2048, 1600, 8, 2) == 0
    assert f(bf, 0, 1, 2048, 1408, 64, 8) == 0  # prefill
    assert f(f32, 1, 1, 2048, 1408, 64, 8) == 0
    assert f(bf, 1, 0, 2048, 1408, 64, 8) == 0
    call = "moe_ffn_down_combine"
    a = (FAKE, FAKE, FAKE, FAKE, FAKE)  # act, w2, topk_w, offsets, slot_to_sorted
    # y may be NULL only where the call is fused
    assert status(lib, call, bf, 1, *a, 33, 128, 128, 8, 1, None, FAKE,
                  None) == _lib.MOE_ERR_INVALID_ARG
    assert status(lib, call, bf, 0, *a, 1, 128, 128, 8, 2, None, FAKE,
                  None) == _lib.MOE_ERR_INVALID_ARG
    assert status(lib, call, bf, 1, *a, 1, 128, 128, 8, 2, FAKE, None,
                  None) == _lib.MOE_ERR_INVALID_ARG  # no out
    # fused: 16-byte aligned act, w2 and out
    assert status(lib, call, bf, 1, ctypes.c_void_p(0x1002), *a[1:], 1, 128, 128, 8, 2, None,
                  FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert status(lib, call, bf, 1, *a, 1, 128, 128, 8, 2, None, ctypes.c_void_p(0x1008),
                  None) == _lib.MOE_ERR_INVALID_ARG
    assert status(lib, call, bf, 1, *a, 65, 128, 128, 8, 2, FAKE, FAKE,
                  None) == _lib.MOE_ERR_UNSUPPORTED  # decode T limit
    assert status(lib, call, bf, 1, *a, 1, 100, 128, 8, 2, FAKE, FAKE,
                  None) == _lib.MOE_ERR_UNSUPPORTED  # H % 64
    assert status(lib, call, bf, 1, None, None, None, None, None, 0, 128, 128, 8, 2, None,
                  None, None) == _lib.MOE_OK  # T = 0


def test_last_error_is_thread_local(lib):
    import threading
    status(lib, "moe_route", FAKE, 4, 8, 9, 1, FAKE, FAKE, None)
    seen = []

    def other():
        seen.append(lib.moe_last_error())

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen == [b""]
    assert b"k = 9" in lib.moe_last_error()


def test_even_mtile_split_never_empty():
    """The grouped GEMMs deal an expert's cn rows to mt = ceil(cn / 320)
    m-tiles in equal shares rounded up to whole 32-row fragments; every tile
    must get at least one row and none more than 320."""
    bm = 320
    for cn in range(1, 200000):
        mt = -(-cn // bm)
        q = -(-cn // (32 * mt)) * 32
        assert q <= bm and (mt - 1) * q < cn <= mt * q, cn


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU; asking for more exits with status 2 and a JSON
    message before anything touches a GPU."""
    import json
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_traffic_records_match_their_sources():
    """Every committed HBM-traffic record (profiles/traffic_*.json: the
    copy-calibrated FETCH_SIZE / WRITE_SIZE counter runs that bench.py reports
    as roofline.traffic) holds the hash of the kernel sources it was taken on.
    bench.py reports null for a record whose sources changed since, so none
    may be stale; each names one of bench.py's kernel source sets, positive
    bytes, its calibration and the commands that made it."""
    import glob
    import json
    import sys
    sys.path.insert(0, ROOT)
    import bench
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json")))
    assert paths
    for path in paths:
        with open(path) as f:
            rec = json.load(f)
        assert rec["source"] in list(bench.KERNEL_SRC.values()), path
        assert rec["source_sha256_16"] == bench.source_hash(rec["source"]), f"stale: {path}"
        assert rec["hbm_bytes_per_launch"] > 0 and rec["algorithmic_bytes_per_launch"] > 0, path
        cal = rec["copy_calibration"]
        assert cal["fetch_factor"] > 0 and cal["write_factor"] > 0, path
        assert any("FETCH_SIZE" in c for c in rec["commands"]), path
        assert any("WRITE_SIZE" in c for c in rec["commands"]), path


def test_route_backward_validation(lib):
    I = _lib.MOE_ERR_INVALID_ARG

    def rb(T=4, E=8, k=2, lg=FAKE, ids=FAKE, w=FAKE, g=FAKE, out=FAKE):
        return lib.moe_route_backward(lg, ids, w, g, T, E, k, 1, out, None)

    assert rb(k=9) == I  # k > E
    assert rb(E=0) == I
    assert rb(T=-1) == I
    assert rb(out=None) == I
    assert rb(g=None) == I
    assert rb(T=0, lg=None, ids=None, w=None, g=None, out=None) == _lib.MOE_OK


def test_ffn_backward_validation(lib):
    I, U, W = _lib.MOE_ERR_INVALID_ARG, _lib.MOE_ERR_UNSUPPORTED, _lib.MOE_ERR_WORKSPACE
    B = _lib.MOE_BF16
    T, H, Im, E, k = 100, 128, 192, 8, 2
    need = lib.moe_expert_ffn_backward_workspace_size(T, H, Im, E, k)
    assert need >= T * k * (10 * Im + 12 * H)
    assert lib.moe_expert_ffn_backward_workspace_size(0, H, Im, E, k) == 0

    def fb(dt=B, T=T, H=H, I=Im, E=E, k=k, x=FAKE, dx=FAKE, ws=FAKE, wsb=need):
        return lib.moe_expert_ffn_backward(dt, x, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           T, H, I, E, k, dx, FAKE, FAKE, FAKE, ws, wsb, None)

    need32 = T * k * (6 * Im + H) * 4  # the float32 path's need, covered by the size call
    assert need32 <= need
    assert fb(dt=_lib.MOE_F32, wsb=need32 - 1) == W
    assert fb(dt=7) == I  # unknown dtype
    assert fb(H=96) == U  # H % 64
    assert fb(I=100) == U
    assert fb(k=65) == I  # k > MOE_MAX_TOPK
    assert fb(x=None) == I
    assert fb(dx=None) == I
    assert fb(x=ctypes.c_void_p(0x1008)) == I  # not 16-byte aligned
    assert fb(wsb=T * k * (10 * Im + 12 * H) - 1) == W  # below the bfloat16 path's need
    assert fb(ws=None) == W
    assert fb(T=0, x=None, dx=None, ws=None, wsb=0) == _lib.MOE_OK


def test_router_backward_validation(lib):
    I, U, W = _lib.MOE_ERR_INVALID_ARG, _lib.MOE_ERR_UNSUPPORTED, _lib.MOE_ERR_WORKSPACE
    B = _lib.MOE_BF16
    T, H, E = 300, 128, 64
    need = lib.moe_router_backward_workspace_size(T, H, E)
    assert need == 2 * E * H * 4  # two chunks of 256 tokens
    assert lib.moe_router_backward_workspace_size(0, H, E) == 0

    def rb(dt=B, T=T, H=H, E=E, x=FAKE, gh=FAKE, ws=FAKE, wsb=need):
        return lib.moe_router_backward(dt, x, FAKE, FAKE, T, H, E, gh, FAKE, ws, wsb, None)

    assert rb(dt=_lib.MOE_F32) == U
    assert rb(H=96) == U
    assert rb(E=0) == I
    assert rb(E=2000) == I
    assert rb(x=None) == I
    assert rb(gh=ctypes.c_void_p(0x1008)) == I
    assert rb(wsb=need - 1) == W
    assert rb(T=0, x=None, gh=None, ws=None, wsb=0) == _lib.MOE_OK

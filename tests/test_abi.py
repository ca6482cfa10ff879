"""The C-ABI library loads, exports every symbol its header declares, and rejects bad
arguments synchronously -- all without a GPU (no call here reaches a launch)."""
import ctypes
import os
import re

import pytest

import oracle
from combine_moe_dispatch_02_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe355.h")


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"MOE355_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_abi.LIB_PATH):
        pytest.fail("libmoe355.so is not built (run __graft_entry__.build())")
    return _abi.load()


def test_header_declares_the_four_calls():
    names = set(declared_symbols())
    assert {"moe_plan", "moe_dispatch", "moe_expert_ffn", "moe_combine"} <= names
    assert len(names) == 21


def test_every_declared_symbol_is_exported(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert {n for n, _, _ in _abi.SIGNATURES} == set(declared_symbols())


def test_status_strings(lib):
    for code in range(5):
        assert lib.moe_status_string(code)
    assert lib.moe_status_string(99) == b"unknown status"


@pytest.mark.parametrize("T,K,E,tile", [(64, 2, 8, 16), (128, 8, 128, 64), (8192, 8, 32, 128),
                                        (16384, 8, 128, 128), (1, 1, 1, 16), (3, 5, 7, 32)])
def test_pool_bound_matches_oracle(lib, T, K, E, tile):
    assert lib.moe_pool_rows_upper_bound(T, K, E, tile) == oracle.pool_rows_bound(T, K, E, tile)


def test_pool_bound_rejects_bad_sizes(lib):
    assert lib.moe_pool_rows_upper_bound(0, 2, 8, 16) == 0
    assert lib.moe_pool_rows_upper_bound(4, 17, 8, 16) == 0
    assert lib.moe_pool_rows_upper_bound(4, 2, 8, 24) == 0
    assert lib.moe_pool_rows_upper_bound(4, 2, 0, 16) == 0


def test_workspace_bytes(lib):
    plan_only = lib.moe_workspace_bytes(16384, 8, 128, 128, 0, 0, 0)
    full_bf16 = lib.moe_workspace_bytes(16384, 8, 128, 128, 0, 1536, 0)
    full_fp8 = lib.moe_workspace_bytes(16384, 8, 128, 128, 0, 1536, 1)
    rows = oracle.pool_rows_bound(16384, 8, 128, 128)
    assert plan_only > 0
    assert full_bf16 - plan_only >= rows * 1536 * 2
    assert full_fp8 - plan_only >= rows * 1536 + rows * 12 * 4
    full_mx = lib.moe_workspace_bytes(16384, 8, 128, 128, 0, 1536, 2)
    assert full_mx - plan_only >= rows * 1536 + rows * 48
    # mxfp4 h scales are ceil(I/128) 4-byte words per row (tile-major): I = 160 needs 8 bytes a row
    r16 = oracle.pool_rows_bound(16, 2, 4, 16)
    assert lib.moe_workspace_bytes(16, 2, 4, 16, 0, 160, 2) - lib.moe_workspace_bytes(16, 2, 4, 16, 0, 0, 0) >= \
        r16 * 160 + r16 * 8
    assert lib.moe_workspace_bytes(16, 2, 4, 16, 0, 100, 1) == 0     # fp8 needs I % 128 == 0
    assert lib.moe_workspace_bytes(16, 2, 4, 16, 0, 48, 2) == 0      # mxfp4 needs I % 32 == 0
    assert lib.moe_workspace_bytes(16, 2, 4, 16, 0, 64, 7) == 0      # unknown dtype


def _fake_plan(**kw):
    # addresses are never dereferenced: every case below fails validation first
    f = dict(T=64, K=2, expert_begin=0, E_local=8, tile=16,
             rows_cap=oracle.pool_rows_bound(64, 2, 8, 16))
    f.update(kw)
    p = _abi.PlanT(f["T"], f["K"], f["expert_begin"], f["E_local"], f["tile"], f["rows_cap"],
                   0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000)
    return p


BAD_PLANS = [dict(T=0), dict(K=0), dict(K=17), dict(E_local=0), dict(E_local=1025), dict(tile=48),
             dict(expert_begin=-1), dict(rows_cap=16)]


@pytest.mark.parametrize("bad", BAD_PLANS)
def test_plan_validation(lib, bad):
    p = _fake_plan(**bad)
    assert lib.moe_plan(ctypes.c_void_p(0x8000), ctypes.byref(p), ctypes.c_void_p(0x9000), 1 << 20,
                        None) == _abi.MOE_ERR_INVALID


def test_plan_null_pointers(lib):
    p = _fake_plan()
    assert lib.moe_plan(None, ctypes.byref(p), ctypes.c_void_p(0x9000), 1 << 20, None) == 1
    assert lib.moe_plan(ctypes.c_void_p(0x8000), None, ctypes.c_void_p(0x9000), 1 << 20, None) == 1
    p.src = None
    assert lib.moe_plan(ctypes.c_void_p(0x8000), ctypes.byref(p), ctypes.c_void_p(0x9000), 1 << 20,
                        None) == 1


def test_plan_small_workspace(lib):
    p = _fake_plan()
    assert lib.moe_plan(ctypes.c_void_p(0x8000), ctypes.byref(p), ctypes.c_void_p(0x9000), 64,
                        None) == _abi.MOE_ERR_INVALID


def test_dispatch_validation(lib):
    p = _fake_plan()
    X, POOL, WS = (ctypes.c_void_p(a) for a in (0x10000, 0x20000, 0x30000))
    big = 1 << 30
    # epoch 0 is reserved
    assert lib.moe_dispatch(X, 128, 0, ctypes.byref(p), 248, POOL, None, 0, WS, big, None) == 1
    # bf16 takes no scale buffer; fp8 needs one
    assert lib.moe_dispatch(X, 128, 0, ctypes.byref(p), 248, POOL, ctypes.c_void_p(8), 1, WS, big, None) == 1
    assert lib.moe_dispatch(X, 128, 1, ctypes.byref(p), 248, POOL, None, 1, WS, big, None) == 1
    # shapes outside the kernels
    assert lib.moe_dispatch(X, 100, 0, ctypes.byref(p), 248, POOL, None, 1, WS, big, None) == 2
    assert lib.moe_dispatch(X, 192, 1, ctypes.byref(p), 248, POOL, ctypes.c_void_p(8), 1, WS, big, None) == 2
    assert lib.moe_dispatch(X, 128, 5, ctypes.byref(p), 248, POOL, None, 1, WS, big, None) == 1
    # mxfp4: needs its E8M0 buffer and whole 32-wide blocks
    assert lib.moe_dispatch(X, 128, 2, ctypes.byref(p), 248, POOL, None, 1, WS, big, None) == 1
    assert lib.moe_dispatch(X, 136, 2, ctypes.byref(p), 248, POOL, ctypes.c_void_p(8), 1, WS, big, None) == 2
    # scaled pools hold whole tiles (tile 16 here): their scale words are tile-major, and a row
    # of a partial last tile would address a word past the buffer
    for dt in (1, 2):
        assert lib.moe_dispatch(X, 128, dt, ctypes.byref(p), 200, POOL, ctypes.c_void_p(8), 1, WS, big,
                                None) == _abi.MOE_ERR_INVALID
    # a bf16 pool of any row count is fine for the checks (it has no scale words)
    assert lib.moe_dispatch(X, 100, 0, ctypes.byref(p), 200, POOL, None, 1, WS, big, None) == 2


def test_ffn_validation(lib):
    p = _fake_plan()
    v = [ctypes.c_void_p(a) for a in range(0x10000, 0x10000 * 9, 0x10000)]
    POOL, W1, W2, WS, Y = v[:5]
    big = 1 << 40

    def call(H=128, I=64, dtype=0, epoch=1, rows=256, ws=big, cfg=None, scales=(None, None, None)):
        ps, w1s, w2s = scales
        return lib.moe_expert_ffn(ctypes.byref(p), rows, POOL, ps, W1, w1s, W2, w2s, H, I, dtype,
                                  epoch, WS, ws, Y, cfg, None)

    assert call(epoch=0) == 1
    assert call(rows=250) == 1                     # not whole tiles
    assert call(dtype=3) == 1
    assert call(H=96) == 2                         # H % 128
    assert call(I=48) == 2                         # I % 64
    assert call(dtype=1, scales=(v[5], v[6], v[7])) == 2   # fp8 needs tile >= 64
    assert call(dtype=1) == 1                      # fp8 without scales
    assert call(scales=(v[5], None, None)) == 1    # bf16 with scales
    assert call(ws=1024) == 1                      # small workspace
    cfg = _abi.TileConfig(192, 0, 0, 0, 0)
    assert call(cfg=ctypes.byref(cfg)) == 1        # block_n must be 128, 256 or 512
    cfg = _abi.TileConfig(0, 0, 0, 0, 3)
    assert call(cfg=ctypes.byref(cfg)) == 1        # unknown weight layout
    cfg = _abi.TileConfig(0, 0, 0, 0, 1)
    assert call(cfg=ctypes.byref(cfg)) == 2        # tiled weights need the big-tile shapes
    cfg = _abi.TileConfig(0, 0, 0, 10, 0)
    assert call(cfg=ctypes.byref(cfg)) == 1        # unit walks are 0..9
    cfg = _abi.TileConfig(0, -1, 0, 0, 0)
    assert call(cfg=ctypes.byref(cfg)) == 1        # negative grid
    cfg = _abi.TileConfig(0, 0, 0, 0, 0, 3)
    assert call(cfg=ctypes.byref(cfg)) == 1        # A pipeline depth is 0, 2 or 4
    mx = (v[5], v[6], v[7])
    assert call(dtype=2) == 1                      # mxfp4 without scales
    assert call(dtype=2, scales=mx) == 2           # mxfp4 runs on tiled weights only
    tiled = _abi.TileConfig(0, 0, 0, 0, 1)
    assert call(H=512, I=256, dtype=2, scales=mx, cfg=ctypes.byref(tiled)) == 2   # tile 128 only
    cfg = _abi.TileConfig(0, 0, 0, 0, 0, 0, -1)
    assert call(cfg=ctypes.byref(cfg)) == 1        # negative dispatch_cus
    cfg = _abi.TileConfig(0, 0, 0, 0, 0, 0, 0, 64)
    assert call(cfg=ctypes.byref(cfg)) == 1        # unit rows are 128 or 256
    cfg = _abi.TileConfig(0, 0, 0, 0, 1, 0, 0, 256)
    assert call(cfg=ctypes.byref(cfg)) == 2        # 256-row units: tile 128 only (this plan has 16)


def test_ffn_unit_rows_validation(lib):
    # the 256 x 256 units: bf16, tiled weights, tile 128, H % 256, I % 128, no combine on completion
    p = _fake_plan(T=64, K=2, E_local=8, tile=128, rows_cap=oracle.pool_rows_bound(64, 2, 8, 128))
    v = [ctypes.c_void_p(a) for a in range(0x10000, 0x10000 * 9, 0x10000)]
    POOL, W1, W2, WS, Y = v[:5]

    def call(H, I, rows, layout):
        cfg = _abi.TileConfig(0, 0, 0, 0, layout, 0, 0, rows)
        return lib.moe_expert_ffn(ctypes.byref(p), 1152, POOL, None, W1, None, W2, None, H, I, 0, 1, WS, 1 << 40,
                                  Y, ctypes.byref(cfg), None)

    assert call(640, 384, 256, 1) == 2             # H % 256
    assert call(1024, 448, 256, 1) == 2            # I % 128
    assert call(1024, 384, 256, 0) == 2            # row-major weights
    # I = 384 with tiled weights has no 128 x 512 kernel (I % 256): only the 256-row units take it
    assert call(1024, 384, 128, 1) == 2
    cfg = _abi.TileConfig(0, 0, 0, 0, 1, 0, 0, 256)
    assert lib.moe_expert_ffn_combine(ctypes.byref(p), 1152, POOL, None, W1, None, W2, None, 1024, 512, 0, 1, WS,
                                      1 << 40, Y, v[5], v[6], ctypes.byref(cfg), None) == 2   # not with combine


def test_ffn_combine_validation(lib):
    p = _fake_plan()
    v = [ctypes.c_void_p(a) for a in range(0x10000, 0x10000 * 9, 0x10000)]
    POOL, W1, W2, WS, Y, TW, OUT = v[:7]

    def call(tw=TW, out=OUT, H=128, epoch=1):
        return lib.moe_expert_ffn_combine(ctypes.byref(p), 256, POOL, None, W1, None, W2, None, H, 64, 0,
                                          epoch, WS, 1 << 40, Y, tw, out, None, None)

    assert call(tw=None) == 1
    assert call(out=None) == 1
    assert call(epoch=0) == 1
    assert call(H=100) == 2


def test_backward_validation(lib):
    p = _fake_plan()
    v = [ctypes.c_void_p(a) for a in range(0x10000, 0x10000 * 12, 0x10000)]
    big = 1 << 40
    # training forward: g_pool required; tile 16 is outside the big-tile kernel
    assert lib.moe_expert_ffn_train(ctypes.byref(p), 256, v[0], v[1], v[2], 512, 512, 1, v[3], big, v[4], None,
                                    None, None) == 1
    assert lib.moe_expert_ffn_train(ctypes.byref(p), 256, v[0], v[1], v[2], 512, 512, 1, v[3], big, v[4], v[5],
                                    None, None) == 2
    # combine backward: null pointer, epoch 0, no workspace, small workspace, H % 8
    assert lib.moe_combine_backward(None, v[1], v[2], 256, ctypes.byref(p), 128, v[3], v[4], 1, v[5], big,
                                    None) == 1
    assert lib.moe_combine_backward(v[0], v[1], v[2], 256, ctypes.byref(p), 128, v[3], v[4], 0, v[5], big,
                                    None) == 1
    assert lib.moe_combine_backward(v[0], v[1], v[2], 256, ctypes.byref(p), 128, v[3], v[4], 1, None, big,
                                    None) == 1
    assert lib.moe_combine_backward(v[0], v[1], v[2], 256, ctypes.byref(p), 128, v[3], v[4], 1, v[5], 64,
                                    None) == 1
    assert lib.moe_combine_backward(v[0], v[1], v[2], 256, ctypes.byref(p), 100, v[3], v[4], 1, v[5], big,
                                    None) == 2
    # expert backward: null pointer, epoch 0, then tile 16 / shapes outside the kernels
    assert lib.moe_expert_ffn_backward(ctypes.byref(p), 256, v[0], None, v[2], v[3], v[4], 512, 512, 1, v[5], big,
                                       v[6], v[7], v[8], None, None) == 1
    assert lib.moe_expert_ffn_backward(ctypes.byref(p), 256, v[0], v[1], v[2], v[3], v[4], 512, 512, 0, v[5], big,
                                       v[6], v[7], v[8], None, None) == 1
    assert lib.moe_expert_ffn_backward(ctypes.byref(p), 256, v[0], v[1], v[2], v[3], v[4], 512, 512, 1, v[5], big,
                                       v[6], v[7], v[8], None, None) == 2
    q = _fake_plan(tile=128, rows_cap=oracle.pool_rows_bound(64, 2, 8, 128))
    assert lib.moe_expert_ffn_backward(ctypes.byref(q), 256, v[0], v[1], v[2], v[3], v[4], 512, 256, 1, v[5], big,
                                       v[6], v[7], v[8], None, None) == 2      # I % 512
    # dispatch backward
    assert lib.moe_dispatch_backward(None, 256, ctypes.byref(p), 128, v[1], None) == 1
    assert lib.moe_dispatch_backward(v[0], 256, ctypes.byref(p), 100, v[1], None) == 2
    # transposed pack: bf16 only, K % 16, rows % 32
    W, OUT = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x100000000)
    assert lib.moe_pack_weights_transposed(W, 1, 32, 16, 1, OUT, None) == 2
    assert lib.moe_pack_weights_transposed(W, 1, 32, 16, 7, OUT, None) == 1
    assert lib.moe_pack_weights_transposed(W, 1, 48, 16, 0, OUT, None) == 2
    assert lib.moe_pack_weights_transposed(W, 1, 32, 24, 0, OUT, None) == 2


def test_combine_validation(lib):
    p = _fake_plan()
    Y, W, OUT = (ctypes.c_void_p(a) for a in (0x10000, 0x20000, 0x30000))
    assert lib.moe_combine(None, 248, W, ctypes.byref(p), 128, OUT, None) == 1
    assert lib.moe_combine(Y, -1, W, ctypes.byref(p), 128, OUT, None) == 1
    assert lib.moe_combine(Y, 248, W, ctypes.byref(p), 100, OUT, None) == 2


def test_pack_weights_validation(lib):
    W, OUT = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x100000000)
    assert lib.moe_pack_weights(None, 1, 16, 32, 0, OUT, None) == 1
    assert lib.moe_pack_weights(W, 1, 16, 32, 9, OUT, None) == 1
    assert lib.moe_pack_weights(W, 1, 24, 32, 0, OUT, None) == 2      # rows % 16
    assert lib.moe_pack_weights(W, 1, 16, 48, 0, OUT, None) == 2      # bf16 K % 32
    assert lib.moe_pack_weights(W, 1, 16, 64, 1, OUT, None) == 2      # fp8 K % 128
    assert lib.moe_pack_weights(W, 4, 64, 256, 0, ctypes.c_void_p(0x10100), None) == 1  # overlap
    assert lib.moe_pack_weights(W, 1, 16, 64, 2, OUT, None) == 2      # mxfp4 K % 128


def test_pack_mx_scales_validation(lib):
    S, OUT = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x100000000)
    assert lib.moe_pack_mx_scales(None, 1, 16, 128, OUT, None) == 1
    assert lib.moe_pack_mx_scales(S, 0, 16, 128, OUT, None) == 1
    assert lib.moe_pack_mx_scales(S, 1, 24, 128, OUT, None) == 2     # rows % 16
    assert lib.moe_pack_mx_scales(S, 1, 16, 96, OUT, None) == 2      # K % 128
    assert lib.moe_pack_mx_scales(S, 2, 16, 256, ctypes.c_void_p(0x10040), None) == 1  # overlap


def test_get_error_validation(lib):
    assert lib.moe_get_error(None, 1 << 20, None) == 1


def test_calibration_validation(lib):
    # the measurement helpers reject bad arguments before any launch
    S = ctypes.c_void_p(0x10000)
    assert lib.moe_calibrate_mfma(0, S, 8, None) == 1            # iters >= 1
    assert lib.moe_calibrate_mfma(10, None, 8, None) == 1        # sink needed
    assert lib.moe_calibrate_mfma(10, S, 0, None) == 1           # workgroups in [1, 65535]
    assert lib.moe_calibrate_mfma(10, S, 65536, None) == 1
    A, B = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    assert lib.moe_calibrate_stream(A, None, 100, 0, S, 8, None) == 1       # not whole 16-byte chunks
    assert lib.moe_calibrate_stream(None, None, 1024, 0, S, 8, None) == 1   # read needs src and sink
    assert lib.moe_calibrate_stream(A, None, 1024, 0, None, 8, None) == 1
    assert lib.moe_calibrate_stream(None, None, 1024, 1, None, 8, None) == 1  # write needs dst
    assert lib.moe_calibrate_stream(A, None, 1024, 2, None, 8, None) == 1     # copy needs both
    assert lib.moe_calibrate_stream(A, ctypes.c_void_p(0x100100), 1024, 2, None, 8, None) == 1  # overlap
    assert lib.moe_calibrate_stream(A, B, 1024, 3, S, 8, None) == 1         # unknown mode


def test_plan_noalloc_validation(lib):
    # the allocation-free plan rejects what moe_plan rejects, and a plan whose histogram would
    # not fit its 4 MiB scratch, before any launch
    p = _fake_plan(T=0)
    assert lib.moe_plan_noalloc(ctypes.c_void_p(0x8000), ctypes.byref(p), None) == _abi.MOE_ERR_INVALID
    p = _fake_plan()
    assert lib.moe_plan_noalloc(None, ctypes.byref(p), None) == _abi.MOE_ERR_INVALID
    # 2^20 pairs x 1024 experts: 1024 columns x 1024 x 4 bytes > 4 MiB
    big = _fake_plan(T=1 << 17, K=8, E_local=1024, tile=128,
                     rows_cap=oracle.pool_rows_bound(1 << 17, 8, 1024, 128))
    assert lib.moe_plan_noalloc(ctypes.c_void_p(0x8000), ctypes.byref(big), None) == _abi.MOE_ERR_UNSUPPORTED


def test_package_exports_the_binding():
    # every name the binding lists is importable from the package
    import combine_moe_dispatch_02_amd as moe
    from combine_moe_dispatch_02_amd import layer
    missing = [n for n in layer.__all__ if not hasattr(moe, n)]
    assert not missing, missing

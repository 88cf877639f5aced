"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, validates arguments before any launch, and its host-only
helpers agree with the oracle."""
import ctypes

import numpy as np
import pytest

import oracle
from video_diffusion_transformer_lvsa_amd import _lib


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _no_gpu():
    import torch

    return torch.cuda.device_count() == 0


def test_exports_every_declared_function(lib):
    names = _lib.header_functions()
    for required in ("lvsa_mask", "draft_mask_and_perm", "block_sparse_attn_fwd", "dense_attn_fwd"):
        assert required in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)
    assert lib.lvsa_version().decode().startswith("lvsa")


@pytest.mark.parametrize("T,C,W,T_per,s", [(4, 3, 2, 2, 0), (126, 21, 5, 8, 0), (126, 21, 5, 8, 7), (21, 21, 5, 8, 3),
                                           (8, 3, 4, 3, 0), (6, 2, 3, 1, 0), (1, 1, 1, 1, 0), (13, 40, 2, 5, 9)])
def test_capacity_matches_oracle(lib, T, C, W, T_per, s):
    assert lib.lvsa_mask_capacity(T, C, W, T_per, s) == oracle.lvsa_capacity(T, C, W, T_per, s)


def test_capacity_sweep(lib):
    for T in (1, 3, 7, 12):
        for C in (1, 4, 9):
            for W in (1, 3):
                for T_per in (1, 2, 5):
                    for s in (0, 3):
                        assert lib.lvsa_mask_capacity(T, C, W, T_per, s) == oracle.lvsa_capacity(T, C, W, T_per, s)


@pytest.mark.parametrize("args", [(0, 3, 2, 2, 0), (4, 0, 2, 2, 0), (4, 3, 0, 2, 0), (4, 3, 2, 0, 0), (4, 3, 2, 2, -1)])
def test_capacity_rejects(lib, args):
    assert lib.lvsa_mask_capacity(*args) == _lib.LVSA_EINVAL
    assert _lib.last_error()


@pytest.mark.parametrize("T,H,W,ph,pw,sp", [(33, 45, 80, 8, 16, 0.9), (2, 5, 7, 2, 4, 0.5), (1, 3, 4, 2, 2, 0.0),
                                            (3, 8, 16, 8, 16, 1.0)])
def test_grid_info_matches_oracle(lib, T, H, W, ph, pw, sp):
    info = _lib.draft_grid_info(T, H, W, ph, pw, sp)
    g = oracle.draft_grid(T, H, W, ph, pw)
    assert info == {"nb": g.nb, "n_pad": g.N_pad, "block_size": g.block_size, "k": oracle.topk_count(sp, g.nb)}
    assert _lib.draft_workspace_bytes(24, T, H, W, 128, ph, pw) == 3 * 24 * g.nb * 128 * 4


def test_grid_info_rejects(lib):
    with pytest.raises(_lib.LvsaError):
        _lib.draft_grid_info(0, 3, 4, 2, 2, 0.5)
    with pytest.raises(_lib.LvsaError):
        _lib.draft_grid_info(1, 3, 4, 2, 2, 1.5)
    with pytest.raises(_lib.LvsaError) as e:
        _lib.draft_grid_info(1, 64, 64, 64, 32, 0.5)  # block size 2048
    assert e.value.code == _lib.LVSA_EUNSUPPORTED


FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every call below fails validation first
MIS = ctypes.c_void_p((1 << 20) + 4)


def test_attention_validation(lib):
    f = lib.block_sparse_attn_fwd
    ok = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, dt=1, heads=2, n=256, d=128, bq=64, bk=64, idx=FAKE, cnt=FAKE, max_kv=4,
              mh=1, bv=None, scale=0.088)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["k"], a["v"], a["o"], a["dt"], a["heads"], a["n"], a["d"], a["bq"], a["bk"], a["idx"],
                 a["cnt"], a["max_kv"], a["mh"], a["bv"], a["scale"], None)

    assert call(d=96) == _lib.LVSA_EUNSUPPORTED
    assert call(dt=7) == _lib.LVSA_EINVAL
    assert call(q=None) == _lib.LVSA_EINVAL
    assert call(k=MIS) == _lib.LVSA_EINVAL
    assert call(bq=0) == _lib.LVSA_EINVAL
    assert call(mh=3) == _lib.LVSA_EINVAL
    assert call(max_kv=-1) == _lib.LVSA_EINVAL
    assert call(cnt=None) == _lib.LVSA_EINVAL
    assert call(bv=FAKE, bk=32) == _lib.LVSA_EINVAL
    assert call(scale=float("inf")) == _lib.LVSA_EINVAL
    assert call(scale=0.0) == _lib.LVSA_EINVAL
    assert call(scale=-0.088) == _lib.LVSA_EINVAL
    assert call(scale=float("nan")) == _lib.LVSA_EINVAL
    assert call(n=1 << 23) == _lib.LVSA_EINVAL  # n*d >= 2^30
    # empty problems are valid no-ops
    assert call(heads=0) == 0
    assert call(n=0) == 0
    g = lib.dense_attn_fwd
    assert g(FAKE, FAKE, FAKE, FAKE, 1, 2, 256, 100, 0.1, None) == _lib.LVSA_EUNSUPPORTED
    assert g(FAKE, FAKE, FAKE, None, 1, 2, 256, 128, 0.1, None) == _lib.LVSA_EINVAL
    assert g(FAKE, FAKE, FAKE, FAKE, 1, 0, 256, 128, 0.1, None) == 0
    for sc in (0.0, -0.1, float("nan")):
        assert g(FAKE, FAKE, FAKE, FAKE, 1, 2, 256, 128, sc, None) == _lib.LVSA_EINVAL


def test_mask_and_permute_validation(lib):
    assert lib.lvsa_mask(126, 21, 5, 8, 0, FAKE, FAKE, 20, None) == _lib.LVSA_ERANGE
    assert "required 21" in _lib.last_error()
    assert lib.lvsa_mask(126, 21, 5, 8, 0, None, FAKE, 21, None) == _lib.LVSA_EINVAL
    assert lib.lvsa_mask(0, 21, 5, 8, 0, FAKE, FAKE, 21, None) == _lib.LVSA_EINVAL
    tp = lib.token_permute
    assert tp(FAKE, FAKE, 1, 2, 10, 10, 12, FAKE, None) == _lib.LVSA_EUNSUPPORTED  # 24-byte rows
    assert tp(FAKE, FAKE, 1, 2, 10, 10, 128, None, None) == _lib.LVSA_EINVAL
    assert tp(FAKE, FAKE, 1, 2, 10, 10, 128, FAKE, None) == _lib.LVSA_EINVAL  # overlap
    assert tp(FAKE, FAKE, 1, 2, 10, 0, 128, FAKE, None) == 0
    assert tp(FAKE, FAKE, 1, 2, 1 << 27, 10, 128, FAKE, None) == _lib.LVSA_EINVAL  # 2^31 chunks per head
    dm = lib.draft_mask_and_perm
    base = [FAKE, FAKE, FAKE, 1, 2, 2, 10, 16, 128, 4, 8, 0.5, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]
    need = lib.draft_workspace_bytes(2, 2, 10, 16, 128, 4, 8)
    assert dm(*base, FAKE, need - 4, None) == _lib.LVSA_ENOMEM
    bad = list(base)
    bad[12] = 2  # pool mode
    assert dm(*bad, FAKE, need, None) == _lib.LVSA_EINVAL
    assert "pool_mode" in _lib.last_error()
    bad = list(base)
    bad[19] = None  # k_perm NULL but q_perm set
    assert dm(*bad, FAKE, need, None) == _lib.LVSA_EINVAL
    bad = list(base)
    bad[8] = 80
    assert dm(*bad, FAKE, need, None) == _lib.LVSA_EUNSUPPORTED
    bad = list(base)
    bad[11] = -0.1
    assert dm(*bad, FAKE, need, None) == _lib.LVSA_EINVAL
    ds = lib.draft_scores
    assert ds(FAKE, FAKE, 1, 2, 3, 0, FAKE, None) == _lib.LVSA_EINVAL
    da = lib.draft_attn_fwd
    ok = [FAKE, FAKE, FAKE, FAKE, 1, 2, 3, 45, 80, 128, 8, 16, FAKE, FAKE, 99, 0.088, None]
    for i, val, code in [(9, 64, _lib.LVSA_EUNSUPPORTED),   # d = 64
                         (4, 0, _lib.LVSA_EUNSUPPORTED),    # fp32
                         (10, 4, _lib.LVSA_EUNSUPPORTED),   # 4x16 = 64 slots: fine; pool 4x8 below
                         (14, -1, _lib.LVSA_EINVAL),        # max_kv < 0
                         (15, float("inf"), _lib.LVSA_EINVAL),
                         (15, 0.0, _lib.LVSA_EINVAL),        # scale must be positive
                         (15, -0.088, _lib.LVSA_EINVAL)]:
        bad = list(ok)
        bad[i] = val
        if i == 10:
            bad[11] = 8  # 4x8 = 32 slots: not a multiple of 64
        assert da(*bad) == code, (i, val)
    bad = list(ok)
    bad[11] = 24  # 8x24 = 192 slots, but 24 does not divide 64
    assert da(*bad) == _lib.LVSA_EUNSUPPORTED
    bad = list(ok)
    bad[13] = None  # kv_cnt
    assert da(*bad) == _lib.LVSA_EINVAL


def test_fp8_validation(lib):
    qz = lib.quantize_fp8_e4m3
    ok = [FAKE, 1, 2, 256, 128, 1, 256, FAKE, FAKE, None]
    for i, val, code in [(1, 7, _lib.LVSA_EINVAL),          # dtype
                         (4, 96, _lib.LVSA_EUNSUPPORTED),   # d
                         (5, 2, _lib.LVSA_EINVAL),          # transpose flag
                         (6, 200, _lib.LVSA_EINVAL),        # ld < n
                         (6, 264, _lib.LVSA_EINVAL),        # ld not a multiple of 16
                         (0, None, _lib.LVSA_EINVAL),       # src
                         (7, MIS, _lib.LVSA_EINVAL),        # dst misaligned
                         (8, None, _lib.LVSA_EINVAL),       # scales
                         (3, 1 << 23, _lib.LVSA_EINVAL),    # n*d >= 2^30
                         (2, 65536, _lib.LVSA_EUNSUPPORTED)]:  # heads
        bad = list(ok)
        bad[i] = val
        assert qz(*bad) == code, (i, val)
    row = list(ok)
    row[5], row[6] = 0, 16  # ld must be 0 without transpose
    assert qz(*row) == _lib.LVSA_EINVAL
    empty = list(ok)
    empty[2] = 0
    assert qz(*empty) == 0

    bs = lib.block_sparse_attn_fwd_fp8
    ok = [FAKE, FAKE, FAKE, 1568, FAKE, FAKE, FAKE, FAKE, 2, 1560, 128, 1560, 1560, FAKE, FAKE, 3, 1, None, 0.088,
          None]
    for i, val, code in [(10, 64, _lib.LVSA_EUNSUPPORTED),   # d
                         (9, 1558, _lib.LVSA_EUNSUPPORTED),  # n not a multiple of 4
                         (3, 1552, _lib.LVSA_EINVAL),        # ldv < n
                         (3, 1570, _lib.LVSA_EINVAL),        # ldv not a multiple of 16
                         (12, 32, _lib.LVSA_EUNSUPPORTED),   # block_k < 64
                         (12, 66, _lib.LVSA_EUNSUPPORTED),   # block_k not a multiple of 4
                         (11, 0, _lib.LVSA_EINVAL),          # block_q
                         (16, 3, _lib.LVSA_EINVAL),          # mask_heads
                         (15, -1, _lib.LVSA_EINVAL),         # max_kv
                         (18, float("nan"), _lib.LVSA_EINVAL),
                         (18, 0.0, _lib.LVSA_EINVAL),
                         (18, -0.088, _lib.LVSA_EINVAL),
                         (4, None, _lib.LVSA_EINVAL),        # q_scale
                         (0, MIS, _lib.LVSA_EINVAL),         # q8 misaligned
                         (14, None, _lib.LVSA_EINVAL)]:      # kv_cnt
        bad = list(ok)
        bad[i] = val
        assert bs(*bad) == code, (i, val)
    bad = list(ok)
    bad[11], bad[17] = 128, FAKE  # block_valid needs block_q == block_k
    assert bs(*bad) == _lib.LVSA_EINVAL
    empty = list(ok)
    empty[8] = 0
    assert bs(*empty) == 0
    da = lib.draft_attn_fwd_fp8
    ok = [FAKE, FAKE, FAKE, 118800, FAKE, FAKE, FAKE, FAKE, 2, 33, 45, 80, 128, 8, 16, FAKE, FAKE, 99, 0.088, None]
    for i, val, code in [(12, 64, _lib.LVSA_EUNSUPPORTED),   # d
                         (11, 78, _lib.LVSA_EUNSUPPORTED),   # grid_w not a multiple of 4
                         (14, 2, _lib.LVSA_EUNSUPPORTED),    # pool_w = 2 (pool 8x2 = 16 slots as well)
                         (3, 118784, _lib.LVSA_EINVAL),      # ldv < n
                         (17, -1, _lib.LVSA_EINVAL),         # max_kv
                         (16, None, _lib.LVSA_EINVAL),       # kv_cnt
                         (18, 0.0, _lib.LVSA_EINVAL),        # scale
                         (4, None, _lib.LVSA_EINVAL)]:       # q_scale
        bad = list(ok)
        bad[i] = val
        assert da(*bad) == code, (i, val)
    bad = list(ok)
    bad[13], bad[14] = 32, 2  # 64 slots, but pool_w = 2
    assert da(*bad) == _lib.LVSA_EUNSUPPORTED
    empty = list(ok)
    empty[8] = 0
    assert da(*empty) == 0
    dn = lib.dense_attn_fwd_fp8
    ok = [FAKE, FAKE, FAKE, 1008, FAKE, FAKE, FAKE, FAKE, 2, 1000, 128, 0.088, None]
    assert dn(*(ok[:10] + [64] + ok[11:])) == _lib.LVSA_EUNSUPPORTED
    assert dn(*(ok[:9] + [1002] + ok[10:])) == _lib.LVSA_EUNSUPPORTED
    assert dn(*(ok[:3] + [1000] + ok[4:])) == _lib.LVSA_EINVAL
    assert dn(*(ok[:6] + [None] + ok[7:])) == _lib.LVSA_EINVAL
    assert dn(*(ok[:8] + [0] + ok[9:])) == 0
    assert dn(*(ok[:11] + [-0.088] + ok[12:])) == _lib.LVSA_EINVAL


@pytest.mark.skipif(not _no_gpu(), reason="checks the no-device error path")
def test_no_device_is_reported(lib):
    assert lib.lvsa_mask(4, 3, 2, 2, 0, FAKE, FAKE, 3, None) == _lib.LVSA_EDEVICE
    assert "GPU" in _lib.last_error()
    assert lib.dense_attn_fwd(FAKE, FAKE, FAKE, FAKE, 1, 2, 256, 128, 0.1, None) == _lib.LVSA_EDEVICE
    assert lib.quantize_fp8_e4m3(FAKE, 1, 2, 256, 128, 1, 256, FAKE, FAKE, None) == _lib.LVSA_EDEVICE
    assert lib.dense_attn_fwd_fp8(FAKE, FAKE, FAKE, 256, FAKE, FAKE, FAKE, FAKE, 2, 256, 128, 0.1,
                                  None) == _lib.LVSA_EDEVICE

"""The Python binding checks every tensor against the scalar arguments the
kernels size their index ranges from, and raises ValueError before any call
into the library. These run on host tensors (no GPU): each case is wrong in
exactly one way, and the message names the tensor at fault."""
import pytest
import torch

from video_diffusion_transformer_lvsa_amd import _lib

bf = torch.bfloat16
i32 = torch.int32
f32 = torch.float32
u8 = torch.uint8


def _qkv(heads=2, n=256, d=128, dt=bf):
    return (torch.zeros(heads, n, d, dtype=dt) for _ in range(3))


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_lvsa_mask_buffer_checks():
    T = 10
    # a caller's buffer sets the row pitch: a cap that disagrees with it is refused
    _raises("cap=5 differs", _lib.lvsa_mask, T, 3, 2, 4, 0, cap=5, kv_idx=torch.zeros(T, 4, dtype=i32))
    _raises(r"kv_idx: expected shape \(10, cap\)", _lib.lvsa_mask, T, 3, 2, 4, 0, kv_idx=torch.zeros(9, 5, dtype=i32))
    _raises("kv_idx: expected dtype", _lib.lvsa_mask, T, 3, 2, 4, 0, kv_idx=torch.zeros(T, 5, dtype=torch.int64))
    _raises("kv_cnt: expected shape", _lib.lvsa_mask, T, 3, 2, 4, 0, kv_idx=torch.zeros(T, 5, dtype=i32),
            kv_cnt=torch.zeros(T + 1, dtype=i32))
    # a matching host buffer passes the shape checks and is refused as not on the GPU
    _raises("CUDA", _lib.lvsa_mask, T, 3, 2, 4, 0, kv_idx=torch.zeros(T, 5, dtype=i32),
            kv_cnt=torch.zeros(T, dtype=i32))


def test_block_sparse_checks():
    q, k, v = _qkv()
    idx = torch.zeros(2, 4, 3, dtype=i32)
    cnt = torch.zeros(2, 4, dtype=i32)
    f = _lib.block_sparse_attn_fwd
    _raises("k: expected shape", f, q, torch.zeros(2, 255, 128, dtype=bf), v, 64, 64, idx, cnt, mask_heads=2)
    _raises("v: expected dtype", f, q, k, torch.zeros(2, 256, 128, dtype=f32), 64, 64, idx, cnt, mask_heads=2)
    _raises("out: expected dtype", f, q, k, v, 64, 64, idx, cnt, mask_heads=2, out=torch.zeros(2, 256, 128, dtype=bf))
    _raises("out: expected shape", f, q, k, v, 64, 64, idx, cnt, mask_heads=2, out=torch.zeros(2, 256, 64))
    _raises("mask_heads", f, q, k, v, 64, 64, idx, cnt, mask_heads=3)
    _raises("kv_cnt: expected 8 elements", f, q, k, v, 64, 64, idx, torch.zeros(2, 3, dtype=i32), mask_heads=2)
    _raises("kv_idx: expected shape", f, q, k, v, 64, 64, torch.zeros(2, 3, 3, dtype=i32), cnt, mask_heads=2)
    _raises("kv_idx: expected shape", f, q, k, v, 64, 64, torch.zeros(1, 4, 3, dtype=i32), cnt, mask_heads=2)
    _raises("kv_idx: expected dtype", f, q, k, v, 64, 64, idx.long(), cnt, mask_heads=2)
    _raises("kv_cnt: expected dtype", f, q, k, v, 64, 64, idx, cnt.long(), mask_heads=2)
    # 256 rows in blocks of 32 keys = 8 key blocks: block_valid must cover them
    _raises("block_valid: expected at least 8", f, q, k, v, 64, 32, idx, cnt, mask_heads=2,
            block_valid=torch.zeros(7, dtype=i32))
    # one shared list: [nqb, max_kv] or [1, nqb, max_kv]
    _raises("CUDA", f, q, k, v, 64, 64, torch.zeros(4, 3, dtype=i32), torch.zeros(4, dtype=i32))
    _raises("CUDA", f, q, k, v, 64, 64, torch.zeros(1, 4, 3, dtype=i32), torch.zeros(1, 4, dtype=i32))


def test_dense_checks():
    q, k, v = _qkv()
    _raises("k: expected shape", _lib.dense_attn_fwd, q, torch.zeros(2, 256, 64, dtype=bf), v)
    _raises("out: expected shape", _lib.dense_attn_fwd, q, k, v, out=torch.zeros(1, 256, 128))
    _raises(r"q: expected \[heads, n, d\]", _lib.dense_attn_fwd, torch.zeros(256, 128, dtype=bf), k, v)


def test_draft_attention_checks():
    T, H, W, ph, pw = 2, 16, 32, 8, 16  # 2 x 2 x 2 = 8 tiles
    n = T * H * W
    q, k, v = _qkv(n=n)
    idx = torch.zeros(2, 8, 3, dtype=i32)
    cnt = torch.zeros(2, 8, dtype=i32)
    f = _lib.draft_attn_fwd
    _raises("tokens; the grid", f, q, k, v, T, H + 1, W, ph, pw, idx, cnt)
    _raises("kv_cnt: expected 16 elements", f, q, k, v, T, H, W, ph, pw, idx, torch.zeros(2, 7, dtype=i32))
    _raises("kv_idx: expected shape", f, q, k, v, T, H, W, ph, pw, torch.zeros(1, 8, 3, dtype=i32), cnt)
    _raises("CUDA", f, q, k, v, T, H, W, ph, pw, idx, cnt)


def test_draft_mask_checks():
    T, H, W = 2, 16, 32
    q, k, v = _qkv(n=T * H * W)
    f = _lib.draft_mask_and_perm
    _raises("tokens; the grid", f, q, k, v, T, H, W + 1, 8, 16, 0.9)
    _raises("k: expected shape", f, q, torch.zeros(2, T * H * W, 64, dtype=bf), v, T, H, W, 8, 16, 0.9)
    _raises("pool must be", f, q, k, v, T, H, W, 8, 16, 0.9, pool="median")


def test_token_permute_and_scores_checks():
    src = torch.zeros(2, 100, 128, dtype=bf)
    m = torch.zeros(120, dtype=i32)
    _raises("dst_to_src: expected dtype", _lib.token_permute, src, m.long())
    _raises("out: expected shape", _lib.token_permute, src, m, out=torch.zeros(2, 100, 128, dtype=bf))
    _raises("out: expected dtype", _lib.token_permute, src, m, out=torch.zeros(2, 120, 128))
    _raises("kbar: expected shape", _lib.draft_scores, torch.zeros(2, 10, 128), torch.zeros(2, 10, 64))
    _raises("qbar: expected dtype", _lib.draft_scores, torch.zeros(2, 10, 128, dtype=bf), torch.zeros(2, 10, 128))


def test_fp8_checks():
    heads, n, d = 2, 256, 128
    q8 = torch.zeros(heads, n, d, dtype=u8)
    k8 = torch.zeros_like(q8)
    vt8 = torch.zeros(heads, d, 256, dtype=u8)
    s = torch.ones(heads)
    idx = torch.zeros(1, 2, 3, dtype=i32)
    cnt = torch.zeros(1, 2, dtype=i32)
    f = _lib.block_sparse_attn_fwd_fp8
    _raises("k8: expected shape", f, q8, torch.zeros(heads, n - 4, d, dtype=u8), vt8, s, s, s, 128, 128, idx, cnt)
    _raises("vt8: expected", f, q8, k8, torch.zeros(heads, d, 128, dtype=u8), s, s, s, 128, 128, idx, cnt)
    _raises("vt8: expected", f, q8, k8, torch.zeros(heads, 64, 256, dtype=u8), s, s, s, 128, 128, idx, cnt)
    _raises("v_scale: expected 2 elements", f, q8, k8, vt8, s, s, torch.ones(3), 128, 128, idx, cnt)
    _raises("q_scale: expected dtype", f, q8, k8, vt8, s.double(), s, s, 128, 128, idx, cnt)
    _raises("kv_idx: expected shape", f, q8, k8, vt8, s, s, s, 128, 128, torch.zeros(1, 3, 3, dtype=i32), cnt)
    _raises("block_valid: expected at least 2", f, q8, k8, vt8, s, s, s, 128, 128, idx, cnt,
            block_valid=torch.zeros(1, dtype=i32))
    _raises("out: expected dtype", _lib.dense_attn_fwd_fp8, q8, k8, vt8, s, s, s, out=torch.zeros(heads, n, d, dtype=bf))
    _raises("k8: expected dtype", _lib.dense_attn_fwd_fp8, q8, k8.to(torch.int8), vt8, s, s, s)
    T, H, W = 1, 16, 16
    _raises("tokens; the grid", _lib.draft_attn_fwd_fp8, q8, k8, vt8, s, s, s, T, H, W + 4, 8, 16, idx, cnt)
    _raises("kv_cnt: expected 4 elements", _lib.draft_attn_fwd_fp8, q8, k8, vt8, s, s, s, T, H, W, 8, 16,
            torch.zeros(2, 2, 3, dtype=i32), cnt)


def test_quantize_checks():
    x = torch.zeros(2, 100, 128, dtype=bf)
    _raises("out: expected shape", _lib.quantize_fp8_e4m3, x, out=torch.zeros(2, 100, 64, dtype=u8))
    _raises("out: expected dtype", _lib.quantize_fp8_e4m3, x, out=torch.zeros(2, 100, 128, dtype=torch.int8))
    _raises("scales: expected 2 elements", _lib.quantize_fp8_e4m3, x, scales=torch.ones(1))
    # the transposed pitch comes from the given buffer; a pitch that disagrees is refused
    _raises("out: expected shape", _lib.quantize_fp8_e4m3, x, transpose=True, ld=128,
            out=torch.zeros(2, 128, 256, dtype=u8))
    _raises("CUDA", _lib.quantize_fp8_e4m3, x, transpose=True, out=torch.zeros(2, 128, 256, dtype=u8))

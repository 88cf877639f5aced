"""Pins for the fp64 attention oracle: pure-Python brute force, torch's fp64
scaled_dot_product_attention with a boolean mask, closed forms and the
reorder's permutation invariance."""
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import bf16_decode_fields
from video_diffusion_transformer_lvsa_amd import synth


def _f64(x):
    """Inputs for the library cross-checks, decoded apart from the oracle:
    bf16 bit patterns through the field-definition decoder, floats by a cast."""
    x = np.asarray(x)
    return bf16_decode_fields(x) if x.dtype == np.uint16 else x.astype(np.float64)


def _py_attention(q, k, v, keys, scale):
    """Pure-Python loops with math.exp, for tiny inputs."""
    d = len(q[0])
    out = []
    for qi in q:
        s = [scale * sum(qi[c] * k[j][c] for c in range(d)) for j in keys]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = sum(w)
        out.append([sum(w[a] * v[j][c] for a, j in enumerate(keys)) / z for c in range(d)])
    return np.array(out)


def test_brute_force_tiny():
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((1, 7, 3)) for _ in range(3))
    keys = [0, 2, 3, 6]
    got = oracle.attention_keyset(q[0], k[0, keys], v[0, keys], 0.7)
    want = _py_attention(q[0].tolist(), k[0].tolist(), v[0].tolist(), keys, 0.7)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    dense = oracle.dense_attention(q, k, v, scale=0.7)
    assert np.allclose(dense[0], _py_attention(q[0].tolist(), k[0].tolist(), v[0].tolist(), list(range(7)), 0.7),
                       rtol=1e-12, atol=1e-12)


def _sdpa_masked(q, k, v, allowed):
    """torch fp64 SDPA with a boolean [n, n] mask (True = attend)."""
    qt, kt, vt = (torch.from_numpy(_f64(x)) for x in (q, k, v))
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(allowed)).numpy()


@pytest.mark.parametrize("s", [0, 1, 2, 3])
def test_lvsa_tiny_vs_sdpa(s):
    w = synth.WORKLOADS["tiny"]
    q, k, v = synth.iid_qkv(w.seed, w.heads, w.N, w.d)
    idx, cnt = oracle.lvsa_mask(w.T, w.C, w.window, w.T_per, s)
    got = oracle.block_sparse_attention(q, k, v, w.P, w.P, idx, cnt)
    allowed = np.zeros((w.N, w.N), dtype=bool)
    for t in range(w.T):
        for f in idx[t, : cnt[t]]:
            allowed[t * w.P : (t + 1) * w.P, f * w.P : (f + 1) * w.P] = True
    want = _sdpa_masked(q, k, v, allowed)
    assert np.allclose(got, want, rtol=1e-11, atol=1e-12)


def test_full_mask_equals_dense():
    w = synth.WORKLOADS["tiny"]
    q, k, v = synth.iid_qkv(w.seed, w.heads, w.N, w.d)
    idx = np.tile(np.arange(w.T, dtype=np.int32), (w.T, 1))
    cnt = np.full(w.T, w.T, dtype=np.int32)
    bs = oracle.block_sparse_attention(q, k, v, w.P, w.P, idx, cnt)
    dense = oracle.dense_attention(q, k, v)
    assert np.allclose(bs, dense, rtol=1e-12, atol=1e-13)
    want = torch.nn.functional.scaled_dot_product_attention(*(torch.from_numpy(x.astype(np.float64)) for x in (q, k, v)))
    assert np.allclose(dense, want.numpy(), rtol=1e-11, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(5)
    n, d = 40, 8
    q = rng.standard_normal((1, n, d))
    k = rng.standard_normal((1, n, d))
    vconst = np.tile(rng.standard_normal(d), (1, n, 1))
    # constant V -> O = v
    assert np.allclose(oracle.dense_attention(q, k, vconst)[0], vconst[0], atol=1e-13)
    # Q = 0 -> uniform weights: O = mean of V over the key set
    v = rng.standard_normal((1, n, d))
    idx = np.array([[1, 3], [0, 4]], dtype=np.int32)  # blocks of 8 rows; 5 blocks
    cnt = np.array([2, 1], dtype=np.int32)
    o = oracle.block_sparse_attention(np.zeros((1, n, d)), k, v, 20, 8, idx, cnt)
    assert np.allclose(o[0, :20], v[0, np.r_[8:16, 24:32]].mean(axis=0), atol=1e-14)
    assert np.allclose(o[0, 20:], v[0, 0:8].mean(axis=0), atol=1e-14)
    # a single visited valid key -> O = that v
    bv = np.array([1, 8, 8, 8, 8], dtype=np.int32)
    o1 = oracle.block_sparse_attention(q, k, v, 8, 8, np.zeros((5, 1), np.int32), np.ones(5, np.int32),
                                       block_valid=bv)
    assert np.allclose(o1[0, 8:], np.tile(v[0, 0], (32, 1)), atol=1e-14)
    assert np.allclose(o1[0, 0], v[0, 0]) and np.all(o1[0, 1:8] == 0)  # pad query rows -> 0
    # an empty key set -> 0
    o0 = oracle.block_sparse_attention(q, k, v, 8, 8, np.zeros((5, 1), np.int32), np.zeros(5, np.int32))
    assert np.all(o0 == 0)


def _draft_case(T=2, H=10, W=16, ph=4, pw=8, heads=2, d=32, sparsity=0.6, seed=7):
    g = oracle.draft_grid(T, H, W, ph, pw)
    q, k, v = synth.video_qkv(seed, heads, T, H, W, d)
    kv, cnt, *_ = oracle.draft_mask(synth.bf16_to_f32(q), synth.bf16_to_f32(k), g, sparsity)
    perm, inv, bv = oracle.draft_permutation(g)
    return g, q, k, v, kv, cnt, perm, inv, bv


def _permute(x, perm):
    out = np.zeros((x.shape[0], len(perm), x.shape[2]), dtype=x.dtype)
    live = perm >= 0
    out[:, live] = x[:, perm[live]]
    return out


def test_draft_reorder_invariance():
    g, q, k, v, kv, cnt, perm, inv, bv = _draft_case()
    bs = g.block_size
    o_perm = oracle.block_sparse_attention(_permute(q, perm), _permute(k, perm), _permute(v, perm), bs, bs, kv, cnt,
                                           mask_heads=q.shape[0], block_valid=bv)
    back = o_perm[:, inv]
    direct = oracle.draft_attention_original_order(q, k, v, perm, inv, bv, bs, kv, cnt)
    assert np.allclose(back, direct, rtol=1e-12, atol=1e-13)
    # pad rows of the reordered output are zero
    assert np.all(o_perm[:, perm < 0] == 0)
    # an independent check: token-level boolean mask in the original order through torch SDPA
    allowed = np.zeros((q.shape[0], g.N, g.N), dtype=bool)
    for h in range(q.shape[0]):
        for b in range(g.nb):
            rows = perm[b * bs : b * bs + bv[b]]
            for bb in kv[h, b, : cnt[h, b]]:
                cols = perm[bb * bs : bb * bs + bv[bb]]
                allowed[h][np.ix_(rows, cols)] = True
    want = _sdpa_masked(q, k, v, allowed)
    assert np.allclose(direct, want, rtol=1e-11, atol=1e-12)


def test_draft_original_order_empty_and_repeated_lists():
    """An empty key list gives an empty key set (output 0, the convention of
    block_sparse_attention); a listed block repeated r times weighs its keys r
    times; both equal the reordered computation mapped back."""
    g, q, k, v, kv, cnt, perm, inv, bv = _draft_case()
    kv, cnt = kv.copy(), cnt.copy()
    cnt[0, 1] = 0
    kv[1, 2, 1] = kv[1, 2, 0]
    bs = g.block_size
    direct = oracle.draft_attention_original_order(q, k, v, perm, inv, bv, bs, kv, cnt)
    rows1 = perm[bs : bs + bv[1]]
    assert np.all(direct[0, rows1] == 0)
    o_perm = oracle.block_sparse_attention(_permute(q, perm), _permute(k, perm), _permute(v, perm), bs, bs, kv, cnt,
                                           mask_heads=q.shape[0], block_valid=bv)
    assert np.allclose(o_perm[:, inv], direct, rtol=1e-12, atol=1e-13)
    # the repeated block: attention over the key multiset, written out with explicit weights
    rows2 = perm[2 * bs : 2 * bs + bv[2]]
    blocks = list(kv[1, 2, : cnt[1, 2]])
    keys = np.concatenate([perm[b * bs : b * bs + bv[b]] for b in blocks])
    qf, kf, vf = (synth.bf16_to_f32(x[1]).astype(np.float64) for x in (q, k, v))
    s = qf[rows2] @ kf[keys].T / np.sqrt(q.shape[2])
    w = np.exp(s - s.max(axis=1, keepdims=True))
    want = (w @ vf[keys]) / w.sum(axis=1, keepdims=True)
    assert np.allclose(direct[1, rows2], want, rtol=1e-12, atol=1e-13)


def test_draft_all_blocks_equals_dense():
    g, q, k, v, *_ = _draft_case(sparsity=0.0)
    kv, cnt, *_ = oracle.draft_mask(synth.bf16_to_f32(q), synth.bf16_to_f32(k), g, 0.0)
    assert kv.shape[2] == g.nb
    perm, inv, bv = oracle.draft_permutation(g)
    direct = oracle.draft_attention_original_order(q, k, v, perm, inv, bv, g.block_size, kv, cnt)
    assert np.allclose(direct, oracle.dense_attention(q, k, v), rtol=1e-12, atol=1e-13)


def test_lvsa_frame_gather_equals_dense_on_gathered_frames():
    """LVSA per query frame = dense attention over the concatenation of its frames."""
    T, H, W, d = 6, 3, 4, 16
    q, k, v = synth.video_qkv(9, 1, T, H, W, d)
    P = H * W
    idx, cnt = oracle.lvsa_mask(T, 3, 2, 3, 1)
    got = oracle.block_sparse_attention(q, k, v, P, P, idx, cnt)
    for t in range(T):
        cols = np.concatenate([np.arange(f * P, (f + 1) * P) for f in idx[t, : cnt[t]]])
        qt = torch.from_numpy(_f64(q)[:, t * P : (t + 1) * P])
        kt = torch.from_numpy(_f64(k)[:, cols])
        vt = torch.from_numpy(_f64(v)[:, cols])
        want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).numpy()
        assert np.allclose(got[:, t * P : (t + 1) * P], want, rtol=1e-11, atol=1e-12)


def test_sampled_rows_match_full():
    w = synth.WORKLOADS["tiny"]
    q, k, v = synth.iid_qkv(w.seed, w.heads, w.N, w.d)
    idx, cnt = oracle.lvsa_mask(w.T, w.C, w.window, w.T_per, 2)
    full = oracle.block_sparse_attention(q, k, v, w.P, w.P, idx, cnt)
    rows = np.array([0, 5, 63, 64, 200, 255])
    part = oracle.block_sparse_attention(q, k, v, w.P, w.P, idx, cnt, rows=rows, heads=[1])
    assert np.allclose(part[0], full[1, rows], rtol=1e-13, atol=1e-15)  # BLAS blocking may differ by shape


def test_planted_dropped_scale_is_caught(monkeypatch):
    """An attention that forgets 1/sqrt(d) must fail the torch SDPA pin."""
    import oracle.attention as A

    real = A.attention_keyset
    monkeypatch.setattr(A, "attention_keyset", lambda q, k, v, scale: real(q, k, v, 1.0))
    w = synth.WORKLOADS["tiny"]
    q, k, v = synth.iid_qkv(w.seed, w.heads, w.N, w.d)
    dense = A.dense_attention(q, k, v)
    want = torch.nn.functional.scaled_dot_product_attention(*(torch.from_numpy(x.astype(np.float64)) for x in (q, k, v)))
    assert not np.allclose(dense, want.numpy(), rtol=1e-6, atol=1e-6)

"""Planted mistakes: each case replaces one oracle function by a plausible
wrong version (a dropped term, a wrong index or tie rule, a transposed
operand, a wrong constant) and checks that the pins already in the suite
catch it -- at least one of the listed pin tests must fail under the
mutation. This is how the pins are shown to be stronger than the oracle's
own restatement."""
import math

import numpy as np
import pytest

import oracle
import oracle.attention as A
import oracle.draft as D
import oracle.fp8 as F
import oracle.lvsa as L
import test_oracle_attention as TA
import test_oracle_bf16 as TB
import test_oracle_draft as TD
import test_oracle_fp8 as TF
import test_oracle_lvsa as TL


def _patch(monkeypatch, module, name, fn):
    """Replace a function in its module and in the package namespace."""
    monkeypatch.setattr(module, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)


def _some_pin_fails(pins):
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


def _pool_counts_pads(real):
    def pool(x, g, mode="mean"):
        out = real(x, g, mode)
        _, _, bv = D.draft_permutation(g)
        return (out * (bv[None, :, None] / g.block_size)).astype(np.float32) if mode == "mean" else out
    return pool


def _scores_drop_first_channel(real):
    return lambda qbar, kbar: real(qbar[..., 1:], kbar[..., 1:])


def _scores_fused(real):
    return lambda qbar, kbar: np.einsum("hic,hjc->hij", qbar.astype(np.float64), kbar.astype(np.float64)).astype(np.float32)


def _topk_ties_high(real):
    def topk(scores, k):
        s = np.asarray(scores, dtype=np.float32)[..., ::-1]
        out = real(s, k)
        return np.sort(s.shape[-1] - 1 - out, axis=-1).astype(np.int32)
    return topk


def _topk_count_floor(real):
    return lambda sparsity, nb: max(1, min(nb, math.floor((1.0 - sparsity) * nb)))


def _perm_column_major(real):
    def perm(g):
        p, inv, bv = real(g)
        p = p.copy()
        for b in range(g.nb):
            blk = p[b * g.block_size : (b + 1) * g.block_size]
            n = int(bv[b])
            if n > 1:
                blk[:n] = blk[:n][::-1]
        inv = np.empty(g.N, dtype=np.int32)
        live = p >= 0
        inv[p[live]] = np.nonzero(live)[0]
        return p, inv, bv
    return perm


def _encode_ties_away(real):
    t = F.e4m3_decode_table()
    pos = t[:0x7F]

    def enc(x):
        x = np.asarray(x, dtype=np.float32)
        out = real(x)
        a = np.abs(x.astype(np.float64))
        i = np.searchsorted(pos, a)
        mid = (i > 0) & (i < len(pos)) & (a == (pos[np.clip(i - 1, 0, len(pos) - 1)] + pos[np.clip(i, 0, len(pos) - 1)]) / 2)
        up = np.where(mid, i, out & 0x7F).astype(np.uint8)
        return np.where(mid, up | (out & 0x80), out).astype(np.uint8)
    return enc


def _quant_scale_240(real):
    def quant(x, transpose=False):
        codes, s = real(np.asarray(x, np.float32) * np.float32(240.0 / 448.0), transpose)
        return codes, s * np.float32(448.0 / 240.0)
    return quant


def _bound_no_subnormal_term(real):
    def bound(q_rows, k_sel, v_sel, scale):
        qr = np.asarray(q_rows, np.float64)
        ks = np.asarray(k_sel, np.float64)
        if ks.shape[0] == 0:
            return np.zeros((qr.shape[0], np.asarray(v_sel).shape[1]))
        s = (qr @ ks.T) * scale
        e = np.exp(s - s.max(axis=1, keepdims=True))
        w = e / e.sum(axis=1, keepdims=True)
        return 2.0 ** -4 * (w @ np.abs(np.asarray(v_sel, np.float64)))
    return bound


def _p_e4m3_rounded_sum(real):
    def attn(q_rows, k_sel, v_sel, scale):
        qr = np.asarray(q_rows, np.float64)
        ks = np.asarray(k_sel, np.float64)
        vs = np.asarray(v_sel, np.float64)
        s = (qr @ ks.T) * scale
        p = np.exp(s - s.max(axis=1, keepdims=True))
        pr = F.e4m3_decode_table()[F.e4m3_encode(p.astype(np.float32))]
        return (pr @ vs) / pr.sum(axis=1, keepdims=True)
    return attn


def _keyset_scale_sqrt_dk(real):
    # 1/d instead of 1/sqrt(d)
    return lambda q, k, v, scale: real(q, k, v, scale * scale * math.sqrt(np.asarray(q).shape[1]))


def _block_keys_off_by_one(real):
    def keys(blocks, block_k, n, block_valid):
        got = real(blocks, block_k, n, block_valid)
        return np.minimum(got + 1, n - 1) if len(got) else got
    return keys


def _attend_no_expansion(real):
    def attend(t, T, C, window, T_per, s):
        if T <= C:
            return list(range(T))
        anchors = set(L.anchors(T, T_per, s))
        win = set(L.nearest_order(t, T)[:window])
        return sorted(anchors | win)
    return attend


def _to_f64_shift8(real):
    def to_f64(x):
        x = np.asarray(x)
        if x.dtype == np.uint16:
            return (x.astype(np.uint32) << np.uint32(8)).view(np.float32).astype(np.float64)
        return real(x)
    return to_f64


def _anchors_shifted(real):
    return lambda T, T_per, s: real(T, T_per, (s + 1) % T_per)


MUTATIONS = [
    ("Draft pool divides by the tile size (pads counted as zeros)", D, "draft_pool", _pool_counts_pads,
     lambda gd: [lambda: TD.test_pool_matches_fp64_within_bound(2, 5, 7, 2, 4)]),
    ("Draft map drops a channel", D, "draft_scores", _scores_drop_first_channel,
     lambda gd: [TD.test_scores_exact_on_integers]),
    ("Draft map fuses multiply and add", D, "draft_scores", _scores_fused,
     lambda gd: [TD.test_scores_no_fused_multiply_add]),
    ("Top-k ties go to the higher block index", D, "draft_topk", _topk_ties_high,
     lambda gd: [TD.test_topk_brute_force, TD.test_topk_known_sets]),
    ("Top-k count rounds down", D, "topk_count", _topk_count_floor, lambda gd: [TD.test_topk_count_rule]),
    ("Reorder reverses the token order inside a tile", D, "draft_permutation", _perm_column_major,
     lambda gd: [lambda: TD.test_permutation_worked_example(gd)]),
    ("E4M3 ties round away from zero", F, "e4m3_encode", _encode_ties_away,
     lambda gd: [TF.test_encode_round_trip_and_ties_to_even, TF.test_encode_brute_force_nearest]),
    ("FP8 scale taken against 240 instead of 448", F, "quantize_per_head", _quant_scale_240,
     lambda gd: [TF.test_quantize_per_head_scales_and_layout]),
    ("FP8 bound without its subnormal term", F, "p_rounding_bound", _bound_no_subnormal_term,
     lambda gd: [TF.test_p_rounding_bound_subnormal_term]),
    ("FP8 row sum over the rounded probabilities", F, "attention_p_e4m3", _p_e4m3_rounded_sum,
     lambda gd: [TF.test_attention_p_e4m3_worked_examples]),
    ("Attention scaled by 1/d", A, "attention_keyset", _keyset_scale_sqrt_dk,
     lambda gd: [TA.test_brute_force_tiny, lambda: TA.test_lvsa_tiny_vs_sdpa(0)]),
    ("Block keys shifted by one row", A, "_block_keys", _block_keys_off_by_one,
     lambda gd: [lambda: TA.test_lvsa_tiny_vs_sdpa(1), TA.test_full_mask_equals_dense]),
    ("LVSA window never widened", L, "attend_set", _attend_no_expansion,
     lambda gd: [lambda: TL.test_worked_examples(gd)]),
    ("bf16 decode shifts by 8 instead of 16", A, "to_f64", _to_f64_shift8,
     lambda gd: [TB.test_fixed_patterns, TA.test_lvsa_frame_gather_equals_dense_on_gathered_frames,
                 TA.test_draft_reorder_invariance]),
    ("LVSA anchors one step off", L, "anchors", _anchors_shifted,
     lambda gd: [lambda: TL.test_worked_examples(gd)]),
]


@pytest.mark.parametrize("what,module,name,mutate,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(what, module, name, mutate, pins, monkeypatch, golden_dir):
    real = getattr(module, name)
    _patch(monkeypatch, module, name, mutate(real))
    assert _some_pin_fails(pins(golden_dir)), f"no pin caught: {what}"


@pytest.mark.parametrize("what,module,name,mutate,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_pass_without_the_mistake(what, module, name, mutate, pins, golden_dir):
    """The same pins pass on the oracle as it is (so a failure above is the mutation's)."""
    for pin in pins(golden_dir):
        pin()

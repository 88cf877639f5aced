"""Writes input_stats.json: statistics of the seeded synthetic inputs of every
workload, computed by the oracle (test infrastructure) on sampled query rows.

For each workload, a few heads and a few query rows per head (seeded): the
standard deviation of the scaled logits over all N keys, the entropy of the
dense softmax, the entropy of the softmax over the keys the workload's mask
keeps, and the share of the dense softmax mass on those keys. The masks are
the oracle's: LVSA with shift s = 0 (frame lists, one frame per block), Draft
Attention from the pooled draft map of that head.

Run from the repository root: python3 tests/golden/input_stats.py
It calls only oracle/ and the seeded generators; nothing here reads results of
the HIP library.
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from video_diffusion_transformer_lvsa_amd import synth  # noqa: E402

ROWS_PER_HEAD = 48
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_stats.json")


def head_inputs(w, h):
    if w.dtype == "f32":
        q, k, _ = synth.iid_qkv(w.seed, w.heads, w.N, w.d)
        return q[h].astype(np.float64), k[h].astype(np.float64)
    q, k, _ = synth.video_qkv_head(w.seed, h, w.heads, w.T, w.H, w.W, w.d)
    return oracle.to_f64(q), oracle.to_f64(k)


def keep_rows(w, rows, qh, kh):
    """Boolean [len(rows), N]: the keys the workload's mask gives each row."""
    n = w.N
    keep = np.zeros((len(rows), n), dtype=bool)
    if w.kind == "lvsa":
        kv, cnt = oracle.lvsa_mask(w.T, w.C, w.window, w.T_per, 0)
        for i, r in enumerate(rows):
            t = r // w.P
            for f in kv[t, : cnt[t]]:
                keep[i, f * w.P : (f + 1) * w.P] = True
        return keep
    g = oracle.draft_grid(w.T, w.H, w.W, w.pool_h, w.pool_w)
    perm, inv, bv = oracle.draft_permutation(g)
    kv, cnt, *_ = oracle.draft_mask(qh[None].astype(np.float32), kh[None].astype(np.float32), g, w.sparsity)
    for i, r in enumerate(rows):
        b = inv[r] // g.block_size
        for bb in kv[0, b, : cnt[0, b]]:
            keep[i, perm[bb * g.block_size : bb * g.block_size + int(bv[bb])]] = True
    return keep


def workload_stats(w):
    heads = sorted({0, w.heads // 2, w.heads - 1})
    rng = np.random.default_rng(1000 + w.seed)
    acc = {"logit_std": [], "entropy_dense": [], "entropy_kept": [], "mass_kept": []}
    for h in heads:
        qh, kh = head_inputs(w, h)
        rows = np.sort(rng.choice(w.N, size=min(ROWS_PER_HEAD, w.N), replace=False))
        st = oracle.attention_statistics(qh[rows], kh, keep_rows(w, rows, qh, kh), 1.0 / np.sqrt(w.d))
        for key in acc:
            acc[key].append(st[key])
    cat = {key: np.concatenate(v) for key, v in acc.items()}
    return {
        "seed": w.seed,
        "heads_sampled": heads,
        "rows_per_head": int(min(ROWS_PER_HEAD, w.N)),
        "keys": w.N,
        "log_keys": round(float(np.log(w.N)), 4),
        "logit_std_mean": round(float(cat["logit_std"].mean()), 4),
        "entropy_dense_mean": round(float(cat["entropy_dense"].mean()), 4),
        "entropy_kept_mean": round(float(cat["entropy_kept"].mean()), 4),
        "mass_kept_mean": round(float(cat["mass_kept"].mean()), 4),
        "mass_kept_min": round(float(cat["mass_kept"].min()), 4),
    }


def main():
    out = {}
    for name, w in synth.WORKLOADS.items():
        print(f"{name} ...", flush=True)
        out[name] = workload_stats(w)
        print(f"  {out[name]}", flush=True)
    with open(OUT, "w") as f:
        json.dump({"generator": "tests/golden/input_stats.py", "workloads": out}, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()

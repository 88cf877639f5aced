"""The attention paths captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: the library launches only kernels on the caller's stream (no
memsets, no allocations, no host synchronisation), so a whole step can be
captured once and replayed. Each replay runs between eager work and
synchronisations and must equal the eager result bit for bit (the kernels
are deterministic)."""
import pytest

from video_diffusion_transformer_lvsa_amd import _lib, synth

from helpers import note, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _torch():
    import torch

    return torch


def _replay_and_check(capture, outputs, what):
    """capture() enqueues the step on the current stream and writes `outputs`
    (preallocated tensors). Runs it eagerly, captures it, replays it."""
    torch = _torch()
    capture()
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        capture()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for o in outputs:
            o.fill_(float("nan") if o.is_floating_point() else 77)
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        note(f"{what}: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        for o, wnt in zip(outputs, want):
            assert torch.equal(o, wnt), f"{what}: replay {r} differs from the eager result"
        del junk


def test_graph_lvsa_step():
    torch = _torch()
    T, H, W, heads, C, win, T_per, s = 12, 30, 52, 2, 5, 3, 4, 1
    P = H * W
    q, k, v = (to_dev(x) for x in synth.video_qkv(5, heads, T, H, W, 128))
    cap = _lib.lvsa_mask_capacity(T, C, win, T_per, s)
    idx = torch.empty((T, cap), dtype=torch.int32, device="cuda")
    cnt = torch.empty((T,), dtype=torch.int32, device="cuda")
    o = torch.empty((heads, T * P, 128), dtype=torch.float32, device="cuda")

    def step():
        _lib.lvsa_mask(T, C, win, T_per, s, cap=cap, kv_idx=idx, kv_cnt=cnt)
        _lib.block_sparse_attn_fwd(q, k, v, P, P, idx, cnt, out=o)

    _replay_and_check(step, [idx, cnt, o], "lvsa step")


def test_graph_lvsa_step_fp8():
    torch = _torch()
    T, H, W, heads, C, win, T_per, s = 12, 30, 52, 2, 5, 3, 4, 2
    P, n = H * W, T * H * W
    q, k, v = (to_dev(x) for x in synth.video_qkv(6, heads, T, H, W, 128))
    cap = _lib.lvsa_mask_capacity(T, C, win, T_per, s)
    idx = torch.empty((T, cap), dtype=torch.int32, device="cuda")
    cnt = torch.empty((T,), dtype=torch.int32, device="cuda")
    q8 = torch.empty((heads, n, 128), dtype=torch.uint8, device="cuda")
    k8 = torch.empty_like(q8)
    vt8 = torch.empty((heads, 128, _lib.fp8_pitch(n)), dtype=torch.uint8, device="cuda")
    sc = torch.empty((3, heads), dtype=torch.float32, device="cuda")
    o = torch.empty((heads, n, 128), dtype=torch.float32, device="cuda")

    def step():
        _lib.quantize_fp8_e4m3(q, out=q8, scales=sc[0])
        _lib.quantize_fp8_e4m3(k, out=k8, scales=sc[1])
        _lib.quantize_fp8_e4m3(v, transpose=True, out=vt8, scales=sc[2])
        _lib.lvsa_mask(T, C, win, T_per, s, cap=cap, kv_idx=idx, kv_cnt=cnt)
        _lib.block_sparse_attn_fwd_fp8(q8, k8, vt8, sc[0], sc[1], sc[2], P, P, idx, cnt, out=o)

    _replay_and_check(step, [q8, k8, vt8, sc, idx, cnt, o], "fp8 lvsa step")


def test_graph_draft_raster_step():
    torch = _torch()
    T, H, W, ph, pw, heads, sp = 3, 45, 80, 8, 16, 2, 0.9
    q, k, v = (to_dev(x) for x in synth.video_qkv(7, heads, T, H, W, 128))
    info = _lib.draft_grid_info(T, H, W, ph, pw, sp)
    kv_idx = torch.empty((heads, info["nb"], info["k"]), dtype=torch.int32, device="cuda")
    kv_cnt = torch.empty((heads, info["nb"]), dtype=torch.int32, device="cuda")
    o = torch.empty((heads, T * H * W, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty((_lib.draft_workspace_bytes(heads, T, H, W, 128, ph, pw) // 4,), dtype=torch.float32,
                     device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    bufs = {"kv_idx": kv_idx, "kv_cnt": kv_cnt, "workspace": ws, "perm": torch.empty((info["n_pad"],), **i32),
            "inv_perm": torch.empty((T * H * W,), **i32), "block_valid": torch.empty((info["nb"],), **i32)}

    def step():
        _lib.draft_mask_and_perm(q, k, v, T, H, W, ph, pw, sp, reorder=False, buffers=bufs)
        _lib.draft_attn_fwd(q, k, v, T, H, W, ph, pw, kv_idx, kv_cnt, out=o)

    _replay_and_check(step, [kv_idx, kv_cnt, o], "draft raster step")


def test_graph_draft_reorder_step():
    """The Draft step as the article lays it out: mask and reorder, block-
    sparse attention on the reordered tensors, scatter back to token order."""
    torch = _torch()
    T, H, W, ph, pw, heads, sp = 3, 45, 80, 8, 16, 2, 0.9
    q, k, v = (to_dev(x) for x in synth.video_qkv(7, heads, T, H, W, 128))
    info = _lib.draft_grid_info(T, H, W, ph, pw, sp)
    nb, n_pad, n, bs = info["nb"], info["n_pad"], T * H * W, ph * pw
    i32 = dict(dtype=torch.int32, device="cuda")
    bufs = {"kv_idx": torch.empty((heads, nb, info["k"]), **i32), "kv_cnt": torch.empty((heads, nb), **i32),
            "perm": torch.empty((n_pad,), **i32), "inv_perm": torch.empty((n,), **i32),
            "block_valid": torch.empty((nb,), **i32),
            "workspace": torch.empty((_lib.draft_workspace_bytes(heads, T, H, W, 128, ph, pw) // 4,),
                                     dtype=torch.float32, device="cuda")}
    for name in ("q_perm", "k_perm", "v_perm"):
        bufs[name] = torch.empty((heads, n_pad, 128), dtype=q.dtype, device="cuda")
    o_perm = torch.empty((heads, n_pad, 128), dtype=torch.float32, device="cuda")
    o = torch.empty((heads, n, 128), dtype=torch.float32, device="cuda")

    def step():
        _lib.draft_mask_and_perm(q, k, v, T, H, W, ph, pw, sp, buffers=bufs)
        _lib.block_sparse_attn_fwd(bufs["q_perm"], bufs["k_perm"], bufs["v_perm"], bs, bs, bufs["kv_idx"],
                                   bufs["kv_cnt"], mask_heads=heads, block_valid=bufs["block_valid"], out=o_perm)
        _lib.token_permute(o_perm, bufs["inv_perm"], out=o)

    _replay_and_check(step, [bufs["kv_idx"], bufs["q_perm"], o_perm, o], "draft reorder step")

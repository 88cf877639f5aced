"""ctypes binding of liblvsa.so (the C ABI in include/lvsa.h).

Argument marshalling only: every step of the path runs in the HIP library.
torch is used for device memory and the current stream. The functions carry
the ABI's names and take torch tensors; outputs are allocated with torch when
not given. There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblvsa.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "lvsa.h")

LVSA_OK, LVSA_EINVAL, LVSA_ERANGE, LVSA_EDEVICE, LVSA_ENOMEM, LVSA_EUNSUPPORTED = 0, -1, -2, -3, -4, -5
LVSA_F32, LVSA_BF16 = 0, 1

_c_int, _c_sz, _c_dbl, _c_flt, _p = ctypes.c_int, ctypes.c_size_t, ctypes.c_double, ctypes.c_float, ctypes.c_void_p
_pint = ctypes.POINTER(ctypes.c_int)

SIGNATURES = {
    "lvsa_last_error": (ctypes.c_char_p, []),
    "lvsa_version": (ctypes.c_char_p, []),
    "lvsa_mask_capacity": (_c_int, [_c_int] * 5),
    "lvsa_mask": (_c_int, [_c_int] * 5 + [_p, _p, _c_int, _p]),
    "draft_grid_info": (_c_int, [_c_int] * 5 + [_c_dbl, _pint, _pint, _pint, _pint]),
    "draft_workspace_bytes": (_c_sz, [_c_int] * 7),
    "draft_mask_and_perm": (_c_int, [_p, _p, _p] + [_c_int] * 8 + [_c_dbl, _c_int] + [_p] * 9 + [_c_sz, _p]),
    "draft_mask_and_perm_noalloc": (_c_int, [_p, _p, _p] + [_c_int] * 8 + [_c_dbl, _c_int] + [_p] * 8 + [_p]),
    "draft_scores": (_c_int, [_p, _p] + [_c_int] * 4 + [_p, _p]),
    "token_permute": (_c_int, [_p, _p] + [_c_int] * 5 + [_p, _p]),
    "block_sparse_attn_fwd": (_c_int, [_p] * 4 + [_c_int] * 6 + [_p, _p, _c_int, _c_int, _p, _c_flt, _p]),
    "dense_attn_fwd": (_c_int, [_p] * 4 + [_c_int] * 4 + [_c_flt, _p]),
    "draft_attn_fwd": (_c_int, [_p] * 4 + [_c_int] * 8 + [_p, _p, _c_int, _c_flt, _p]),
    "quantize_fp8_e4m3": (_c_int, [_p] + [_c_int] * 6 + [_p, _p, _p]),
    "block_sparse_attn_fwd_fp8": (_c_int, [_p] * 3 + [_c_int] + [_p] * 4 + [_c_int] * 5
                                  + [_p, _p, _c_int, _c_int, _p, _c_flt, _p]),
    "draft_attn_fwd_fp8": (_c_int, [_p] * 3 + [_c_int] + [_p] * 4 + [_c_int] * 7 + [_p, _p, _c_int, _c_flt, _p]),
    "dense_attn_fwd_fp8": (_c_int, [_p] * 3 + [_c_int] + [_p] * 4 + [_c_int] * 3 + [_c_flt, _p]),
}

_lib = None


class LvsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"lvsa error {code}: {msg}")
        self.code = code


def load() -> ctypes.CDLL:
    """Load liblvsa.so (built in-tree by build.py; LVSA_LIBRARY may name another
    build of the same library). Raises if it is missing."""
    global _lib
    if _lib is None:
        path = os.environ.get("LVSA_LIBRARY", LIB_PATH)
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m video_diffusion_transformer_lvsa_amd.build`")
        # torch ships its own HIP runtime. Loading it first makes the library
        # bind to that same runtime (one device context; torch's streams and
        # pointers are valid in the library). Opened first, the library would
        # pull in the system runtime and torch would then load a second one,
        # which finds no device.
        _torch()
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/lvsa.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def last_error() -> str:
    return load().lvsa_last_error().decode()


def _check(rc: int):
    if rc != 0:
        raise LvsaError(rc, last_error())
    return rc


# --------------------------------------------------------------------------
# torch-facing wrappers
# --------------------------------------------------------------------------
def _torch():
    import torch

    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LVSA_BF16
    if t.dtype == torch.float32:
        return LVSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _contig_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous CUDA (HIP) tensors")


def _expect(t, name: str, shape=None, dtype=None, device=None, numel=None, min_numel=None):
    """Raise ValueError unless tensor t has the given shape, dtype, device and size.
    The kernels size their index ranges from the scalar arguments, so a tensor
    that disagrees with them would be read or written out of bounds."""
    if t is None:
        raise ValueError(f"{name} is required")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name}: expected at least {min_numel} elements, got {t.numel()}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")


def _check_qkv(q, k, v, out=None, what="q"):
    """q [heads, n, d] and k, v of the same shape, dtype and device; out fp32 [heads, n, d]."""
    torch = _torch()
    if q.dim() != 3:
        raise ValueError(f"{what}: expected [heads, n, d], got shape {tuple(q.shape)}")
    for name, t in (("k", k), ("v", v)):
        _expect(t, name, q.shape, q.dtype, q.device)
    if out is not None:
        _expect(out, "out", q.shape, torch.float32, q.device)


def _check_lists(kv_idx, kv_cnt, lead: tuple, device, kv_idx_required: bool = True):
    """kv_idx int32 [*lead, max_kv] and kv_cnt int32 [*lead] (a leading 1 may be dropped)."""
    torch = _torch()
    _expect(kv_cnt, "kv_cnt", dtype=torch.int32, device=device, numel=math.prod(lead))
    if kv_idx is None:
        if kv_idx_required:
            raise ValueError("kv_idx is required")
        return 0
    _expect(kv_idx, "kv_idx", dtype=torch.int32, device=device)
    got = tuple(kv_idx.shape[:-1])
    ok = got == tuple(lead) or (len(lead) > 1 and lead[0] == 1 and got == tuple(lead[1:]))
    if kv_idx.dim() < 2 or not ok:
        raise ValueError(f"kv_idx: expected shape {tuple(lead)} + (max_kv,), got {tuple(kv_idx.shape)}")
    return int(kv_idx.shape[-1])


def lvsa_mask_capacity(T: int, C: int, window: int, T_per: int, step: int) -> int:
    rc = load().lvsa_mask_capacity(T, C, window, T_per, step)
    if rc < 0:
        raise LvsaError(rc, last_error())
    return rc


def lvsa_mask(T: int, C: int, window: int, T_per: int, step: int, cap: int | None = None, kv_idx=None, kv_cnt=None,
              device="cuda", stream=None):
    """LVSA frame lists on the GPU: (kv_idx [T, cap] int32, kv_cnt [T] int32)."""
    torch = _torch()
    if kv_idx is not None:
        # the lists are written at the buffer's row pitch, which the attention reads back
        if kv_idx.dim() != 2 or kv_idx.shape[0] != T:
            raise ValueError(f"kv_idx: expected shape ({T}, cap), got {tuple(kv_idx.shape)}")
        if cap is not None and cap != kv_idx.shape[1]:
            raise ValueError(f"cap={cap} differs from kv_idx's row length {kv_idx.shape[1]}")
        cap = int(kv_idx.shape[1])
        _expect(kv_idx, "kv_idx", dtype=torch.int32)
    elif cap is None:
        cap = lvsa_mask_capacity(T, C, window, T_per, step)
    if kv_idx is None:
        kv_idx = torch.empty((T, cap), dtype=torch.int32, device=device)
    if kv_cnt is None:
        kv_cnt = torch.empty((T,), dtype=torch.int32, device=kv_idx.device)
    _expect(kv_cnt, "kv_cnt", (T,), torch.int32, kv_idx.device)
    _contig_cuda(kv_idx, kv_cnt)
    _check(load().lvsa_mask(T, C, window, T_per, step, _ptr(kv_idx), _ptr(kv_cnt), cap, _stream(stream)))
    return kv_idx, kv_cnt


def draft_grid_info(T: int, H: int, grid_w: int, pool_h: int, pool_w: int, sparsity: float) -> dict:
    nb, n_pad, bs, k = (ctypes.c_int() for _ in range(4))
    _check(load().draft_grid_info(T, H, grid_w, pool_h, pool_w, sparsity, ctypes.byref(nb), ctypes.byref(n_pad),
                                  ctypes.byref(bs), ctypes.byref(k)))
    return {"nb": nb.value, "n_pad": n_pad.value, "block_size": bs.value, "k": k.value}


def draft_workspace_bytes(heads: int, T: int, H: int, grid_w: int, d: int, pool_h: int, pool_w: int) -> int:
    return int(load().draft_workspace_bytes(heads, T, H, grid_w, d, pool_h, pool_w))


POOL_MODES = {"mean": 0, "max": 1}


def draft_mask_and_perm(q, k, v, T: int, H: int, grid_w: int, pool_h: int, pool_w: int, sparsity: float,
                        reorder: bool = True, pool: str = "mean", buffers: dict | None = None, stream=None) -> dict:
    """Draft mask builder + reorder. q, k, v: [heads, T*H*grid_w, d] on the GPU;
    pool is "mean" or "max".

    Returns a dict with kv_idx, kv_cnt, perm, inv_perm, block_valid, the
    reordered q_perm/k_perm/v_perm (if reorder) and qbar/kbar (views of the
    workspace). `buffers` may hold any of these outputs and "workspace"
    (float32, draft_workspace_bytes / 4 elements), preallocated by the caller
    (for instance for a captured graph); the others are allocated."""
    torch = _torch()
    _check_qkv(q, k, v)
    heads, n, d = q.shape
    if n != T * H * grid_w:
        raise ValueError(f"q has {n} tokens; the grid {T}x{H}x{grid_w} has {T * H * grid_w}")
    if pool not in POOL_MODES:
        raise ValueError(f"pool must be one of {sorted(POOL_MODES)}")
    _contig_cuda(q, k, v)
    info = draft_grid_info(T, H, grid_w, pool_h, pool_w, sparsity)
    nb, n_pad, topk = info["nb"], info["n_pad"], info["k"]
    dev = q.device
    i32 = dict(dtype=torch.int32, device=dev)
    given = buffers or {}

    def buf(name, shape, **kw):
        t = given.get(name)
        if t is None:
            return torch.empty(shape, **kw)
        if tuple(t.shape) != tuple(shape) or t.dtype != kw["dtype"]:
            raise ValueError(f"{name}: expected {kw['dtype']} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
        _expect(t, name, device=dev)
        return t

    out = {
        "kv_idx": buf("kv_idx", (heads, nb, topk), **i32),
        "kv_cnt": buf("kv_cnt", (heads, nb), **i32),
        "perm": buf("perm", (n_pad,), **i32),
        "inv_perm": buf("inv_perm", (n,), **i32),
        "block_valid": buf("block_valid", (nb,), **i32),
        "info": info,
    }
    if reorder:
        for name in ("q_perm", "k_perm", "v_perm"):
            out[name] = buf(name, (heads, n_pad, d), dtype=q.dtype, device=dev)
    ws_bytes = draft_workspace_bytes(heads, T, H, grid_w, d, pool_h, pool_w)
    ws = buf("workspace", (ws_bytes // 4,), dtype=torch.float32, device=dev)
    _contig_cuda(*(t for key, t in out.items() if key != "info"), ws)
    _check(load().draft_mask_and_perm(
        _ptr(q), _ptr(k), _ptr(v), _dt(q), heads, T, H, grid_w, d, pool_h, pool_w, sparsity, POOL_MODES[pool],
        _ptr(out["kv_idx"]), _ptr(out["kv_cnt"]), _ptr(out["perm"]), _ptr(out["inv_perm"]), _ptr(out["block_valid"]),
        _ptr(out.get("q_perm")), _ptr(out.get("k_perm")), _ptr(out.get("v_perm")), _ptr(ws), ws_bytes,
        _stream(stream)))
    out["qbar"] = ws[: heads * nb * d].view(heads, nb, d)
    out["kbar"] = ws[heads * nb * d : 2 * heads * nb * d].view(heads, nb, d)
    return out


NOALLOC_SCRATCH_BYTES = 48 << 20  # LVSA_NOALLOC_SCRATCH_BYTES


def draft_mask_and_perm_noalloc(q, k, v, T: int, H: int, grid_w: int, pool_h: int, pool_w: int, sparsity: float,
                                out: dict, pool: str = "mean", stream=None) -> dict:
    """draft_mask_and_perm without a workspace: the library's own device
    scratch holds the pooled Q and K, so nothing is allocated, here or in the
    library. `out` must hold every output, preallocated: kv_idx, kv_cnt,
    perm, inv_perm, block_valid and, to reorder, q_perm, k_perm, v_perm (all
    three, or none of them)."""
    torch = _torch()
    _check_qkv(q, k, v)
    heads, n, d = q.shape
    if n != T * H * grid_w:
        raise ValueError(f"q has {n} tokens; the grid {T}x{H}x{grid_w} has {T * H * grid_w}")
    if pool not in POOL_MODES:
        raise ValueError(f"pool must be one of {sorted(POOL_MODES)}")
    info = draft_grid_info(T, H, grid_w, pool_h, pool_w, sparsity)
    nb, n_pad, topk = info["nb"], info["n_pad"], info["k"]
    want = {"kv_idx": ((heads, nb, topk), torch.int32), "kv_cnt": ((heads, nb), torch.int32),
            "perm": ((n_pad,), torch.int32), "inv_perm": ((n,), torch.int32), "block_valid": ((nb,), torch.int32)}
    perm_names = [x for x in ("q_perm", "k_perm", "v_perm") if out.get(x) is not None]
    if perm_names and len(perm_names) != 3:
        raise ValueError("q_perm, k_perm, v_perm: give all three or none")
    for name in perm_names:
        want[name] = ((heads, n_pad, d), q.dtype)
    for name, (shape, dt) in want.items():
        _expect(out.get(name), name, shape, dt, q.device)
    _contig_cuda(q, k, v, *(out[x] for x in want))
    _check(load().draft_mask_and_perm_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _dt(q), heads, T, H, grid_w, d, pool_h, pool_w, sparsity, POOL_MODES[pool],
        _ptr(out["kv_idx"]), _ptr(out["kv_cnt"]), _ptr(out["perm"]), _ptr(out["inv_perm"]), _ptr(out["block_valid"]),
        _ptr(out.get("q_perm")), _ptr(out.get("k_perm")), _ptr(out.get("v_perm")), _stream(stream)))
    return out


def draft_scores(qbar, kbar, stream=None):
    torch = _torch()
    if qbar.dim() != 3 or kbar.dim() != 3:
        raise ValueError("qbar and kbar must be [heads, nb, d]")
    heads, nbq, d = qbar.shape
    nbk = kbar.shape[1]
    _expect(qbar, "qbar", dtype=torch.float32)
    _expect(kbar, "kbar", (heads, nbk, d), torch.float32, qbar.device)
    _contig_cuda(qbar, kbar)
    s = torch.empty((heads, nbq, nbk), dtype=torch.float32, device=qbar.device)
    _check(load().draft_scores(_ptr(qbar), _ptr(kbar), heads, nbq, nbk, d, _ptr(s), _stream(stream)))
    return s


def token_permute(src, dst_to_src, out=None, stream=None):
    """out[h, i] = src[h, dst_to_src[i]] (zeros where the map is -1)."""
    torch = _torch()
    if src.dim() != 3 or dst_to_src.dim() != 1:
        raise ValueError("src must be [heads, n_src, d] and dst_to_src one-dimensional")
    heads, n_src, d = src.shape
    n_dst = dst_to_src.shape[0]
    _expect(dst_to_src, "dst_to_src", dtype=torch.int32, device=src.device)
    if out is None:
        out = torch.empty((heads, n_dst, d), dtype=src.dtype, device=src.device)
    _expect(out, "out", (heads, n_dst, d), src.dtype, src.device)
    _contig_cuda(src, dst_to_src, out)
    _check(load().token_permute(_ptr(src), _ptr(out), _dt(src), heads, n_src, n_dst, d, _ptr(dst_to_src),
                                _stream(stream)))
    return out


def block_sparse_attn_fwd(q, k, v, block_q: int, block_k: int, kv_idx, kv_cnt, mask_heads: int = 1, block_valid=None,
                          scale: float | None = None, out=None, stream=None):
    """Block-sparse attention; returns O fp32 [heads, n, d]."""
    torch = _torch()
    _check_qkv(q, k, v, out)
    heads, n, d = q.shape
    if mask_heads not in (1, heads):
        raise ValueError(f"mask_heads={mask_heads} must be 1 or heads={heads}")
    if block_q < 1 or block_k < 1:
        raise ValueError("block_q and block_k must be >= 1")
    max_kv = _check_lists(kv_idx, kv_cnt, (mask_heads, -(-n // block_q)), q.device)
    if block_valid is not None:
        _expect(block_valid, "block_valid", dtype=torch.int32, device=q.device, min_numel=-(-n // block_k))
    if out is None:
        out = torch.empty((heads, n, d), dtype=torch.float32, device=q.device)
    _contig_cuda(q, k, v, out, kv_idx, kv_cnt, block_valid)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(load().block_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dt(q), heads, n, d, block_q, block_k,
                                        _ptr(kv_idx), _ptr(kv_cnt), max_kv, mask_heads, _ptr(block_valid), scale,
                                        _stream(stream)))
    return out


def dense_attn_fwd(q, k, v, scale: float | None = None, out=None, stream=None):
    """Dense attention; returns O fp32 [heads, n, d]."""
    torch = _torch()
    _check_qkv(q, k, v, out)
    heads, n, d = q.shape
    if out is None:
        out = torch.empty((heads, n, d), dtype=torch.float32, device=q.device)
    _contig_cuda(q, k, v, out)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(load().dense_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dt(q), heads, n, d, scale, _stream(stream)))
    return out


def _draft_blocks(n: int, T: int, H: int, grid_w: int, pool_h: int, pool_w: int) -> int:
    """Pool tiles of the grid (raster order), after checking the grid matches n tokens."""
    if n != T * H * grid_w:
        raise ValueError(f"{n} tokens; the grid {T}x{H}x{grid_w} has {T * H * grid_w}")
    if pool_h < 1 or pool_w < 1:
        raise ValueError("pool sizes must be >= 1")
    return T * (-(-H // pool_h)) * (-(-grid_w // pool_w))


def draft_attn_fwd(q, k, v, T: int, H: int, grid_w: int, pool_h: int, pool_w: int, kv_idx, kv_cnt,
                   scale: float | None = None, out=None, stream=None):
    """Draft attention on the raster layout (no reorder): q, k, v [heads, T*H*grid_w, 128]
    bf16, per-head lists kv_idx [heads, nb, k], kv_cnt [heads, nb]; returns O fp32."""
    torch = _torch()
    _check_qkv(q, k, v, out)
    heads, n, d = q.shape
    nb = _draft_blocks(n, T, H, grid_w, pool_h, pool_w)
    _check_lists(kv_idx, kv_cnt, (heads, nb), q.device)
    if out is None:
        out = torch.empty((heads, n, d), dtype=torch.float32, device=q.device)
    _contig_cuda(q, k, v, out, kv_idx, kv_cnt)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(load().draft_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _dt(q), heads, T, H, grid_w, d, pool_h, pool_w,
                                 _ptr(kv_idx), _ptr(kv_cnt), kv_idx.shape[-1], scale, _stream(stream)))
    return out


# --------------------------------------------------------------------------
# FP8 (E4M3) variant
# --------------------------------------------------------------------------
def fp8_pitch(n: int) -> int:
    """Row pitch (bytes) of a transposed code tensor: n rounded up to 128, so
    every row starts on a cache line (the ABI needs only a multiple of 16)."""
    return (n + 127) // 128 * 128


def quantize_fp8_e4m3(x, transpose: bool = False, ld: int | None = None, out=None, scales=None, stream=None):
    """Per-head E4M3 codes of x [heads, n, d] (bf16 or fp32). Returns (codes, scales):
    codes uint8 [heads, n, d], or [heads, d, ld] when transpose (ld defaults to
    fp8_pitch(n)); scales fp32 [heads] (the value of a code is decode(code) * scale)."""
    torch = _torch()
    if x.dim() != 3:
        raise ValueError(f"x: expected [heads, n, d], got shape {tuple(x.shape)}")
    heads, n, d = x.shape
    if transpose:
        if ld is None:
            ld = fp8_pitch(n) if out is None else int(out.shape[-1])
        shape = (heads, d, ld)
    else:
        ld = 0
        shape = (heads, n, d)
    if out is None:
        out = torch.empty(shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((heads,), dtype=torch.float32, device=x.device)
    _expect(out, "out", shape, torch.uint8, x.device)
    _expect(scales, "scales", dtype=torch.float32, device=x.device, numel=heads)
    _contig_cuda(x, out, scales)
    _check(load().quantize_fp8_e4m3(_ptr(x), _dt(x), heads, n, d, int(transpose), ld, _ptr(out), _ptr(scales),
                                    _stream(stream)))
    return out, scales


def quantize_qkv_fp8(q, k, v, stream=None) -> dict:
    """Codes and scales the FP8 attention takes: q8, k8 row-major, vt8 transposed."""
    q8, qs = quantize_fp8_e4m3(q, stream=stream)
    k8, ks = quantize_fp8_e4m3(k, stream=stream)
    vt8, vs = quantize_fp8_e4m3(v, transpose=True, stream=stream)
    return {"q8": q8, "k8": k8, "vt8": vt8, "q_scale": qs, "k_scale": ks, "v_scale": vs}


def _check_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, out):
    """q8, k8 uint8 [heads, n, d]; vt8 uint8 [heads, d, ldv] with ldv >= n; scales fp32 [heads]; out fp32."""
    torch = _torch()
    if q8.dim() != 3:
        raise ValueError(f"q8: expected [heads, n, d], got shape {tuple(q8.shape)}")
    heads, n, d = q8.shape
    _expect(q8, "q8", dtype=torch.uint8)
    _expect(k8, "k8", q8.shape, torch.uint8, q8.device)
    _expect(vt8, "vt8", dtype=torch.uint8, device=q8.device)
    if vt8.dim() != 3 or vt8.shape[0] != heads or vt8.shape[1] != d or vt8.shape[2] < n:
        raise ValueError(f"vt8: expected [{heads}, {d}, ldv >= {n}], got {tuple(vt8.shape)}")
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _expect(t, name, dtype=torch.float32, device=q8.device, numel=heads)
    if out is not None:
        _expect(out, "out", q8.shape, torch.float32, q8.device)


def block_sparse_attn_fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, block_q: int, block_k: int, kv_idx, kv_cnt,
                              mask_heads: int = 1, block_valid=None, scale: float | None = None, out=None,
                              stream=None):
    """Block-sparse attention on E4M3 codes (vt8 [heads, 128, ldv]); returns O fp32 [heads, n, 128]."""
    torch = _torch()
    _check_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, out)
    heads, n, d = q8.shape
    if mask_heads not in (1, heads):
        raise ValueError(f"mask_heads={mask_heads} must be 1 or heads={heads}")
    if block_q < 1 or block_k < 1:
        raise ValueError("block_q and block_k must be >= 1")
    _check_lists(kv_idx, kv_cnt, (mask_heads, -(-n // block_q)), q8.device)
    if block_valid is not None:
        _expect(block_valid, "block_valid", dtype=torch.int32, device=q8.device, min_numel=-(-n // block_k))
    if out is None:
        out = torch.empty((heads, n, d), dtype=torch.float32, device=q8.device)
    _contig_cuda(q8, k8, vt8, q_scale, k_scale, v_scale, out, kv_idx, kv_cnt, block_valid)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(load().block_sparse_attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(vt8), vt8.shape[-1], _ptr(q_scale),
                                            _ptr(k_scale), _ptr(v_scale), _ptr(out), heads, n, d, block_q, block_k,
                                            _ptr(kv_idx), _ptr(kv_cnt), kv_idx.shape[-1], mask_heads,
                                            _ptr(block_valid), scale, _stream(stream)))
    return out


def draft_attn_fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, T: int, H: int, grid_w: int, pool_h: int,
                       pool_w: int, kv_idx, kv_cnt, scale: float | None = None, out=None, stream=None):
    """FP8 Draft attention on the raster layout: codes of q, k [heads, T*H*grid_w, 128] and
    vt8 [heads, 128, ldv], per-head lists kv_idx [heads, nb, k], kv_cnt [heads, nb]; returns O fp32."""
    torch = _torch()
    _check_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, out)
    heads, n, d = q8.shape
    nb = _draft_blocks(n, T, H, grid_w, pool_h, pool_w)
    _check_lists(kv_idx, kv_cnt, (heads, nb), q8.device)
    if out is None:
        out = torch.empty((heads, n, d), dtype=torch.float32, device=q8.device)
    _contig_cuda(q8, k8, vt8, q_scale, k_scale, v_scale, out, kv_idx, kv_cnt)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(load().draft_attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(vt8), vt8.shape[-1], _ptr(q_scale), _ptr(k_scale),
                                     _ptr(v_scale), _ptr(out), heads, T, H, grid_w, d, pool_h, pool_w, _ptr(kv_idx),
                                     _ptr(kv_cnt), kv_idx.shape[-1], scale, _stream(stream)))
    return out


def dense_attn_fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, scale: float | None = None, out=None, stream=None):
    """Dense attention on E4M3 codes; returns O fp32 [heads, n, 128]."""
    torch = _torch()
    _check_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, out)
    heads, n, d = q8.shape
    if out is None:
        out = torch.empty((heads, n, d), dtype=torch.float32, device=q8.device)
    _contig_cuda(q8, k8, vt8, q_scale, k_scale, v_scale, out)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    _check(load().dense_attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(vt8), vt8.shape[-1], _ptr(q_scale), _ptr(k_scale),
                                     _ptr(v_scale), _ptr(out), heads, n, d, scale, _stream(stream)))
    return out

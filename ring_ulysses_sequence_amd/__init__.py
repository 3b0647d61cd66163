"""Python binding of libringattn.so (ring-order block attention and Ulysses
transposes for MI355X / gfx950).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels.  Tensors are torch tensors on the GPU (PyTorch supplies device
memory and the current stream); shapes follow the C ABI in
include/ringattn.h:

    block_attn_fwd(q, k, v, ...)   -> (o fp32, lse, m, l)     one ring round
    ring_merge(o_acc, lse_acc, o_blk, lse_blk, ...)           LSE combine
    ring_attn_fwd(q_r, k_blocks, v_blocks, rank, ...) -> (o, lse)
    seq2head(x) / head2seq(x)                                 Ulysses layout
    ring_schedule(P, rank, block_len, causal, valid_len)      host only
    padded_len(S, P), shard_range(S, P, rank), classify_block(...)

Errors: RA_ERR_SHAPE raises ValueError (as the Ulysses guideline's
divisibility check does), every other status RuntimeError.  If the shared
library has not been built the import succeeds but every call raises; there
is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libringattn.so")

RA_OK, RA_ERR_NULL, RA_ERR_SHAPE, RA_ERR_DTYPE, RA_ERR_RANGE, RA_ERR_UNSUPPORTED, RA_ERR_HIP = range(7)
RA_BF16, RA_FP32 = 0, 1
RA_SKIP, RA_FULL, RA_DIAG = 0, 1, 2
RA_MAX_P = 64
RA_PAD_MULTIPLE = 16
RA_OPT_ATTN_KERNEL, RA_OPT_ATTN_WAVES = 0, 1
RA_KERNEL_AUTO, RA_KERNEL_ROWMAX = 0, 1

# Every symbol include/ringattn.h declares.
EXPORTED = (
    "ra_abi_version", "ra_set_option", "ra_get_option", "ra_last_error", "ra_padded_len", "ra_shard_range",
    "ra_classify_block", "ra_ring_schedule", "ra_block_attn_fwd",
    "ra_ring_merge", "ra_ring_attn_fwd", "ra_seq2head", "ra_head2seq",
    "ra_zigzag_padded_len", "ra_zigzag_schedule", "ra_zigzag_attn_fwd", "ra_ring_attn_bwd",
    "ra_ring_attn_fwd_gqa", "ra_ring_attn_fwd_varlen", "ra_block_attn_bwd",
    "ra_ring_attn_fwd_split", "ra_ring_split_plan", "ra_zigzag_attn_bwd", "ra_ring_attn_bwd_gqa",
    "ra_ring_attn_bwd_varlen", "ra_ring_attn_fwd_split_noalloc", "ra_block_attn_fwd_acc",
    "ra_lockstep_order",
)

_lib = None


class LibraryMissing(RuntimeError):
    pass


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(
            f"{LIB_PATH} is not built; run `python -m ring_ulysses_sequence_amd.build` "
            "(hipcc for gfx950). There is no CPU fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    c_ll, c_int, c_vp, c_float = ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p, ctypes.c_float
    c_fp = ctypes.POINTER(ctypes.c_float)
    sig = {
        "ra_abi_version": (c_int, []),
        "ra_set_option": (c_int, [c_int, c_int]),
        "ra_get_option": (c_int, [c_int]),
        "ra_last_error": (ctypes.c_char_p, []),
        "ra_padded_len": (c_ll, [c_ll, c_int, c_int]),
        "ra_shard_range": (c_int, [c_ll, c_int, c_int, ctypes.POINTER(c_ll), ctypes.POINTER(c_ll)]),
        "ra_classify_block": (c_int, [c_ll, c_ll, c_ll, c_ll, c_int, c_ll, ctypes.POINTER(c_int)]),
        "ra_ring_schedule": (c_int, [c_int, c_int, c_ll, c_int, c_ll,
                                     ctypes.POINTER(c_int), ctypes.POINTER(c_int)]),
        "ra_block_attn_fwd": (c_int, [c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_int,
                                      c_int, c_float, c_ll, c_ll, c_int, c_ll,
                                      c_vp, c_vp, c_vp, c_vp, c_vp]),
        "ra_block_attn_fwd_acc": (c_int, [c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_int,
                                          c_int, c_float, c_ll, c_ll, c_int, c_ll,
                                          c_vp, c_vp, c_vp, c_vp]),
        "ra_ring_merge": (c_int, [c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int,
                                  c_vp, c_int, c_vp]),
        "ra_ring_attn_fwd": (c_int, [c_vp, ctypes.POINTER(c_vp), ctypes.POINTER(c_vp),
                                     c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                     c_float, c_int, c_ll, c_vp, c_vp, c_vp]),
        "ra_zigzag_padded_len": (c_ll, [c_ll, c_int]),
        "ra_zigzag_schedule": (c_int, [c_int, c_int, c_ll, c_int, c_ll,
                                       ctypes.POINTER(c_int), ctypes.POINTER(c_int)]),
        "ra_zigzag_attn_fwd": (c_int, [c_vp, ctypes.POINTER(c_vp), ctypes.POINTER(c_vp),
                                       c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                       c_float, c_int, c_ll, c_vp, c_vp, c_vp]),
        "ra_ring_attn_fwd_gqa": (c_int, [c_vp, ctypes.POINTER(c_vp), ctypes.POINTER(c_vp),
                                         c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                         c_float, c_int, c_ll, c_vp, c_vp, c_vp]),
        "ra_ring_attn_fwd_varlen": (c_int, [c_vp, ctypes.POINTER(c_vp), ctypes.POINTER(c_vp),
                                            c_int, c_int, c_int, c_int, c_int, c_int, c_float,
                                            c_int, ctypes.POINTER(c_ll), c_int, c_vp, c_vp,
                                            c_vp]),
        "ra_ring_attn_bwd_varlen": (c_int, [c_vp, ctypes.POINTER(c_vp), ctypes.POINTER(c_vp), c_vp,
                                            c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                            c_float, c_int, ctypes.POINTER(c_ll), c_int, c_vp,
                                            ctypes.POINTER(c_vp), ctypes.POINTER(c_vp), c_vp,
                                            c_vp]),
        "ra_ring_attn_bwd_gqa": (c_int, [c_vp, ctypes.POINTER(c_vp), ctypes.POINTER(c_vp), c_vp,
                                         c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                         c_int, c_int, c_float, c_int, c_ll, c_vp,
                                         ctypes.POINTER(c_vp), ctypes.POINTER(c_vp), c_vp, c_vp]),
        "ra_zigzag_attn_bwd": (c_int, [c_vp, ctypes.POINTER(c_vp), ctypes.POINTER(c_vp), c_vp,
                                       c_vp, c_vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                       c_int, c_float, c_int, c_ll, c_vp, ctypes.POINTER(c_vp),
                                       ctypes.POINTER(c_vp), c_vp, c_vp]),
        "ra_ring_attn_bwd": (c_int, [c_vp, ctypes.POINTER(c_vp), ctypes.POINTER(c_vp), c_vp, c_vp,
                                     c_vp, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                     c_float, c_int, c_ll, c_vp, ctypes.POINTER(c_vp),
                                     ctypes.POINTER(c_vp), c_vp, c_vp]),
        "ra_ring_attn_fwd_split": (c_int, [c_vp, ctypes.POINTER(c_vp), ctypes.POINTER(c_vp),
                                           c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                           c_int, c_float, c_int, c_ll, c_int, c_vp, c_ll, c_vp,
                                           c_vp, c_vp]),
        "ra_ring_attn_fwd_split_noalloc": (c_int, [c_vp, ctypes.POINTER(c_vp),
                                                   ctypes.POINTER(c_vp), c_int, c_int, c_int,
                                                   c_int, c_int, c_int, c_int, c_int, c_float,
                                                   c_int, c_ll, c_int, c_vp, c_vp, c_vp]),
        "ra_ring_split_plan": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_ll,
                                       c_int, ctypes.POINTER(c_ll)]),
        "ra_lockstep_order": (c_int, [c_int, c_int, c_int, c_int, ctypes.POINTER(c_int),
                                      ctypes.POINTER(c_int), ctypes.POINTER(c_int)]),
        "ra_block_attn_bwd": (c_int, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int,
                                      c_int, c_int, c_int, c_float, c_ll, c_ll, c_int, c_ll,
                                      c_vp, c_vp, c_vp, c_vp, c_vp]),
        "ra_seq2head": (c_int, [c_vp, c_vp, c_int, c_int, c_ll, c_int, c_int, c_int, c_vp]),
        "ra_head2seq": (c_int, [c_vp, c_vp, c_int, c_int, c_ll, c_int, c_int, c_int, c_vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def lib():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


def _check(status: int, what: str):
    if status == RA_OK:
        return
    msg = _load().ra_last_error().decode(errors="replace")
    if status == RA_ERR_SHAPE:
        raise ValueError(f"{what}: {msg}")
    raise RuntimeError(f"{what}: status {status}: {msg}")


# --------------------------------------------------------------- host helpers
def abi_version() -> int:
    return _load().ra_abi_version()


def set_attn_kernel(choice: int) -> None:
    """How the bf16 kernels keep the row max: RA_KERNEL_AUTO (reference set
    once per row, tiles over the weight bound redone) or RA_KERNEL_ROWMAX
    (row max of every tile)."""
    _check(_load().ra_set_option(RA_OPT_ATTN_KERNEL, choice), "set_attn_kernel")


def get_attn_kernel() -> int:
    return _load().ra_get_option(RA_OPT_ATTN_KERNEL)


def set_attn_waves(waves: int) -> None:
    """Waves per bf16 attention workgroup: 0 (the library's choice), 4 or 8."""
    _check(_load().ra_set_option(RA_OPT_ATTN_WAVES, waves), "set_attn_waves")


def get_attn_waves() -> int:
    return _load().ra_get_option(RA_OPT_ATTN_WAVES)


def padded_len(S: int, P: int, pad_multiple: int = RA_PAD_MULTIPLE) -> int:
    r = _load().ra_padded_len(S, P, pad_multiple)
    if r < 0:
        raise ValueError(_load().ra_last_error().decode())
    return r


def shard_range(S: int, P: int, rank: int):
    b, e = ctypes.c_longlong(), ctypes.c_longlong()
    _check(_load().ra_shard_range(S, P, rank, ctypes.byref(b), ctypes.byref(e)), "shard_range")
    return b.value, e.value


def classify_block(q0: int, q1: int, k0: int, k1: int, causal: bool, valid_len: int = -1) -> int:
    c = ctypes.c_int()
    _check(_load().ra_classify_block(q0, q1, k0, k1, int(causal), valid_len, ctypes.byref(c)),
           "classify_block")
    return c.value


def ring_schedule(P: int, rank: int, block_len: int, causal: bool, valid_len: int = -1):
    """(sources, classes) of rank's ring; sources[t] = (rank - t) mod P."""
    src = (ctypes.c_int * max(P, 1))()
    cls = (ctypes.c_int * max(P, 1))()
    _check(_load().ra_ring_schedule(P, rank, block_len, int(causal), valid_len, src, cls),
           "ring_schedule")
    return list(src)[:P], list(cls)[:P]


def zigzag_padded_len(S: int, P: int) -> int:
    """Smallest multiple of 2P*64 >= S (zigzag chunks of a multiple of 64 rows)."""
    r = _load().ra_zigzag_padded_len(S, P)
    if r < 0:
        raise ValueError(_load().ra_last_error().decode())
    return r


def zigzag_schedule(P: int, rank: int, chunk_len: int, causal: bool, valid_len: int = -1):
    """(sources, classes) of rank's zigzag ring: sources[t] = (rank - t) mod P,
    classes[t] = (class of chunk sources[t], class of chunk 2P-1-sources[t])."""
    src = (ctypes.c_int * max(P, 1))()
    cls = (ctypes.c_int * max(2 * P, 2))()
    _check(_load().ra_zigzag_schedule(P, rank, chunk_len, int(causal), valid_len, src, cls),
           "zigzag_schedule")
    return list(src)[:P], [(cls[2 * t], cls[2 * t + 1]) for t in range(P)]


# --------------------------------------------------------------- device calls
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return RA_BF16
    if t.dtype == torch.float32:
        return RA_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _dev(t, name, like=None):
    """Device pointer of a contiguous GPU tensor; with ``like``, the tensor
    must also sit on like's device."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if like is not None and t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, expected {like.device}")
    return ctypes.c_void_p(t.data_ptr())


def _out(t, name, shape, dtype, like):
    """Check a caller-supplied output buffer before the library writes into
    it: the C ABI cannot see buffer sizes, so a wrong shape or dtype would
    mean writes past its end."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {tuple(shape)} of {dtype}, got "
                         f"{tuple(t.shape)} of {t.dtype}")
    return _dev(t, name, like)


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class _on:
    """Make the launch stream current while temporaries and default outputs
    are allocated (and zero-filled), so the caching allocator ties them to
    the stream the kernels run on and the fills are ordered before them."""

    def __init__(self, stream):
        self.stream = stream
        self.ctx = None

    def __enter__(self):
        if self.stream is not None:
            self.ctx = _torch().cuda.stream(self.stream)
            self.ctx.__enter__()
        return self

    def __exit__(self, *exc):
        if self.ctx is not None:
            self.ctx.__exit__(*exc)
        return False


def block_attn_fwd(q, k, v, *, scale: float = 0.0, q_pos0: int = 0, k_pos0: int = 0,
                   causal: bool = False, valid_len: int = -1, want_ml: bool = True,
                   out=None, stream=None):
    """One ring round: (o fp32 [B,Sq,H,D], lse, m, l [B,Sq,H]) of q over one block."""
    torch = _torch()
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if k.shape != (B, Sk, H, D) or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    dt = _dtype_code(q)
    if out is None:
        with _on(stream):
            o = torch.empty((B, Sq, H, D), dtype=torch.float32, device=q.device)
            lse = torch.empty((B, Sq, H), dtype=torch.float32, device=q.device)
            m = torch.empty_like(lse) if want_ml else None
            l = torch.empty_like(lse) if want_ml else None
    else:
        o, lse, m, l = out
    f32, row = torch.float32, (B, Sq, H)
    st = _load().ra_block_attn_fwd(
        _dev(q, "q"), _dev(k, "k", q), _dev(v, "v", q), B, Sq, Sk, H, D, dt, float(scale),
        q_pos0, k_pos0, int(causal), valid_len, _out(o, "o", (B, Sq, H, D), f32, q),
        _out(lse, "lse", row, f32, q),
        _out(m, "m", row, f32, q) if m is not None else None,
        _out(l, "l", row, f32, q) if l is not None else None,
        _stream(stream))
    _check(st, "ra_block_attn_fwd")
    return o, lse, m, l


def block_attn_fwd_acc(q, k, v, o_acc, lse_acc, *, scale: float = 0.0, q_pos0: int = 0,
                       k_pos0: int = 0, causal: bool = False, valid_len: int = -1,
                       out_final=None, stream=None):
    """One ring round folded into the running partial (o_acc fp32 [B,Sq,H,D],
    lse_acc [B,Sq,H]) in the same launch; with ``out_final`` (q's dtype and
    shape) the combined output goes there and o_acc is left as it was.
    Returns (o_acc, lse_acc) or (out_final, lse_acc)."""
    torch = _torch()
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if k.shape != (B, Sk, H, D) or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    dt = _dtype_code(q)
    f32, row = torch.float32, (B, Sq, H)
    st = _load().ra_block_attn_fwd_acc(
        _dev(q, "q"), _dev(k, "k", q), _dev(v, "v", q), B, Sq, Sk, H, D, dt, float(scale),
        q_pos0, k_pos0, int(causal), valid_len, _out(o_acc, "o_acc", (B, Sq, H, D), f32, q),
        _out(lse_acc, "lse_acc", row, f32, q),
        _out(out_final, "out_final", (B, Sq, H, D), q.dtype, q) if out_final is not None
        else None,
        _stream(stream))
    _check(st, "ra_block_attn_fwd_acc")
    return (o_acc if out_final is None else out_final), lse_acc


def ring_merge(o_acc, lse_acc, o_blk, lse_blk, *, out_final=None, stream=None):
    """In-place LSE combine of (o_blk, lse_blk) into (o_acc, lse_acc)."""
    torch = _torch()
    B, Sq, H, D = o_acc.shape
    for t, n in ((o_acc, "o_acc"), (o_blk, "o_blk"), (lse_acc, "lse_acc"), (lse_blk, "lse_blk")):
        if t.dtype != torch.float32:
            raise TypeError(f"{n} must be fp32")
    if o_blk.shape != o_acc.shape or lse_acc.shape != (B, Sq, H) or lse_blk.shape != (B, Sq, H):
        raise ValueError("merge operands have inconsistent shapes")
    fdt = RA_FP32
    fptr = None
    if out_final is not None:
        if out_final.shape != o_acc.shape:
            raise ValueError("out_final shape mismatch")
        fdt = _dtype_code(out_final)
        fptr = _dev(out_final, "out_final")
    if out_final is not None:
        _dev(out_final, "out_final", o_acc)
    st = _load().ra_ring_merge(_dev(o_acc, "o_acc"), _dev(lse_acc, "lse_acc", o_acc),
                               _dev(o_blk, "o_blk", o_acc), _dev(lse_blk, "lse_blk", o_acc),
                               B, Sq, H, D, fptr, fdt, _stream(stream))
    _check(st, "ra_ring_merge")
    return o_acc, lse_acc


def ring_split_plan(B: int, Sb: int, H: int, D: int, P: int, rank: int, causal: bool = False,
                    valid_len: int = -1, nsplit: int = 0):
    """(runs per query tile, workspace floats) of the split ring for this
    share; 1 run means the single pass (see ra_ring_split_plan)."""
    ws = ctypes.c_longlong(0)
    n = _load().ra_ring_split_plan(B, Sb, H, D, P, rank, int(causal), valid_len,
                                   int(nsplit), ctypes.byref(ws))
    if n < 0:
        raise ValueError(_load().ra_last_error().decode())
    return n, ws.value


def lockstep_order(Q: int, BH: int, later_rot: int = 1):
    """The lockstep workgroup order of the 8-wave kernels for Q query tiles
    of 256 rows times BH (batch, head) problems (see ra_lockstep_order):
    (applies, bh[id], qt[id], rot[id]) over the dispatch index id, the lists
    meaningful only when it applies."""
    n = Q * BH
    arr = ctypes.c_int * max(n, 1)
    bh, qt, rot = arr(), arr(), arr()
    st = _load().ra_lockstep_order(n, Q, BH, later_rot, bh, qt, rot)
    if st < 0:
        raise ValueError(_load().ra_last_error().decode())
    return st == 1, list(bh)[:n], list(qt)[:n], list(rot)[:n]


def ring_attn_fwd(q_r, k_blocks: Sequence, v_blocks: Sequence, rank: int, *,
                  causal: bool = False, valid_len: int = -1, scale: float = 0.0,
                  want_lse: bool = True, out=None, lse_out=None, stream=None, split=None):
    """Rank ``rank``'s whole ring: (o [B,Sb,H,D] in q's dtype, lse).
    K/V blocks with fewer heads than q_r (a divisor of H) select the grouped-query
    form: query head h reads K/V head h / (H / H_kv).  ``split``: runs per
    query tile of the split ring (None: ra_ring_split_plan's choice for bf16,
    1: the single pass)."""
    torch = _torch()
    B, Sb, H, D = q_r.shape
    P = len(k_blocks)
    if len(v_blocks) != P:
        raise ValueError("k_blocks and v_blocks differ in length")
    if P > RA_MAX_P:
        raise RuntimeError(f"P={P} exceeds {RA_MAX_P}")
    dt = _dtype_code(q_r)
    Hkv = k_blocks[0].shape[2] if P else H
    kv_shape = (B, Sb, Hkv, D)
    kp = (ctypes.c_void_p * max(P, 1))()
    vp = (ctypes.c_void_p * max(P, 1))()
    for j in range(P):
        for t, n in ((k_blocks[j], "k"), (v_blocks[j], "v")):
            if tuple(t.shape) != kv_shape or t.dtype != q_r.dtype:
                raise ValueError(f"{n}_blocks[{j}] must be {kv_shape} of q_r's dtype")
        kp[j] = _dev(k_blocks[j], f"k_blocks[{j}]", q_r).value
        vp[j] = _dev(v_blocks[j], f"v_blocks[{j}]", q_r).value
    with _on(stream):
        o = torch.empty_like(q_r) if out is None else out
        lse = lse_out
        if lse is None and want_lse:
            lse = torch.empty((B, Sb, H), dtype=torch.float32, device=q_r.device)
    args = (float(scale), int(causal), valid_len, _out(o, "out", q_r.shape, q_r.dtype, q_r),
            _out(lse, "lse_out", (B, Sb, H), torch.float32, q_r) if lse is not None else None,
            _stream(stream))
    if split is not None and split < 1:
        raise ValueError(f"split must be >= 1 (got {split})")
    runs, ws_floats = 1, 0
    if dt == RA_BF16 and split != 1:
        runs, ws_floats = ring_split_plan(B, Sb, H, D, P, rank, causal, valid_len, split or 0)
    if runs > 1:
        with _on(stream):
            ws = torch.empty(ws_floats, dtype=torch.float32, device=q_r.device)
        st = _load().ra_ring_attn_fwd_split(_dev(q_r, "q_r"), kp, vp, B, Sb, H, Hkv, D, P, rank,
                                            dt, float(scale), int(causal), valid_len, runs,
                                            _dev(ws, "ws"), ws_floats, *args[3:])
        _check(st, "ra_ring_attn_fwd_split")
    elif Hkv == H:
        st = _load().ra_ring_attn_fwd(_dev(q_r, "q_r"), kp, vp, B, Sb, H, D, P, rank, dt, *args)
        _check(st, "ra_ring_attn_fwd")
    else:
        st = _load().ra_ring_attn_fwd_gqa(_dev(q_r, "q_r"), kp, vp, B, Sb, H, Hkv, D, P, rank,
                                          dt, *args)
        _check(st, "ra_ring_attn_fwd_gqa")
    return o, lse


def ring_attn_fwd_split_noalloc(q_r, k_blocks: Sequence, v_blocks: Sequence, rank: int, out,
                                lse_out=None, *, causal: bool = False, valid_len: int = -1,
                                scale: float = 0.0, nsplit: int = 0, stream=None):
    """The split ring with its partials in the library's fixed device
    scratch (ra_ring_attn_fwd_split_noalloc): nothing is allocated, so the
    caller passes ``out`` (q_r's shape and dtype) and, optionally,
    ``lse_out`` (fp32 [B, Sb, H]).  Calls on one GPU share the scratch and
    must not overlap.  Returns (out, lse_out)."""
    torch = _torch()
    B, Sb, H, D = q_r.shape
    P = len(k_blocks)
    if len(v_blocks) != P:
        raise ValueError("k_blocks and v_blocks differ in length")
    if P > RA_MAX_P:
        raise RuntimeError(f"P={P} exceeds {RA_MAX_P}")
    dt = _dtype_code(q_r)
    Hkv = k_blocks[0].shape[2] if P else H
    kv_shape = (B, Sb, Hkv, D)
    kp = (ctypes.c_void_p * max(P, 1))()
    vp = (ctypes.c_void_p * max(P, 1))()
    for j in range(P):
        for t, n in ((k_blocks[j], "k"), (v_blocks[j], "v")):
            if tuple(t.shape) != kv_shape or t.dtype != q_r.dtype:
                raise ValueError(f"{n}_blocks[{j}] must be {kv_shape} of q_r's dtype")
        kp[j] = _dev(k_blocks[j], f"k_blocks[{j}]", q_r).value
        vp[j] = _dev(v_blocks[j], f"v_blocks[{j}]", q_r).value
    st = _load().ra_ring_attn_fwd_split_noalloc(
        _dev(q_r, "q_r"), kp, vp, B, Sb, H, Hkv, D, P, rank, dt, float(scale), int(causal),
        valid_len, int(nsplit), _out(out, "out", q_r.shape, q_r.dtype, q_r),
        _out(lse_out, "lse_out", (B, Sb, H), torch.float32, q_r) if lse_out is not None else None,
        _stream(stream))
    _check(st, "ra_ring_attn_fwd_split_noalloc")
    return out, lse_out


def ring_attn_fwd_varlen(q_r, k_blocks: Sequence, v_blocks: Sequence, rank: int,
                         cu_seqlens: Sequence, *, causal: bool = True, scale: float = 0.0,
                         want_lse: bool = True, out=None, lse_out=None, stream=None):
    """Rank ``rank``'s ring over a packed sequence (B = 1): sample i holds
    global positions [cu_seqlens[i], cu_seqlens[i+1]) and attends only within
    itself.  Returns (o, lse); rows outside every sample are left as allocated
    (zero-filled here when the outputs are not given)."""
    torch = _torch()
    B, Sb, H, D = q_r.shape
    if B != 1:
        raise ValueError("packed sequences need B = 1")
    P = len(k_blocks)
    if len(v_blocks) != P:
        raise ValueError("k_blocks and v_blocks differ in length")
    if P > RA_MAX_P:
        raise RuntimeError(f"P={P} exceeds {RA_MAX_P}")
    dt = _dtype_code(q_r)
    kp = (ctypes.c_void_p * max(P, 1))()
    vp = (ctypes.c_void_p * max(P, 1))()
    for j in range(P):
        for t, n in ((k_blocks[j], "k"), (v_blocks[j], "v")):
            if t.shape != q_r.shape or t.dtype != q_r.dtype:
                raise ValueError(f"{n}_blocks[{j}] must match q_r in shape and dtype")
        kp[j] = _dev(k_blocks[j], f"k_blocks[{j}]", q_r).value
        vp[j] = _dev(v_blocks[j], f"v_blocks[{j}]", q_r).value
    with _on(stream):
        o = torch.zeros_like(q_r) if out is None else out
        lse = lse_out
        if lse is None and want_lse:
            lse = torch.full((B, Sb, H), float("-inf"), dtype=torch.float32, device=q_r.device)
    n = len(cu_seqlens) - 1
    cu = (ctypes.c_longlong * max(n + 1, 1))(*[int(x) for x in cu_seqlens])
    st = _load().ra_ring_attn_fwd_varlen(
        _dev(q_r, "q_r"), kp, vp, Sb, H, D, P, rank, dt, float(scale), int(causal), cu,
        max(n, 0), _out(o, "out", q_r.shape, q_r.dtype, q_r),
        _out(lse, "lse_out", (B, Sb, H), torch.float32, q_r) if lse is not None else None,
        _stream(stream))
    _check(st, "ra_ring_attn_fwd_varlen")
    return o, lse


def zigzag_attn_fwd(q_r, k_shares: Sequence, v_shares: Sequence, rank: int, *,
                    causal: bool = True, valid_len: int = -1, scale: float = 0.0,
                    want_lse: bool = True, out=None, lse_out=None, stream=None):
    """Rank ``rank``'s whole ring over zigzag shares in one launch.  q_r and
    every share are [B, Sr, H, D]: chunk r then chunk 2P-1-r of the sequence.
    Returns (o [B,Sr,H,D] in q's dtype, lse [B,Sr,H] fp32)."""
    torch = _torch()
    B, Sr, H, D = q_r.shape
    P = len(k_shares)
    if len(v_shares) != P:
        raise ValueError("k_shares and v_shares differ in length")
    if 2 * P > RA_MAX_P:
        raise RuntimeError(f"P={P} exceeds {RA_MAX_P // 2}")
    dt = _dtype_code(q_r)
    kp = (ctypes.c_void_p * max(P, 1))()
    vp = (ctypes.c_void_p * max(P, 1))()
    for j in range(P):
        for t, n in ((k_shares[j], "k"), (v_shares[j], "v")):
            if t.shape != q_r.shape or t.dtype != q_r.dtype:
                raise ValueError(f"{n}_shares[{j}] must match q_r in shape and dtype")
        kp[j] = _dev(k_shares[j], f"k_shares[{j}]", q_r).value
        vp[j] = _dev(v_shares[j], f"v_shares[{j}]", q_r).value
    with _on(stream):
        o = torch.empty_like(q_r) if out is None else out
        lse = lse_out
        if lse is None and want_lse:
            lse = torch.empty((B, Sr, H), dtype=torch.float32, device=q_r.device)
    st = _load().ra_zigzag_attn_fwd(
        _dev(q_r, "q_r"), kp, vp, B, Sr, H, D, P, rank, dt, float(scale), int(causal),
        valid_len, _out(o, "out", q_r.shape, q_r.dtype, q_r),
        _out(lse, "lse_out", (B, Sr, H), torch.float32, q_r) if lse is not None else None,
        _stream(stream))
    _check(st, "ra_zigzag_attn_fwd")
    return o, lse


def block_attn_bwd(q, k, v, o, do, lse, *, scale: float = 0.0, q_pos0: int = 0,
                   k_pos0: int = 0, causal: bool = False, valid_len: int = -1,
                   dq=None, dk=None, dv=None, stream=None):
    """Backward of one round: accumulates this K/V block's gradient terms
    into (dq [B,Sq,H,D], dk, dv [B,Sk,H,D]) (fp32, zero-initialised when not
    given), with ``lse`` the natural log-sum-exp of the whole forward.
    Returns (dq, dk, dv)."""
    torch = _torch()
    B, Sq, H, D = q.shape
    Sk = k.shape[1]
    if k.shape != (B, Sk, H, D) or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == do.dtype):
        raise TypeError("q, k, v, o, do must share a dtype")
    if o.shape != q.shape or do.shape != q.shape:
        raise ValueError("o and do must match q in shape")
    if lse.shape != (B, Sq, H) or lse.dtype != torch.float32:
        raise ValueError("lse must be fp32 [B, Sq, H]")
    dt = _dtype_code(q)
    f32 = dict(dtype=torch.float32, device=q.device)
    with _on(stream):
        dq = torch.zeros(q.shape, **f32) if dq is None else dq
        dk = torch.zeros(k.shape, **f32) if dk is None else dk
        dv = torch.zeros(k.shape, **f32) if dv is None else dv
        stats = torch.empty((2, B, H, Sq), **f32)
    for t, n, shp in ((dq, "dq", q.shape), (dk, "dk", k.shape), (dv, "dv", k.shape)):
        _out(t, n, shp, torch.float32, q)
    st = _load().ra_block_attn_bwd(
        _dev(q, "q"), _dev(k, "k", q), _dev(v, "v", q), _dev(o, "o", q), _dev(do, "do", q),
        _dev(lse, "lse", q), B, Sq, Sk, H, D, dt, float(scale), q_pos0, k_pos0, int(causal),
        valid_len, _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"), _dev(stats, "stats"),
        _stream(stream))
    _check(st, "ra_block_attn_bwd")
    return dq, dk, dv


def ring_attn_bwd(q_r, k_blocks: Sequence, v_blocks: Sequence, o_r, do_r, lse_r, rank: int, *,
                  causal: bool = False, valid_len: int = -1, scale: float = 0.0,
                  dq=None, dk_blocks=None, dv_blocks=None, stream=None):
    """Backward of rank ``rank``'s ring: accumulates into (dq [B,Sb,H,D],
    dk_blocks[j], dv_blocks[j]) (fp32, zero-initialised when not given) the
    gradients of the rank's queries and of the blocks it visits.  K/V blocks
    with fewer heads than q_r select the grouped-query form.  Returns
    (dq, dk_blocks, dv_blocks)."""
    return _ring_bwd("ra_ring_attn_bwd", q_r, k_blocks, v_blocks, o_r, do_r, lse_r, rank,
                     causal, valid_len, scale, dq, dk_blocks, dv_blocks, stream)


def zigzag_attn_bwd(q_r, k_shares: Sequence, v_shares: Sequence, o_r, do_r, lse_r, rank: int, *,
                    causal: bool = True, valid_len: int = -1, scale: float = 0.0,
                    dq=None, dk_shares=None, dv_shares=None, stream=None):
    """Backward of rank ``rank``'s zigzag ring (shares as in zigzag_attn_fwd):
    accumulates into (dq [B,Sr,H,D], dk_shares[j], dv_shares[j]) (fp32,
    zero-initialised when not given).  Returns (dq, dk_shares, dv_shares)."""
    return _ring_bwd("ra_zigzag_attn_bwd", q_r, k_shares, v_shares, o_r, do_r, lse_r, rank,
                     causal, valid_len, scale, dq, dk_shares, dv_shares, stream)


def ring_attn_bwd_varlen(q_r, k_blocks: Sequence, v_blocks: Sequence, o_r, do_r, lse_r,
                         rank: int, cu_seqlens: Sequence, *, causal: bool = True,
                         scale: float = 0.0, dq=None, dk_blocks=None, dv_blocks=None,
                         stream=None):
    """Backward over packed samples (B = 1; see ring_attn_fwd_varlen):
    accumulates into (dq, dk_blocks[j], dv_blocks[j]) (fp32, zero-initialised
    when not given).  Returns (dq, dk_blocks, dv_blocks)."""
    torch = _torch()
    B, Sb, H, D = q_r.shape
    if B != 1:
        raise ValueError("packed samples need B = 1")
    P = len(k_blocks)
    dt = _dtype_code(q_r)
    f32 = dict(dtype=torch.float32, device=q_r.device)
    with _on(stream):
        dq = torch.zeros(q_r.shape, **f32) if dq is None else dq
        dk_blocks = ([torch.zeros(q_r.shape, **f32) for _ in range(P)] if dk_blocks is None
                     else dk_blocks)
        dv_blocks = ([torch.zeros(q_r.shape, **f32) for _ in range(P)] if dv_blocks is None
                     else dv_blocks)
        stats = torch.empty((2, 1, H, Sb), **f32)
    if len(dk_blocks) != P or len(dv_blocks) != P or len(v_blocks) != P:
        raise ValueError("v_blocks, dk_blocks and dv_blocks must hold one buffer per K block")
    for t, n in ((o_r, "o_r"), (do_r, "do_r")):
        if t.shape != q_r.shape or t.dtype != q_r.dtype:
            raise ValueError(f"{n} must match q_r in shape and dtype")
    if lse_r.shape != (1, Sb, H) or lse_r.dtype != torch.float32:
        raise ValueError("lse_r must be fp32 [1, Sb, H]")
    if dq.shape != q_r.shape or dq.dtype != torch.float32:
        raise ValueError("dq must be fp32 of q_r's shape")
    arrs = [(ctypes.c_void_p * max(P, 1))() for _ in range(4)]
    for j in range(P):
        for t, n in ((k_blocks[j], "k"), (v_blocks[j], "v")):
            if t.shape != q_r.shape or t.dtype != q_r.dtype:
                raise ValueError(f"{n}_blocks[{j}] must match q_r in shape and dtype")
        for t, n in ((dk_blocks[j], "dk"), (dv_blocks[j], "dv")):
            if t.shape != q_r.shape or t.dtype != torch.float32:
                raise ValueError(f"{n}_blocks[{j}] must be fp32 of q_r's shape")
        for arr, t, n in zip(arrs, (k_blocks[j], v_blocks[j], dk_blocks[j], dv_blocks[j]),
                             ("k", "v", "dk", "dv")):
            arr[j] = _dev(t, f"{n}_blocks[{j}]", q_r).value
    _dev(dq, "dq", q_r)
    cu = list(cu_seqlens)
    table = (ctypes.c_longlong * max(len(cu), 1))(*cu)
    st = _load().ra_ring_attn_bwd_varlen(_dev(q_r, "q_r"), arrs[0], arrs[1], _dev(o_r, "o_r", q_r),
                                         _dev(do_r, "do_r", q_r), _dev(lse_r, "lse_r", q_r),
                                         Sb, H, D, P,
                                         rank, dt, float(scale), int(causal), table,
                                         len(cu) - 1, _dev(dq, "dq"), arrs[2], arrs[3],
                                         _dev(stats, "stats"), _stream(stream))
    _check(st, "ra_ring_attn_bwd_varlen")
    return dq, dk_blocks, dv_blocks


def _ring_bwd(fn_name, q_r, k_blocks, v_blocks, o_r, do_r, lse_r, rank, causal, valid_len,
              scale, dq, dk_blocks, dv_blocks, stream):
    torch = _torch()
    B, Sb, H, D = q_r.shape
    P = len(k_blocks)
    if len(v_blocks) != P:
        raise ValueError("k_blocks and v_blocks differ in length")
    if P > RA_MAX_P:
        raise RuntimeError(f"P={P} exceeds {RA_MAX_P}")
    dt = _dtype_code(q_r)
    Hkv = k_blocks[0].shape[2] if P else H
    kv_shape = (B, Sb, Hkv, D)
    for t, n in ((o_r, "o_r"), (do_r, "do_r")):
        if t.shape != q_r.shape or t.dtype != q_r.dtype:
            raise ValueError(f"{n} must match q_r in shape and dtype")
    if lse_r.shape != (B, Sb, H) or lse_r.dtype != torch.float32:
        raise ValueError("lse_r must be fp32 [B, Sb, H]")
    f32 = dict(dtype=torch.float32, device=q_r.device)
    with _on(stream):
        dq = torch.zeros(q_r.shape, **f32) if dq is None else dq
        dk_blocks = ([torch.zeros(kv_shape, **f32) for _ in range(P)] if dk_blocks is None
                     else dk_blocks)
        dv_blocks = ([torch.zeros(kv_shape, **f32) for _ in range(P)] if dv_blocks is None
                     else dv_blocks)
        stats = torch.empty((2, B, H, Sb), **f32)
    if len(dk_blocks) != P or len(dv_blocks) != P:
        raise ValueError("dk and dv buffers must hold one buffer per K block")
    kp = (ctypes.c_void_p * max(P, 1))()
    vp = (ctypes.c_void_p * max(P, 1))()
    dkp = (ctypes.c_void_p * max(P, 1))()
    dvp = (ctypes.c_void_p * max(P, 1))()
    for j in range(P):
        for t, n in ((k_blocks[j], "k"), (v_blocks[j], "v")):
            if tuple(t.shape) != kv_shape or t.dtype != q_r.dtype:
                raise ValueError(f"{n}_blocks[{j}] must be {kv_shape} of q_r's dtype")
        for t, n in ((dk_blocks[j], "dk"), (dv_blocks[j], "dv")):
            if tuple(t.shape) != kv_shape or t.dtype != torch.float32:
                raise ValueError(f"{n}_blocks[{j}] must be fp32 {kv_shape}")
        kp[j] = _dev(k_blocks[j], f"k_blocks[{j}]", q_r).value
        vp[j] = _dev(v_blocks[j], f"v_blocks[{j}]", q_r).value
        dkp[j] = _dev(dk_blocks[j], f"dk_blocks[{j}]", q_r).value
        dvp[j] = _dev(dv_blocks[j], f"dv_blocks[{j}]", q_r).value
    _out(dq, "dq", q_r.shape, torch.float32, q_r)
    head = (B, Sb, H, D, P, rank) if Hkv == H else (B, Sb, H, Hkv, D, P, rank)
    if Hkv != H:
        if fn_name != "ra_ring_attn_bwd":
            raise ValueError("grouped-query K/V heads are supported by the ring backward only")
        fn_name = "ra_ring_attn_bwd_gqa"
    st = getattr(_load(), fn_name)(_dev(q_r, "q_r"), kp, vp, _dev(o_r, "o_r", q_r),
                                   _dev(do_r, "do_r", q_r), _dev(lse_r, "lse_r", q_r), *head,
                                   dt, float(scale),
                                   int(causal), valid_len, _dev(dq, "dq"), dkp, dvp,
                                   _dev(stats, "stats"), _stream(stream))
    _check(st, fn_name)
    return dq, dk_blocks, dv_blocks


def _perm(fn_name, x, out_shape, P, B, S, H, D, out, stream):
    torch = _torch()
    with _on(stream):
        y = torch.empty(out_shape, dtype=x.dtype, device=x.device) if out is None else out
    st = getattr(_load(), fn_name)(_dev(x, "src"), _out(y, "out", out_shape, x.dtype, x),
                                   P, B, S, H, D,
                                   x.element_size(), _stream(stream))
    _check(st, fn_name)
    return y


def seq2head(x, *, out=None, stream=None):
    """[P, B, S/P, H, D] -> [P, B, S, H/P, D] (bit copy)."""
    P, B, Sl, H, D = x.shape
    if H % P:
        raise ValueError(f"head count H={H} is not divisible by P={P}")
    return _perm("ra_seq2head", x, (P, B, Sl * P, H // P, D), P, B, Sl * P, H, D, out, stream)


def head2seq(x, *, out=None, stream=None):
    """[P, B, S, H/P, D] -> [P, B, S/P, H, D] (bit copy)."""
    P, B, S, Hl, D = x.shape
    if S % P:
        raise ValueError(f"sequence length {S} is not divisible by P={P}")
    return _perm("ra_head2seq", x, (P, B, S // P, Hl * P, D), P, B, S, Hl * P, D, out, stream)


def ring_attn_composable(q_r, k_blocks, v_blocks, rank: int, *, causal: bool = False,
                         valid_len: int = -1, scale: float = 0.0, stream=None):
    """The same ring as ``ring_attn_fwd`` done round by round: the first
    visited block by ``block_attn_fwd``, every later one folded into that
    partial by ``block_attn_fwd_acc`` in its own launch (the last one writing
    the output in q's dtype).  With a single visited block (or none) the
    output is written by folding in an empty block."""
    torch = _torch()
    B, Sb, H, D = q_r.shape
    P = len(k_blocks)
    srcs, classes = ring_schedule(P, rank, Sb, causal, valid_len)
    visit = [j for j, c in zip(srcs, classes) if c != RA_SKIP]
    with _on(stream):
        final = torch.empty_like(q_r)
    kw = dict(scale=scale, q_pos0=rank * Sb, causal=causal, valid_len=valid_len,
              stream=stream)
    empty = q_r[:, :0]
    first = visit[0] if visit else None
    o_acc, lse_acc, _, _ = (
        block_attn_fwd(q_r, k_blocks[first], v_blocks[first], k_pos0=first * Sb,
                       want_ml=False, **kw) if first is not None
        else block_attn_fwd(q_r, empty, empty, want_ml=False, **kw))
    rest = visit[1:]
    if not rest:
        block_attn_fwd_acc(q_r, empty, empty, o_acc, lse_acc, out_final=final, **kw)
        return final, lse_acc
    for n, j in enumerate(rest):
        block_attn_fwd_acc(q_r, k_blocks[j], v_blocks[j], o_acc, lse_acc, k_pos0=j * Sb,
                           out_final=final if n == len(rest) - 1 else None, **kw)
    return final, lse_acc


__all__ = [
    "lib", "abi_version", "set_attn_kernel", "get_attn_kernel", "set_attn_waves",
    "get_attn_waves", "padded_len", "shard_range", "classify_block", "ring_schedule",
    "block_attn_fwd", "block_attn_fwd_acc", "ring_merge", "ring_attn_fwd", "seq2head", "head2seq",
    "zigzag_padded_len", "zigzag_schedule", "zigzag_attn_fwd", "ring_attn_bwd",
    "ring_attn_fwd_varlen", "ring_attn_fwd_split_noalloc",
    "ring_attn_composable", "block_attn_bwd", "ring_split_plan", "zigzag_attn_bwd", "ring_attn_bwd_varlen",
    "EXPORTED", "LIB_PATH", "LibraryMissing",
    "RA_BF16", "RA_FP32", "RA_SKIP", "RA_FULL", "RA_DIAG", "RA_MAX_P", "RA_PAD_MULTIPLE",
    "RA_KERNEL_AUTO", "RA_KERNEL_ROWMAX", "RA_OPT_ATTN_WAVES",
]

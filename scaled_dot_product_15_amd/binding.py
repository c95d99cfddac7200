"""ctypes binding of libsdpa_mi355x.so (declared in include/sdpa_attn.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.  If
the library is missing this module raises; it never falls back to another
implementation.

Names follow the pages' module arguments (TransformerEngine "JAX: Single-GPU
Attention" sections 2 and 4 and "Other attention knobs"; PR #2225
softmax_type / softmax_offset).
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsdpa_mi355x.so")

ATTN_F32, ATTN_BF16, ATTN_FP8 = 0, 1, 2
FP8_FORMATS = {"e4m3": 0, "e5m2": 1}
MASKS = {"no_mask": 0, "none": 0, "causal": 1}
SOFTMAX = {"vanilla": 0, "off_by_one": 1, "learnable": 2}
STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "workspace", -4: "hip error",
          -5: "too large for the allocation-free scratch"}
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024  # ATTN_NOALLOC_SCRATCH_BYTES

_c_i32 = ctypes.c_int32
_vp = ctypes.c_void_p


class Params(ctypes.Structure):
    _fields_ = [("batch", _c_i32), ("seqlen", _c_i32), ("num_heads", _c_i32),
                ("num_gqa_groups", _c_i32), ("head_dim_qk", _c_i32), ("head_dim_v", _c_i32),
                ("dtype", _c_i32), ("mask_type", _c_i32), ("window_left", _c_i32),
                ("window_right", _c_i32), ("scale_factor", ctypes.c_float),
                ("softmax_type", _c_i32), ("dropout_p", ctypes.c_float),
                ("dropout_seed_lo", ctypes.c_uint32), ("dropout_seed_hi", ctypes.c_uint32),
                ("dropout_offset", ctypes.c_uint32)]


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({STATUS.get(status, 'unknown')})")


EXPORTS = {
    "attn_validate": (ctypes.c_int, [ctypes.POINTER(Params)]),
    "attn_fwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Params)]),
    "attn_bwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Params)]),
    "attn_bwd_ds_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Params)]),
    "attn_fwd": (ctypes.c_int, [ctypes.POINTER(Params), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                ctypes.c_size_t, _vp]),
    "attn_bwd": (ctypes.c_int, [ctypes.POINTER(Params), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "attn_bwd_stage": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(Params), _vp, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "attn_fwd_bias": (ctypes.c_int, [ctypes.POINTER(Params), _vp, _vp, _vp, _vp, _c_i32, _c_i32, _vp, _vp, _vp,
                                     _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "attn_bwd_bias": (ctypes.c_int, [ctypes.POINTER(Params), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32,
                                     _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "attn_bwd_noalloc": (ctypes.c_int, [ctypes.POINTER(Params), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _vp, _vp, _vp, _vp, _vp]),
    "attn_fwd_fp8": (ctypes.c_int, [ctypes.POINTER(Params), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    ctypes.c_size_t, _vp]),
    "attn_bwd_fp8": (ctypes.c_int, [ctypes.POINTER(Params), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "attn_fp8_quantize": (ctypes.c_int, [_vp, _c_i32, ctypes.c_size_t, _c_i32, _vp, _vp, _vp, _vp]),
    "attn_fp8_update_scale": (ctypes.c_int, [_vp, _c_i32, _vp, _c_i32, _c_i32, _vp, _vp, _vp]),
    "attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "attn_fwd_tile_shape": (ctypes.c_int, [ctypes.POINTER(Params), ctypes.POINTER(_c_i32),
                                           ctypes.POINTER(_c_i32)]),
    "attn_debug_tile_map": (ctypes.c_int, [ctypes.POINTER(Params), _vp, _c_i32, _c_i32, _vp, _vp]),
    "attn_debug_mask_probe": (ctypes.c_int, [ctypes.POINTER(Params), _vp, _vp, _vp]),
    "attn_debug_dropout_mask": (ctypes.c_int, [ctypes.POINTER(Params), _vp, _vp]),
    "attn_host_tile_map": (ctypes.c_int, [ctypes.POINTER(Params), _vp, _c_i32, _c_i32, _vp]),
    "attn_host_key_range": (ctypes.c_int, [ctypes.POINTER(Params), _c_i32, _c_i32, _c_i32,
                                           ctypes.POINTER(_c_i32), ctypes.POINTER(_c_i32)]),
    "attn_host_query_range": (ctypes.c_int, [ctypes.POINTER(Params), _c_i32, _c_i32, _c_i32,
                                             ctypes.POINTER(_c_i32), ctypes.POINTER(_c_i32)]),
    "attn_host_full_key_tiles": (ctypes.c_int, [ctypes.POINTER(Params), _c_i32, _c_i32, _c_i32, _c_i32,
                                                ctypes.POINTER(_c_i32), ctypes.POINTER(_c_i32)]),
    "attn_host_dkdv_splits": (ctypes.c_int, [ctypes.POINTER(Params)]),
}

_lib = None


def load_library(path: str | None = None):
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m scaled_dot_product_15_amd.build` (there is no fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


def make_params(B, S, Hq, Hkv, d_qk, d_v, dtype="bf16", attn_mask_type="causal",
                window_size=(-1, -1), scale_factor=None, softmax_type="vanilla", dropout_p=0.0,
                rng_state=(0, 0)) -> Params:
    """rng_state = (seed, offset): the 64-bit generator key and the 32-bit
    counter word of attention dropout (same values for forward and backward)."""
    seed, offset = (int(x) for x in rng_state)
    return Params(B, S, Hq, Hkv, d_qk, d_v, {"bf16": ATTN_BF16, "f32": ATTN_F32, "fp8": ATTN_FP8}[dtype],
                  MASKS[attn_mask_type], int(window_size[0]), int(window_size[1]),
                  float(scale_factor or 0.0), SOFTMAX[softmax_type], float(dropout_p),
                  seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF, offset & 0xFFFFFFFF)


def _check(rc, where):
    if rc != 0:
        raise AttnError(rc, where)


def attn_validate(p: Params) -> int:
    return load_library().attn_validate(ctypes.byref(p))


def attn_fwd_workspace_size(p: Params) -> int:
    return load_library().attn_fwd_workspace_size(ctypes.byref(p))


def attn_bwd_workspace_size(p: Params) -> int:
    return load_library().attn_bwd_workspace_size(ctypes.byref(p))


def attn_bwd_ds_workspace_size(p: Params) -> int:
    return load_library().attn_bwd_ds_workspace_size(ctypes.byref(p))


# Largest workspace attn_bwd allocates by itself to keep dS (store_ds=None).
DS_WORKSPACE_LIMIT = 8 << 30
# Smallest Q/K head dim for which attn_bwd keeps dS by default (store_ds=None).
# Measured on one MI355X (fwd + bwd step, both paths in one run): 192/128 heads
# (causal, S=4096, 128 heads) 7.49 -> 6.10 ms with stored dS, since the dQ
# kernel that recomputes S and dP runs one wave per SIMD there; 128/128 heads
# 1-3 % faster (GQA with a 1024-key window at S=4096: 1.253 -> 1.216 ms; a
# 4096-key window at S=8192: 4.08 -> 4.04 ms) for 1.1-6.6 GB more workspace, so
# left to the caller (store_ds=True); 64/64 heads (causal, S=4096..8192)
# 9-12 % slower: the dK/dV kernel's dS stores cost more than recomputing the
# cheap 64-dim products saves.
DS_DEFAULT_MIN_HEAD_DIM = 192


def prefers_stored_ds(p: Params, bias=None) -> bool:
    """Whether attn_bwd keeps dS by default (store_ds=None) for problem p
    (with the attention bias tensor bias, or None).

    A bias shared over batches or heads always takes the stored dS when it
    fits: dBias is then a sum of the stored blocks, where the recomputing
    path runs S and dP once more for every sharing (batch, head) pair
    (measured, GQA 32:8 with a 1024-key window at S=4096, head dim 128:
    backward 2.4-2.7 -> 1.2-1.5 ms).  A bias per (batch, head) gains little
    (2.09 -> 2.0 ms) and follows the head-dim rule.  With dropout the
    recomputing dQ kernel also regenerates every random byte, and from head
    dim 128 the stored dS is the faster path (same workload, p = 0.1: step
    1.55 -> 1.44 ms; sink + padding S=8192, 6.6 GB of dS: 5.97 -> 5.65 ms);
    at head dim 64 it is 2 % slower."""
    size = attn_bwd_ds_workspace_size(p)
    if not 0 < size <= DS_WORKSPACE_LIMIT:
        return False
    if bias is not None and (bias.shape[0] == 1 < p.batch or bias.shape[1] == 1 < p.num_heads):
        return True
    if math.floor(256.0 * p.dropout_p + 0.5) > 0 and p.head_dim_qk >= 128:
        return True
    return p.head_dim_qk >= DS_DEFAULT_MIN_HEAD_DIM


def attn_status_string(rc: int) -> str:
    return load_library().attn_status_string(rc).decode()


def fwd_tile_shape(p: Params):
    bm, bn = _c_i32(), _c_i32()
    _check(load_library().attn_fwd_tile_shape(ctypes.byref(p), ctypes.byref(bm), ctypes.byref(bn)),
           "attn_fwd_tile_shape")
    return bm.value, bn.value


# --------------------------------------------------------------- torch level

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _packed_layout(q, seq_offsets, seqlens, max_seqlen):
    """Host checks of packed (THD) segment metadata; returns (B, S).

    seq_offsets [B+1] int32 on the device: 0 = off[0] <= off[1] <= ... <=
    off[B] <= T.  S = max_seqlen, or the largest segment when None; every
    segment must fit in S tokens and every seqlens[b] in its segment.
    """
    torch = _torch()
    if seq_offsets.dtype != torch.int32 or seq_offsets.dim() != 1 or seq_offsets.numel() < 2 \
            or not seq_offsets.is_cuda:
        raise ValueError("seq_offsets must be an int32 device tensor of shape [B+1]")
    off = seq_offsets.cpu().to(torch.int64)
    sizes = off[1:] - off[:-1]
    if int(off[0]) != 0 or bool((sizes < 0).any()) or int(off[-1]) > q.shape[0]:
        raise ValueError("seq_offsets must start at 0, not decrease and end at or below T")
    S = int(sizes.max()) if max_seqlen is None else int(max_seqlen)
    S = max(S, 1)
    if bool((sizes > S).any()):
        raise ValueError(f"a segment holds more than max_seqlen = {S} tokens")
    if seqlens is not None:
        if seqlens.dtype != torch.int32 or seqlens.numel() != sizes.numel() or not seqlens.is_cuda:
            raise ValueError("seqlens must be an int32 device tensor of shape [B]")
        sl = seqlens.cpu().to(torch.int64)
        if bool((sl < 0).any()) or bool((sl > sizes).any()):
            raise ValueError("seqlens values must lie in [0, segment size]")
    return int(sizes.numel()), S


def _problem(q, k, v, num_gqa_groups, attn_mask_type, window_size, scale_factor, softmax_type,
             packed=None, dropout_p=0.0, rng_state=(0, 0)):
    """Params for BSHD tensors, or for packed [T, H, D] tensors when
    packed = (B, S) comes from _packed_layout."""
    torch = _torch()
    if packed is None:
        if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
            raise ValueError("q, k, v must be BSHD tensors (or pass seq_offsets for packed THD)")
        B, S, Hq, dqk = q.shape
        Hkv = k.shape[2] if num_gqa_groups is None else int(num_gqa_groups)
        lead = (B, S)
    else:
        if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
            raise ValueError("packed q, k, v must be [T, heads, dim] tensors")
        B, S = packed
        T, Hq, dqk = q.shape
        Hkv = k.shape[1] if num_gqa_groups is None else int(num_gqa_groups)
        lead = (T,)
    if tuple(k.shape) != lead + (Hkv, dqk) or tuple(v.shape[:-1]) != lead + (Hkv,):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError("q, k, v must be contiguous device tensors of one dtype")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("dtype must be bfloat16 or float32")
    dtype = "bf16" if q.dtype == torch.bfloat16 else "f32"
    return make_params(B, S, Hq, Hkv, dqk, v.shape[-1], dtype, attn_mask_type, window_size,
                       scale_factor, softmax_type, dropout_p, rng_state)


def _check_buffer(t, shape, dtype, name):
    """Caller-supplied output / workspace buffers: the library sees only their
    pointers, so their size, dtype and layout are checked here."""
    if not t.is_cuda or not t.is_contiguous() or t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous {dtype} device tensor of shape {list(shape)}, "
                         f"got {t.dtype} {list(t.shape)}")


def _sink_offsets(softmax_offset, Hq, q):
    """The learnable sink logits as a contiguous float32 [Hq] device tensor on
    q's device (a copy when the caller's tensor has another dtype or layout).
    The kernels read softmax_offset[h] for every query head h, so a host
    tensor or a short one is refused here."""
    torch = _torch()
    if softmax_offset is None:
        raise ValueError("learnable softmax needs softmax_offset [Hq]")
    if not isinstance(softmax_offset, torch.Tensor) or not softmax_offset.is_cuda \
            or softmax_offset.device != q.device:
        raise ValueError("softmax_offset must be a device tensor on q's device")
    if softmax_offset.numel() != Hq:
        raise ValueError(f"softmax_offset must hold num_heads = {Hq} values, got {softmax_offset.numel()}")
    return softmax_offset.reshape(-1).to(torch.float32).contiguous()


def _check_bias(bias, q, B, Hq, S):
    """An additive bias [1 or B, 1 or Hq, S, S] of q's dtype on q's device;
    returns (bias_batch, bias_heads)."""
    torch = _torch()
    if not isinstance(bias, torch.Tensor) or not bias.is_cuda or bias.device != q.device \
            or bias.dtype != q.dtype or not bias.is_contiguous() or bias.dim() != 4 \
            or bias.shape[0] not in (1, B) or bias.shape[1] not in (1, Hq) or tuple(bias.shape[2:]) != (S, S):
        raise ValueError(f"bias must be a contiguous {q.dtype} device tensor of shape [1 or {B}, 1 or {Hq}, "
                         f"{S}, {S}]")
    return int(bias.shape[0]), int(bias.shape[1])


def _on_stream(stream):
    """Context for the call's torch work (allocations, dtype copies): on the
    launch stream, so that memory freed when the call returns is reused only
    after the kernels queued on that stream, and copies precede the kernels."""
    torch = _torch()
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _check_seqlens(seqlens, B, S):
    torch = _torch()
    if seqlens is None:
        return None
    if seqlens.dtype != torch.int32 or seqlens.numel() != B or not seqlens.is_cuda:
        raise ValueError("seqlens must be an int32 device tensor of shape [B]")
    host = seqlens.cpu()
    if bool((host < 0).any()) or bool((host > S).any()):
        raise ValueError(f"seqlens values must lie in [0, {S}]")
    return seqlens


def _layout(q, seq_offsets, seqlens, max_seqlen, check):
    """(B, S) of packed inputs, or None for BSHD.  With check, the offsets and
    lengths are copied to the host and checked; without (timed loops), S must
    be given as max_seqlen and the caller vouches for the values."""
    if seq_offsets is None:
        if max_seqlen is not None:
            raise ValueError("max_seqlen applies to packed inputs (seq_offsets) only")
        return None
    if not check:
        if max_seqlen is None:
            raise ValueError("packed inputs without host checks need max_seqlen")
        return seq_offsets.numel() - 1, int(max_seqlen)
    return _packed_layout(q, seq_offsets, seqlens, max_seqlen)


def attn_fwd(q, k, v, *, num_gqa_groups=None, attn_mask_type="causal", window_size=(-1, -1),
             scale_factor=None, softmax_type="vanilla", softmax_offset=None, seqlens=None,
             seq_offsets=None, max_seqlen=None, dropout_p=0.0, rng_state=(0, 0), out=None, lse=None,
             stream=None, check_seqlens=True, bias=None):
    """Forward attention.  Returns (O, LSE [B,Hq,S]).

    BSHD: q [B,S,Hq,Dqk], k/v [B,S,Hkv,D], O [B,S,Hq,Dv].  Packed (THD, when
    seq_offsets [B+1] is given): q [T,Hq,Dqk], k/v [T,Hkv,D], O [T,Hq,Dv];
    S = max_seqlen or the largest segment.  dropout_p > 0 applies attention
    dropout with the generator state rng_state = (seed, offset); pass the
    same values to attn_bwd.  bias: an additive post-scale bias
    [1 or B, 1 or Hq, S, S] of q's dtype (attn_fwd_bias).
    """
    with _on_stream(stream):
        return _attn_fwd(q, k, v, num_gqa_groups, attn_mask_type, window_size, scale_factor, softmax_type,
                         softmax_offset, seqlens, seq_offsets, max_seqlen, dropout_p, rng_state, out, lse,
                         stream, check_seqlens, bias)


def _attn_fwd(q, k, v, num_gqa_groups, attn_mask_type, window_size, scale_factor, softmax_type,
              softmax_offset, seqlens, seq_offsets, max_seqlen, dropout_p, rng_state, out, lse, stream,
              check_seqlens, bias):
    torch = _torch()
    packed = _layout(q, seq_offsets, seqlens, max_seqlen, check_seqlens)
    p = _problem(q, k, v, num_gqa_groups, attn_mask_type, window_size, scale_factor, softmax_type, packed,
                 dropout_p, rng_state)
    B, S, Hq = p.batch, p.seqlen, p.num_heads
    if check_seqlens and packed is None:
        _check_seqlens(seqlens, B, S)
    softmax_offset = _sink_offsets(softmax_offset, Hq, q) if softmax_type == "learnable" else None
    o_shape = tuple(q.shape[:-1]) + (p.head_dim_v,)
    o = out if out is not None else torch.empty(o_shape, dtype=q.dtype, device=q.device)
    l = lse if lse is not None else torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _check_buffer(o, o_shape, q.dtype, "out")
    _check_buffer(l, (B, Hq, S), torch.float32, "lse")
    lib = load_library()
    if bias is not None:
        bb, bh = _check_bias(bias, q, B, Hq, S)
        _check(lib.attn_fwd_bias(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(bias), bb, bh,
                                 _ptr(softmax_offset), _ptr(seqlens), _ptr(seq_offsets), _ptr(o), _ptr(l), None, 0,
                                 _stream(stream)), "attn_fwd_bias")
        return o, l
    _check(lib.attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(softmax_offset),
                        _ptr(seqlens), _ptr(seq_offsets), _ptr(o), _ptr(l), None, 0, _stream(stream)),
           "attn_fwd")
    return o, l


def attn_bwd(q, k, v, o, lse, d_o, *, num_gqa_groups=None, attn_mask_type="causal",
             window_size=(-1, -1), scale_factor=None, softmax_type="vanilla", softmax_offset=None,
             seqlens=None, seq_offsets=None, max_seqlen=None, dropout_p=0.0, rng_state=(0, 0),
             want_d_offset=None, workspace=None, outs=None, stream=None, check_seqlens=True, stage=0,
             bias=None, d_bias=None, want_d_bias=True, store_ds=None):
    """Backward attention.  Returns (dQ, dK, dV, d_softmax_offset or None),
    and with a bias (dQ, dK, dV, d_softmax_offset or None, d_bias or None).

    store_ds (without a caller workspace): True allocates the workspace that
    lets the library keep dS and compute dQ from it (attn_bwd_ds_workspace_size;
    ValueError if the problem has no such path), False the smaller one with
    which dQ recomputes S and dP, None whichever prefers_stored_ds picks.  A
    caller workspace decides by its size.

    d_softmax_offset is returned for learnable softmax (always) and for
    off-by-one when want_d_offset is true; vanilla returns None.  Layouts as
    for attn_fwd (packed THD when seq_offsets is given); dropout_p and
    rng_state must match the forward's.
    """
    with _on_stream(stream):
        return _attn_bwd(q, k, v, o, lse, d_o, num_gqa_groups, attn_mask_type, window_size, scale_factor,
                         softmax_type, softmax_offset, seqlens, seq_offsets, max_seqlen, dropout_p,
                         rng_state, want_d_offset, workspace, outs, stream, check_seqlens, stage, bias, d_bias,
                         want_d_bias, store_ds)


def _attn_bwd(q, k, v, o, lse, d_o, num_gqa_groups, attn_mask_type, window_size, scale_factor,
              softmax_type, softmax_offset, seqlens, seq_offsets, max_seqlen, dropout_p, rng_state,
              want_d_offset, workspace, outs, stream, check_seqlens, stage, bias, d_bias, want_d_bias,
              store_ds=None):
    torch = _torch()
    packed = _layout(q, seq_offsets, seqlens, max_seqlen, check_seqlens)
    p = _problem(q, k, v, num_gqa_groups, attn_mask_type, window_size, scale_factor, softmax_type, packed,
                 dropout_p, rng_state)
    B, S, Hq, Hkv = p.batch, p.seqlen, p.num_heads, p.num_gqa_groups
    if check_seqlens and packed is None:
        _check_seqlens(seqlens, B, S)
    o_shape = tuple(q.shape[:-1]) + (p.head_dim_v,)
    for t in (o, d_o):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype or tuple(t.shape) != o_shape:
            raise ValueError(f"o and d_o must be contiguous {list(o_shape)} tensors of q's dtype")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, S) or not lse.is_contiguous() \
            or not lse.is_cuda:
        raise ValueError("lse must be a contiguous float32 [B,Hq,S] device tensor")
    if bias is not None:
        bias_dims = _check_bias(bias, q, B, Hq, S)
        if stage:
            raise ValueError("the staged backward takes no bias")
        if d_bias is not None:
            _check_buffer(d_bias, bias.shape, bias.dtype, "d_bias")
        elif want_d_bias:
            d_bias = torch.empty_like(bias)
    softmax_offset = _sink_offsets(softmax_offset, Hq, q) if softmax_type == "learnable" else None
    want = softmax_type == "learnable" or (softmax_type == "off_by_one" and bool(want_d_offset))
    if outs is not None:
        dq, dk, dv, doff = outs
        _check_buffer(dq, q.shape, q.dtype, "dq")
        _check_buffer(dk, k.shape, q.dtype, "dk")
        _check_buffer(dv, v.shape, q.dtype, "dv")
        if want and doff is not None:
            _check_buffer(doff, (Hq,), torch.float32, "d_softmax_offset")
        if want and doff is None:
            doff = torch.empty(Hq, dtype=torch.float32, device=q.device)
    else:
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
        doff = torch.empty(Hq, dtype=torch.float32, device=q.device) if want else None
    if not want:
        doff = None
    lib = load_library()
    ws_bytes = lib.attn_bwd_workspace_size(ctypes.byref(p))
    if workspace is not None and (not workspace.is_cuda or workspace.numel() * workspace.element_size() < ws_bytes):
        raise ValueError(f"workspace must be a device tensor of at least {ws_bytes} bytes")
    if workspace is None:
        if not stage and store_ds is not False:
            ds_bytes = lib.attn_bwd_ds_workspace_size(ctypes.byref(p))
            if store_ds and ds_bytes == 0:
                raise ValueError("this problem has no stored-dS backward")
            if store_ds or prefers_stored_ds(p, bias):
                ws_bytes = ds_bytes
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    args = (ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse),
            _ptr(softmax_offset), _ptr(seqlens), _ptr(seq_offsets), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(doff), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if bias is not None:
        _check(lib.attn_bwd_bias(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse),
                                 _ptr(bias), bias_dims[0], bias_dims[1], _ptr(d_bias), _ptr(softmax_offset),
                                 _ptr(seqlens), _ptr(seq_offsets), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(doff),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
               "attn_bwd_bias")
        return dq, dk, dv, doff, d_bias
    if stage:
        _check(lib.attn_bwd_stage(stage, *args), f"attn_bwd_stage({stage})")
    else:
        _check(lib.attn_bwd(*args), "attn_bwd")
    return dq, dk, dv, doff


def attn_bwd_noalloc(q, k, v, o, lse, d_o, *, outs, num_gqa_groups=None, attn_mask_type="causal",
                     window_size=(-1, -1), scale_factor=None, softmax_type="vanilla", softmax_offset=None,
                     seqlens=None, seq_offsets=None, max_seqlen=None, dropout_p=0.0, rng_state=(0, 0),
                     stream=None, check_seqlens=True):
    """The allocation-free backward: attn_bwd's result in the caller's
    outs = (dq, dk, dv, d_softmax_offset or None), with the library's static
    per-GPU scratch as workspace.  Allocates nothing: every output must be
    given, and a learnable softmax_offset must already be a contiguous float32
    [Hq] device tensor.  Calls that overlap on one GPU race (they share the
    scratch); calls on one stream are ordered."""
    torch = _torch()
    packed = _layout(q, seq_offsets, seqlens, max_seqlen, check_seqlens)
    p = _problem(q, k, v, num_gqa_groups, attn_mask_type, window_size, scale_factor, softmax_type, packed,
                 dropout_p, rng_state)
    B, S, Hq = p.batch, p.seqlen, p.num_heads
    if check_seqlens and packed is None:
        _check_seqlens(seqlens, B, S)
    o_shape = tuple(q.shape[:-1]) + (p.head_dim_v,)
    for t in (o, d_o):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != q.dtype or tuple(t.shape) != o_shape:
            raise ValueError(f"o and d_o must be contiguous {list(o_shape)} tensors of q's dtype")
    _check_buffer(lse, (B, Hq, S), torch.float32, "lse")
    if softmax_type == "learnable":
        if not isinstance(softmax_offset, torch.Tensor) or not softmax_offset.is_cuda \
                or softmax_offset.device != q.device or softmax_offset.dtype != torch.float32 \
                or not softmax_offset.is_contiguous() or softmax_offset.numel() != Hq:
            raise ValueError(f"softmax_offset must be a contiguous float32 tensor of {Hq} values on q's "
                             "device (no copy is made)")
        softmax_offset = softmax_offset.reshape(-1)
    else:
        softmax_offset = None
    dq, dk, dv, doff = outs
    _check_buffer(dq, q.shape, q.dtype, "dq")
    _check_buffer(dk, k.shape, q.dtype, "dk")
    _check_buffer(dv, v.shape, q.dtype, "dv")
    if softmax_type == "vanilla":
        doff = None
    elif doff is not None:
        _check_buffer(doff, (Hq,), torch.float32, "d_softmax_offset")
    _check(load_library().attn_bwd_noalloc(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse), _ptr(softmax_offset),
        _ptr(seqlens), _ptr(seq_offsets), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(doff), _stream(stream)),
        "attn_bwd_noalloc")
    return dq, dk, dv, doff


# ------------------------------------------------------------------- FP8

def fp8_quantize(x, scale, fmt="e4m3", out=None, amax=None, stream=None):
    """Per-tensor quantization on the device: codes (uint8, x's shape) of
    clamp(x * scale, -max, max) in fmt ("e4m3" / "e5m2"), and amax = max |x|
    (float32 [1]).  x: contiguous bf16 or float32 device tensor; scale: float32
    device tensor of one element."""
    torch = _torch()
    if not x.is_cuda or not x.is_contiguous() or x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("x must be a contiguous bf16 or float32 device tensor")
    if not isinstance(scale, torch.Tensor) or not scale.is_cuda or scale.dtype != torch.float32 or scale.numel() != 1:
        raise ValueError("scale must be a float32 device tensor of one element")
    with _on_stream(stream):
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if out is None else out
        amax = torch.empty(1, dtype=torch.float32, device=x.device) if amax is None else amax
    _check_buffer(out, x.shape, torch.uint8, "out")
    _check_buffer(amax, (1,), torch.float32, "amax")
    _check(load_library().attn_fp8_quantize(_ptr(x), ATTN_BF16 if x.dtype == torch.bfloat16 else ATTN_F32,
                                            x.numel(), FP8_FORMATS[fmt], _ptr(scale), _ptr(out), _ptr(amax),
                                            _stream(stream)), "attn_fp8_quantize")
    return out, amax


def fp8_update_scale(amax_history, amax, scale, descale, fmt="e4m3", margin=0, stream=None):
    """One delayed-scaling step on the device (updates amax_history, scale and
    descale in place): the new amax enters the history newest first; scale =
    fmt_max / max(history) / 2^margin while that max is positive and finite."""
    torch = _torch()
    for name, t in (("amax_history", amax_history), ("amax", amax), ("scale", scale), ("descale", descale)):
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 device tensor")
    _check(load_library().attn_fp8_update_scale(_ptr(amax_history), amax_history.numel(), _ptr(amax),
                                                FP8_FORMATS[fmt], int(margin), _ptr(scale), _ptr(descale),
                                                _stream(stream)), "attn_fp8_update_scale")


def attn_fwd_fp8(q8, k8, v8, descale_qkv, *, num_gqa_groups=None, attn_mask_type="causal", window_size=(-1, -1),
                 scale_factor=None, softmax_type="vanilla", softmax_offset=None, seqlens=None, seq_offsets=None,
                 max_seqlen=None, out=None, lse=None, workspace=None, stream=None, check_seqlens=True):
    """FP8 forward: q8, k8, v8 are E4M3 codes (uint8, the layouts of attn_fwd),
    descale_qkv a float32 device tensor [3] (descales of q, k, v).  Returns
    (O bf16, LSE [B,Hq,S])."""
    torch = _torch()
    for t in (q8, k8, v8):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.uint8:
            raise ValueError("q8, k8, v8 must be contiguous uint8 device tensors (E4M3 codes)")
    if not descale_qkv.is_cuda or descale_qkv.dtype != torch.float32 or descale_qkv.numel() != 3:
        raise ValueError("descale_qkv must be a float32 device tensor of 3 elements")
    with _on_stream(stream):
        packed = _layout(q8, seq_offsets, seqlens, max_seqlen, check_seqlens)
        if packed is None:
            B, S, Hq, dqk = q8.shape
            Hkv = k8.shape[2] if num_gqa_groups is None else int(num_gqa_groups)
        else:
            B, S = packed
            Hq, dqk = q8.shape[1], q8.shape[2]
            Hkv = k8.shape[1] if num_gqa_groups is None else int(num_gqa_groups)
        lead = tuple(q8.shape[:-2])
        if tuple(k8.shape) != lead + (Hkv, dqk) or tuple(v8.shape[:-1]) != lead + (Hkv,):
            raise ValueError(f"shape mismatch q{tuple(q8.shape)} k{tuple(k8.shape)} v{tuple(v8.shape)}")
        p = make_params(B, S, Hq, Hkv, dqk, v8.shape[-1], "fp8", attn_mask_type, window_size, scale_factor,
                        softmax_type)
        if check_seqlens and packed is None:
            _check_seqlens(seqlens, B, S)
        offs = _sink_offsets(softmax_offset, Hq, q8) if softmax_type == "learnable" else None
        o_shape = tuple(q8.shape[:-1]) + (p.head_dim_v,)
        o = out if out is not None else torch.empty(o_shape, dtype=torch.bfloat16, device=q8.device)
        l = lse if lse is not None else torch.empty((B, Hq, S), dtype=torch.float32, device=q8.device)
        _check_buffer(o, o_shape, torch.bfloat16, "out")
        _check_buffer(l, (B, Hq, S), torch.float32, "lse")
        lib = load_library()
        ws_bytes = lib.attn_fwd_workspace_size(ctypes.byref(p))
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q8.device)
        elif not workspace.is_cuda or workspace.numel() * workspace.element_size() < ws_bytes:
            raise ValueError(f"workspace must be a device tensor of at least {ws_bytes} bytes")
        _check(lib.attn_fwd_fp8(ctypes.byref(p), _ptr(q8), _ptr(k8), _ptr(v8), _ptr(descale_qkv), _ptr(offs),
                                _ptr(seqlens), _ptr(seq_offsets), _ptr(o), _ptr(l), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)), "attn_fwd_fp8")
    return o, l


def attn_bwd_fp8(q8, k8, v8, o, do8, lse, descale_qkvdo, ds_scale, *, num_gqa_groups=None, attn_mask_type="causal",
                 window_size=(-1, -1), scale_factor=None, softmax_type="vanilla", softmax_offset=None, seqlens=None,
                 seq_offsets=None, max_seqlen=None, want_d_offset=None, outs=None, amax=None, workspace=None,
                 stream=None, check_seqlens=True):
    """FP8 backward: q8, k8, v8 the forward's E4M3 codes, o its bf16 output,
    do8 E5M2 codes of dO (q's layout with Dv), lse the forward's LSE;
    descale_qkvdo float32 device [4]; ds_scale float32 device [1] (the scale
    of dS before its E5M2 encoding).  Returns (dQ, dK, dV bf16,
    d_softmax_offset or None, amax of dS float32 [1])."""
    torch = _torch()
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8), ("do8", do8)):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.uint8:
            raise ValueError(f"{name} must be a contiguous uint8 device tensor (FP8 codes)")
    for name, t, n in (("descale_qkvdo", descale_qkvdo, 4), ("ds_scale", ds_scale, 1)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.float32 or t.numel() != n:
            raise ValueError(f"{name} must be a float32 device tensor of {n} element(s)")
    with _on_stream(stream):
        packed = _layout(q8, seq_offsets, seqlens, max_seqlen, check_seqlens)
        if packed is None:
            B, S, Hq, dqk = q8.shape
            Hkv = k8.shape[2] if num_gqa_groups is None else int(num_gqa_groups)
        else:
            B, S = packed
            Hq, dqk = q8.shape[1], q8.shape[2]
            Hkv = k8.shape[1] if num_gqa_groups is None else int(num_gqa_groups)
        lead = tuple(q8.shape[:-2])
        if tuple(k8.shape) != lead + (Hkv, dqk) or tuple(v8.shape[:-1]) != lead + (Hkv,):
            raise ValueError(f"shape mismatch q{tuple(q8.shape)} k{tuple(k8.shape)} v{tuple(v8.shape)}")
        p = make_params(B, S, Hq, Hkv, dqk, v8.shape[-1], "fp8", attn_mask_type, window_size, scale_factor,
                        softmax_type)
        if check_seqlens and packed is None:
            _check_seqlens(seqlens, B, S)
        o_shape = tuple(q8.shape[:-1]) + (p.head_dim_v,)
        if tuple(do8.shape) != o_shape:
            raise ValueError(f"do8 must have shape {list(o_shape)}")
        if not o.is_cuda or not o.is_contiguous() or o.dtype != torch.bfloat16 or tuple(o.shape) != o_shape:
            raise ValueError(f"o must be a contiguous bf16 {list(o_shape)} device tensor")
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, S) or not lse.is_contiguous() \
                or not lse.is_cuda:
            raise ValueError("lse must be a contiguous float32 [B,Hq,S] device tensor")
        offs = _sink_offsets(softmax_offset, Hq, q8) if softmax_type == "learnable" else None
        want = softmax_type == "learnable" or (softmax_type == "off_by_one" and bool(want_d_offset))
        if outs is not None:
            dq, dk, dv, doff = outs
            for name, t, shape in (("dq", dq, q8.shape), ("dk", dk, k8.shape), ("dv", dv, v8.shape)):
                _check_buffer(t, shape, torch.bfloat16, name)
            if want and doff is None:
                doff = torch.empty(Hq, dtype=torch.float32, device=q8.device)
            elif want:
                _check_buffer(doff, (Hq,), torch.float32, "d_softmax_offset")
        else:
            dq = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
            dk = torch.empty(k8.shape, dtype=torch.bfloat16, device=q8.device)
            dv = torch.empty(v8.shape, dtype=torch.bfloat16, device=q8.device)
            doff = torch.empty(Hq, dtype=torch.float32, device=q8.device) if want else None
        if not want:
            doff = None
        amax = torch.empty(1, dtype=torch.float32, device=q8.device) if amax is None else amax
        _check_buffer(amax, (1,), torch.float32, "amax")
        lib = load_library()
        ws_bytes = lib.attn_bwd_workspace_size(ctypes.byref(p))
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q8.device)
        elif not workspace.is_cuda or workspace.numel() * workspace.element_size() < ws_bytes:
            raise ValueError(f"workspace must be a device tensor of at least {ws_bytes} bytes")
        _check(lib.attn_bwd_fp8(ctypes.byref(p), _ptr(q8), _ptr(k8), _ptr(v8), _ptr(o), _ptr(do8), _ptr(lse),
                                _ptr(descale_qkvdo), _ptr(ds_scale), _ptr(amax), _ptr(offs), _ptr(seqlens),
                                _ptr(seq_offsets), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(doff), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)), "attn_bwd_fp8")
    return dq, dk, dv, doff, amax


def debug_tile_map(p: Params, seqlens, block_m, block_n, stream=None):
    torch = _torch()
    nqt = -(-p.seqlen // block_m)
    nkt = -(-p.seqlen // block_n)
    out = torch.empty((p.batch, nqt, nkt), dtype=torch.int8, device="cuda")
    _check(load_library().attn_debug_tile_map(ctypes.byref(p), _ptr(seqlens), block_m, block_n,
                                              _ptr(out), _stream(stream)), "attn_debug_tile_map")
    return out


def debug_mask_probe(p: Params, seqlens, stream=None):
    torch = _torch()
    out = torch.empty((p.batch, p.seqlen, p.seqlen), dtype=torch.uint8, device="cuda")
    _check(load_library().attn_debug_mask_probe(ctypes.byref(p), _ptr(seqlens), _ptr(out),
                                                _stream(stream)), "attn_debug_mask_probe")
    return out


def debug_dropout_mask(p: Params, stream=None):
    """Device keep decisions of attention dropout, uint8 [B, Hq, S, S]."""
    torch = _torch()
    out = torch.empty((p.batch, p.num_heads, p.seqlen, p.seqlen), dtype=torch.uint8, device="cuda")
    _check(load_library().attn_debug_dropout_mask(ctypes.byref(p), _ptr(out), _stream(stream)),
           "attn_debug_dropout_mask")
    return out


def host_tile_map(p: Params, seqlens, block_m, block_n):
    import numpy as np
    nqt = -(-p.seqlen // block_m)
    nkt = -(-p.seqlen // block_n)
    out = np.zeros((p.batch, nqt, nkt), dtype=np.int8)
    sl = None if seqlens is None else np.ascontiguousarray(seqlens, dtype=np.int32)
    _check(load_library().attn_host_tile_map(
        ctypes.byref(p), None if sl is None else sl.ctypes.data_as(ctypes.c_void_p), block_m,
        block_n, out.ctypes.data_as(ctypes.c_void_p)), "attn_host_tile_map")
    return out


def host_key_range(p: Params, L, i0, i1):
    lo, hi = _c_i32(), _c_i32()
    ok = load_library().attn_host_key_range(ctypes.byref(p), L, i0, i1, ctypes.byref(lo), ctypes.byref(hi))
    return (lo.value, hi.value) if ok else None


def host_query_range(p: Params, L, j0, j1):
    lo, hi = _c_i32(), _c_i32()
    ok = load_library().attn_host_query_range(ctypes.byref(p), L, j0, j1, ctypes.byref(lo), ctypes.byref(hi))
    return (lo.value, hi.value) if ok else None


def host_full_key_tiles(p: Params, L, i0, block_m, block_n):
    f0, f1 = _c_i32(), _c_i32()
    ok = load_library().attn_host_full_key_tiles(ctypes.byref(p), L, i0, block_m, block_n, ctypes.byref(f0),
                                                 ctypes.byref(f1))
    return (f0.value, f1.value) if ok else None


def host_dkdv_splits(p: Params) -> int:
    """Query-head splits of a GQA group in the bf16 dK/dV stage (0 if p is invalid)."""
    return load_library().attn_host_dkdv_splits(ctypes.byref(p))

"""The allocation-free backward (attn_bwd_noalloc) against attn_bwd.

attn_bwd_noalloc runs attn_bwd's kernels with the library's static per-GPU
scratch as workspace (the minimum workspace size: dQ recomputes S and dP).
Two calls in a row, the second on a smaller problem, each equal bitwise to
attn_bwd's result with that workspace (both are deterministic and run the
same kernels), so the second call cannot be reading anything the first left in
the scratch; a third case has dK/dV head splits, whose fp32 partials also live
in the scratch.
"""
import numpy as np
import pytest

from scaled_dot_product_15_amd import binding, inputs
from tests import gpu_cases as gc

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gc.gpu_available(), reason="needs a GPU and the built library")]


def _case(p, seed, seqlens=None):
    import torch
    arr = inputs.draw(p, seed)
    if seqlens is not None:
        arr["seqlens"] = np.asarray(seqlens, dtype=np.int32)
    t = inputs.to_torch(arr, p.dtype, "cuda")
    kw = dict(num_gqa_groups=p.Hkv, attn_mask_type="causal" if p.causal else "no_mask",
              window_size=p.window, softmax_type=p.softmax_type,
              softmax_offset=t["alpha"] if p.softmax_type == "learnable" else None, seqlens=t["seqlens"])
    o, lse = binding.attn_fwd(t["q"], t["k"], t["v"], **kw)
    ref = binding.attn_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], want_d_offset=True, store_ds=False, **kw)
    torch.cuda.synchronize()
    return t, kw, o, lse, ref


def _noalloc(t, kw, o, lse, ref):
    import torch
    outs = tuple(None if r is None else torch.full_like(r, float("nan")) for r in ref)
    got = binding.attn_bwd_noalloc(t["q"], t["k"], t["v"], o, lse, t["do"], outs=outs, **kw)
    torch.cuda.synchronize()
    return got


def _equal(got, ref, name):
    import torch
    for n, a, b in zip(("dq", "dk", "dv", "d_offset"), got, ref):
        assert (a is None) == (b is None), (name, n)
        if a is not None:
            assert torch.equal(a, b), (name, n, float((a.float() - b.float()).abs().max()))


def test_noalloc_two_calls_second_smaller():
    big = inputs.Problem(B=2, S=1024, Hq=8, Hkv=2, d_qk=128, d_v=128, dtype="bf16", causal=True,
                         window=(256, 0), softmax_type="learnable")
    small = inputs.Problem(B=1, S=300, Hq=4, Hkv=1, d_qk=128, d_v=128, dtype="bf16", causal=True,
                           window=(-1, -1), softmax_type="off_by_one")
    gc.log("noalloc: first call, B=2 S=1024 Hq=8 Hkv=2 d=128 learnable, lengths (1024, 700)")
    c1 = _case(big, 9101, seqlens=[1024, 700])
    _equal(_noalloc(*c1), c1[4], "first")
    gc.log("noalloc: second call, B=1 S=300 Hq=4 Hkv=1 d=128 off-by-one")
    c2 = _case(small, 9102)
    _equal(_noalloc(*c2), c2[4], "second")


def test_noalloc_with_dkdv_head_splits():
    # One KV head for 16 query heads over 2048 keys: the dK/dV stage splits the
    # group's heads and keeps fp32 partials in the workspace.
    p = inputs.Problem(B=1, S=2048, Hq=16, Hkv=1, d_qk=64, d_v=64, dtype="bf16", causal=True,
                       window=(-1, -1), softmax_type="vanilla")
    pp = binding.make_params(p.B, p.S, p.Hq, p.Hkv, p.d_qk, p.d_v, "bf16", "causal")
    assert binding.host_dkdv_splits(pp) > 1
    assert binding.attn_bwd_workspace_size(pp) <= binding.NOALLOC_SCRATCH_BYTES
    gc.log("noalloc: B=1 S=2048 Hq=16 Hkv=1 d=64 (dK/dV head splits)")
    c = _case(p, 9103)
    _equal(_noalloc(*c), c[4], "splits")

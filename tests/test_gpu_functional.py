"""The autograd wrapper (scaled_dot_product_15_amd.functional.attention): its
forward and the gradients torch.autograd gets from it are bitwise the direct
attn_fwd / attn_bwd results (same kernels, same backward path), for a
learnable sink, GQA with a window and padded batches, a shared bias with
dropout, and packed inputs; inputs that do not require grad get none."""
import numpy as np
import pytest

from scaled_dot_product_15_amd import binding, inputs
from tests import gpu_cases as gc

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gc.gpu_available(), reason="needs a GPU and the built library")]


def _leaves(t, names):
    return {n: t[n].detach().clone().requires_grad_(True) for n in names}


def test_autograd_matches_direct_calls_sink_gqa_padded():
    import torch
    from scaled_dot_product_15_amd.functional import attention
    p = inputs.Problem(B=3, S=300, Hq=8, Hkv=2, d_qk=128, d_v=128, dtype="bf16", causal=True, window=(90, 0),
                       softmax_type="learnable")
    arr = inputs.draw(p, 81_000)
    arr["seqlens"] = np.array([300, 171, 0], dtype=np.int32)
    t = inputs.to_torch(arr, "bf16", "cuda")
    gc.log("autograd: learnable sink, GQA 8:2, window 90, padded")
    kw = dict(num_gqa_groups=p.Hkv, attn_mask_type="causal", window_size=p.window, softmax_type="learnable",
              seqlens=t["seqlens"])
    x = _leaves(t, ("q", "k", "v", "alpha"))
    o = attention(x["q"], x["k"], x["v"], softmax_offset=x["alpha"], **kw)
    o.backward(t["do"])
    ro, rlse = binding.attn_fwd(t["q"], t["k"], t["v"], softmax_offset=t["alpha"], **kw)
    dq, dk, dv, doff = binding.attn_bwd(t["q"], t["k"], t["v"], ro, rlse, t["do"], softmax_offset=t["alpha"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), ro)
    for name, ref in (("q", dq), ("k", dk), ("v", dv)):
        assert torch.equal(x[name].grad, ref), name
    assert torch.equal(x["alpha"].grad, doff.to(x["alpha"].dtype))


@pytest.mark.parametrize("store_default", ("shared", "full"))
def test_autograd_bias_and_dropout(store_default):
    """A bias that requires grad gets dBias (shared: the stored-dS backward by
    default; full: the recomputing one); Q, K, V with dropout."""
    import torch
    from scaled_dot_product_15_amd.functional import attention
    p = inputs.Problem(B=2, S=256, Hq=4, Hkv=2, d_qk=64, d_v=64, dtype="bf16", causal=True, window=(-1, -1),
                       softmax_type="vanilla")
    t = inputs.to_torch(inputs.draw(p, 81_100), "bf16", "cuda")
    shape = (1, 1, p.S, p.S) if store_default == "shared" else (p.B, p.Hq, p.S, p.S)
    g = torch.Generator(device="cuda").manual_seed(81_101)
    bias = torch.randn(shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    gc.log(f"autograd: bias {shape} + dropout 0.2")
    kw = dict(num_gqa_groups=p.Hkv, attn_mask_type="causal", dropout_p=0.2, rng_state=(77, 3))
    x = _leaves(t, ("q", "k", "v"))
    xb = bias.clone().requires_grad_(True)
    o = attention(x["q"], x["k"], x["v"], bias=xb, **kw)
    o.backward(t["do"])
    ro, rlse = binding.attn_fwd(t["q"], t["k"], t["v"], bias=bias, **kw)
    dq, dk, dv, _, db = binding.attn_bwd(t["q"], t["k"], t["v"], ro, rlse, t["do"], bias=bias, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), ro)
    for name, ref in (("q", dq), ("k", dk), ("v", dv)):
        assert torch.equal(x[name].grad, ref), name
    assert torch.equal(xb.grad, db)


def test_autograd_packed_and_partial_requires_grad():
    """Packed (THD) inputs; only Q requires grad, so K and V get none."""
    import torch
    from scaled_dot_product_15_amd.functional import attention
    p = inputs.Problem(B=3, S=200, Hq=4, Hkv=1, d_qk=64, d_v=64, dtype="bf16", causal=True, window=(50, 0),
                       softmax_type="off_by_one")
    arr = inputs.draw(p, 81_200)
    sizes = [200, 33, 120]
    arr["seqlens"] = np.array(sizes, dtype=np.int32)
    tp = inputs.to_torch_packed(inputs.pack(arr, sizes), "bf16", "cuda")
    gc.log("autograd: packed, off-by-one, only Q requires grad")
    kw = dict(num_gqa_groups=p.Hkv, window_size=p.window, softmax_type="off_by_one",
              seq_offsets=tp["seq_offsets"], max_seqlen=p.S)
    q = tp["q"].detach().clone().requires_grad_(True)
    o = attention(q, tp["k"], tp["v"], **kw)
    o.backward(tp["do"])
    ro, rlse = binding.attn_fwd(tp["q"], tp["k"], tp["v"], **kw)
    dq, _, _, _ = binding.attn_bwd(tp["q"], tp["k"], tp["v"], ro, rlse, tp["do"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), ro) and torch.equal(q.grad, dq)
    assert tp["k"].grad is None and tp["v"].grad is None

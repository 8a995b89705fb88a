"""dspark_pack_w: the r x V right factor converted to the [V][r] layout the calls read.  Bit-exact
against torch's transpose for both dtypes and sizes that leave partial 64 x 64 tiles; a draft
through the packed factor equals the draft through a factor built in [V][r] directly; the
conversion of the headline factor (r = 256, V = 151936, bfloat16) is timed."""
import numpy as np
import pytest
import torch

from draft_head_verification_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("r,V", [(16, 1024), (96, 1000), (256, 2392), (1, 8), (130, 70)])
def test_pack_matches_transpose(dtype, r, V):
    from draft_head_verification_amd import dspark as D
    g = torch.Generator(device="cuda").manual_seed(r * 7 + V)
    w_rv = torch.randn(r, V, generator=g, device="cuda").to(dtype)
    out = D.dspark_pack_w(w_rv)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                       w_rv.T.contiguous().view(torch.int16 if dtype == torch.bfloat16 else torch.int32))


def test_draft_through_packed_factor():
    from draft_head_verification_amd import dspark as D
    w = synth.shrink(synth.WORKLOADS["moderate"], V=2392, B=40, K=5)
    inp = synth.make_inputs(w, device="cuda", strong_bias=True)
    Z = inp["Z_ext"][:, : w.K].contiguous()
    w_rv = inp["W"].T.contiguous()  # the factorisation's own r x V shape
    packed = D.dspark_pack_w(w_rv)
    a = D.draft_block(Z, inp["U"], inp["W"], inp["prev_token"], inp["temperature"], inp["seed"],
                      req_id=inp["req_id"])
    b = D.draft_block(Z, inp["U"], packed, inp["prev_token"], inp["temperature"], inp["seed"],
                      req_id=inp["req_id"])
    for k in ("tokens", "q_tok", "q_lse"):
        assert torch.equal(a[k], b[k])


def test_pack_headline_factor_time():
    from draft_head_verification_amd import dspark as D
    r, V = 256, 151936
    w_rv = torch.randn(r, V, device="cuda").to(torch.bfloat16)
    out = torch.empty(V, r, dtype=torch.bfloat16, device="cuda")
    D.dspark_pack_w(w_rv, out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        D.dspark_pack_w(w_rv, out)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / 10 * 1e3
    gbs = 2 * r * V * 2 / (us * 1e-6) / 1e9
    print(f"[pack] r={r} V={V} bf16: {us:.1f} us per conversion ({gbs:.0f} GB/s read+write)",
          flush=True)
    assert torch.equal(out[:1000], w_rv[:, :1000].T.contiguous())

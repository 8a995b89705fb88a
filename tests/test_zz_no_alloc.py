"""The allocation-free draft entry point (dspark_draft_block_static) against dspark_draft_block:
the same kernels on the same inputs, so tokens, q_tok and q_lse are identical, for two calls
in a row on one device (the second smaller, so the static scratch holds the previous call's
leftovers), on the matrix-core path (bfloat16, rank 256, both samplers) and the vector path
(float32, rank 16); device status bits land in the caller's word; sizes beyond the static
scratch are rejected before anything is launched."""
import pytest
import torch

from draft_head_verification_amd import synth

pytestmark = pytest.mark.gpu


def _both(w, T, sampler):
    from draft_head_verification_amd import dspark as D
    inp = synth.make_inputs(w, device="cuda", temperature=T, strong_bias=True)
    Z = inp["Z_ext"][:, : w.K].contiguous()
    ref = D.draft_block(Z, inp["U"], inp["W"], inp["prev_token"], inp["temperature"], inp["seed"],
                        draft_len=inp["draft_len"], req_id=inp["req_id"], sampler=sampler)
    B, K = w.B, w.K
    out = dict(tokens=torch.full((B, K), -7, dtype=torch.int32, device="cuda"),
               q_tok=torch.full((B, K), -7.0, device="cuda"),
               q_lse=torch.full((B, K), -7.0, device="cuda"))
    status = torch.full((1,), 0x7FFF, dtype=torch.int32, device="cuda")
    D.dspark_draft_block_static(Z, inp["U"], inp["W"], inp["prev_token"], inp["temperature"],
                                inp["seed"], out["tokens"], out["q_tok"], out["q_lse"], status,
                                draft_len=inp["draft_len"], req_id=inp["req_id"], sampler=sampler)
    assert D.dspark_query_device_status(status) == 0
    for k in ("tokens", "q_tok", "q_lse"):
        assert torch.equal(out[k], ref[k]), k


@pytest.mark.parametrize("sampler", ["token", "block16"])
def test_static_draft_matches_workspace_draft_twice(sampler):
    big = synth.shrink(synth.WORKLOADS["ragged"], B=300, V=6000)  # two request groups
    small = synth.shrink(synth.WORKLOADS["moderate"], B=20, K=5, V=2392)
    _both(big, None, sampler)
    _both(small, None, sampler)


def test_static_draft_vector_path_and_status_bits():
    from draft_head_verification_amd import dspark as D
    w = synth.WORKLOADS["tiny"]
    _both(w, 1.0, "token")
    _both(synth.shrink(w, B=2, K=3), 0.0, "token")
    inp = synth.make_inputs(w, device="cuda")
    Z = inp["Z_ext"][:, : w.K].contiguous()
    prev = inp["prev_token"].clone()
    prev[1] = -3  # flagged, read as token 0
    toks = torch.empty(w.B, w.K, dtype=torch.int32, device="cuda")
    qt = torch.empty(w.B, w.K, device="cuda")
    ql = torch.empty(w.B, w.K, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    D.dspark_draft_block_static(Z, inp["U"], inp["W"], prev, inp["temperature"], inp["seed"],
                                toks, qt, ql, status, req_id=inp["req_id"])
    assert D.dspark_query_device_status(status) & D.DEV_BAD_TOKEN


def test_static_draft_rejects_sizes_beyond_its_scratch():
    from draft_head_verification_amd import dspark as D
    B, K, V, r = 4096, 16, 262144, 256
    assert D.dspark_draft_workspace_size(B, K, V, r) > D.STATIC_SCRATCH_BYTES
    tiny = torch.zeros(1, device="cuda")  # never read: the call is rejected before any launch
    a = D.DraftArgs(B, K, V, r, 0, 0, tiny.data_ptr(), tiny.data_ptr(), tiny.data_ptr(),
                    tiny.data_ptr(), None, tiny.data_ptr(), None, 1, tiny.data_ptr(),
                    tiny.data_ptr(), tiny.data_ptr(), None, None)
    import ctypes as C
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert D._lib.dspark_draft_block_static(C.byref(a), status.data_ptr(), None) == D.DSPARK_ESCRATCH
    assert D._lib.dspark_draft_block_static(C.byref(a), None, None) == D.DSPARK_EINVAL

"""The C-ABI library loads, exports every entry point include/dspark.h declares, and rejects
invalid host-visible arguments before touching the GPU (no compute calls here)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")
LIB = os.path.join(ROOT, "draft_head_verification_amd", "libdspark.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libdspark.so is not built (run __graft_entry__.build())")
    return C.CDLL(LIB)


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"dspark_draft_block", "dspark_schedule", "dspark_verify"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in dspark.h but not exported"


def test_binding_structs_match_header():
    """The ctypes structs in the binding list the same fields, in order, as the C structs."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for cname, pyname in (("dspark_draft_args", "DraftArgs"), ("dspark_schedule_args", "ScheduleArgs"),
                          ("dspark_verify_args", "VerifyArgs"),
                          ("dspark_calibrate_args", "CalibrateArgs")):
        body = re.search(r"typedef struct \{([^{}]*)\}\s*" + cname + ";", src).group(1)
        fields = []
        for decl in body.split(";"):
            decl = decl.strip()
            if not decl:
                continue
            decl = re.sub(r"^(const\s+)?[a-z_0-9]+\s*", "", decl)
            for part in decl.split(","):
                fields.append(part.strip().lstrip("*").strip())
        pysrc = open(os.path.join(ROOT, "draft_head_verification_amd", "dspark.py")).read()
        block = re.search(r"class " + pyname + r"\(C\.Structure\):\s*_fields_ = \[(.*?)\]\n\n", pysrc, re.S).group(1)
        pyfields = re.findall(r'\("(\w+)"', block)
        assert pyfields == fields, (cname, pyfields, fields)


def test_workspace_queries_and_strings(lib):
    lib.dspark_draft_workspace_size.restype = C.c_size_t
    lib.dspark_verify_workspace_size.restype = C.c_size_t
    lib.dspark_schedule_workspace_size.restype = C.c_size_t
    lib.dspark_status_string.restype = C.c_char_p
    assert lib.dspark_draft_workspace_size(256, 16, 151936, 256) > 256 * 4
    assert lib.dspark_verify_workspace_size(256, 16, 151936, 256) > 256 * 17 * 16
    # status word, then 8-byte products and 4-byte ranks of up to 8192 items
    assert lib.dspark_schedule_workspace_size(512, 16) == 256 + 8192 * 8 + 8192 * 4
    assert lib.dspark_schedule_workspace_size(8192, 64) == 256 + 8192 * 8 + 8192 * 4
    assert lib.dspark_schedule_workspace_size(3, 5) == 256 + 256 + 256
    # invalid sizes give 0
    assert lib.dspark_draft_workspace_size(4, 0, 1024, 16) == 0
    assert lib.dspark_draft_workspace_size(4, 4, 1020, 16) == 0  # V % 8 != 0
    assert lib.dspark_draft_workspace_size(4, 65, 1024, 16) == 0
    assert lib.dspark_draft_workspace_size(4, 4, 1024, 2048) == 0
    assert lib.dspark_schedule_workspace_size(9000, 4) == 0
    for s in (0, -1, -2, -3, -4, -5):
        assert lib.dspark_status_string(s)
    lib.dspark_version.restype = C.c_char_p
    assert b"gfx950" in lib.dspark_version()


def test_host_validation_without_gpu():
    """Argument errors come back before any HIP call, so they are testable on the CPU."""
    import torch  # noqa: F401  (the binding module needs torch for its types only)
    from draft_head_verification_amd import dspark as D
    lib = D._lib
    fake = 0x1000  # never dereferenced: validation fails first
    a = D.DraftArgs(4, 4, 1024, 16, 0, 0, fake, fake, fake, fake, None, fake, None, 1,
                    fake, fake, fake, None, None)
    assert lib.dspark_draft_block(None, None, 0, None) == D.DSPARK_EINVAL
    bad = D.DraftArgs(*[getattr(a, f) for f, _ in a._fields_])
    bad.K = 0
    assert lib.dspark_draft_block(C.byref(bad), None, 0, None) == D.DSPARK_EINVAL
    bad.K, bad.V = 4, 1020
    assert lib.dspark_draft_block(C.byref(bad), None, 0, None) == D.DSPARK_EINVAL
    bad.V, bad.z_dtype = 1024, 7
    assert lib.dspark_draft_block(C.byref(bad), None, 0, None) == D.DSPARK_EDTYPE
    bad.z_dtype, bad.Z = 0, None
    assert lib.dspark_draft_block(C.byref(bad), None, 0, None) == D.DSPARK_EINVAL
    # an unknown sampler
    bad.Z, bad.sampler = fake, 2
    assert lib.dspark_draft_block(C.byref(bad), fake, 1 << 30, None) == D.DSPARK_EINVAL
    bad.sampler = -1
    assert lib.dspark_draft_block(C.byref(bad), fake, 1 << 30, None) == D.DSPARK_EINVAL
    assert a.sampler == D.SAMPLERS["token"] == 0  # a zero-initialised field is the default
    # missing / misaligned / short workspace
    assert lib.dspark_draft_block(C.byref(a), None, 0, None) == D.DSPARK_EWORKSPACE
    assert lib.dspark_draft_block(C.byref(a), fake + 8, 1 << 30, None) == D.DSPARK_EWORKSPACE
    assert lib.dspark_draft_block(C.byref(a), fake, 16, None) == D.DSPARK_EWORKSPACE
    # recurrent head: all four GRU arrays, bfloat16 factors of a matrix-core rank; head_state
    # only with it (a has float32 factors of rank 16)
    rnn = D.DraftArgs(*[getattr(a, f) for f, _ in a._fields_])
    rnn.gru_wi = fake
    assert lib.dspark_draft_block(C.byref(rnn), fake, 1 << 30, None) == D.DSPARK_EINVAL
    rnn.gru_wh = rnn.gru_bi = rnn.gru_bh = fake
    assert lib.dspark_draft_block(C.byref(rnn), fake, 1 << 30, None) == D.DSPARK_EINVAL
    rnn.uw_dtype, rnn.r = 1, 100
    assert lib.dspark_draft_block(C.byref(rnn), fake, 1 << 30, None) == D.DSPARK_EINVAL
    hs = D.DraftArgs(*[getattr(a, f) for f, _ in a._fields_])
    hs.head_state = fake
    assert lib.dspark_draft_block(C.byref(hs), fake, 1 << 30, None) == D.DSPARK_EINVAL
    # B = 0 is a no-op
    empty = D.DraftArgs(*[getattr(a, f) for f, _ in a._fields_])
    empty.B = 0
    assert lib.dspark_draft_block(C.byref(empty), None, 0, None) == D.DSPARK_OK

    s = D.ScheduleArgs(4, 4, fake, None, 0, None, None, 1, fake, None, None, None)
    assert lib.dspark_schedule(C.byref(s), fake, 256, None) == D.DSPARK_EINVAL  # no knots
    s.n_knots, s.knot_tokens, s.knot_tps = 2, fake, fake
    s.B = 600  # B*K > 8192 with scheduling on
    s.K = 16
    assert lib.dspark_schedule(C.byref(s), fake, 256, None) == D.DSPARK_EINVAL
    s.B, s.K = 4, 4
    assert lib.dspark_schedule(C.byref(s), fake, 8, None) == D.DSPARK_EWORKSPACE

    v = D.VerifyArgs(4, 4, 1024, 16, 0, 0, 0, fake, fake, fake, fake, fake, fake, fake, fake,
                     fake, fake, None, 1, fake, fake, None, None)
    assert lib.dspark_verify(C.byref(v), None, 0, None) == D.DSPARK_EWORKSPACE
    v.y_dtype = 3
    assert lib.dspark_verify(C.byref(v), None, 0, None) == D.DSPARK_EDTYPE
    v.y_dtype, v.Y = 0, None
    assert lib.dspark_verify(C.byref(v), None, 0, None) == D.DSPARK_EINVAL
    v.Y, v.head_state = fake, fake  # recurrent-head operands need matrix-core factors
    assert lib.dspark_verify(C.byref(v), fake, 1 << 30, None) == D.DSPARK_EINVAL
    v.head_state, v.sampler = None, 5
    assert lib.dspark_verify(C.byref(v), fake, 1 << 30, None) == D.DSPARK_EINVAL

    c = D.CalibrateArgs(4, 4, fake, fake, fake, fake, 1.0, 1e-3, None)
    assert lib.dspark_calibrate(None, None, 0, None) == D.DSPARK_EINVAL
    for field, value in (("K", 0), ("K", 65), ("step", 0.0), ("step", 1.5), ("ridge", 0.0),
                         ("inv_temp", None)):
        bad = D.CalibrateArgs(*[getattr(c, f) for f, _ in c._fields_])
        setattr(bad, field, value)
        assert lib.dspark_calibrate(C.byref(bad), fake, 256, None) == D.DSPARK_EINVAL, field
    assert lib.dspark_calibrate(C.byref(c), fake, 8, None) == D.DSPARK_EWORKSPACE
    empty = D.CalibrateArgs(*[getattr(c, f) for f, _ in c._fields_])
    empty.B = 0
    assert lib.dspark_calibrate(C.byref(empty), None, 0, None) == D.DSPARK_OK
    assert D.dspark_calibrate_workspace_size(8, 16) == 256 and D.dspark_calibrate_workspace_size(8, 0) == 0


def test_binding_rejects_host_workspaces_and_counts_bytes():
    """The binding hands the library device pointers only: a host tensor as workspace (or as
    the workspace whose status is queried) is refused before any call, and a workspace's size
    is passed in bytes whatever its element type."""
    import pytest
    import torch
    from draft_head_verification_amd import dspark as D
    with pytest.raises(TypeError, match="workspace must be a device tensor"):
        D._ws(torch.zeros(1024, dtype=torch.uint8), 256, torch.device("cuda", 0))
    with pytest.raises(TypeError, match="workspace must be a device tensor"):
        D.dspark_query_device_status(torch.zeros(256, dtype=torch.uint8))
    assert D._nbytes(torch.zeros(64, dtype=torch.float32)) == 256
    assert D._nbytes(torch.zeros(64, dtype=torch.uint8)) == 64
    # tensors on another device than the first input are refused
    with pytest.raises(ValueError, match="is on cpu"):
        D._same_device(torch.device("cuda", 0), U=torch.zeros(1))
    D._same_device(torch.device("cpu"), U=torch.zeros(1), W=None)

"""Thin ctypes binding of libdspark.so (C ABI in include/dspark.h).

Argument marshalling only: every step of the round runs in the HIP library.  Tensors are
PyTorch device tensors (PyTorch provides device memory and streams); the binding checks
their dtype / shape / contiguity, takes their data pointers and the current HIP stream, and
raises DSparkError on a non-OK status.  The library must be built (draft_head_verification_amd
/build.py); importing this module without it raises immediately -- there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdspark.so")

DSPARK_OK, DSPARK_EINVAL, DSPARK_EDTYPE, DSPARK_EWORKSPACE, DSPARK_EHIP, DSPARK_EDEVICE = \
    0, -1, -2, -3, -4, -5
DSPARK_ESCRATCH = -6
STATIC_SCRATCH_BYTES = 8 << 20  # DSPARK_STATIC_SCRATCH_BYTES
DSPARK_F32, DSPARK_BF16 = 0, 1
# samplers (include/dspark.h): the per-token Gumbel-max (default) and the opt-in block race
SAMPLERS = {"token": 0, "block16": 1}
DEV_BAD_TOKEN, DEV_BAD_TEMPERATURE, DEV_BAD_LENGTH, DEV_BAD_PROFILE = 0x1, 0x2, 0x4, 0x8


class DSparkError(RuntimeError):
    def __init__(self, status: int, where: str, bits: int = 0):
        self.status = status
        self.bits = bits
        super().__init__(f"{where}: {status_string(status)} (status {status}, device bits {bits:#x})")


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m draft_head_verification_amd.build`")
_lib = C.CDLL(LIB_PATH)

_p = C.c_void_p
_i32 = C.c_int32


class DraftArgs(C.Structure):
    _fields_ = [("B", _i32), ("K", _i32), ("V", _i32), ("r", _i32),
                ("z_dtype", _i32), ("uw_dtype", _i32),
                ("Z", _p), ("U", _p), ("W", _p),
                ("prev_token", _p), ("draft_len", _p), ("temperature", _p), ("req_id", _p),
                ("seed", C.c_uint64),
                ("draft_tokens", _p), ("q_tok", _p), ("q_lse", _p), ("corrected", _p),
                ("trace", _p), ("gru_wi", _p), ("gru_wh", _p), ("gru_bi", _p), ("gru_bh", _p),
                ("head_state", _p), ("sampler", _i32)]


class ScheduleArgs(C.Structure):
    _fields_ = [("B", _i32), ("K", _i32), ("conf_logits", _p), ("draft_len", _p),
                ("n_knots", _i32), ("knot_tokens", _p), ("knot_tps", _p), ("enabled", _i32),
                ("verify_len", _p), ("expected_tokens", _p), ("conf_inv_temp", _p), ("trace", _p)]


class CalibrateArgs(C.Structure):
    _fields_ = [("B", _i32), ("K", _i32), ("conf_logits", _p), ("verify_len", _p),
                ("accept_len", _p), ("inv_temp", _p), ("step", C.c_double), ("ridge", C.c_double),
                ("trace", _p)]


class VerifyArgs(C.Structure):
    _fields_ = [("B", _i32), ("K", _i32), ("V", _i32), ("r", _i32),
                ("y_dtype", _i32), ("z_dtype", _i32), ("uw_dtype", _i32),
                ("Y", _p), ("draft_tokens", _p), ("q_tok", _p), ("q_lse", _p),
                ("Z", _p), ("U", _p), ("W", _p), ("prev_token", _p), ("verify_len", _p),
                ("temperature", _p), ("req_id", _p), ("seed", C.c_uint64),
                ("accept_len", _p), ("next_token", _p), ("p_tok", _p), ("trace", _p),
                ("head_state", _p), ("sampler", _i32)]


_lib.dspark_draft_workspace_size.restype = C.c_size_t
_lib.dspark_draft_workspace_size.argtypes = [_i32] * 4
_lib.dspark_verify_workspace_size.restype = C.c_size_t
_lib.dspark_verify_workspace_size.argtypes = [_i32] * 4
_lib.dspark_schedule_workspace_size.restype = C.c_size_t
_lib.dspark_schedule_workspace_size.argtypes = [_i32] * 2
_lib.dspark_calibrate_workspace_size.restype = C.c_size_t
_lib.dspark_calibrate_workspace_size.argtypes = [_i32] * 2
_lib.dspark_calibrate.restype = C.c_int
_lib.dspark_calibrate.argtypes = [C.POINTER(CalibrateArgs), _p, C.c_size_t, _p]
_lib.dspark_draft_block.restype = C.c_int
_lib.dspark_draft_block.argtypes = [C.POINTER(DraftArgs), _p, C.c_size_t, _p]
_lib.dspark_draft_block_static.restype = C.c_int
_lib.dspark_draft_block_static.argtypes = [C.POINTER(DraftArgs), _p, _p]
_lib.dspark_schedule.restype = C.c_int
_lib.dspark_schedule.argtypes = [C.POINTER(ScheduleArgs), _p, C.c_size_t, _p]
_lib.dspark_verify.restype = C.c_int
_lib.dspark_verify.argtypes = [C.POINTER(VerifyArgs), _p, C.c_size_t, _p]
_lib.dspark_pack_w.restype = C.c_int
_lib.dspark_pack_w.argtypes = [_p, _p, _i32, _i32, _i32, _p]
_lib.dspark_query_device_status.restype = C.c_int
_lib.dspark_query_device_status.argtypes = [_p, _p, C.POINTER(C.c_uint32)]
_lib.dspark_status_string.restype = C.c_char_p
_lib.dspark_status_string.argtypes = [C.c_int]
_lib.dspark_version.restype = C.c_char_p
_lib.dspark_trace_create.restype = _p
_lib.dspark_trace_create.argtypes = [_i32]
_lib.dspark_trace_destroy.argtypes = [_p]
_lib.dspark_trace_reset.argtypes = [_p]
_lib.dspark_trace_count.restype = _i32
_lib.dspark_trace_count.argtypes = [_p]
_lib.dspark_trace_get.restype = C.c_int
_lib.dspark_trace_get.argtypes = [_p, _i32, C.POINTER(C.c_char_p), C.POINTER(C.c_float)]


def status_string(status: int) -> str:
    return _lib.dspark_status_string(int(status)).decode()


def version() -> str:
    return _lib.dspark_version().decode()


# ----------------------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------------------

_DT = {torch.float32: DSPARK_F32, torch.bfloat16: DSPARK_BF16}


def _dev(t: torch.Tensor, name: str, dtypes=None, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)


def _ws(ws: torch.Tensor | None, need: int, device) -> torch.Tensor:
    """The caller's workspace (a contiguous device tensor on the inputs' device; its size is
    checked by the library), or a new one of the queried size."""
    if ws is None:
        return torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    _dev(ws, "workspace")
    if ws.device != torch.device(device):
        raise ValueError(f"workspace is on {ws.device}, the inputs on {device}")
    return ws


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _same_device(device, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, the first input on {device}")


_INT = (torch.int32,)
_F32 = (torch.float32,)
_LOGIT = (torch.float32, torch.bfloat16)


class Trace:
    """Per-kernel HIP-event timing of the calls it is passed to (dspark_trace_*)."""

    def __init__(self, capacity: int = 4096):
        self.handle = _lib.dspark_trace_create(int(capacity))
        if not self.handle:
            raise DSparkError(DSPARK_EHIP, "dspark_trace_create")

    def reset(self):
        _lib.dspark_trace_reset(self.handle)

    def records(self):
        out = []
        for i in range(_lib.dspark_trace_count(self.handle)):
            name, ms = C.c_char_p(), C.c_float()
            st = _lib.dspark_trace_get(self.handle, i, C.byref(name), C.byref(ms))
            if st != DSPARK_OK:
                raise DSparkError(st, "dspark_trace_get")
            out.append((name.value.decode(), float(ms.value)))
        return out

    def close(self):
        """Release the events now (also done when the object is collected)."""
        handle, self.handle = getattr(self, "handle", None), None
        lib = _lib
        if handle and lib is not None:
            lib.dspark_trace_destroy(handle)

    def __del__(self):
        # at interpreter exit the module globals may already be gone: then the process is
        # ending and the events go with it
        try:
            self.close()
        except Exception:
            pass


def _trace(trace):
    return None if trace is None else trace.handle


# ----------------------------------------------------------------------------------------
# the C entry points
# ----------------------------------------------------------------------------------------

def dspark_draft_workspace_size(B, K, V, r) -> int:
    return int(_lib.dspark_draft_workspace_size(B, K, V, r))


def dspark_verify_workspace_size(B, K, V, r) -> int:
    return int(_lib.dspark_verify_workspace_size(B, K, V, r))


def dspark_schedule_workspace_size(B, K) -> int:
    return int(_lib.dspark_schedule_workspace_size(B, K))


def _sampler(sampler) -> int:
    if sampler not in SAMPLERS:
        raise ValueError(f"sampler must be one of {sorted(SAMPLERS)}")
    return SAMPLERS[sampler]


def _draft_args(Z, U, W, prev_token, temperature, seed, draft_tokens, q_tok, q_lse, draft_len,
                req_id, corrected, trace, gru, head_state, sampler) -> DraftArgs:
    B, K, V = Z.shape
    r = U.shape[1]
    _dev(Z, "Z", _LOGIT)
    _dev(U, "U", _LOGIT, (V, r))
    _dev(W, "W", (U.dtype,), (V, r))
    _dev(prev_token, "prev_token", _INT, (B,))
    _dev(temperature, "temperature", _F32, (B,))
    _dev(draft_tokens, "draft_tokens", _INT, (B, K))
    _dev(q_tok, "q_tok", _F32, (B, K))
    _dev(q_lse, "q_lse", _F32, (B, K))
    if draft_len is not None:
        _dev(draft_len, "draft_len", _INT, (B,))
    if req_id is not None:
        _dev(req_id, "req_id", _INT, (B,))
    if corrected is not None:
        _dev(corrected, "corrected", _F32, (B, K, V))
    g = (None,) * 4
    if gru is not None:
        g = tuple(gru)
        for t, n, shape in zip(g, ("gru_wi", "gru_wh", "gru_bi", "gru_bh"),
                               ((3 * r, r), (3 * r, r), (3 * r,), (3 * r,))):
            _dev(t, n, _F32, shape)
    if head_state is not None:
        _dev(head_state, "head_state", (torch.bfloat16,), (B, K, r))
    _same_device(Z.device, U=U, W=W, prev_token=prev_token, temperature=temperature,
                 draft_tokens=draft_tokens, q_tok=q_tok, q_lse=q_lse, draft_len=draft_len,
                 req_id=req_id, corrected=corrected, head_state=head_state,
                 **{n: t for n, t in zip(("gru_wi", "gru_wh", "gru_bi", "gru_bh"), g)})
    return DraftArgs(B, K, V, r, _DT[Z.dtype], _DT[U.dtype], _ptr(Z), _ptr(U), _ptr(W),
                     _ptr(prev_token), _ptr(draft_len), _ptr(temperature), _ptr(req_id),
                     int(seed) & (2**64 - 1), _ptr(draft_tokens), _ptr(q_tok), _ptr(q_lse),
                     _ptr(corrected), _trace(trace), *(_ptr(t) for t in g), _ptr(head_state),
                     _sampler(sampler))


def dspark_draft_block(Z, U, W, prev_token, temperature, seed, draft_tokens, q_tok, q_lse,
                       draft_len=None, req_id=None, corrected=None, workspace=None, stream=None,
                       trace=None, gru=None, head_state=None, sampler="token"):
    """Draft one block (see dspark_draft_block in include/dspark.h).  Returns the workspace
    (reusable; it also carries the device status word).  gru: None (Markov head) or the
    recurrent head's (Wi [3r,r], Wh [3r,r], bi [3r], bh [3r]) float32 device tensors;
    head_state: optional [B,K,r] bfloat16 output of the recurrent head's operands;
    sampler: "token" (per-token Gumbel-max) or "block16" (the two-level block race)."""
    B, K, V = Z.shape
    r = U.shape[1]
    a = _draft_args(Z, U, W, prev_token, temperature, seed, draft_tokens, q_tok, q_lse,
                    draft_len, req_id, corrected, trace, gru, head_state, sampler)
    need = dspark_draft_workspace_size(B, K, V, r)
    ws = _ws(workspace, need, Z.device)
    st = _lib.dspark_draft_block(C.byref(a), _ptr(ws), _nbytes(ws), _stream(stream))
    if st != DSPARK_OK:
        raise DSparkError(st, "dspark_draft_block")
    return ws


def dspark_draft_block_static(Z, U, W, prev_token, temperature, seed, draft_tokens, q_tok,
                              q_lse, device_status, draft_len=None, req_id=None, corrected=None,
                              stream=None, trace=None, gru=None, head_state=None,
                              sampler="token"):
    """Allocation-free draft (see dspark_draft_block_static in include/dspark.h): the library's
    static scratch replaces the workspace; device_status is a one-element int32 / uint32
    device tensor that receives the device status bits (dspark_query_device_status reads it)."""
    a = _draft_args(Z, U, W, prev_token, temperature, seed, draft_tokens, q_tok, q_lse,
                    draft_len, req_id, corrected, trace, gru, head_state, sampler)
    _dev(device_status, "device_status", (torch.int32,), (1,))
    st = _lib.dspark_draft_block_static(C.byref(a), _ptr(device_status), _stream(stream))
    if st != DSPARK_OK:
        raise DSparkError(st, "dspark_draft_block_static")
    return device_status


def dspark_schedule(conf_logits, verify_len, knot_tokens=None, knot_tps=None, enabled=True,
                    draft_len=None, expected_tokens=None, workspace=None, stream=None, trace=None,
                    inv_temp=None):
    """Per-request verification lengths (see dspark_schedule in include/dspark.h)."""
    B, K = conf_logits.shape
    _dev(conf_logits, "conf_logits", _F32)
    _dev(verify_len, "verify_len", _INT, (B,))
    if inv_temp is not None:
        _dev(inv_temp, "inv_temp", (torch.float64,), (K,))
    n_knots = 0
    if enabled:
        _dev(knot_tokens, "knot_tokens", (torch.float64,))
        _dev(knot_tps, "knot_tps", (torch.float64,), knot_tokens.shape)
        n_knots = knot_tokens.numel()
    if draft_len is not None:
        _dev(draft_len, "draft_len", _INT, (B,))
    if expected_tokens is not None:
        _dev(expected_tokens, "expected_tokens", (torch.float64,), (B,))
    _same_device(conf_logits.device, verify_len=verify_len, inv_temp=inv_temp,
                 knot_tokens=knot_tokens if enabled else None,
                 knot_tps=knot_tps if enabled else None, draft_len=draft_len,
                 expected_tokens=expected_tokens)
    ws = _ws(workspace, dspark_schedule_workspace_size(B, K), conf_logits.device)
    a = ScheduleArgs(B, K, _ptr(conf_logits), _ptr(draft_len), n_knots,
                     _ptr(knot_tokens) if enabled else None, _ptr(knot_tps) if enabled else None,
                     int(bool(enabled)), _ptr(verify_len), _ptr(expected_tokens), _ptr(inv_temp),
                     _trace(trace))
    st = _lib.dspark_schedule(C.byref(a), _ptr(ws), _nbytes(ws), _stream(stream))
    if st != DSPARK_OK:
        raise DSparkError(st, "dspark_schedule")
    return ws


def dspark_calibrate_workspace_size(B, K) -> int:
    return int(_lib.dspark_calibrate_workspace_size(B, K))


def dspark_calibrate(conf_logits, verify_len, accept_len, inv_temp, step=1.0, ridge=1e-3,
                     workspace=None, stream=None, trace=None):
    """One online calibration step (see dspark_calibrate in include/dspark.h); inv_temp [K]
    float64 is updated in place.  Returns the workspace (it carries the status word)."""
    B, K = conf_logits.shape
    _dev(conf_logits, "conf_logits", _F32)
    _dev(verify_len, "verify_len", _INT, (B,))
    _dev(accept_len, "accept_len", _INT, (B,))
    _dev(inv_temp, "inv_temp", (torch.float64,), (K,))
    _same_device(conf_logits.device, verify_len=verify_len, accept_len=accept_len,
                 inv_temp=inv_temp)
    ws = _ws(workspace, dspark_calibrate_workspace_size(B, K), conf_logits.device)
    a = CalibrateArgs(B, K, _ptr(conf_logits), _ptr(verify_len), _ptr(accept_len), _ptr(inv_temp),
                      float(step), float(ridge), _trace(trace))
    st = _lib.dspark_calibrate(C.byref(a), _ptr(ws), _nbytes(ws), _stream(stream))
    if st != DSPARK_OK:
        raise DSparkError(st, "dspark_calibrate")
    return ws


def dspark_verify(Y, draft_tokens, q_tok, q_lse, Z, U, W, prev_token, verify_len, temperature,
                  seed, accept_len, next_token, req_id=None, p_tok=None, workspace=None,
                  stream=None, trace=None, head_state=None, sampler="token"):
    """Rejection-sampling verification (see dspark_verify in include/dspark.h).  head_state:
    the [B,K,r] bfloat16 operands of a recurrent-head draft, or None (Markov head); sampler:
    how the residual / bonus tokens are drawn ("token" or "block16")."""
    B, K, V = Z.shape
    r = U.shape[1]
    _dev(Y, "Y", _LOGIT, (B, K + 1, V))
    _dev(draft_tokens, "draft_tokens", _INT, (B, K))
    _dev(q_tok, "q_tok", _F32, (B, K))
    _dev(q_lse, "q_lse", _F32, (B, K))
    _dev(Z, "Z", _LOGIT)
    _dev(U, "U", _LOGIT, (V, r))
    _dev(W, "W", (U.dtype,), (V, r))
    _dev(prev_token, "prev_token", _INT, (B,))
    _dev(verify_len, "verify_len", _INT, (B,))
    _dev(temperature, "temperature", _F32, (B,))
    _dev(accept_len, "accept_len", _INT, (B,))
    _dev(next_token, "next_token", _INT, (B,))
    if req_id is not None:
        _dev(req_id, "req_id", _INT, (B,))
    if p_tok is not None:
        _dev(p_tok, "p_tok", _F32, (B, K))
    if head_state is not None:
        _dev(head_state, "head_state", (torch.bfloat16,), (B, K, r))
    _same_device(Z.device, Y=Y, draft_tokens=draft_tokens, q_tok=q_tok, q_lse=q_lse, U=U, W=W,
                 prev_token=prev_token, verify_len=verify_len, temperature=temperature,
                 accept_len=accept_len, next_token=next_token, req_id=req_id, p_tok=p_tok,
                 head_state=head_state)
    ws = _ws(workspace, dspark_verify_workspace_size(B, K, V, r), Z.device)
    a = VerifyArgs(B, K, V, r, _DT[Y.dtype], _DT[Z.dtype], _DT[U.dtype], _ptr(Y),
                   _ptr(draft_tokens), _ptr(q_tok), _ptr(q_lse), _ptr(Z), _ptr(U), _ptr(W),
                   _ptr(prev_token), _ptr(verify_len), _ptr(temperature), _ptr(req_id),
                   int(seed) & (2**64 - 1), _ptr(accept_len), _ptr(next_token), _ptr(p_tok),
                   _trace(trace), _ptr(head_state), _sampler(sampler))
    st = _lib.dspark_verify(C.byref(a), _ptr(ws), _nbytes(ws), _stream(stream))
    if st != DSPARK_OK:
        raise DSparkError(st, "dspark_verify")
    return ws


def dspark_pack_w(w_rv: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """The r x V right factor -> the [V, r] layout the calls read (see dspark_pack_w in
    include/dspark.h).  Returns the packed tensor (a new one unless `out` is given)."""
    _dev(w_rv, "w_rv", _LOGIT)
    r, V = w_rv.shape
    if out is None:
        out = torch.empty(V, r, dtype=w_rv.dtype, device=w_rv.device)
    _dev(out, "out", (w_rv.dtype,), (V, r))
    st = _lib.dspark_pack_w(_ptr(w_rv), _ptr(out), r, V, _DT[w_rv.dtype], _stream(stream))
    if st != DSPARK_OK:
        raise DSparkError(st, "dspark_pack_w")
    return out


def dspark_query_device_status(workspace: torch.Tensor, stream=None) -> int:
    """Synchronise and return the device status bits of a workspace (0 = clean)."""
    _dev(workspace, "workspace")
    bits = C.c_uint32(0)
    st = _lib.dspark_query_device_status(_ptr(workspace), _stream(stream), C.byref(bits))
    if st not in (DSPARK_OK, DSPARK_EDEVICE):
        raise DSparkError(st, "dspark_query_device_status")
    return int(bits.value)


# ----------------------------------------------------------------------------------------
# convenience: allocate outputs, run one call
# ----------------------------------------------------------------------------------------

def draft_block(Z, U, W, prev_token, temperature, seed, draft_len=None, req_id=None,
                want_corrected=False, workspace=None, trace=None, gru=None, sampler="token"):
    """gru: None (Markov head) or (Wi, Wh, bi, bh) for the recurrent head, whose operands are
    returned as head_state [B,K,r] bfloat16 (positions past a draft are zero)."""
    B, K, V = Z.shape
    r = U.shape[1]
    dev = Z.device
    out = dict(tokens=torch.empty(B, K, dtype=torch.int32, device=dev),
               q_tok=torch.empty(B, K, dtype=torch.float32, device=dev),
               q_lse=torch.empty(B, K, dtype=torch.float32, device=dev),
               corrected=(torch.empty(B, K, V, dtype=torch.float32, device=dev)
                          if want_corrected else None),
               head_state=(torch.zeros(B, K, r, dtype=torch.bfloat16, device=dev)
                           if gru is not None else None))
    out["workspace"] = dspark_draft_block(Z, U, W, prev_token, temperature, seed, out["tokens"],
                                          out["q_tok"], out["q_lse"], draft_len=draft_len,
                                          req_id=req_id, corrected=out["corrected"],
                                          workspace=workspace, trace=trace, gru=gru,
                                          head_state=out["head_state"], sampler=sampler)
    return out


def schedule(conf_logits, knot_tokens=None, knot_tps=None, enabled=True, draft_len=None,
             workspace=None, trace=None, inv_temp=None):
    B, K = conf_logits.shape
    dev = conf_logits.device
    out = dict(verify_len=torch.empty(B, dtype=torch.int32, device=dev),
               expected_tokens=torch.empty(B, dtype=torch.float64, device=dev))
    out["workspace"] = dspark_schedule(conf_logits, out["verify_len"], knot_tokens, knot_tps,
                                       enabled, draft_len, out["expected_tokens"], workspace,
                                       trace=trace, inv_temp=inv_temp)
    return out


def calibrate(conf_logits, verify_len, accept_len, inv_temp, step=1.0, ridge=1e-3,
              workspace=None, trace=None):
    """One online calibration step; inv_temp (device float64 [K]) is updated in place."""
    ws = dspark_calibrate(conf_logits, verify_len, accept_len, inv_temp, step, ridge, workspace,
                          trace=trace)
    return dict(inv_temp=inv_temp, workspace=ws)


def verify(Y, draft_tokens, q_tok, q_lse, Z, U, W, prev_token, verify_len, temperature, seed,
           req_id=None, want_p=True, workspace=None, trace=None, head_state=None, sampler="token"):
    B, K = draft_tokens.shape
    dev = Y.device
    out = dict(accept_len=torch.empty(B, dtype=torch.int32, device=dev),
               next_token=torch.empty(B, dtype=torch.int32, device=dev),
               p_tok=torch.empty(B, K, dtype=torch.float32, device=dev) if want_p else None)
    out["workspace"] = dspark_verify(Y, draft_tokens, q_tok, q_lse, Z, U, W, prev_token,
                                     verify_len, temperature, seed, out["accept_len"],
                                     out["next_token"], req_id=req_id, p_tok=out["p_tok"],
                                     workspace=workspace, trace=trace, head_state=head_state,
                                     sampler=sampler)
    return out

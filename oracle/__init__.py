"""CPU oracle for the DSpark draft / schedule / verify round -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The product path (the HIP library and its Python binding) never does,
and this package never imports anything from the product package.

The arithmetic lives in ``dspark_oracle.c`` (plain C, double precision, one loop per step of
the definition).  This module only marshals numpy / torch-CPU arrays into that library and
back.  ``build()`` compiles it with gcc; ``lib()`` loads it, building it once if it is absent.

Every function documents the definition it implements; the C file cites the pages.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dspark_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
STREAM_DRAFT, STREAM_ACCEPT, STREAM_RESIDUAL, STREAM_BONUS = 0, 1, 2, 3
# samplers: the per-token Gumbel-max (the definition), and the optional two-level block race
SAMPLERS = {"token": 0, "block16": 1}

_lib = None


def build() -> str:
    """Compile the oracle with gcc (-O2, scalar code, OpenMP over requests)."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        p = C.c_void_p
        i32 = C.c_int
        u64 = C.c_uint64
        L.oracle_philox4x32_10.argtypes = [p, p, p]
        L.oracle_philox_batch.argtypes = [i32, p, p, p]
        L.oracle_uniform.restype = C.c_double
        L.oracle_uniform.argtypes = [u64, C.c_uint32, C.c_uint32, C.c_uint32, C.c_uint32]
        L.oracle_gumbel.restype = C.c_double
        L.oracle_gumbel.argtypes = [u64, C.c_uint32, C.c_uint32, C.c_uint32, C.c_uint32]
        L.oracle_uniform_batch.argtypes = [i32, u64, p, p, p, C.c_uint32, p]
        L.oracle_block_uniform.restype = C.c_double
        L.oracle_block_uniform.argtypes = [u64, C.c_uint32, C.c_uint32, C.c_uint32, C.c_uint32]
        L.oracle_two_level_sample.restype = i32
        L.oracle_two_level_sample.argtypes = [i32, p, u64, C.c_uint32, C.c_uint32, C.c_uint32,
                                              C.c_uint32, p]
        L.oracle_token_sample.restype = i32
        L.oracle_token_sample.argtypes = [i32, p, u64, C.c_uint32, C.c_uint32, C.c_uint32, p]
        L.oracle_corrected_row.argtypes = [i32, i32, i32, p, i32, p, p, i32, p]
        L.oracle_draft_block.restype = i32
        L.oracle_draft_block.argtypes = [i32, i32, i32, i32, i32, p, i32, p, p, p, p, p, p, u64,
                                         p, i32, p, p, p, p, p, i32]
        L.oracle_profile.restype = C.c_double
        L.oracle_profile.argtypes = [i32, p, p, C.c_double]
        L.oracle_prefix_expected.argtypes = [i32, i32, p, p]
        L.oracle_schedule.restype = i32
        L.oracle_schedule.argtypes = [i32, i32, p, p, i32, p, p, i32, p, p, p, p]
        L.oracle_calibrate_step.restype = i32
        L.oracle_calibrate_step.argtypes = [i32, i32, p, p, p, C.c_double, C.c_double, p]
        L.oracle_ece.restype = C.c_double
        L.oracle_ece.argtypes = [i32, p, p, i32]
        L.oracle_verify.restype = i32
        L.oracle_verify.argtypes = [i32, i32, i32, i32, i32, p, p, p, p, i32, p, i32, p, p, p, p,
                                    p, p, u64, p, i32, p, p, p, p, i32]
        L.oracle_gru_cell.argtypes = [i32, p, p, p, p, p, p, p]
        L.oracle_float_to_bf16.restype = C.c_uint16
        L.oracle_float_to_bf16.argtypes = [C.c_float]
        L.oracle_corrected_row_operand.argtypes = [i32, i32, i32, p, p, i32, p, p]
        L.oracle_draft_block_head.restype = i32
        L.oracle_draft_block_head.argtypes = [i32, i32, i32, i32, i32, p, i32, p, p, p, p, p, p,
                                              p, p, p, p, u64, p, i32, p, p, p, p, p, p, i32]
        L.oracle_verify_head.restype = i32
        L.oracle_verify_head.argtypes = [i32, i32, i32, i32, i32, p, p, p, p, i32, p, i32, p,
                                         p, p, p, p, p, p, u64, p, i32, p, p, p, p, i32]
        L.oracle_num_threads.restype = i32
        _lib = L
    return _lib


# ----------------------------------------------------------------------------------------
# array marshalling
# ----------------------------------------------------------------------------------------

def _as_logits(a):
    """Return (contiguous numpy array, dtype code) for float32 or bfloat16 data.

    bfloat16 arrives as a torch tensor (numpy has no bfloat16); its raw 16-bit patterns are
    handed to C, which widens them exactly."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                return a.view(torch.int16).numpy().view(np.uint16), BF16
            if a.dtype == torch.float32:
                return a.numpy(), F32
            raise TypeError(f"unsupported logits dtype {a.dtype}")
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"unsupported logits dtype {a.dtype}")


def _np(a, dtype):
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _subset(a, rows):
    """Rows of a leading-batch array (keeps bfloat16 tensors as tensors)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            idx = torch.as_tensor(rows, dtype=torch.long, device=a.device)
            return a.detach()[idx].cpu().contiguous()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a)[rows])


# ----------------------------------------------------------------------------------------
# random numbers
# ----------------------------------------------------------------------------------------

def philox(ctrs, key):
    """Philox4x32-10 blocks for counters ctrs [n,4] (uint32) under key [2] -> [n,4] uint32."""
    ctrs = _np(ctrs, np.uint32).reshape(-1, 4)
    key = _np(key, np.uint32).reshape(2)
    out = np.empty_like(ctrs)
    lib().oracle_philox_batch(len(ctrs), _ptr(ctrs), _ptr(key), _ptr(out))
    return out


def uniform(seed, req, pos, v, stream):
    """Uniforms in (0,1) at (request key, position, vocab index) on a stream (broadcasting)."""
    req, pos, v = np.broadcast_arrays(np.asarray(req), np.asarray(pos), np.asarray(v))
    shape = req.shape
    req = _np(req, np.uint32).ravel()
    pos = _np(pos, np.uint32).ravel()
    v = _np(v, np.uint32).ravel()
    out = np.empty(len(req), np.float64)
    lib().oracle_uniform_batch(len(req), C.c_uint64(seed), _ptr(req), _ptr(pos), _ptr(v),
                               stream, _ptr(out))
    return out.reshape(shape)


def block_uniform(seed, req, pos, beta, stream):
    """Uniform of 16-token block beta of the two-level sampler (scalar arguments)."""
    return lib().oracle_block_uniform(C.c_uint64(seed), req, pos, beta, stream)


def token_sample(log_w, seed, req, pos, stream):
    """Per-token Gumbel-max draw argmax_v(log_w_v + G_v) on `stream` -> (token, margin)."""
    a = _np(log_w, np.float64)
    gap = np.zeros(1, np.float64)
    x = lib().oracle_token_sample(len(a), _ptr(a), C.c_uint64(seed), req, pos, stream, _ptr(gap))
    return int(x), float(gap[0])


def two_level_sample(log_w, seed, req, pos, race_stream, within_stream):
    """Two-level Gumbel-max draw from log-weights log_w [n] -> (token, margin)."""
    a = _np(log_w, np.float64)
    gap = np.zeros(1, np.float64)
    x = lib().oracle_two_level_sample(len(a), _ptr(a), C.c_uint64(seed), req, pos, race_stream,
                                      within_stream, _ptr(gap))
    return int(x), float(gap[0])


# stream ids of the random draws (race / within-block pairs of the two-level sampler)
STREAM_DRAFT, STREAM_ACCEPT, STREAM_RESIDUAL, STREAM_BONUS = 0, 1, 2, 3
STREAM_DRAFT_WITHIN, STREAM_RESIDUAL_WITHIN, STREAM_BONUS_WITHIN = 4, 5, 6


# ----------------------------------------------------------------------------------------
# the three steps of a round
# ----------------------------------------------------------------------------------------

def corrected_row(z_row, U, W, prev):
    """c_v = Z_v + sum_i U[prev][i] * W[v][i] (double accumulation, float result) -> [V]."""
    z, zdt = _as_logits(z_row)
    u, udt = _as_logits(U)
    w, wdt = _as_logits(W)
    assert udt == wdt
    V = z.shape[-1]
    r = u.shape[-1]
    out = np.empty(V, np.float32)
    lib().oracle_corrected_row(V, r, zdt, _ptr(z), udt, _ptr(u), _ptr(w), int(prev), _ptr(out))
    return out


def _gru_arrays(gru, r):
    wi, wh, bi, bh = (_np(x, np.float32) for x in gru)
    assert wi.shape == (3 * r, r) and wh.shape == (3 * r, r), "GRU weights are [3r, r]"
    assert bi.shape == (3 * r,) and bh.shape == (3 * r,), "GRU biases are [3r]"
    return wi, wh, bi, bh


def gru_cell(e, h, gru):
    """One GRU update (oracle_gru_cell): e, h [r] -> h' [r], float64."""
    e = _np(e, np.float64)
    h = _np(h, np.float64)
    r = e.shape[0]
    wi, wh, bi, bh = _gru_arrays(gru, r)
    out = np.empty(r, np.float64)
    lib().oracle_gru_cell(r, _ptr(wi), _ptr(wh), _ptr(bi), _ptr(bh), _ptr(e), _ptr(h), _ptr(out))
    return out


def float_to_bf16(x):
    """bfloat16 bit patterns (uint16) of float32 values, nearest with ties to even."""
    x = _np(x, np.float32).ravel()
    f = lib().oracle_float_to_bf16
    return np.array([f(float(v)) for v in x], dtype=np.uint16)


def draft_block(Z, U, W, prev_token, temperature, seed, draft_len=None, req_id=None, rows=None,
                want_corrected=False, gru=None, sampler="token"):
    """Draft tokens for a block (see oracle_draft_block_head in dspark_oracle.c).

    sampler: "token" (the per-token Gumbel-max, the definition) or "block16" (the optional
    two-level block race).

    Z [B,K,V] (float32 or bfloat16), U [V,r], W [V,r] (row v = column v of the r x V factor),
    prev_token [B], temperature [B], draft_len [B] or None (= K), req_id [B] or None (= b).
    gru: None (Markov head) or (Wi [3r,r], Wh [3r,r], bi [3r], bh [3r]) float32 for the
    recurrent head.
    rows: optional list of requests to compute; the result arrays then have len(rows) rows.
    Returns a dict with tokens [n,K] int32, q_tok / q_lse [n,K] float64, gap [n,K] float64,
    when asked corrected [n,K,V] float32, and with the recurrent head state [n,K,r] uint16
    (the bfloat16 operand of each drafted position; zero elsewhere).
    """
    B = int(Z.shape[0])
    rows = np.arange(B) if rows is None else np.asarray(rows, dtype=np.int64)
    n = len(rows)
    z, zdt = _as_logits(_subset(Z, rows))
    u, udt = _as_logits(U)
    w, wdt = _as_logits(W)
    assert udt == wdt, "U and W must share a dtype"
    K, V = z.shape[1], z.shape[2]
    r = u.shape[1]
    prev = _np(prev_token, np.int32)[rows]
    temp = _np(temperature, np.float32)[rows]
    dlen = None if draft_len is None else _np(draft_len, np.int32)[rows]
    req = (rows.astype(np.uint32) if req_id is None else _np(req_id, np.uint32)[rows])
    req = np.ascontiguousarray(req, dtype=np.uint32)
    sub_rows = np.arange(n, dtype=np.int32)
    tokens = np.empty((n, K), np.int32)
    q_tok = np.empty((n, K), np.float64)
    q_lse = np.empty((n, K), np.float64)
    gap = np.empty((n, K), np.float64)
    corrected = np.empty((n, K, V), np.float32) if want_corrected else None
    g = (None,) * 4 if gru is None else _gru_arrays(gru, r)
    state = None if gru is None else np.zeros((n, K, r), np.uint16)
    st = lib().oracle_draft_block_head(n, K, V, r, zdt, _ptr(z), udt, _ptr(u), _ptr(w),
                                       *(_ptr(x) for x in g), _ptr(prev), _ptr(dlen), _ptr(temp),
                                       _ptr(req), C.c_uint64(seed), _ptr(sub_rows), n,
                                       _ptr(tokens), _ptr(q_tok), _ptr(q_lse), _ptr(corrected),
                                       _ptr(gap), _ptr(state), SAMPLERS[sampler])
    if st != 0:
        raise ValueError("oracle_draft_block: token index out of range")
    return dict(tokens=tokens, q_tok=q_tok, q_lse=q_lse, gap=gap, corrected=corrected,
                state=state)


def profile(knot_tokens, knot_tps, N):
    kt = _np(knot_tokens, np.float64)
    kp = _np(knot_tps, np.float64)
    return lib().oracle_profile(len(kt), _ptr(kt), _ptr(kp), float(N))


def prefix_expected(B, P_sorted):
    """E(n) = B + sum of the first n of P_sorted, n = 0..len, each rounded once from the exact
    sum (see oracle_prefix_expected in dspark_oracle.c) -> float64 [len + 1]."""
    P = _np(P_sorted, np.float64)
    out = np.empty(len(P) + 1, np.float64)
    lib().oracle_prefix_expected(int(B), len(P), _ptr(P), _ptr(out))
    return out


def schedule(conf_logits, knot_tokens, knot_tps, enabled=True, draft_len=None, inv_temp=None):
    """Per-request verification lengths (see oracle_schedule in dspark_oracle.c); inv_temp
    [K] float64 are the per-position inverse temperatures of the confidence logits.

    Returns dict(verify_len [B] int32, expected_tokens [B] float64, n_star, margin)."""
    c = _np(conf_logits, np.float32)
    B, K = c.shape
    dlen = None if draft_len is None else _np(draft_len, np.int32)
    kt = _np(knot_tokens, np.float64)
    kp = _np(knot_tps, np.float64)
    th = None if inv_temp is None else _np(inv_temp, np.float64)
    vl = np.empty(B, np.int32)
    et = np.empty(B, np.float64)
    diag = np.empty(2, np.float64)
    st = lib().oracle_schedule(B, K, _ptr(c), _ptr(dlen), len(kt), _ptr(kt), _ptr(kp),
                               int(bool(enabled)), _ptr(th), _ptr(vl), _ptr(et), _ptr(diag))
    if st != 0:
        raise ValueError("oracle_schedule: invalid argument")
    return dict(verify_len=vl, expected_tokens=et, n_star=int(diag[0]), margin=float(diag[1]))


def calibrate_step(conf_logits, verify_len, accept_len, inv_temp, step=1.0, ridge=1e-3):
    """One online calibration step (see oracle_calibrate_step in dspark_oracle.c).

    Returns the updated inverse temperatures [K] float64 (the input is not modified)."""
    c = _np(conf_logits, np.float32)
    B, K = c.shape
    vl = _np(verify_len, np.int32)
    al = _np(accept_len, np.int32)
    th = np.array(_np(inv_temp, np.float64), dtype=np.float64, copy=True)
    st = lib().oracle_calibrate_step(B, K, _ptr(c), _ptr(vl), _ptr(al), float(step), float(ridge),
                                     _ptr(th))
    if st != 0:
        raise ValueError("oracle_calibrate_step: invalid argument")
    return th


def ece(s, y, n_bins=10):
    """Expected calibration error (see oracle_ece in dspark_oracle.c)."""
    s = np.ascontiguousarray(np.asarray(s, dtype=np.float64).ravel())
    y = np.ascontiguousarray(np.asarray(y, dtype=np.float64).ravel())
    assert s.shape == y.shape
    return float(lib().oracle_ece(len(s), _ptr(s), _ptr(y), int(n_bins)))


def verify(Y, draft_tokens, q_tok, q_lse, Z, U, W, prev_token, verify_len, temperature, seed,
           req_id=None, rows=None, head_state=None, sampler="token"):
    """Rejection-sampling verification (see oracle_verify_head in dspark_oracle.c).

    sampler: "token" (per-token Gumbel-max draws) or "block16" (the two-level block race).

    Y [B,K+1,V] (float32 or bfloat16); draft_tokens [B,K]; q_tok, q_lse [B,K] (taken as
    float32, the precision the draft hands over); Z, U, W, prev_token as for draft_block;
    head_state [B,K,r] (uint16 bfloat16 bits, or a bfloat16 tensor) from a recurrent-head
    draft, or None for the Markov head.
    Returns dict(accept_len [n], next_token [n], p_tok [n,K], accept_margin [n],
    sample_margin [n]) for the listed rows (all by default)."""
    B = int(Y.shape[0])
    rows = np.arange(B) if rows is None else np.asarray(rows, dtype=np.int64)
    n = len(rows)
    y, ydt = _as_logits(_subset(Y, rows))
    z, zdt = _as_logits(_subset(Z, rows))
    u, udt = _as_logits(U)
    w, wdt = _as_logits(W)
    assert udt == wdt
    K = z.shape[1]
    V = z.shape[2]
    r = u.shape[1]
    assert y.shape[1] == K + 1 and y.shape[2] == V
    toks = _np(draft_tokens, np.int32)[rows]
    qt = _np(q_tok, np.float32)[rows]
    ql = _np(q_lse, np.float32)[rows]
    prev = _np(prev_token, np.int32)[rows]
    vl = _np(verify_len, np.int32)[rows]
    temp = _np(temperature, np.float32)[rows]
    req = (rows.astype(np.uint32) if req_id is None else _np(req_id, np.uint32)[rows])
    req = np.ascontiguousarray(req, dtype=np.uint32)
    sub_rows = np.arange(n, dtype=np.int32)
    acc = np.empty(n, np.int32)
    nxt = np.empty(n, np.int32)
    p_tok = np.zeros((n, K), np.float64)
    diag = np.empty((n, 2), np.float64)
    hs = None
    if head_state is not None:
        hs, hdt = _as_logits(_subset(head_state, rows))
        assert hdt == BF16 and hs.shape == (n, K, r), "head_state is [B,K,r] bfloat16"
    st = lib().oracle_verify_head(n, K, V, r, ydt, _ptr(y), _ptr(toks), _ptr(qt), _ptr(ql), zdt,
                                  _ptr(z), udt, _ptr(u), _ptr(w), _ptr(hs), _ptr(prev), _ptr(vl),
                                  _ptr(temp), _ptr(req), C.c_uint64(seed), _ptr(sub_rows), n,
                                  _ptr(acc), _ptr(nxt), _ptr(p_tok), _ptr(diag),
                                  SAMPLERS[sampler])
    if st != 0:
        raise ValueError("oracle_verify: token index out of range")
    return dict(accept_len=acc, next_token=nxt, p_tok=p_tok, accept_margin=diag[:, 0],
                sample_margin=diag[:, 1])


def num_threads() -> int:
    return int(lib().oracle_num_threads())

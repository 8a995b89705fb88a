"""Seeded synthetic workloads for the draft / schedule / verify round.

This module only draws random numbers and lays them out.  It holds none of the method's
arithmetic: it never forms the Markov bias, a softmax, a survival product or an accept test.
The target logits of a workload are "corrected draft logits plus noise"; the corrected part
depends on the draft chain and is therefore supplied by the caller (the oracle in the tests,
the library itself in the benchmark) to ``target_logits``, which only adds the noise drawn
here and casts.

Workloads (the pages name no dataset for this path; these shapes stand in for the serving
traffic the articles describe, with a vocabulary of 151936 or 262144 and rank-256 factors):

  tiny        B=4   K=4  V=1024   r=16  fp32 everything; base 2N(0,1) + 6 on one id per row;
              target noise 0.5; confidence N(1,1); linear throughput profile; greedy or T=1.
  single      B=1   K=8  V=151936 r=256 bf16 base/factors, fp32 target; Zipf peak; noise 0.3;
              greedy; scheduling off.
  moderate    B=64  K=16 V=151936 r=256 bf16 base/factors/target; Zipf; noise 0.6; T=1;
              confidence N(1.5,1) - 0.15k; scheduling off.
  concurrent  B=512 K=16 V=151936 r=256 bf16 base/factors/target; Zipf; noise 0.3 for the
              first half of the requests, 1.0 for the rest; T=0.8; confidence as moderate;
              scheduling on with a throughput knee at 2048 tokens.
  ragged      B=256 K=16 V=262144 r=256 bf16 base/factors, fp32 target; Zipf; noise 0.5;
              draft lengths uniform in [2,16]; temperature per request from {0, 0.7, 1.0};
              verify length = draft length.
  headline    B=256 K=16 V=151936 r=256 bf16 base/factors, fp32 target; Zipf; noise 0.6;
              T=1; confidence as moderate; scheduling off.
  headline_sched  the headline inputs with scheduling on against the concurrent workload's
              knee profile.

Factor entries are N(0, sd) with sd = 0.5/sqrt(r) ("std" reading).  ``strong_bias=True`` uses
sd = sqrt(0.5/sqrt(r)) instead (the "variance" reading), which makes the Markov bias large
enough to change which token wins; it is used to exercise the token chain.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

KNEE_PROFILE = ((1.0, 1e5 / 2048.0), (2048.0, 1e5), (8704.0, 1e5))
LINEAR_PROFILE = ((4.0, 600.0), (20.0, 2200.0))


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    K: int
    V: int
    r: int
    z_dtype: torch.dtype
    uw_dtype: torch.dtype
    y_dtype: torch.dtype
    base: str  # "one_hot6" or "zipf"
    noise: tuple  # sigma for the first half / second half of the requests
    conf: tuple  # (mean, sd, per-position decay)
    temperature: tuple  # choices; one value means every request uses it
    ragged: bool  # draft lengths uniform in [2, K]
    schedule: bool
    profile: tuple = field(default=())
    data_seed: int = 0
    philox_seed: int = 0


BF16, F32 = torch.bfloat16, torch.float32

WORKLOADS = {
    "tiny": Workload("tiny", 4, 4, 1024, 16, F32, F32, F32, "one_hot6", (0.5, 0.5), (1.0, 1.0, 0.0),
                     (1.0,), False, True, LINEAR_PROFILE, 101, 0xD5A0000000000001),
    "single": Workload("single", 1, 8, 151936, 256, BF16, BF16, F32, "zipf", (0.3, 0.3),
                       (1.0, 1.0, 0.0), (0.0,), False, False, (), 102, 0xD5A0000000000002),
    "moderate": Workload("moderate", 64, 16, 151936, 256, BF16, BF16, BF16, "zipf", (0.6, 0.6),
                         (1.5, 1.0, 0.15), (1.0,), False, False, (), 103, 0xD5A0000000000003),
    "concurrent": Workload("concurrent", 512, 16, 151936, 256, BF16, BF16, BF16, "zipf",
                           (0.3, 1.0), (1.5, 1.0, 0.15), (0.8,), False, True, KNEE_PROFILE, 104,
                           0xD5A0000000000004),
    "ragged": Workload("ragged", 256, 16, 262144, 256, BF16, BF16, F32, "zipf", (0.5, 0.5),
                       (1.5, 1.0, 0.15), (0.0, 0.7, 1.0), True, False, (), 105, 0xD5A0000000000005),
    "headline": Workload("headline", 256, 16, 151936, 256, BF16, BF16, F32, "zipf", (0.6, 0.6),
                         (1.5, 1.0, 0.15), (1.0,), False, False, (), 106, 0xD5A0000000000006),
    # the headline inputs with the confidence schedule on, against the knee profile
    "headline_sched": Workload("headline_sched", 256, 16, 151936, 256, BF16, BF16, F32, "zipf",
                               (0.6, 0.6), (1.5, 1.0, 0.15), (1.0,), False, True, KNEE_PROFILE,
                               106, 0xD5A0000000000006),
}


def shrink(w: Workload, **kw) -> Workload:
    """Same recipe at other sizes (used for oracle-sized parity cases)."""
    d = dict(w.__dict__)
    d.update(kw)
    return Workload(**d)


def _distinct_ids(gen, rows: int, count: int, V: int, device) -> torch.Tensor:
    """`count` distinct ids in [0, V) per row (Floyd's sampling, vectorised over rows)."""
    chosen = torch.empty(rows, count, dtype=torch.long, device=device)
    for i, j in enumerate(range(V - count, V)):
        t = torch.randint(0, j + 1, (rows,), generator=gen, device=device)
        dup = (chosen[:, :i] == t[:, None]).any(dim=1) if i else torch.zeros_like(t, dtype=torch.bool)
        chosen[:, i] = torch.where(dup, torch.full_like(t, j), t)
    return chosen


def make_inputs(w: Workload, device="cpu", temperature=None, strong_bias=False) -> dict:
    """Draw every input of one round of workload `w` on `device` (seeded by w.data_seed).

    Returns a dict of tensors:
      Z_ext [B,K+1,V] base logits (rows 0..K-1 feed the draft; row K is the extra base row the
            bonus position's target logits are built on), Z = Z_ext[:, :K] (a view),
      U, W [V,r] factors (row v of W is column v of the r x V right factor),
      prev_token [B] int32, draft_len [B] int32, temperature [B] float32, req_id [B] int32,
      conf_logits [B,K] float32, noise [B,K+1,V] float32 (already scaled by each request's
      sigma), knot_tokens / knot_tps float64 (empty when scheduling is off), seed (int).
    `temperature` overrides the workload's temperature for every request.
    """
    B, K, V, r = w.B, w.K, w.V, w.r
    gen = torch.Generator(device=device)
    gen.manual_seed(w.data_seed)
    rows = B * (K + 1)

    z = 2.0 * torch.randn(B, K + 1, V, generator=gen, device=device, dtype=torch.float32)
    zf = z.view(rows, V)
    if w.base == "one_hot6":
        ids = torch.randint(0, V, (rows,), generator=gen, device=device)
        zf[torch.arange(rows, device=device), ids] += 6.0
    elif w.base == "zipf":
        ids = _distinct_ids(gen, rows, 32, V, device)
        boost = 8.0 / torch.arange(1, 33, device=device, dtype=torch.float32)
        zf.scatter_add_(1, ids, boost.expand(rows, 32).contiguous())
    else:
        raise ValueError(w.base)
    Z_ext = z.to(w.z_dtype)
    del z, zf

    sd = math.sqrt(0.5 / math.sqrt(r)) if strong_bias else 0.5 / math.sqrt(r)
    U = (sd * torch.randn(V, r, generator=gen, device=device)).to(w.uw_dtype)
    W = (sd * torch.randn(V, r, generator=gen, device=device)).to(w.uw_dtype)

    prev_token = torch.randint(0, V, (B,), generator=gen, device=device, dtype=torch.int32)
    mean, csd, decay = w.conf
    kpos = torch.arange(K, device=device, dtype=torch.float32)
    conf = mean + csd * torch.randn(B, K, generator=gen, device=device) - decay * kpos

    sig = torch.full((B,), w.noise[0], device=device)
    sig[B // 2:] = w.noise[1]
    noise = torch.randn(B, K + 1, V, generator=gen, device=device) * sig[:, None, None]

    if temperature is not None:
        temp = torch.full((B,), float(temperature), device=device)
    elif len(w.temperature) == 1:
        temp = torch.full((B,), float(w.temperature[0]), device=device)
    else:
        choice = torch.randint(0, len(w.temperature), (B,), generator=gen, device=device)
        temp = torch.tensor(w.temperature, device=device, dtype=torch.float32)[choice]
    if w.ragged:
        draft_len = torch.randint(2, K + 1, (B,), generator=gen, device=device, dtype=torch.int32)
    else:
        draft_len = torch.full((B,), K, device=device, dtype=torch.int32)
    req_id = torch.arange(B, device=device, dtype=torch.int32) + 1000 * (w.data_seed - 100)
    kt = torch.tensor([k[0] for k in w.profile], dtype=torch.float64, device=device)
    kp = torch.tensor([k[1] for k in w.profile], dtype=torch.float64, device=device)
    return dict(Z_ext=Z_ext, Z=Z_ext[:, :K], U=U, W=W, prev_token=prev_token, draft_len=draft_len,
                temperature=temp.float(), req_id=req_id, conf_logits=conf.float(), noise=noise,
                knot_tokens=kt, knot_tps=kp, seed=w.philox_seed, workload=w)


def target_logits(corrected_ext: torch.Tensor, noise: torch.Tensor, dtype: torch.dtype):
    """Target logits of the workload: corrected draft logits [B,K+1,V] plus the drawn noise."""
    return (corrected_ext.float() + noise.to(corrected_ext.device)).to(dtype)


def make_gru(r: int, seed: int, device="cpu") -> tuple:
    """Seeded weights of a recurrent head's GRU cell: Wi, Wh [3r, r] and bi, bh [3r], float32,
    uniform in (-1/sqrt(r), 1/sqrt(r)) (the usual initialisation of a GRU of width r)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    a = 1.0 / float(r) ** 0.5

    def u(*shape):
        return (2.0 * torch.rand(*shape, generator=gen, device=device) - 1.0) * a

    return u(3 * r, r), u(3 * r, r), u(3 * r), u(3 * r)

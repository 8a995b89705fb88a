import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU statistics test")


def pytest_sessionfinish(session, exitstatus):
    """Write the parity tallies (near-ties counted by tests/parity.py) as JSON lines into
    $DSPARK_TALLY_DIR/parity_tallies.jsonl when that variable names a directory."""
    out_dir = os.environ.get("DSPARK_TALLY_DIR")
    if not out_dir:
        return
    try:
        import json
        import parity
    except Exception:
        return
    if not parity.REPORTS:
        return
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "parity_tallies.jsonl"), "a") as f:
        for r in parity.REPORTS:
            f.write(json.dumps(r) + "\n")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


PIN_SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "pins", "rocrand_philox_pin.cpp")


@pytest.fixture(scope="session")
def rocrand_pin():
    """rocRAND's public host-callable Philox4x32-10 engine, built from its installed header and
    run as a separate program: run(keys [n,2], ctrs [n,4]) -> the four output words [n,4]."""
    import numpy as np
    out = os.path.join(tempfile.gettempdir(), "dspark_rocrand_pin")
    if not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(PIN_SRC):
        subprocess.run(["hipcc", "-O1", PIN_SRC, "-o", out], check=True,
                       stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)

    def run(keys, ctrs):
        lines = "".join(
            f"{k[0]:08x} {k[1]:08x} {c[0]:08x} {c[1]:08x} {c[2]:08x} {c[3]:08x}\n"
            for k, c in zip(keys, ctrs))
        res = subprocess.run([out], input=lines, capture_output=True, text=True, check=True)
        return np.array([[int(w, 16) for w in ln.split()] for ln in res.stdout.strip().splitlines()],
                        dtype=np.uint64).astype(np.uint32)
    return run


@pytest.fixture(scope="session")
def rocrand_gumbel(rocrand_pin):
    """Gumbel draws of tokens 0..n-1 at (seed, request key, position, stream) computed from
    rocRAND's Philox words with the documented keying: word v & 3 of the block at counter
    (v >> 2, position, request key, stream) under key (seed low, seed high),
    u = ((word >> 8) + 0.5) 2^-24, G = -log(-log u)."""
    import numpy as np

    def gumbel(seed, req, pos, n, stream):
        v = np.arange(n)
        key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint64).astype(np.uint32)
        ctrs = np.stack([v >> 2, np.full(n, pos), np.full(n, req), np.full(n, stream)],
                        1).astype(np.uint32)
        words = rocrand_pin(np.repeat(key[None], n, 0), ctrs)[v, v & 3]
        u = ((words >> 8).astype(np.float64) + 0.5) / 2.0**24
        return -np.log(-np.log(u))
    return gumbel

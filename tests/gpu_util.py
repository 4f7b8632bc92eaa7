"""Helpers for the GPU parity tests: run the HIP path, compare with the oracle.

Tolerances (floating point, element by element):
  out       |gpu - ref| <= 2e-3 + 1e-2 |ref|
  page mass |gpu - ref| <= 1e-4
  lse       |gpu - ref| <= 1e-3 + 1e-4 |ref|     (-inf must match exactly)
  s_next    |gpu - ref| <= 1e-6 + 1e-6 |ref|
  page max  |gpu - ref| <= 1e-4 + 1e-4 |ref|     (-inf must match exactly)
Queue, offsets and indexing are compared bit for bit.
"""

import sys

import numpy as np

from oracle import kvref

TOL = {
    "out": (2e-3, 1e-2),
    "mass": (1e-4, 0.0),
    "lse": (1e-3, 1e-4),
    "s_next": (1e-6, 1e-6),
    "page_max": (1e-4, 1e-4),
}


def say(*args):
    """Name the case before a GPU step, flushed so it survives a crash."""
    print("[gpu-case]", *args, flush=True)
    sys.stdout.flush()


def assert_close(name, got, ref, mask=None):
    atol, rtol = TOL[name]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    sel = ~np.isnan(ref) if mask is None else (mask & ~np.isnan(ref))
    ninf = sel & np.isinf(ref)
    if np.any(ninf):
        assert np.array_equal(got[ninf], ref[ninf]), f"{name}: infinite entries differ"
    fin = sel & np.isfinite(ref)
    assert np.all(np.isfinite(got[fin])), f"{name}: non-finite where reference is finite"
    err = np.abs(got[fin] - ref[fin])
    bound = atol + rtol * np.abs(ref[fin])
    bad = err > bound
    if np.any(bad):
        i = np.argmax(err - bound)
        raise AssertionError(f"{name}: {bad.sum()} of {fin.sum()} entries out of tolerance; "
                             f"worst err {err[i]:.3e} vs bound {bound[i]:.3e} (ref {ref[fin][i]:.4e})")
    return float(err.max()) if err.size else 0.0


def compare_step(res, ref, budget=True, rows=None, label=""):
    """Compare a DecodeStep result with an oracle step (optionally on rows)."""
    assert res["n_tasks"] == ref["n_tasks"], label
    assert np.array_equal(res["tasks"], ref["tasks"]), label
    assert np.array_equal(res["group_offsets"], ref["group_offsets"]), label
    errs = {}
    errs["out"] = assert_close("out", res["out"], ref["out"])
    errs["lse"] = assert_close("lse", res["lse"], ref["lse"])
    if budget:
        errs["mass"] = assert_close("mass", res["mass"], ref["mass"])
        errs["s_next"] = assert_close("s_next", res["s_next"], ref["s_next"])
        errs["page_max"] = assert_close("page_max", res["page_max"], ref["page_max"])
    return errs


def sample_rows(wl, n, seed=0):
    """n (b, h) rows: the longest and shortest sequences plus random ones."""
    rng = np.random.default_rng(seed)
    rows = {(int(np.argmax(wl.ctx_lens)), 0), (int(np.argmin(wl.ctx_lens)), wl.Hq - 1)}
    while len(rows) < n:
        rows.add((int(rng.integers(0, wl.B)), int(rng.integers(0, wl.Hq))))
    return sorted(rows)


def group_rows(wl, extra=0, seed=0):
    """One query head of every (sequence, KV head) group (the head index
    rotates with b + g), plus ``extra`` sampled rows."""
    rows = {(b, g * wl.G + (b + g) % wl.G) for b in range(wl.B) for g in range(wl.Hkv)}
    if extra:
        rows |= set(sample_rows(wl, extra, seed))
    return sorted(rows)


def oracle_step(wl, rows=None, q=None, s_prev=None, split_tokens=None):
    if split_tokens is not None and split_tokens != wl.split_tokens:
        import dataclasses
        wl = dataclasses.replace(wl, split_tokens=split_tokens)
    return kvref.decode_step(wl, rows=rows, q=q, s_prev=s_prev)

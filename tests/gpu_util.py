"""Helpers for GPU tests: moving seeded numpy inputs to the device and back,
and the attention tolerance.

Tolerances (element-wise, |o - r| <= atol + rtol * |r| against the fp64
oracle):
  bf16 inputs: atol 2e-3, rtol 1e-2 -- the bound the decode path is held to;
               bf16 output rounding alone is <= 2^-9 |r| ~ 2e-3 |r|.
  fp32 inputs: atol 1e-4, rtol 1e-4 -- fp32 accumulation over <= 32768
               tokens of head_dim <= 128 products leaves errors near 1e-6;
               the bound keeps two orders of magnitude of headroom while
               staying 20x tighter than the bf16 one.
"""

from __future__ import annotations

import numpy as np
import torch

TOL = {"bf16": (2e-3, 1e-2), "f32": (1e-4, 1e-4)}


def dev(a: np.ndarray, dtype: str = None, device="cuda"):
    """numpy -> device tensor.  uint16 arrays become bfloat16 (same bits)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def host(t) -> np.ndarray:
    """device tensor -> numpy; bfloat16 comes back as uint16 bits."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def check_close(out_bits: np.ndarray, ref: np.ndarray, dtype: str, where=None):
    """Assert the tolerance; return (max_abs, max_rel over |r| >= 0.2)."""
    o = as_f64(out_bits)
    if where is not None:
        o, ref = o[where], ref[where]
    atol, rtol = TOL[dtype]
    err = np.abs(o - ref)
    bad = ~(err <= atol + rtol * np.abs(ref))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{int(bad.sum())} elements out of tolerance ({dtype}); first at {idx.tolist()}: "
            f"got {o[tuple(idx[0])]}, want {ref[tuple(idx[0])]}")
    big = np.abs(ref) >= 0.2
    max_rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    return float(err.max()) if err.size else 0.0, max_rel


def scatter_histories(pool_shape, dtype: str, tables, lens, hist_k, hist_v, B: int):
    """Expected pools: token t of sequence i at block tables[i][t // B], offset
    t % B; every other slot 0."""
    import datagen

    kc = np.zeros(pool_shape, dtype=datagen.np_dtype(dtype))
    vc = np.zeros(pool_shape, dtype=datagen.np_dtype(dtype))
    for i, n in enumerate(lens):
        n = int(n)
        t = np.arange(n)
        blk = np.asarray(tables[i])[t // B]
        kc[blk, :, t % B, :] = hist_k[i][:n]
        vc[blk, :, t % B, :] = hist_v[i][:n]
    return kc, vc


def live_rows(pool: np.ndarray, tables, lens, B: int) -> np.ndarray:
    """Rows [tokens, Hkv, D] of every sequence's live slots, concatenated."""
    rows = []
    for i, n in enumerate(lens):
        t = np.arange(int(n))
        rows.append(pool[np.asarray(tables[i])[t // B], :, t % B, :])
    return np.concatenate(rows)

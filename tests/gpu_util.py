"""Helpers shared by the GPU tests: device copies of seeded inputs, error
metrics, TwELL arrays to numpy."""
import sys

import numpy as np

from workloads import bf16_bits


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def rel_fro(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def mat_to_numpy(m):
    """Host copies of a TwellMat's arrays (val as float32 or raw bf16 bits)."""
    import torch
    out = {
        "cnt": m.cnt.cpu().numpy().astype(np.int64),
        "width": m.width.cpu().numpy().astype(np.int64),
        "idx": m.idx.cpu().numpy(),
        "mask": None if m.mask is None else m.mask.cpu().numpy().view(np.uint64),
    }
    if m.val.dtype == torch.bfloat16:
        out["val_bits"] = m.val.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        out["val_bits"] = m.val.cpu().numpy().view(np.uint32)
    return out


def masks_from_positive(P: np.ndarray, C: int = 64) -> np.ndarray:
    """[T, F] boolean -> [T, F/C] uint64 bitmaps (bit c = column j*C+c)."""
    T, F = P.shape
    w = (np.uint64(1) << np.arange(C, dtype=np.uint64))
    return (P.reshape(T, F // C, C).astype(np.uint64) * w).sum(axis=2, dtype=np.uint64)


def oracle_val_bits(val: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits(val.astype(np.float32))
    return np.ascontiguousarray(val.astype(np.float32)).view(np.uint32)


def compare_twell(gpu: dict, ref, dtype: str, row_tiles=None, rows=None):
    """Bit-exact comparison of a GPU TwELL against the oracle's on the listed
    row tiles (all if None): counts, widths, and every slot below the width."""
    NR = ref.width.shape[0]
    tiles = np.arange(NR) if row_tiles is None else np.asarray(row_tiles)
    rows_all = np.arange(ref.T) if rows is None else np.asarray(rows)
    np.testing.assert_array_equal(gpu["cnt"][rows_all], ref.cnt[rows_all], err_msg="cnt")
    np.testing.assert_array_equal(gpu["width"][tiles], ref.width[tiles], err_msg="width")
    vref = oracle_val_bits(ref.val, dtype)
    for i in tiles:
        for j in range(ref.width.shape[1]):
            w = int(ref.width[i, j])
            if w == 0:
                continue
            np.testing.assert_array_equal(gpu["idx"][i, j, :w], ref.idx[i, j, :w], err_msg=f"idx tile {i},{j}")
            np.testing.assert_array_equal(gpu["val_bits"][i, j, :w], vref[i, j, :w], err_msg=f"val tile {i},{j}")

"""Helpers shared by the GPU parity tests (device transfer, oracle operands)."""
import numpy as np


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a: np.ndarray):
    """numpy (uint16 BF16 patterns / uint8 / int / float) -> cuda tensor, bits unchanged."""
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def upload_nvfp4(q, bbs, n_scales=None):
    """Oracle NVFP4 copy -> device NVFP4Tensor with the same bytes."""
    import torch
    s = np.atleast_1d(np.asarray(q.s_dec if n_scales is None else n_scales, np.float32))
    return bbs.NVFP4Tensor(to_dev(q.codes), to_dev(q.scales), to_dev(s), q.rows, q.cols,
                           q.tile2d)


def upload_mxfp8(m, bbs):
    return bbs.MXFP8Tensor(to_dev(m.codes), to_dev(m.scales), m.rows, m.cols)


def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def announce(msg: str):
    print(f"\n[gpu case] {msg}", flush=True)


# ---------------------------------------------------------------------------
# Accumulation bounds.  An FP32 sum of K exact products, in any order, with
# one more rounding for the output scale, differs from the exact sum by at
# most (K + 4) * 2^-24 * sum |a_k b_k| (the standard bound gamma_n for
# recursive summation, with margin).  The GEMM operands' products are exact
# in FP32 (FP16 x FP16 expansions of NVFP4, E4M3 x E4M3 for MXFP8).
# ---------------------------------------------------------------------------

def accumulation_bound(abs_sum, K):
    return (K + 4) * 2.0 ** -24 * np.asarray(abs_sum, np.float64)


def bf16_key(bits):
    """BF16 bit patterns -> integers ordered like their values (+-0 -> 0)."""
    b = np.asarray(bits, np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def bf16_from_key(key):
    k = np.asarray(key, np.int64)
    return np.where(k < 0, (-k) | 0x8000, k).astype(np.uint16)


def bf16_bits_of(v):
    """Float values that are BF16 numbers -> their bit patterns."""
    return (np.asarray(v, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_window(y64, E):
    """Keys of the lowest and highest BF16 value an FP32 accumulation within
    E of y64, rounded to BF16 (nearest even), can give."""
    import oracle as O
    return (bf16_key(bf16_bits_of(O.bf16_rne(np.asarray(y64) - E))),
            bf16_key(bf16_bits_of(O.bf16_rne(np.asarray(y64) + E))))


def check_bounded_outputs(y, y64, E, bf16, what, tiles=None):
    """Each output within its bound: FP32 |y - y64| <= E; BF16 y inside the
    BF16 rounding of [y64 - E, y64 + E].  Reports the global relative
    Frobenius error and, with `tiles` (the tile id of every sample), the
    worst per-tile normalised deviation; returns that worst value."""
    import oracle as O
    y = np.asarray(y, np.float64)
    ref = O.bf16_rne(y64) if bf16 else np.asarray(y64, np.float64)
    err = O.rel_fro(y, ref)
    if bf16:
        lo, hi = bf16_window(y64, E)
        k = bf16_key(bf16_bits_of(y))
        inside = (k >= lo) & (k <= hi)
        dev_ = np.abs(y - y64) / np.maximum(E, 1e-300)
    else:
        dev_ = np.abs(y - y64) / np.maximum(E, 1e-300)
        inside = np.abs(y - y64) <= E
    worst = float(dev_.max()) if dev_.size else 0.0
    if tiles is not None and dev_.size:
        per = np.zeros(int(tiles.max()) + 1)
        np.maximum.at(per, tiles, dev_)
        worst_tile = int(per.argmax())
        print(f"  {what}: rel err {err:.3e}; {int(np.unique(tiles).size)} tiles sampled; "
              f"worst tile {worst_tile}: |y - ref| / bound {per[worst_tile]:.3f}", flush=True)
    else:
        print(f"  {what}: rel err {err:.3e}; worst |y - ref| / bound {worst:.3f}", flush=True)
    bad = np.nonzero(~inside)[0]
    assert bad.size == 0, (f"{what}: {bad.size} outputs outside their accumulation bound, "
                           f"first sample {int(bad[0])}: y={y[bad[0]]} ref={y64[bad[0]]} "
                           f"bound={E[bad[0]]}")
    assert err <= 1e-3, f"{what}: relative error {err}"
    return worst


def tile_samples(M, N, per_tile, seed, tile=256, extra=None):
    """(rows, cols, tile ids): per_tile random outputs inside every tile x
    tile output tile, plus the last row and column when given `extra`."""
    rng = np.random.default_rng(seed)
    tm, tn = (M + tile - 1) // tile, (N + tile - 1) // tile
    ti = np.repeat(np.arange(tm), tn * per_tile)
    tj = np.tile(np.repeat(np.arange(tn), per_tile), tm)
    rows = ti * tile + rng.integers(0, tile, ti.size)
    cols = tj * tile + rng.integers(0, tile, tj.size)
    keep = (rows < M) & (cols < N)
    rows, cols = rows[keep], cols[keep]
    if extra:
        r2 = np.concatenate([np.full(N, M - 1), rng.integers(0, M, extra)])
        c2 = np.concatenate([np.arange(N), rng.integers(0, N, extra)])
        rows, cols = np.concatenate([rows, r2]), np.concatenate([cols, c2])
    return rows.astype(np.int64), cols.astype(np.int64), (rows // tile) * tn + cols // tile

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

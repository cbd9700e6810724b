"""Seeded synthetic inputs for the NVFP4 quantized-linear workloads.

This module only draws random numbers and rounds them to BF16 storage; it
holds none of the quantization arithmetic.  Both the HIP path (through the
tests and the benchmark) and the CPU oracle consume what it produces.

Shapes and distributions follow the five workloads of the hot path:
  tiny linear      X, W [256 x 256] N(0,1), 0.5% of entries scaled by 20
  activation SR    X [4096 x 4096] Student-t with 3 degrees of freedom
  dense forward    X [8192 x 4096] N(0,1) + 0.5% x20 outliers, W [14336 x 4096] N(0, 0.02)
  backward         dY [8192 x 14336] Laplace, std 1e-3
  MoE forward      X [65536 x 4096] as above, 64 experts, top-8 of Zipf(1.1),
                   W_up[g] [1536 x 4096], W_down[g] [4096 x 1536] N(0, 0.02)
  MLP hidden       H [8192 x 14336], the pre-activation between the dense
                   layer's two projections: N(0,1) + 0.5% x20 outliers
  MoE combine      Y [524288 x 4096], the routed expert outputs of the MoE
                   forward in expert order (N(0,1) + 0.35% x10 outliers:
                   kurtosis about 55, near the 59 of the pages' MLP outputs),
                   each token's 8 rows and gate weights (softmax of N(0,1))
All generators are numpy PCG64 seeded with fixed integers.
"""
import numpy as np


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float -> float32 -> BF16 bit patterns (uint16), round to nearest even."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    b = f.view(np.uint32)
    r = ((b >> 16) & 1) + np.uint32(0x7FFF)
    return ((b + r) >> 16).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_with_outliers(rows: int, cols: int, seed: int, frac: float = 0.005,
                         factor: float = 20.0) -> np.ndarray:
    """N(0,1) BF16 matrix with round(frac * n) distinct entries multiplied by `factor`."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    n = rows * cols
    k = int(round(frac * n))
    pos = rng.choice(n, size=k, replace=False)
    x.reshape(-1)[pos] *= np.float32(factor)
    return bf16_bits(x)


def normal(rows: int, cols: int, seed: int, std: float) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
    return bf16_bits(x)


def student_t(rows: int, cols: int, seed: int, df: float = 3.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return bf16_bits(rng.standard_t(df, size=(rows, cols)))


def laplace(rows: int, cols: int, seed: int, std: float) -> np.ndarray:
    """Laplace with the given standard deviation (scale b = std / sqrt(2))."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((rows, cols), np.uint16)
    step = max(1, (1 << 24) // cols)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = bf16_bits(rng.laplace(0.0, std / np.sqrt(2.0), size=(r1 - r0, cols)))
    return out


def rht_signs(seed: int) -> int:
    """The one fixed random sign vector of the 16-point RHT, as a 16-bit mask."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return int(rng.integers(0, 1 << 16))


def moe_routing(tokens: int, experts: int, topk: int, seed: int, zipf_s: float = 1.1,
                n_empty: int = 4):
    """Top-k routing drawn from a Zipf(zipf_s) law over a seeded expert order.

    The n_empty lowest-ranked experts get probability 0, so those groups are
    empty.  Returns (row_index, group_offsets): row_index[i] is the token of the
    i-th routed row when rows are sorted by expert; rows of expert g occupy
    [group_offsets[g], group_offsets[g+1])."""
    rng = np.random.Generator(np.random.PCG64(seed))
    order = rng.permutation(experts)
    rank = np.empty(experts, np.int64)
    rank[order] = np.arange(experts)
    p = 1.0 / np.power(rank + 1.0, zipf_s)
    p[rank >= experts - n_empty] = 0.0
    p /= p.sum()
    logp = np.where(p > 0, np.log(np.maximum(p, 1e-300)), -np.inf)
    chosen = np.empty((tokens, topk), np.int64)
    step = 8192
    for t0 in range(0, tokens, step):
        t1 = min(tokens, t0 + step)
        g = rng.gumbel(size=(t1 - t0, experts))
        score = logp[None, :] + g
        chosen[t0:t1] = np.argpartition(-score, topk - 1, axis=1)[:, :topk]
    tok = np.repeat(np.arange(tokens, dtype=np.int64), topk)
    exp = chosen.reshape(-1)
    perm = np.lexsort((tok, exp))
    row_index = tok[perm].astype(np.int32)
    counts = np.bincount(exp, minlength=experts)
    offsets = np.zeros(experts + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    return row_index, offsets


# --------------------------------------------------------------------------
# The five workloads (seeds fixed here, shared by tests and benchmark)
# --------------------------------------------------------------------------

def tiny_linear():
    return {"x": normal_with_outliers(256, 256, 101), "w": normal_with_outliers(256, 256, 102)}


SR_SEED_ACT = 0x2001


def activation_sr(rows: int = 4096, cols: int = 4096):
    return {"x": student_t(rows, cols, 201), "seed": SR_SEED_ACT, "row_stream": 0,
            "col_stream": 1}


def dense_forward(m: int = 8192, k: int = 4096, n: int = 14336):
    return {"x": normal_with_outliers(m, k, 301), "w": normal(n, k, 302, 0.02)}


def combine_values(rows: int, cols: int, seed: int, frac: float = 0.0035,
                   factor: float = 10.0, chunk_rows: int = 4096) -> np.ndarray:
    """BF16 [rows, cols]: N(0,1) with about a fraction `frac` of the entries
    (binomial count, uniform positions) multiplied by `factor`, drawn in row
    chunks (bounded memory)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((rows, cols), np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0) * cols, dtype=np.float32)
        hit = rng.integers(0, x.size, rng.binomial(x.size, frac))
        x[hit] *= np.float32(factor)
        out[r0:r1] = bf16_bits(x).reshape(r1 - r0, cols)
    return out


def combine_values_device(rows: int, cols: int, seed: int, device, frac: float = 0.0035,
                          factor: float = 10.0, chunk_rows: int = 65536):
    """The same distribution as combine_values, drawn on a GPU with torch's
    seeded generator (for sizes the host would take minutes to draw); BF16
    bit patterns as an int16 device tensor."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty((rows, cols), dtype=torch.int16, device=device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = torch.randn((r1 - r0, cols), generator=g, device=device, dtype=torch.float32)
        hit = torch.rand((r1 - r0, cols), generator=g, device=device) < frac
        x = torch.where(hit, x * factor, x)
        out[r0:r1] = x.to(torch.bfloat16).view(torch.int16)
    return out


def moe_combine(tokens: int = 65536, hidden: int = 4096, experts: int = 64, topk: int = 8,
                device=None):
    """Combine inputs of the MoE layer: expert outputs in expert order (a
    device tensor when device is given), the rows of each token (src[t, j])
    and its gate weights."""
    row_index, _ = moe_routing(tokens, experts, topk, 502)
    src = np.argsort(row_index, kind="stable").astype(np.int32).reshape(tokens, topk)
    rng = np.random.Generator(np.random.PCG64(702))
    g = rng.standard_normal((tokens, topk))
    w = np.exp(g - g.max(axis=1, keepdims=True))
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    if device is None:
        y = combine_values(tokens * topk, hidden, 701)
    else:
        y = combine_values_device(tokens * topk, hidden, 701, device)
    return {"y": y, "src": src, "w": w, "signs": int(rng.integers(0, 1 << 32))}


MLP_SEEDS = {"mx8": 602}


def mlp_hidden(m: int = 8192, n: int = 14336):
    return {"h": normal_with_outliers(m, n, 601), "seeds": MLP_SEEDS}


BWD_SEEDS = {"dy_col": 403, "dy_mx8": 404, "x_col": 405, "w_req": 406}


def backward(m: int = 8192, n: int = 14336):
    return {"dy": laplace(m, n, 401, 1e-3), "rht_signs": rht_signs(402), "seeds": BWD_SEEDS}


def moe_weights(experts: int, rows: int, cols: int, seed0: int):
    return [normal(rows, cols, seed0 + g, 0.02) for g in range(experts)]


def moe_forward(tokens: int = 65536, hidden: int = 4096, ffn: int = 1536, experts: int = 64,
                topk: int = 8, with_weights: bool = True):
    d = {"x": normal_with_outliers(tokens, hidden, 501)}
    d["row_index"], d["group_offsets"] = moe_routing(tokens, experts, topk, 502)
    if with_weights:
        d["w_up"] = moe_weights(experts, ffn, hidden, 503)
        d["w_down"] = moe_weights(experts, hidden, ffn, 503 + experts)
    return d

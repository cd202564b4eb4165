"""Seeded synthetic inputs shaped like the workloads of the qwantize "Results"
page (a 2560x9728 bfloat16 ``down_proj`` weight and 244449x9728 calibration
activations) and the other parity configurations.

The real model weights and calibration activations are not available; these
generators stand in for them.  This module holds no arithmetic of the method:
it only draws random numbers (numpy ``Generator(PCG64(seed))``) and rounds them
to bfloat16 with torch's round-to-nearest-even cast.  Both the GPU tests and the
CPU oracle take their inputs from here.

Every generator returns a CPU ``torch.Tensor`` (float32 or bfloat16).  Use
``bits(t)`` to get the numpy view the oracle takes (float32, or the bfloat16
bit patterns as uint16).
"""
import numpy as np
import torch

__all__ = ["weights", "activations", "activation_chunks", "bits", "CONFIGS", "config_inputs"]


def _cast(a32: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t if dtype == torch.float32 else t.to(dtype)


def bits(t: torch.Tensor) -> np.ndarray:
    """numpy view for the oracle: float32 values or bfloat16 bits as uint16."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    raise TypeError(t.dtype)


def weights(kind: str, N: int, K: int, std: float, seed: int, gain_seed=None,
            gain_sigma: float = 0.5, dtype=torch.bfloat16) -> torch.Tensor:
    """W [N, K].  kind: 'normal' (std * N(0,1)), 't4' / 't3' (std * Student-t
    with 4 / 3 degrees of freedom), 'laplace' (Laplace with std `std`, i.e.
    scale std/sqrt(2)).  gain_seed: multiply row n by g_n ~ LogNormal(0, gain_sigma)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "normal":
        w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(std)
    elif kind in ("t4", "t3"):
        w = (rng.standard_t(int(kind[1]), (N, K)) * std).astype(np.float32)
    elif kind == "laplace":
        w = rng.laplace(0.0, std / np.sqrt(2.0), (N, K)).astype(np.float32)
    else:
        raise ValueError(kind)
    if gain_seed is not None:
        g = np.random.Generator(np.random.PCG64(gain_seed)).lognormal(0.0, gain_sigma, N)
        w *= g.astype(np.float32)[:, None]
    return _cast(w, dtype)


def _outlier_idx(K, n_out, idx_seed):
    return np.random.Generator(np.random.PCG64(idx_seed)).choice(K, n_out, replace=False)


def activation_chunks(M: int, K: int, seed: int, n_out: int = 0, out_gain: float = 1.0,
                      idx_seed=None, dtype=torch.bfloat16, rows_per_chunk: int = 16384):
    """Yield X [M, K] in row chunks: N(0,1) with n_out channels scaled by out_gain.
    The concatenation of the chunks does not depend on rows_per_chunk."""
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = _outlier_idx(K, n_out, idx_seed) if n_out else None
    done = 0
    while done < M:
        r = min(rows_per_chunk, M - done)
        x = rng.standard_normal((r, K), dtype=np.float32)
        if idx is not None:
            x[:, idx] *= np.float32(out_gain)
        yield _cast(x, dtype)
        done += r


def activations(M, K, seed, n_out=0, out_gain=1.0, idx_seed=None, dtype=torch.bfloat16):
    return torch.cat(list(activation_chunks(M, K, seed, n_out, out_gain, idx_seed, dtype)), 0)


# The five parity / benchmark configurations.  Shapes follow the pages' layer
# (W 2560x9728, X 244449x9728); distributions are the stated stand-ins.
CONFIGS = {
    1: dict(name="tiny-int8-fp32", W=dict(kind="normal", N=64, K=256, std=0.02, seed=11,
                                          gain_seed=None, dtype=torch.float32),
            X=dict(M=512, K=256, seed=12, n_out=0, out_gain=1.0, idx_seed=None, dtype=torch.float32),
            formats=["INT8_E4M3"], blocks=[32]),
    2: dict(name="int8-e4m3-down_proj-2560x9728",
            W=dict(kind="t4", N=2560, K=9728, std=0.02, seed=21, gain_seed=22, dtype=torch.bfloat16),
            X=dict(M=16384, K=9728, seed=23, n_out=8, out_gain=50.0, idx_seed=24, dtype=torch.bfloat16),
            formats=["INT8_E4M3"], blocks=[32, 64, 128, 256]),
    3: dict(name="nvfp4-down_proj-2560x9728-x244449",
            W=dict(kind="t4", N=2560, K=9728, std=0.02, seed=21, gain_seed=22, dtype=torch.bfloat16),
            X=dict(M=244449, K=9728, seed=33, n_out=16, out_gain=100.0, idx_seed=34, dtype=torch.bfloat16),
            formats=["NVFP4"], blocks=[16, 32]),
    4: dict(name="mx-block-sweep-4096x4096",
            W=dict(kind="laplace", N=4096, K=4096, std=0.02, seed=41, gain_seed=42, dtype=torch.bfloat16),
            X=None, formats=["MXFP4", "NVFP4", "MXFP8", "FP8_E4M3S"], blocks=[8, 16, 32, 64, 128, 256]),
    5: dict(name="large-8192x28672",
            W=dict(kind="t3", N=8192, K=28672, std=0.015, seed=51, gain_seed=None, dtype=torch.bfloat16),
            X=dict(M=65536, K=28672, seed=53, n_out=4, out_gain=1e4, idx_seed=54, dtype=torch.bfloat16),
            formats=["NVFP4", "INT8_E4M3"], blocks=[16, 128]),
}


def config_inputs(i: int, rows=None, x_rows=None):
    """(W, X) of configuration i; rows / x_rows cut W / X to their first rows
    (the draws of the kept rows are the same as in the full tensors);
    x_rows=0 skips X (returned as None)."""
    c = CONFIGS[i]
    wp = dict(c["W"])
    N = wp.pop("N")
    K = wp.pop("K")
    kind = wp.pop("kind")
    W = weights(kind, N, K, **wp)
    if rows is not None:
        W = W[:rows].contiguous()
    X = None
    if c["X"] is not None and x_rows != 0:
        xp = dict(c["X"])
        M = xp.pop("M") if x_rows is None else min(x_rows, xp.pop("M"))
        xp.pop("M", None)
        X = activations(M, xp.pop("K"), **xp)
    return W, X

"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no arithmetic of the attention method: it only draws random tensors with the
shapes and value structure of the workloads (pixel-token sequences of square images, flattened in
row-major order) and rounds them once to the storage dtype.  Both the HIP path and the CPU oracle
read exactly the values produced here.

Recipe
------
* numpy ``Generator(PCG64)`` seeded by ``SeedSequence([seed, slice, stream])`` where ``slice`` is
  ``batch_index * heads + head`` and ``stream`` is 0..5 for Q noise / K noise / V noise / dO /
  field / projection.
* ``"iid"``: Q, K, V are i.i.d. N(0, 1).
* ``"field"``: per slice, ``C`` scalar Gaussian random fields on the periodic ``H x W`` grid with
  covariance proportional to exp(-r^2 / (2 l^2)) (``l`` = length scale in pixels), made by filtering
  white noise in the Fourier domain with exp(-pi^2 l^2 |f|^2) (f in cycles per pixel); each channel
  is standardised, flattened row-major to ``F`` of shape [H*W, C], projected by ``P`` [C, d] with
  entries N(0, 1/C) (the product summed channel by channel, elementwise), and Q = F P + a*eps_Q,
  K = F P + a*eps_K, V = F P + a*eps_V with independent eps ~ N(0, 1) and noise amplitude ``a``.
* ``"hub"``: i.i.d. N(0, 1) rows plus a shared direction ``u`` (entries +-1, drawn per slice from the
  projection stream): every query row gets ``hub_gain * u`` and so do the key rows of the first
  ``hub_tokens`` tokens, so that every unit's selection keeps the blocks that hold them -- a few key
  blocks whose CSC columns hold every query block (the most skewed column lengths there are).
* ``dO`` is i.i.d. N(0, 1).
* Values are drawn in float64, then rounded once (round-to-nearest-even) to fp32 or bf16.
"""
from __future__ import annotations

import concurrent.futures
import math
from dataclasses import dataclass, field

import numpy as np

STREAM_Q, STREAM_K, STREAM_V, STREAM_DO, STREAM_FIELD, STREAM_PROJ = range(6)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: tensor shapes, method parameters and input recipe."""
    name: str
    batch: int
    heads: int
    n: int
    d: int
    dtype: str          # "f32" or "bf16"
    block: int
    topk: int
    levels: int
    backward: bool
    kind: str           # "iid", "field" or "hub"
    seed: int
    grid: tuple = field(default=(0, 0))   # (H, W) pixel grid, H * W == n
    length_scale: float = 16.0
    channels: int = 8
    noise: float = 0.1
    hub_tokens: int = 64
    hub_gain: float = 0.35

    @property
    def bh(self) -> int:
        return self.batch * self.heads


def _grid(n: int) -> tuple:
    s = int(round(math.sqrt(n)))
    assert s * s == n
    return (s, s)


# The five workloads: a tiny fp32 forward on a 64x64 grid, a bf16 forward on 128x128, bf16 forward and
# forward+backward on 256x256 smooth fields, and forward+backward on 512x512 smooth fields.
WORKLOADS = {
    "tiny_fwd_f32_n4096": Workload("tiny_fwd_f32_n4096", 1, 2, 4096, 64, "f32", 16, 8, 2, False, "iid",
                                   1001, _grid(4096)),
    "fwd_bf16_n16384": Workload("fwd_bf16_n16384", 1, 8, 16384, 64, "bf16", 16, 8, 2, False, "iid",
                                1002, _grid(16384)),
    "fwd_bf16_n65536": Workload("fwd_bf16_n65536", 1, 16, 65536, 64, "bf16", 16, 8, 3, False, "field",
                                1003, _grid(65536)),
    "fwdbwd_bf16_n65536": Workload("fwdbwd_bf16_n65536", 1, 16, 65536, 64, "bf16", 16, 8, 3, True,
                                   "field", 1004, _grid(65536)),
    "fwdbwd_bf16_n262144": Workload("fwdbwd_bf16_n262144", 1, 8, 262144, 64, "bf16", 16, 16, 3, True,
                                    "field", 1005, _grid(262144)),
}


def rng(seed: int, slice_: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, slice_, stream])))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> fp32 (RNE) -> bf16 (RNE) bit patterns as uint16."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


@dataclass
class Tensor:
    """A rounded input: ``store`` holds what goes to the device (float32 or uint16 bf16 bits) and
    ``exact`` the same values as float64 for the oracle.  Shape [batch, heads, n, d]."""
    store: np.ndarray
    exact: np.ndarray


def to_dtype(x: np.ndarray, dtype: str) -> Tensor:
    if dtype == "f32":
        s = np.ascontiguousarray(x, dtype=np.float32)
        return Tensor(s, s.astype(np.float64))
    if dtype == "bf16":
        s = round_to_bf16_bits(x)
        return Tensor(s, bf16_bits_to_f64(s))
    raise ValueError(dtype)


def smooth_field(seed: int, slice_: int, grid: tuple, length_scale: float, channels: int) -> np.ndarray:
    """[H*W, C] standardised periodic Gaussian random fields, flattened row-major."""
    H, W = grid
    g = rng(seed, slice_, STREAM_FIELD)
    white = g.standard_normal((channels, H, W))
    fy = np.fft.fftfreq(H)[:, None]
    fx = np.fft.fftfreq(W)[None, :]
    filt = np.exp(-(math.pi ** 2) * length_scale ** 2 * (fx ** 2 + fy ** 2))
    f = np.real(np.fft.ifft2(np.fft.fft2(white) * filt[None]))
    f -= f.mean(axis=(1, 2), keepdims=True)
    f /= f.std(axis=(1, 2), keepdims=True)
    return f.reshape(channels, H * W).T.copy()


def _slice_values(w: Workload, s: int, d: int):
    n = w.n
    if w.kind == "iid":
        return [rng(w.seed, s, st).standard_normal((n, d)) for st in (STREAM_Q, STREAM_K, STREAM_V)]
    if w.kind == "field":
        F = smooth_field(w.seed, s, w.grid, w.length_scale, w.channels)
        P = rng(w.seed, s, STREAM_PROJ).standard_normal((w.channels, d)) / math.sqrt(w.channels)
        # F P as a channel-by-channel sum of elementwise products: the same bits on every run, machine and
        # thread (a BLAS product here gave wrong values when slices were drawn on several threads at once)
        X = F[:, 0:1] * P[0]
        for c in range(1, w.channels):
            X = X + F[:, c:c + 1] * P[c]
        return [X + w.noise * rng(w.seed, s, st).standard_normal((n, d))
                for st in (STREAM_Q, STREAM_K, STREAM_V)]
    if w.kind == "hub":
        q, k, v = (rng(w.seed, s, st).standard_normal((n, d)) for st in (STREAM_Q, STREAM_K, STREAM_V))
        u = rng(w.seed, s, STREAM_PROJ).choice(np.array([-1.0, 1.0]), d)
        q += w.hub_gain * u
        k[:w.hub_tokens] += w.hub_gain * u
        return [q, k, v]
    raise ValueError(w.kind)


def make_inputs(w: Workload, heads: list | None = None, with_dout: bool | None = None) -> dict:
    """Draw Q, K, V (and dO) for workload ``w``.  ``heads`` restricts to a subset of slices
    (bh indices); the values of a slice never depend on which other slices are drawn."""
    slices = list(range(w.bh)) if heads is None else list(heads)
    with_dout = w.backward if with_dout is None else with_dout

    def one(s):
        q, k, v = _slice_values(w, s, w.d)
        do = rng(w.seed, s, STREAM_DO).standard_normal((w.n, w.d)) if with_dout else None
        return q, k, v, do

    # slices are independent streams, so drawing them concurrently gives the same values
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(slices)) or 1) as ex:
        drawn = list(ex.map(one, slices))
    qs = [t[0] for t in drawn]
    ks = [t[1] for t in drawn]
    vs = [t[2] for t in drawn]
    dos = [t[3] for t in drawn] if with_dout else []
    shape = (1, len(slices), w.n, w.d) if heads is not None else (w.batch, w.heads, w.n, w.d)
    out = {name: to_dtype(np.stack(arr).reshape(shape), w.dtype)
           for name, arr in (("q", qs), ("k", ks), ("v", vs)) if arr}
    if with_dout:
        out["dout"] = to_dtype(np.stack(dos).reshape(shape), w.dtype)
    return out


def custom(batch: int, heads: int, n: int, d: int, dtype: str, seed: int, kind: str = "iid",
           block: int = 16, topk: int = 8, levels: int = 0, backward: bool = False, **kw) -> Workload:
    """A workload of any shape (parity tests at small sizes and ragged tails)."""
    grid = kw.pop("grid", None)
    if grid is None and kind == "field":
        grid = _grid(n)
    return Workload(f"custom_n{n}", batch, heads, n, d, dtype, block, topk, levels, backward, kind, seed,
                    grid or (0, 0), **kw)

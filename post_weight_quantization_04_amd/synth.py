"""Seeded synthetic inputs for the GPTQ layer quantizer.

This module only draws random numbers and stores them as fp32 or bf16 bytes.
It holds none of the quantizer's arithmetic, so both the HIP path and the
CPU oracle may be fed from it.

Workloads (Llama-shaped linear layers, calibration activations X of shape
[tokens, d_in], weights W of shape [d_out, d_in]):

  toy        W fp32 256x512 ~ N(0, 0.02^2); X fp32 2048x512 ~ N(0, 1) with
             four seeded channels multiplied by 20.
  q_proj     W bf16 4096x4096 ~ N(0, 0.02^2) with exactly round(0.001*size)
             distinct seeded entries multiplied by 10; X bf16 262144x4096,
             x[t, c] = z[t, c] * exp(g_c), z, g ~ N(0, 1) (log-normal channel
             scale, sigma = 1).
  down_proj  W as q_proj at 4096x11008; X bf16 262144x11008, i.i.d.
             Student-t with 3 degrees of freedom.
  up_proj    W as q_proj at 11008x4096; X identical to q_proj's.
  down70b    W bf16 8192x28672 ~ N(0, 0.015^2), no outliers; X bf16
             131072x28672 with log-normal channel scales (sigma = 1).

Seeding: numpy PCG64 streams keyed by SeedSequence([tag, stream, index]) with
stream 1 = W, 2 = X (index = 8192-token chunk), 3 = picks (index 0: channel
scales / outlier channels, index 1: outlier positions).  The tag is the
workload's number (1..5); reduced-size variants of a workload use their own
tag so that their draws are independent of the full-size ones.

bf16 values are produced from fp32 draws by round-to-nearest-even on the bit
pattern and kept as uint16 arrays (numpy has no bf16 type).
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, replace

import numpy as np

CHUNK_TOKENS = 8192
STREAM_W, STREAM_X, STREAM_PICKS = 1, 2, 3


@dataclass(frozen=True)
class Workload:
    tag: int            # seed tag
    name: str
    d_out: int
    d_in: int
    n: int              # calibration tokens
    dtype: str          # "f32" or "bf16" (both W and X)
    bits: int
    group_size: int
    block_size: int
    damp: float
    act_order: bool
    w_std: float
    w_outlier_frac: float   # fraction of W entries multiplied by 10
    x_kind: str             # "gauss_outlier_ch", "lognormal_ch", "student_t"
    x_outlier_channels: int = 0

    def with_shape(self, tag: int, d_out: int, d_in: int, n: int, **kw) -> "Workload":
        return replace(self, tag=tag, d_out=d_out, d_in=d_in, n=n, **kw)


WORKLOADS = {
    "toy": Workload(1, "toy", 256, 512, 2048, "f32", 4, 128, 128, 0.01, False,
                    0.02, 0.0, "gauss_outlier_ch", 4),
    "q_proj": Workload(2, "q_proj", 4096, 4096, 262144, "bf16", 4, 128, 128, 0.01, False,
                       0.02, 0.001, "lognormal_ch"),
    "down_proj": Workload(3, "down_proj", 4096, 11008, 262144, "bf16", 4, 128, 128, 0.01, True,
                          0.02, 0.001, "student_t"),
    "up_proj": Workload(4, "up_proj", 11008, 4096, 262144, "bf16", 3, 32, 128, 0.01, True,
                        0.02, 0.001, "lognormal_ch"),
    "down70b": Workload(5, "down70b", 8192, 28672, 131072, "bf16", 4, 128, 256, 0.01, False,
                        0.015, 0.0, "lognormal_ch"),
}


# Transformer blocks: the linear layers of one Llama block grouped by the input
# they read (layers of a group share that input's Hessian).  Each entry:
# (input, d_in, x law, x tag, [(layer, d_out, w tag), ...]).  The attention
# input uses q_proj's activation draws and the MLP's inner activations
# down_proj's; the other inputs have tags of their own.  Weights follow the
# q_proj law (the 70B block the 70B down_proj's).
BLOCKS = {
    "llama7b_block": dict(n=262144, bits=4, group_size=128, block_size=128, act_order=False, w_std=0.02,
                          w_outlier_frac=0.001, groups=[
        ("attn_in", 4096, "lognormal_ch", 2, [("q_proj", 4096, 31), ("k_proj", 4096, 32), ("v_proj", 4096, 33)]),
        ("attn_out", 4096, "lognormal_ch", 21, [("o_proj", 4096, 34)]),
        ("mlp_in", 4096, "lognormal_ch", 22, [("gate_proj", 11008, 35), ("up_proj", 11008, 36)]),
        ("mlp_mid", 11008, "student_t", 3, [("down_proj", 4096, 37)]),
    ]),
    "llama70b_block": dict(n=131072, bits=4, group_size=128, block_size=256, act_order=False, w_std=0.015,
                           w_outlier_frac=0.0, groups=[
        ("attn_in", 8192, "lognormal_ch", 51, [("q_proj", 8192, 61), ("k_proj", 1024, 62), ("v_proj", 1024, 63)]),
        ("attn_out", 8192, "lognormal_ch", 52, [("o_proj", 8192, 64)]),
        ("mlp_in", 8192, "lognormal_ch", 53, [("gate_proj", 28672, 65), ("up_proj", 28672, 66)]),
        ("mlp_mid", 28672, "lognormal_ch", 5, [("down_proj", 8192, 67)]),
    ]),
}


def block_workloads(name: str, n: int | None = None):
    """[(input workload, [layer workloads])] of a block; the input workload
    carries the X law and the layer workloads the W law (same d_in)."""
    b = BLOCKS[name]
    n = n or b["n"]
    out = []
    for inp, d_in, law, xtag, layers in b["groups"]:
        xw = Workload(xtag, inp, 1, d_in, n, "bf16", b["bits"], b["group_size"], b["block_size"], 0.01,
                      b["act_order"], b["w_std"], b["w_outlier_frac"], law)
        lws = [replace(xw, tag=wtag, name=lname, d_out=d_out) for lname, d_out, wtag in layers]
        out.append((xw, lws))
    return out


def _rng(tag: int, stream: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([tag, stream, index])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32, exact."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _x_tag(wl: Workload) -> int:
    # up_proj reuses q_proj's activations (same draws) so H can be shared.
    if wl.name == "up_proj" and wl.tag == 4:
        return 2
    return wl.tag


def channel_scales(wl: Workload) -> np.ndarray | None:
    """Per-channel multipliers applied to X (None for i.i.d. channels)."""
    r = _rng(_x_tag(wl), STREAM_PICKS, 0)
    if wl.x_kind == "lognormal_ch":
        return np.exp(r.standard_normal(wl.d_in)).astype(np.float32)
    if wl.x_kind == "gauss_outlier_ch":
        s = np.ones(wl.d_in, dtype=np.float32)
        ch = r.choice(wl.d_in, size=min(wl.x_outlier_channels, wl.d_in), replace=False)
        s[ch] = 20.0
        return s
    return None


def make_w(wl: Workload) -> np.ndarray:
    """Weights [d_out, d_in]: float32 array for f32 workloads, uint16 bf16 bits otherwise."""
    r = _rng(wl.tag, STREAM_W, 0)
    w = (r.standard_normal((wl.d_out, wl.d_in), dtype=np.float32) * np.float32(wl.w_std))
    k = int(round(wl.w_outlier_frac * wl.d_out * wl.d_in))
    if k > 0:
        pos = _rng(wl.tag, STREAM_PICKS, 1).choice(wl.d_out * wl.d_in, size=k, replace=False)
        w.reshape(-1)[pos] *= np.float32(10.0)
    if wl.dtype == "f32":
        return w
    return f32_to_bf16_bits(w)


def n_chunks(wl: Workload) -> int:
    return (wl.n + CHUNK_TOKENS - 1) // CHUNK_TOKENS


def make_x_chunk(wl: Workload, c: int, scales: np.ndarray | None = None) -> np.ndarray:
    """Tokens [c*8192, min((c+1)*8192, n)) of X, shape [rows, d_in]."""
    rows = min(CHUNK_TOKENS, wl.n - c * CHUNK_TOKENS)
    if rows <= 0:
        raise IndexError(c)
    r = _rng(_x_tag(wl), STREAM_X, c)
    if wl.x_kind == "student_t":
        x = r.standard_t(3.0, size=(rows, wl.d_in)).astype(np.float32)
    else:
        x = r.standard_normal((rows, wl.d_in), dtype=np.float32)
    if scales is None:
        scales = channel_scales(wl)
    if scales is not None:
        x *= scales[None, :]
    if wl.dtype == "f32":
        return x
    return f32_to_bf16_bits(x)


def make_x(wl: Workload, threads: int | None = None, out: np.ndarray | None = None) -> np.ndarray:
    """The whole X [n, d_in] (fp32 or bf16 bits), generated chunk-parallel."""
    dt = np.float32 if wl.dtype == "f32" else np.uint16
    if out is None:
        out = np.empty((wl.n, wl.d_in), dtype=dt)
    scales = channel_scales(wl)
    threads = threads or min(16, os.cpu_count() or 1)

    def fill(c):
        out[c * CHUNK_TOKENS: c * CHUNK_TOKENS + min(CHUNK_TOKENS, wl.n - c * CHUNK_TOKENS)] = \
            make_x_chunk(wl, c, scales)

    with _cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill, range(n_chunks(wl))))
    return out


def to_float32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored bytes -> fp32 values (exact)."""
    return a if dtype == "f32" else bf16_bits_to_f32(a)

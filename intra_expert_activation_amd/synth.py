"""Seeded synthetic inputs shaped like the MoE layers the method is evaluated on.

This module holds no arithmetic of the method itself: it only draws weights,
hidden states and router logits with numpy's PCG64 generator and rounds them
to bf16 (round to nearest even).  The tests feed the same arrays to the CPU
oracle and to the GPU library; the benchmark feeds them to the GPU library.

Streams of ``numpy.random.default_rng([config_id, stream, ...])``:
  0  expert weights (and the gate bias channel)
  1  calibration tokens and logits (64 tokens)
  2  evaluation tokens and logits (batch sweeps take prefixes of one draw)
  3  the shared token direction of the correlated-token generator
  4  the rank permutation behind Zipf expert popularity
The workloads stand in for the pages' real models (Qwen-, Mixtral- and
DeepSeek-style MoE layers); no real weights or datasets are used.
"""
from __future__ import annotations

import math

import numpy as np

CALIB_TOKENS = 64

# Shapes and distributions of the synthetic layers.
CONFIGS = {
    1: dict(name="tiny-fp32", H=256, E=8, I=512, K=2, S=0, I_shared=0, dtype="f32",
            renormalize=1, T=(16,), q=(0.80,), tokens="iid", logits="normal"),
    2: dict(name="qwen-moe-decode", H=2048, E=128, I=768, K=8, S=0, I_shared=0, dtype="bf16",
            renormalize=1, T=(1, 8, 32, 64), q=(0.85,), tokens="correlated", logits="normal",
            bias=(-1.5, 0.5), rho=0.9),
    3: dict(name="mixtral-style", H=4096, E=8, I=14336, K=2, S=0, I_shared=0, dtype="bf16",
            renormalize=1, T=(1, 16, 128, 256), q=(0.70, 0.90), tokens="iid", logits="normal"),
    4: dict(name="deepseek-v2-lite-style", H=2048, E=64, I=1408, K=6, S=2, I_shared=1408,
            dtype="bf16", renormalize=0, T=(1, 8, 32, 64), q=(0.85, 0.70), tokens="iid",
            logits="zipf", zipf=1.1),
    5: dict(name="qwen-moe-prefill", H=2048, E=128, I=768, K=8, S=0, I_shared=0, dtype="bf16",
            renormalize=1, T=(4096,), q=(0.50, 0.70, 0.90), tokens="correlated", logits="normal",
            bias=(-1.5, 0.5), rho=0.9),
}

WEIGHT_STD = 0.02


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    out = ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def config(cfg_id: int, **overrides) -> dict:
    """A config dict with optional shape overrides (used for reduced-size cases)."""
    c = dict(CONFIGS[cfg_id])
    c.update(overrides)
    c["id"] = cfg_id
    c["overridden"] = tuple(sorted(k for k in overrides))
    return c


def _seed(c: dict, stream: int):
    base = [c["id"], stream]
    if c["overridden"]:
        base += [c["H"], c["E"], c["I"], c["K"], c["S"], c["I_shared"]]
    return np.random.default_rng(base)


def _finish(w32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(w32) if dtype == "bf16" else np.ascontiguousarray(w32, np.float32)


def _normal_matrix(rng, shape, std, dtype):
    out = np.empty(shape, np.uint16 if dtype == "bf16" else np.float32)
    for e in range(shape[0]):  # one expert at a time keeps the float32 temporaries small
        w = rng.standard_normal(shape[1:], dtype=np.float32)
        w *= np.float32(std)
        out[e] = _finish(w, dtype)
    return out


def make_layer(c: dict) -> dict:
    """Weights of one MoE layer, all neuron-major [experts, rows, H].

    The down matrix is stored neuron-major too: row j is neuron j's output
    weights (the transpose of the usual [H, I] layout).  With a ``bias`` entry
    the gate's last input channel carries a per-neuron offset drawn from
    N(mean, std); the token generator pins that channel to 1.
    """
    rng = _seed(c, 0)
    H, E, I, S, Is, dt = c["H"], c["E"], c["I"], c["S"], c["I_shared"], c["dtype"]
    layer = {k: c[k] for k in ("H", "E", "I", "K", "S", "I_shared", "renormalize", "dtype")}
    wg = np.empty((E, I, H), np.uint16 if dt == "bf16" else np.float32)
    for e in range(E):
        w = rng.standard_normal((I, H), dtype=np.float32)
        w *= np.float32(WEIGHT_STD)
        if "bias" in c:
            mean, std = c["bias"]
            w[:, H - 1] = rng.normal(mean, std, size=I).astype(np.float32)
        wg[e] = _finish(w, dt)
    layer["w_gate"] = wg
    layer["w_up"] = _normal_matrix(rng, (E, I, H), WEIGHT_STD, dt)
    layer["w_down"] = _normal_matrix(rng, (E, I, H), WEIGHT_STD, dt)
    if S > 0:
        layer["ws_gate"] = _normal_matrix(rng, (S, Is, H), WEIGHT_STD, dt)
        layer["ws_up"] = _normal_matrix(rng, (S, Is, H), WEIGHT_STD, dt)
        layer["ws_down"] = _normal_matrix(rng, (S, Is, H), WEIGHT_STD, dt)
    return layer


def _zipf_log_popularity(c: dict) -> np.ndarray:
    rng = _seed(c, 4)
    ranks = rng.permutation(c["E"]) + 1
    p = ranks.astype(np.float64) ** (-c["zipf"])
    p /= p.sum()
    return np.log(p)


def make_tokens(c: dict, stream: int, T: int | None = None):
    """(x [T,H], logits [T,E] float32) for the calibration (1) or evaluation (2) stream.

    The draw always covers the config's largest batch (or ``T`` if larger), so
    smaller batches are prefixes of the same tokens.
    """
    T_max = CALIB_TOKENS if stream == 1 else max(c["T"])
    if T is None:
        T = T_max
    n = max(T, T_max)
    rng = _seed(c, stream)
    H, E = c["H"], c["E"]
    z = rng.standard_normal((n, H), dtype=np.float32)
    if c["tokens"] == "correlated":
        rho = c["rho"]
        direction = _seed(c, 3).standard_normal(H, dtype=np.float32)
        z = (np.float32(math.sqrt(rho)) * direction[None, :]
             + np.float32(math.sqrt(1.0 - rho)) * z).astype(np.float32)
    if "bias" in c:
        z[:, H - 1] = 1.0
    if c["logits"] == "zipf":
        g = rng.gumbel(size=(n, E))
        logits = (_zipf_log_popularity(c)[None, :] + g).astype(np.float32)
    else:
        logits = rng.standard_normal((n, E), dtype=np.float32)
    x = _finish(z[:T], c["dtype"])
    return x, np.ascontiguousarray(logits[:T])


def to_float(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 view of a weight or token array of the given dtype."""
    return bf16_bits_to_f32(a) if dtype == "bf16" else np.asarray(a, np.float32)

"""CPU oracle for the intra-expert-sparse MoE SwiGLU layer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``moe_oracle.c`` (plain C,
double precision, no BLAS) through ctypes and shares no code with the GPU
library.  All arithmetic lives in the C file; this module only marshals numpy
arrays.

Every function follows arXiv 2605.08575 "Uncovering Intra-expert Activation
Sparsity for Efficient Mixture-of-Expert Model Execution" as explained on its
gist.science page (Technical Summary, Methodology: Gate Projection, Activation
Masking, Fused Up-Down Projection) -- see the C file's comments for the step
each loop follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc (IEEE arithmetic: no -ffast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-std=c99", "-Wall", "-shared",
             "-fPIC", _SRC, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        lib.oracle_route.argtypes = [vp, i32, i32, i32, i32, vp, vp]
        lib.oracle_route.restype = i32
        lib.oracle_moe.argtypes = [i32] * 9 + [vp] * 9 + [i32, vp] + [vp] * 7 + [i32]
        lib.oracle_moe.restype = i32
        lib.oracle_calibrate.argtypes = [i32] * 8 + [vp] * 4 + [ctypes.c_double, i32, vp, i32]
        lib.oracle_topk_mask.argtypes = [i32, i32, vp, vp, i32, vp]
        lib.oracle_calibrate.restype = i32
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


@dataclass
class OracleResult:
    y: np.ndarray          # [T, H] float64
    mask_bits: np.ndarray  # [T, K+S, W] uint32
    scores: np.ndarray | None  # [T, K+S, Imax] float64 (SiLU(gate), signed)
    union_idx: np.ndarray  # [E+S, Imax] int32 (first union_cnt[e] valid)
    union_cnt: np.ndarray  # [E+S] int32
    ids: np.ndarray        # [T, K] int32
    w: np.ndarray          # [T, K] float64


def route(logits: np.ndarray, K: int, renormalize: bool):
    """Top-K softmax routing.  Returns (ids [T,K] int32, w [T,K] float64)."""
    lib = _load()
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.zeros((T, K), np.int32)
    w = np.zeros((T, K), np.float64)
    rc = lib.oracle_route(_ptr(logits), T, E, K, int(renormalize), _ptr(ids), _ptr(w))
    if rc:
        raise ValueError(f"oracle_route: invalid arguments (rc={rc})")
    return ids, w


def _check_layer(layer):
    """(is_bf16, dict of C-contiguous weight arrays of the layer's dtype)."""
    bf16 = layer["dtype"] == "bf16"
    want = np.uint16 if bf16 else np.float32
    names = ("w_gate", "w_up", "w_down") + (("ws_gate", "ws_up", "ws_down") if layer.get("S", 0) > 0 else ())
    ws = {}
    for k in names:
        assert layer[k].dtype == want, k
        ws[k] = np.ascontiguousarray(layer[k])
    return bf16, ws


def moe(layer: dict, x: np.ndarray, logits: np.ndarray, tau, *, dense: bool = False,
        force_mask: np.ndarray | None = None, want_scores: bool = False,
        threads: int | None = None) -> OracleResult:
    """The layer output, masks and per-expert unions, in float64.

    ``layer`` holds the shapes (H, E, I, K, S, I_shared, renormalize, dtype) and
    the neuron-major weights; ``x`` is [T,H] (uint16 bf16 bits or float32) and
    ``logits`` [T,E] float32.  ``tau`` is a scalar or an [E+S] array.
    """
    lib = _load()
    bf16, ws = _check_layer(layer)
    H, E, I, K = layer["H"], layer["E"], layer["I"], layer["K"]
    S, Is = layer.get("S", 0), layer.get("I_shared", 0)
    x = np.ascontiguousarray(x)
    assert x.dtype == (np.uint16 if bf16 else np.float32)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T = x.shape[0]
    assert x.shape == (T, H) and logits.shape == (T, E)
    slots = K + S
    Imax = max(I, Is) if S > 0 else I
    W = (Imax + 31) // 32
    tau_arr = np.ascontiguousarray(np.broadcast_to(np.asarray(tau, np.float64), (E + S,)))
    fm = None
    if force_mask is not None:
        fm = np.ascontiguousarray(force_mask, dtype=np.uint32)
        assert fm.shape == (T, slots, W)
    y = np.zeros((T, H), np.float64)
    mb = np.zeros((T, slots, W), np.uint32)
    sc = np.zeros((T, slots, Imax), np.float64) if want_scores else None
    uidx = np.full((E + S, Imax), -1, np.int32)
    ucnt = np.zeros((E + S,), np.int32)
    ids = np.zeros((T, K), np.int32)
    w = np.zeros((T, K), np.float64)
    rc = lib.oracle_moe(
        T, H, E, I, K, S, Is, int(layer["renormalize"]), int(bf16),
        _ptr(x), _ptr(logits), _ptr(ws["w_gate"]), _ptr(ws["w_up"]), _ptr(ws["w_down"]),
        _ptr(ws.get("ws_gate")), _ptr(ws.get("ws_up")), _ptr(ws.get("ws_down")),
        _ptr(tau_arr), int(dense), _ptr(fm),
        _ptr(y), _ptr(mb), _ptr(sc), _ptr(uidx), _ptr(ucnt), _ptr(ids), _ptr(w),
        int(threads or default_threads()))
    if rc:
        raise ValueError(f"oracle_moe failed (rc={rc})")
    return OracleResult(y, mb, sc, uidx, ucnt, ids, w)


def calibrate(layer: dict, x_calib: np.ndarray, logits_calib: np.ndarray, q: float,
              per_expert: bool = False, threads: int | None = None) -> np.ndarray:
    """Threshold per expert [E+S] (float64) for target sparsity q.

    ``q`` is rounded to float32 first, because the library's boundary takes a
    float; the order-statistic index is floor(q*N) in double precision.
    """
    lib = _load()
    bf16, ws = _check_layer(layer)
    H, E, I, K = layer["H"], layer["E"], layer["I"], layer["K"]
    S, Is = layer.get("S", 0), layer.get("I_shared", 0)
    x_calib = np.ascontiguousarray(x_calib)
    logits_calib = np.ascontiguousarray(logits_calib, dtype=np.float32)
    Tc = x_calib.shape[0]
    tau = np.zeros((E + S,), np.float64)
    q32 = float(np.float32(q))
    rc = lib.oracle_calibrate(Tc, H, E, I, K, S, Is, int(bf16), _ptr(x_calib), _ptr(logits_calib),
                              _ptr(ws["w_gate"]), _ptr(ws.get("ws_gate")), q32,
                              int(per_expert), _ptr(tau), int(threads or default_threads()))
    if rc:
        raise ValueError(f"oracle_calibrate: invalid arguments (rc={rc})")
    return tau


def topk_masks(scores: np.ndarray, rows: np.ndarray, budget: int) -> np.ndarray:
    """Top-k neuron masks [..., W] uint32 from scores a [..., Imax] (oracle_moe's
    ``want_scores`` output) and each pair's expert row count ``rows`` [...]:
    the ``budget`` largest |a| of a pair are active (see oracle_topk_mask)."""
    lib = _load()
    sc = np.ascontiguousarray(scores, dtype=np.float64)
    lead, Imax = sc.shape[:-1], sc.shape[-1]
    rw = np.ascontiguousarray(np.broadcast_to(np.asarray(rows, np.int32), lead))
    n = int(np.prod(lead)) if lead else 1
    W = (Imax + 31) // 32
    out = np.zeros(lead + (W,), np.uint32)
    if lib.oracle_topk_mask(n, Imax, _ptr(sc), _ptr(rw), int(budget), _ptr(out)):
        raise ValueError("oracle_topk_mask: invalid arguments")
    return out


def moe_topk(layer: dict, x: np.ndarray, logits: np.ndarray, budget: int,
             threads: int | None = None) -> OracleResult:
    """The layer with per-pair top-k neuron selection instead of the threshold:
    the scores of every pair (the dense pass), their top-``budget`` masks, then
    the layer under those masks.  ``scores`` of the result are the dense pass's."""
    E, S = layer["E"], layer.get("S", 0)
    d = moe(layer, x, logits, 0.0, dense=True, want_scores=True, threads=threads)
    exp = np.concatenate([d.ids, np.broadcast_to(E + np.arange(S, dtype=np.int32), (d.ids.shape[0], S))], axis=1)
    rows = np.where(exp < E, layer["I"], layer.get("I_shared", 0))
    m = topk_masks(d.scores, rows, budget)
    o = moe(layer, x, logits, 0.0, force_mask=m, threads=threads)
    return OracleResult(o.y, o.mask_bits, d.scores, o.union_idx, o.union_cnt, o.ids, o.w)

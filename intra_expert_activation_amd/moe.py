"""Thin ctypes binding of libmoesparse (include/moe_sparse.h).

Argument marshalling only: shapes are read from the tensors, output tensors and
the workspace are allocated with PyTorch on the tensors' device, and every step
of the computation runs in the library's HIP kernels on the current stream.
There is no fallback: if ``libmoesparse.so`` is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoesparse.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_SPARSE, MOE_DENSE, MOE_TOPK = 0, 1, 2

# every symbol include/moe_sparse.h declares
EXPORTS = (
    "moe_route_topk", "moe_workspace_size", "moe_sparse_expert_ffn", "moe_sparse_expert_ffn_noalloc",
    "moe_calibrate_workspace_size", "moe_calibrate_threshold", "moe_status_string",
)
# bytes of the fixed scratch array moe_sparse_expert_ffn_noalloc uses
NOALLOC_SCRATCH_BYTES = 64 << 20
# every symbol include/moe_sparse_prof.h declares (measurement hooks)
PROF_EXPORTS = (
    "moe_sparse_expert_ffn_profiled", "moe_timer_create", "moe_timer_destroy", "moe_timer_elapsed_ms",
)


class MoeShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "H", "E", "I", "K", "S", "I_shared", "x_dtype", "w_dtype", "renormalize")]


class MoeFfnArgs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x", "router_logits", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down", "tau",
        "y", "mask_bits", "union_idx", "union_cnt", "topk_ids", "topk_w", "workspace")] + [
        ("workspace_bytes", ctypes.c_size_t),
        ("neuron_budget", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {status_string(code)}")
        self.code = code


_lib = None


def lib():
    """The loaded library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                "(hipcc for gfx950); there is no non-HIP fallback")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        sp = ctypes.POINTER(MoeShape)
        L.moe_route_topk.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
        L.moe_workspace_size.argtypes = [sp, i32, ctypes.POINTER(sz)]
        L.moe_sparse_expert_ffn.argtypes = [sp, i32, ctypes.POINTER(MoeFfnArgs), vp]
        L.moe_sparse_expert_ffn_profiled.argtypes = [sp, i32, ctypes.POINTER(MoeFfnArgs), vp, vp, vp]
        L.moe_sparse_expert_ffn_noalloc.argtypes = [sp, i32, ctypes.POINTER(MoeFfnArgs), vp]
        L.moe_calibrate_workspace_size.argtypes = [sp, i32, ctypes.POINTER(sz)]
        L.moe_calibrate_threshold.argtypes = [sp, vp, vp, i32, vp, vp, ctypes.c_float, i32, vp, vp, sz, vp]
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_timer_create.argtypes = [ctypes.POINTER(vp)]
        L.moe_timer_destroy.argtypes = [vp]
        L.moe_timer_elapsed_ms.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_float)]
        for n in EXPORTS + PROF_EXPORTS:
            if n != "moe_status_string":
                getattr(L, n).restype = i32
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().moe_status_string(int(code)).decode()


def _check(code: int, where: str):
    if code != MOE_OK:
        raise MoeError(code, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def make_shape(T, H, E, I, K, S=0, I_shared=0, dtype=MOE_BF16, renormalize=1, x_dtype=None) -> MoeShape:
    """x_dtype defaults to the weights' dtype."""
    return MoeShape(T, H, E, I, K, S, I_shared, dtype if x_dtype is None else x_dtype, dtype, renormalize)


def layer_shape(x, w_gate, K, renormalize, ws_gate=None) -> MoeShape:
    T, H = x.shape
    E, I, _ = w_gate.shape
    S, Is = (ws_gate.shape[0], ws_gate.shape[1]) if ws_gate is not None else (0, 0)
    return make_shape(T, H, E, I, K, S, Is, _dtype_code(w_gate), int(renormalize), x_dtype=_dtype_code(x))


# ---------------------------------------------------------------------------
# Argument checks.  The C ABI receives bare pointers and cannot see sizes,
# element types or devices, so every tensor is checked here before the call:
# a wrong one would make the kernels read or write past a buffer.
# ---------------------------------------------------------------------------
def _need(cond: bool, msg: str, exc=ValueError):
    if not cond:
        raise exc(msg)


def _check_tensor(name, t, dtype=None, shape=None, min_numel=None, ndim=None):
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch.Tensor", TypeError)
    if dtype is not None:
        _need(t.dtype in (dtype if isinstance(dtype, tuple) else (dtype,)),
              f"{name} has dtype {t.dtype}, expected {dtype}", TypeError)
    if ndim is not None:
        _need(t.dim() == ndim, f"{name} must have {ndim} dimensions, has shape {tuple(t.shape)}")
    if shape is not None:
        _need(tuple(t.shape) == tuple(shape), f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if min_numel is not None:
        _need(t.dim() == 1 and t.numel() >= min_numel,
              f"{name} must be 1-D with at least {min_numel} elements, has shape {tuple(t.shape)}")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def _check_devices(named):
    devs = {n: t.device for n, t in named if t is not None}
    first = next(iter(devs.values()))
    _need(first.type == "cuda", f"tensors must be on a GPU (cuda) device, found {first}")
    for n, d in devs.items():
        _need(d == first, f"{n} is on {d}, expected {first} like the other tensors")


_FLOAT_TYPES = (torch.bfloat16, torch.float32)


def workspace_size(shape: MoeShape, mode: int = MOE_SPARSE) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_workspace_size(ctypes.byref(shape), int(mode), ctypes.byref(n)), "moe_workspace_size")
    return n.value


def calibrate_workspace_size(shape: MoeShape, Tc: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_calibrate_workspace_size(ctypes.byref(shape), int(Tc), ctypes.byref(n)),
           "moe_calibrate_workspace_size")
    return n.value


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def route_topk(logits: torch.Tensor, K: int, renormalize: bool = True):
    """(topk_ids [T,K] int32, topk_w [T,K] float32) of fp32 router logits [T,E]."""
    _check_tensor("logits", logits, torch.float32, ndim=2)
    _check_devices([("logits", logits)])
    T, E = logits.shape
    ids = torch.empty((T, K), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, K), dtype=torch.float32, device=logits.device)
    _check(lib().moe_route_topk(_ptr(logits), T, E, int(K), int(renormalize), _ptr(ids), _ptr(w),
                                _stream(logits.device)), "moe_route_topk")
    return ids, w


def sparse_expert_ffn(x, router_logits, w_gate, w_up, w_down, tau=None, *, K, renormalize=True,
                      shared=None, mode=MOE_SPARSE, want_masks=True, out=None, workspace=None,
                      prof_events=None, neuron_budget=0, noalloc=False):
    """One MoE layer forward.  ``shared`` = (ws_gate, ws_up, ws_down) or None.

    ``mode`` MOE_TOPK keeps the ``neuron_budget`` largest |SiLU(gate)| neurons
    of every (token, slot) pair instead of thresholding (``tau`` unused).
    Returns a dict with ``y`` [T,H] fp32 and, when ``want_masks``, ``mask_bits``
    [T,K+S,W] int32 (bit patterns), ``union_idx`` [E+S,Imax], ``union_cnt`` [E+S],
    ``topk_ids`` and ``topk_w``.  ``out`` may supply preallocated outputs.
    ``prof_events`` (a pair of library timers' handles) brackets the expert
    projection kernel through moe_sparse_expert_ffn_profiled.  ``noalloc``
    calls moe_sparse_expert_ffn_noalloc, which takes no workspace (the
    library's fixed per-device scratch instead; calls on one GPU must not
    overlap).
    Raises TypeError / ValueError for a tensor of the wrong dtype, shape,
    layout or device before anything is launched.
    """
    ws_gate, ws_up, ws_down = shared if shared is not None else (None, None, None)
    _check_tensor("x", x, _FLOAT_TYPES, ndim=2)
    _check_tensor("w_gate", w_gate, x.dtype, ndim=3)
    T, H = x.shape
    E, I, Hw = w_gate.shape
    _need(Hw == H, f"w_gate has rows of {Hw} elements, x has {H}")
    _check_tensor("w_up", w_up, x.dtype, (E, I, H))
    _check_tensor("w_down", w_down, x.dtype, (E, I, H))  # neuron-major: row j is neuron j's H outputs
    _check_tensor("router_logits", router_logits, torch.float32, (T, E))
    S = 0
    if shared is not None:
        _need(len(shared) == 3, "shared must be (ws_gate, ws_up, ws_down)")
        _check_tensor("ws_gate", ws_gate, x.dtype, ndim=3)
        S, Is_, Hs = ws_gate.shape
        _need(Hs == H, f"ws_gate has rows of {Hs} elements, x has {H}")
        _check_tensor("ws_up", ws_up, x.dtype, (S, Is_, H))
        _check_tensor("ws_down", ws_down, x.dtype, (S, Is_, H))
    if mode == MOE_SPARSE:
        _need(tau is not None, "tau is required in MOE_SPARSE mode")
    if tau is not None:
        _check_tensor("tau", tau, torch.float32, min_numel=E + S)
    shape = layer_shape(x, w_gate, K, renormalize, ws_gate)
    dev = x.device
    Imax = max(shape.I, shape.I_shared) if S else shape.I
    W = Imax // 32
    o = dict(out or {})
    _need(set(o) <= {"y", "mask_bits", "union_idx", "union_cnt", "topk_ids", "topk_w"},
          f"unknown output names {sorted(set(o) - {'y', 'mask_bits', 'union_idx', 'union_cnt', 'topk_ids', 'topk_w'})}")
    out_specs = dict(y=((T, H), torch.float32), mask_bits=((T, K + S, W), torch.int32),
                     union_idx=((E + S, Imax), torch.int32), union_cnt=((E + S,), torch.int32),
                     topk_ids=((T, K), torch.int32), topk_w=((T, K), torch.float32))
    for k, v in o.items():
        _check_tensor(f"out[{k!r}]", v, out_specs[k][1], out_specs[k][0])
    if workspace is not None:
        _check_tensor("workspace", workspace, torch.uint8, ndim=1)
    _check_devices([("x", x), ("router_logits", router_logits), ("w_gate", w_gate), ("w_up", w_up),
                    ("w_down", w_down), ("ws_gate", ws_gate), ("ws_up", ws_up), ("ws_down", ws_down),
                    ("tau", tau), ("workspace", workspace)] + [(f"out[{k!r}]", v) for k, v in o.items()])
    if "y" not in o:
        o["y"] = torch.empty((T, H), dtype=torch.float32, device=dev)
    if want_masks:
        shapes = dict(mask_bits=((T, K + S, W), torch.int32), union_idx=((E + S, Imax), torch.int32),
                      union_cnt=((E + S,), torch.int32), topk_ids=((T, K), torch.int32),
                      topk_w=((T, K), torch.float32))
        for k, (shp, dt) in shapes.items():
            if k not in o:
                o[k] = torch.empty(shp, dtype=dt, device=dev)
    if noalloc:
        _need(workspace is None and prof_events is None, "noalloc takes no workspace and no events")
    else:
        need = workspace_size(shape, mode)
        if workspace is None or workspace.numel() < need:
            workspace = alloc_workspace(need, dev)
    a = MoeFfnArgs()
    a.x, a.router_logits = _ptr(x), _ptr(router_logits)
    a.w_gate, a.w_up, a.w_down = _ptr(w_gate), _ptr(w_up), _ptr(w_down)
    a.ws_gate, a.ws_up, a.ws_down = _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down)
    a.tau = _ptr(tau)
    a.y = _ptr(o["y"])
    a.mask_bits, a.union_idx, a.union_cnt = (_ptr(o.get(k)) for k in ("mask_bits", "union_idx", "union_cnt"))
    a.topk_ids, a.topk_w = _ptr(o.get("topk_ids")), _ptr(o.get("topk_w"))
    a.workspace, a.workspace_bytes = (_ptr(workspace), workspace.numel()) if workspace is not None else (None, 0)
    a.neuron_budget = int(neuron_budget)
    if noalloc:
        _check(lib().moe_sparse_expert_ffn_noalloc(ctypes.byref(shape), int(mode), ctypes.byref(a), _stream(dev)),
               "moe_sparse_expert_ffn_noalloc")
    elif prof_events is not None:
        _check(lib().moe_sparse_expert_ffn_profiled(ctypes.byref(shape), int(mode), ctypes.byref(a),
                                                    prof_events[0], prof_events[1], _stream(dev)),
               "moe_sparse_expert_ffn_profiled")
    else:
        _check(lib().moe_sparse_expert_ffn(ctypes.byref(shape), int(mode), ctypes.byref(a), _stream(dev)),
               "moe_sparse_expert_ffn")
    return o


def calibrate_threshold(x_calib, logits_calib, w_gate, q, *, K, shared_gate=None, per_expert=False,
                        tau_out=None, workspace=None):
    """tau [E+S] fp32 on the device: the floor(q*N)-th smallest |SiLU(gate)| score."""
    _check_tensor("x_calib", x_calib, _FLOAT_TYPES, ndim=2)
    _check_tensor("w_gate", w_gate, x_calib.dtype, ndim=3)
    Tc, H = x_calib.shape
    E, _, Hw = w_gate.shape
    _need(Hw == H, f"w_gate has rows of {Hw} elements, x_calib has {H}")
    _check_tensor("logits_calib", logits_calib, torch.float32, (Tc, E))
    S = 0
    if shared_gate is not None:
        _check_tensor("shared_gate", shared_gate, x_calib.dtype, ndim=3)
        S = shared_gate.shape[0]
        _need(shared_gate.shape[2] == H, f"shared_gate has rows of {shared_gate.shape[2]} elements, x has {H}")
    if tau_out is not None:
        _check_tensor("tau_out", tau_out, torch.float32, min_numel=E + S)
    if workspace is not None:
        _check_tensor("workspace", workspace, torch.uint8, ndim=1)
    _check_devices([("x_calib", x_calib), ("logits_calib", logits_calib), ("w_gate", w_gate),
                    ("shared_gate", shared_gate), ("tau_out", tau_out), ("workspace", workspace)])
    shape = layer_shape(x_calib, w_gate, K, True, shared_gate)
    Tc = shape.T
    dev = x_calib.device
    if tau_out is None:
        tau_out = torch.empty((shape.E + shape.S,), dtype=torch.float32, device=dev)
    need = calibrate_workspace_size(shape, Tc)
    if workspace is None or workspace.numel() < need:
        workspace = alloc_workspace(need, dev)
    _check(lib().moe_calibrate_threshold(ctypes.byref(shape), _ptr(x_calib), _ptr(logits_calib), Tc,
                                         _ptr(w_gate), _ptr(shared_gate), ctypes.c_float(q),
                                         int(per_expert), _ptr(tau_out), _ptr(workspace),
                                         workspace.numel(), _stream(dev)),
           "moe_calibrate_threshold")
    return tau_out


class Timer:
    """A pair of HIP events with timing, created by the library."""

    def __init__(self):
        self.begin, self.end = ctypes.c_void_p(), ctypes.c_void_p()
        _check(lib().moe_timer_create(ctypes.byref(self.begin)), "moe_timer_create")
        _check(lib().moe_timer_create(ctypes.byref(self.end)), "moe_timer_create")

    @property
    def events(self):
        return (self.begin, self.end)

    def elapsed_ms(self) -> float:
        ms = ctypes.c_float()
        _check(lib().moe_timer_elapsed_ms(self.begin, self.end, ctypes.byref(ms)), "moe_timer_elapsed_ms")
        return ms.value

    def close(self):
        for e in (self.begin, self.end):
            if e:
                lib().moe_timer_destroy(e)
        self.begin = self.end = ctypes.c_void_p()

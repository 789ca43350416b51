"""The C ABI without a GPU: the library loads, exports every symbol that
include/*.h declares, and rejects invalid calls before any HIP call (so these
run on a CPU-only host).  Pointers used here are never dereferenced: every
call below fails validation first.  The binding's own argument checks, which
guard what the C ABI cannot see (sizes, element types, devices), run on CPU
tensors and raise before any library call."""
import ctypes
import os
import re

import pytest
import torch

from intra_expert_activation_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from intra_expert_activation_amd import _build
        _build.build()
    return moe.lib()


def _declared(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char \*)\s*\**\s*(moe_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(L):
    names = _declared("moe_sparse.h")
    assert set(names) == set(moe.EXPORTS), names
    prof = _declared("moe_sparse_prof.h")
    assert set(prof) == set(moe.PROF_EXPORTS), prof
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == ["moe_sparse.h", "moe_sparse_prof.h"], headers
    for n in names + prof:
        assert hasattr(L, n), n


def test_product_header_has_no_measurement_hooks():
    text = open(os.path.join(ROOT, "include", "moe_sparse.h")).read()
    assert "timer" not in text and "event" not in text


def test_status_strings(L):
    for code in range(5):
        s = moe.status_string(code)
        assert s.startswith(("MOE_OK", "MOE_ERR_"))
    assert moe.status_string(99) == "unknown moe_status"


def _ws(shape, mode=moe.MOE_SPARSE):
    n = ctypes.c_size_t()
    rc = moe.lib().moe_workspace_size(ctypes.byref(shape), mode, ctypes.byref(n))
    return rc, n.value


GOOD = dict(T=8, H=2048, E=128, I=768, K=8, S=0, I_shared=0, dtype=moe.MOE_BF16, renormalize=1)


def _shape(**kw):
    d = dict(GOOD)
    d.update(kw)
    return moe.make_shape(**d)


def test_workspace_size_valid_and_shape_only(L):
    rc, n = _ws(_shape())
    assert rc == moe.MOE_OK and n > 0 and n % 256 == 0
    assert _ws(_shape())[1] == n                      # deterministic
    assert _ws(_shape(T=64))[1] > n                   # grows with the batch
    assert _ws(_shape(), moe.MOE_DENSE)[0] == moe.MOE_OK
    assert _ws(_shape(T=0))[0] == moe.MOE_OK          # empty batch is valid
    rc, n = _ws(_shape(H=256, E=8, I=512, K=2, dtype=moe.MOE_F32))
    assert rc == moe.MOE_OK


@pytest.mark.parametrize("kw,code", [
    (dict(K=0), moe.MOE_ERR_INVALID_ARG),
    (dict(K=129), moe.MOE_ERR_INVALID_ARG),          # K > E
    (dict(T=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(H=0), moe.MOE_ERR_INVALID_ARG),
    (dict(dtype=7), moe.MOE_ERR_INVALID_ARG),
    (dict(x_dtype=7), moe.MOE_ERR_INVALID_ARG),
    (dict(x_dtype=moe.MOE_F32), moe.MOE_ERR_UNSUPPORTED),      # fp32 x with bf16 weights
    (dict(dtype=moe.MOE_F32, x_dtype=moe.MOE_BF16, H=1024), moe.MOE_ERR_UNSUPPORTED),
    (dict(renormalize=2), moe.MOE_ERR_INVALID_ARG),
    (dict(S=1, I_shared=0), moe.MOE_ERR_INVALID_ARG),
    (dict(H=2000), moe.MOE_ERR_UNSUPPORTED),         # not 64 lanes x 16 bytes
    (dict(H=1536), moe.MOE_ERR_UNSUPPORTED),         # 3 vectors per lane
    (dict(I=770), moe.MOE_ERR_UNSUPPORTED),          # not a multiple of 32
    (dict(I=32768), moe.MOE_ERR_UNSUPPORTED),
    (dict(E=500, S=20, I_shared=64), moe.MOE_ERR_UNSUPPORTED),
    (dict(K=33, E=128), moe.MOE_ERR_UNSUPPORTED),
])
def test_workspace_size_rejects(L, kw, code):
    assert _ws(_shape(**kw))[0] == code


def test_workspace_bounded_at_prefill_size(L):
    # the down projection's pieces after the first exist only for pairs of
    # experts below the MFMA pair threshold (at most 15 pairs each), so at
    # 4096 tokens the workspace stays near the [P, H] fp32 outputs instead of
    # growing with KMAX * P * H (8 pieces: 2.1 GiB)
    T, H, E, I, K = 4096, 2048, 128, 768, 8
    P = T * K
    rc, n = _ws(_shape(T=T, H=H, E=E, I=I, K=K))
    assert rc == moe.MOE_OK
    outputs = P * H * 4                        # piece 0 of every pair
    gemv_pieces = 7 * min(P, E * 15) * H * 4    # pieces 1..7 of the GEMV experts' pairs
    h = P * I * 4                              # h of the GEMV path (the routed pairs' rows)
    max_items = P // 64 + min(P // 16, E)
    mfma_tiles = max_items * (I // 64) * 64 * 64 * 2 * 2   # compacted h per (item, 64-row tile), hi and lo
    assert n < outputs + gemv_pieces + h + mfma_tiles + (16 << 20), n
    assert n < 620 * 2 ** 20, n
    assert n < 8 * P * H * 4 * 0.3


def test_invalid_mode(L):
    assert _ws(_shape(), 5)[0] == moe.MOE_ERR_INVALID_ARG


def _args(**ptrs):
    a = moe.MoeFfnArgs()
    base = dict(x=0x10000, router_logits=0x20000, w_gate=0x30000, w_up=0x40000, w_down=0x50000,
                tau=0x60000, y=0x70000, workspace=0x80000)
    base.update(ptrs)
    for k, v in base.items():
        setattr(a, k, v)
    a.workspace_bytes = ptrs.get("workspace_bytes", 1 << 40)
    return a


def _ffn(shape, a, mode=moe.MOE_SPARSE):
    return moe.lib().moe_sparse_expert_ffn(ctypes.byref(shape), mode, ctypes.byref(a), None)


@pytest.mark.parametrize("missing", ["x", "router_logits", "w_gate", "w_up", "w_down", "y", "workspace"])
def test_ffn_null_pointer(L, missing):
    assert _ffn(_shape(), _args(**{missing: None})) == moe.MOE_ERR_INVALID_ARG


def test_ffn_tau_required_only_when_sparse(L):
    assert _ffn(_shape(), _args(tau=None)) == moe.MOE_ERR_INVALID_ARG
    # dense ignores tau: with a too-small workspace the call stops at that check
    a = _args(tau=None)
    a.workspace_bytes = 16
    assert _ffn(_shape(), a, moe.MOE_DENSE) == moe.MOE_ERR_WORKSPACE


def test_ffn_topk_mode(L):
    # the top-k variant needs no tau; a negative budget is rejected before any HIP call
    assert _ws(_shape(), moe.MOE_TOPK)[0] == moe.MOE_OK
    a = _args(tau=None)
    a.neuron_budget = -1
    assert _ffn(_shape(), a, moe.MOE_TOPK) == moe.MOE_ERR_INVALID_ARG
    a = _args(tau=None)
    a.neuron_budget = 115
    a.workspace_bytes = 16
    assert _ffn(_shape(), a, moe.MOE_TOPK) == moe.MOE_ERR_WORKSPACE
    assert _ws(_shape(), 3)[0] == moe.MOE_ERR_INVALID_ARG


def test_ffn_shared_pointers_required(L):
    assert _ffn(_shape(S=2, I_shared=768), _args()) == moe.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("field,value", [("x", 0x10008), ("w_gate", 0x30004), ("y", 0x70002),
                                         ("router_logits", 0x20002), ("workspace", 0x80080)])
def test_ffn_misaligned(L, field, value):
    assert _ffn(_shape(), _args(**{field: value})) == moe.MOE_ERR_INVALID_ARG


def test_ffn_workspace_too_small(L):
    need = _ws(_shape())[1]
    a = _args()
    a.workspace_bytes = need - 1
    assert _ffn(_shape(), a) == moe.MOE_ERR_WORKSPACE


def test_ffn_empty_batch_is_a_noop(L):
    # T = 0: valid, nothing is enqueued (so no device is needed)
    assert _ffn(_shape(T=0), _args(x=None, y=None)) == moe.MOE_OK


def test_ffn_null_shape_or_args(L):
    assert moe.lib().moe_sparse_expert_ffn(None, 0, ctypes.byref(_args()), None) == moe.MOE_ERR_INVALID_ARG
    assert moe.lib().moe_sparse_expert_ffn(ctypes.byref(_shape()), 0, None, None) == moe.MOE_ERR_INVALID_ARG


def test_route_validation(L):
    f = moe.lib().moe_route_topk
    assert f(0x1000, 4, 8, 9, 1, 0x2000, 0x3000, None) == moe.MOE_ERR_INVALID_ARG   # K > E
    assert f(0x1000, 4, 8, 0, 1, 0x2000, 0x3000, None) == moe.MOE_ERR_INVALID_ARG
    assert f(0x1000, 4, 8, 2, 3, 0x2000, 0x3000, None) == moe.MOE_ERR_INVALID_ARG   # renormalize
    assert f(None, 4, 8, 2, 1, 0x2000, 0x3000, None) == moe.MOE_ERR_INVALID_ARG
    assert f(0x1002, 4, 8, 2, 1, 0x2000, 0x3000, None) == moe.MOE_ERR_INVALID_ARG   # misaligned
    assert f(0x1000, 4, 600, 2, 1, 0x2000, 0x3000, None) == moe.MOE_ERR_UNSUPPORTED  # E > 512
    assert f(None, 0, 8, 2, 1, None, None, None) == moe.MOE_OK                        # empty batch


def _cal(shape, q, Tc=64, per_expert=0, ws_bytes=1 << 40, **ptr):
    p = dict(x=0x10000, logits=0x20000, wg=0x30000, wsg=0x40000, tau=0x50000, ws=0x60000)
    p.update(ptr)
    return moe.lib().moe_calibrate_threshold(ctypes.byref(shape), p["x"], p["logits"], Tc, p["wg"],
                                             p["wsg"], ctypes.c_float(q), per_expert, p["tau"],
                                             p["ws"], ws_bytes, None)


def test_calibrate_validation(L):
    s = _shape()
    for q in (-0.1, 1.5, float("nan")):
        assert _cal(s, q) == moe.MOE_ERR_INVALID_ARG
    assert _cal(s, 0.5, Tc=0) == moe.MOE_ERR_INVALID_ARG
    assert _cal(s, 0.5, per_expert=2) == moe.MOE_ERR_INVALID_ARG
    assert _cal(s, 0.5, tau=None) == moe.MOE_ERR_INVALID_ARG
    assert _cal(_shape(S=1, I_shared=768), 0.5, wsg=None) == moe.MOE_ERR_INVALID_ARG
    assert _cal(s, 0.5, x=0x10004) == moe.MOE_ERR_INVALID_ARG
    assert _cal(s, 0.5, ws_bytes=10) == moe.MOE_ERR_WORKSPACE
    n = ctypes.c_size_t()
    assert moe.lib().moe_calibrate_workspace_size(ctypes.byref(s), 64, ctypes.byref(n)) == moe.MOE_OK
    assert n.value > 0


def test_timer_validation(L):
    assert moe.lib().moe_timer_create(None) == moe.MOE_ERR_INVALID_ARG
    assert moe.lib().moe_timer_destroy(None) == moe.MOE_ERR_INVALID_ARG
    assert moe.lib().moe_timer_elapsed_ms(None, None, None) == moe.MOE_ERR_INVALID_ARG


def test_profiled_call_validates_like_the_plain_one(L):
    f = moe.lib().moe_sparse_expert_ffn_profiled
    assert f(ctypes.byref(_shape()), 0, ctypes.byref(_args(x=None)), None, None, None) == moe.MOE_ERR_INVALID_ARG
    a = _args()
    a.workspace_bytes = 16
    assert f(ctypes.byref(_shape()), 0, ctypes.byref(a), None, None, None) == moe.MOE_ERR_WORKSPACE


# ---------------------------------------------------------------------------
# The binding's argument checks (CPU tensors: every rejection happens before
# the device check, and a well-formed call fails only there)
# ---------------------------------------------------------------------------
def _layer_tensors(T=4, H=512, E=6, I=64, S=0, Is=64, dt=torch.bfloat16):
    t = dict(x=torch.zeros(T, H, dtype=dt), router_logits=torch.zeros(T, E),
             w_gate=torch.zeros(E, I, H, dtype=dt), w_up=torch.zeros(E, I, H, dtype=dt),
             w_down=torch.zeros(E, I, H, dtype=dt), tau=torch.zeros(E + S))
    if S:
        t["shared"] = tuple(torch.zeros(S, Is, H, dtype=dt) for _ in range(3))
    return t


def _call(t, **kw):
    t = dict(t)
    x, lg, wg, wu, wd, tau = (t.pop(k) for k in ("x", "router_logits", "w_gate", "w_up", "w_down", "tau"))
    args = dict(K=2)
    args.update(t)
    args.update(kw)
    return moe.sparse_expert_ffn(x, lg, wg, wu, wd, tau, **args)


def test_binding_accepts_a_well_formed_call_up_to_the_device():
    with pytest.raises(ValueError, match="GPU"):
        _call(_layer_tensors())
    with pytest.raises(ValueError, match="GPU"):
        _call(_layer_tensors(S=2))


@pytest.mark.parametrize("change,exc", [
    (dict(x=torch.zeros(4, 512, dtype=torch.float16)), TypeError),            # unsupported dtype
    (dict(x=torch.zeros(4, 512)), TypeError),                                 # fp32 x, bf16 weights
    (dict(router_logits=torch.zeros(4, 6, dtype=torch.bfloat16)), TypeError), # logits not fp32
    (dict(router_logits=torch.zeros(5, 6)), ValueError),                      # wrong T
    (dict(w_up=torch.zeros(6, 64, 512)), TypeError),                          # fp32 up, bf16 gate
    (dict(w_down=torch.zeros(6, 512, 64, dtype=torch.bfloat16)), ValueError), # [E,H,I], not neuron-major
    (dict(w_gate=torch.zeros(6, 64, 256, dtype=torch.bfloat16)), ValueError), # rows of the wrong width
    (dict(tau=torch.zeros(5)), ValueError),                                   # shorter than E + S
    (dict(tau=torch.zeros(6, dtype=torch.float64)), TypeError),
    (dict(x=torch.zeros(512, 4, dtype=torch.bfloat16).t()), ValueError),      # not contiguous
])
def test_binding_rejects(change, exc):
    t = _layer_tensors()
    t.update(change)
    with pytest.raises(exc):
        _call(t)


def test_binding_rejects_bad_shared_and_outputs():
    t = _layer_tensors(S=2)
    g, u, d = t["shared"]
    t["shared"] = (g, u, torch.zeros(2, 64, 256, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        _call(t)
    t = _layer_tensors(S=2)
    t["tau"] = torch.zeros(6)  # E + S = 8 thresholds are needed
    with pytest.raises(ValueError):
        _call(t)
    with pytest.raises(ValueError):
        _call(_layer_tensors(), out=dict(y=torch.zeros(4, 256)))
    with pytest.raises(TypeError):
        _call(_layer_tensors(), out=dict(mask_bits=torch.zeros(4, 2, 2)))
    with pytest.raises(ValueError):
        _call(_layer_tensors(), out=dict(union_cnt=torch.zeros(5, dtype=torch.int32)))
    t = _layer_tensors()
    t["tau"] = None
    with pytest.raises(ValueError, match="tau is required"):
        _call(t)


def test_binding_rejects_calibration_arguments():
    t = _layer_tensors()
    with pytest.raises(TypeError):
        moe.calibrate_threshold(t["x"], t["router_logits"].to(torch.bfloat16), t["w_gate"], 0.5, K=2)
    with pytest.raises(TypeError):
        moe.calibrate_threshold(t["x"].float(), t["router_logits"], t["w_gate"], 0.5, K=2)
    with pytest.raises(ValueError):
        moe.calibrate_threshold(t["x"], t["router_logits"], t["w_gate"], 0.5, K=2, tau_out=torch.zeros(3))
    with pytest.raises(ValueError, match="GPU"):
        moe.calibrate_threshold(t["x"], t["router_logits"], t["w_gate"], 0.5, K=2)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no non-HIP fallback"):
        moe.lib()

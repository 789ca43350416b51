"""Helpers shared by the GPU parity tests: moving synthetic layers to the
device, running the library, and comparing with the CPU oracle.

Mask comparison.  A neuron whose oracle score lies within 1e-3 * tau of tau
(the "band") may land on either side of the threshold: the GPU accumulates in
fp32 in another order than the float64 oracle.  Masks are compared bit for bit
outside the band.  For the layer output, the oracle is evaluated with its own
mask outside the band and the GPU's reported decision inside it (either
decision is correct there), so that y is compared on the same set of active
neurons; the band decisions are read from the GPU's mask output, which is
itself checked against the oracle everywhere outside the band.
"""
from __future__ import annotations

import functools

import numpy as np
import torch

import oracle
from intra_expert_activation_amd import moe, synth

BAND = 1e-3


def dev_tensor(a: np.ndarray, dtype: str, device="cuda"):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def layer_to_device(L: dict, device="cuda") -> dict:
    d = {k: L[k] for k in ("H", "E", "I", "K", "S", "I_shared", "renormalize", "dtype")}
    for k in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
        if k in L:
            d[k] = dev_tensor(L[k], L["dtype"], device)
    return d


@functools.lru_cache(maxsize=4)
def cached_layer(cfg_id: int, overrides: tuple = ()):
    c = synth.config(cfg_id, **dict(overrides))
    L = synth.make_layer(c)
    return c, L


def gpu_ffn(DL: dict, x: np.ndarray, logits: np.ndarray, tau, mode=moe.MOE_SPARSE, **kw):
    dt = DL["dtype"]
    xd = dev_tensor(x, dt)
    ld = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
    taud = None
    if tau is not None:
        taud = torch.from_numpy(np.array(
            np.broadcast_to(np.asarray(tau, np.float32), (DL["E"] + DL["S"],)))).cuda()
    shared = (DL["ws_gate"], DL["ws_up"], DL["ws_down"]) if DL["S"] else None
    out = moe.sparse_expert_ffn(xd, ld, DL["w_gate"], DL["w_up"], DL["w_down"], taud, K=DL["K"],
                                renormalize=bool(DL["renormalize"]), shared=shared, mode=mode, **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def unpack_bits(mask_bits: np.ndarray, rows: int) -> np.ndarray:
    mb = np.ascontiguousarray(mask_bits).view(np.uint32)
    bits = np.unpackbits(mb.view(np.uint8), bitorder="little")
    return bits.reshape(mb.shape[:-1] + (-1,))[..., :rows].astype(bool)


def pack_bits(m: np.ndarray, words: int) -> np.ndarray:
    rows = m.shape[-1]
    full = np.zeros(m.shape[:-1] + (words * 32,), bool)
    full[..., :rows] = m
    return np.packbits(full, axis=-1, bitorder="little").view(np.uint32)


def slot_experts(ids: np.ndarray, E: int, S: int) -> np.ndarray:
    T = ids.shape[0]
    return np.concatenate([ids, np.broadcast_to(E + np.arange(S), (T, S))], axis=1)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_layer(L, DL, x, logits, tau, *, mode=moe.MOE_SPARSE, tol, rows_idx=None, check_union=True):
    """Run GPU (all rows of x) and oracle (rows ``rows_idx`` or all) and compare.

    Returns a dict of statistics.  Asserts: routing ids exact and weights to
    1e-6, masks bit-exact outside the band, unions consistent with the GPU's
    masks and with the oracle's outside the band (equal when all rows are
    checked, a superset of the sampled pairs' union otherwise), y within
    ``tol`` relative L2."""
    E, S, K = L["E"], L["S"], L["K"]
    Imax = max(L["I"], L["I_shared"]) if S else L["I"]
    W = Imax // 32
    g = gpu_ffn(DL, x, logits, tau, mode=mode)
    idx = np.arange(x.shape[0]) if rows_idx is None else np.asarray(rows_idx)
    dense = mode == moe.MOE_DENSE
    tau_arr = np.broadcast_to(np.asarray(0.0 if tau is None else tau, np.float64), (E + S,))
    o = oracle.moe(L, x[idx], logits[idx], tau_arr, dense=dense, want_scores=True)

    # routing
    np.testing.assert_array_equal(g["topk_ids"][idx], o.ids)
    np.testing.assert_allclose(g["topk_w"][idx], o.w, rtol=1e-5, atol=1e-7)

    # masks outside the band
    exp = slot_experts(o.ids, E, S)                           # [n, slots]
    rows_of = np.where(exp < E, L["I"], L["I_shared"] if S else 0)
    gm = unpack_bits(g["mask_bits"][idx], W * 32)
    om = unpack_bits(o.mask_bits, W * 32)
    tau_slot = tau_arr[exp][..., None]
    score = np.abs(o.scores)
    valid = np.arange(W * 32)[None, None, :] < rows_of[..., None]
    band = np.zeros_like(om)
    if not dense:
        band[..., :Imax] = (np.abs(score - tau_slot) <= BAND * tau_slot) & valid[..., :Imax]
    mismatch = (gm != om) & ~band
    assert not mismatch.any(), f"{mismatch.sum()} mask bits differ outside the band"
    assert not (gm & ~valid).any(), "mask bits set past an expert's rows"

    # y against the oracle on the same active set
    force = np.where(band, gm, om)
    o2 = oracle.moe(L, x[idx], logits[idx], tau_arr, force_mask=pack_bits(force, W))
    err = rel_l2(g["y"][idx], o2.y)
    assert err <= tol, f"y rel-L2 {err:.3e} > {tol:.1e}"

    # unions: exactly the OR of the GPU's own masks over each expert's pairs
    gids = slot_experts(g["topk_ids"], E, S)
    gmall = unpack_bits(g["mask_bits"], W * 32)
    ucnt = g["union_cnt"]
    for e in range(E + S):
        sel = gids == e
        rows = L["I"] if e < E else L["I_shared"]
        want = np.flatnonzero(gmall[sel].any(axis=0)[:rows]) if sel.any() else np.array([], int)
        assert ucnt[e] == len(want), (e, ucnt[e], len(want))
        np.testing.assert_array_equal(g["union_idx"][e, :len(want)], want)
    if check_union:
        # and the oracle's union, up to rows whose only support is in the band.
        # With every row checked the union is pinned from both sides; with
        # sampled rows the oracle sees only the sampled pairs, so every row
        # they definitely activate must be in the GPU's union (the rest of the
        # union comes from pairs the oracle did not evaluate; it is still
        # checked above against the GPU's own masks)
        for e in range(E + S):
            sel = exp == e
            if not sel.any():
                continue
            rows = L["I"] if e < E else L["I_shared"]
            definite = (om & ~band)[sel].any(axis=0)[:rows]
            possible = (om | band)[sel].any(axis=0)[:rows]
            gu = np.zeros(rows, bool)
            gu[g["union_idx"][e, :ucnt[e]]] = True
            assert not (definite & ~gu).any(), e
            if rows_idx is None:
                assert not (gu & ~possible).any(), e
    return dict(err=err, band=int(band.sum()), flips=int(((gm != om) & band).sum()),
                active=float(gm[valid].mean()) if valid.any() else 0.0, gpu=g, oracle=o2)

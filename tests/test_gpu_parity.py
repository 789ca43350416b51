"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Bars (checked in parity_util.check_layer): routing ids exact, masks and
per-expert unions bit-exact outside the +-1e-3*tau band, layer output within
relative L2 2e-3 for bf16 weights (fp32 accumulation) and 1e-5 for the fp32
layer.  The thresholds fed to both sides are the oracle's own calibration.
"""
import numpy as np
import pytest
import torch

import oracle
from intra_expert_activation_amd import moe, synth

from parity_util import (cached_layer, check_layer, dev_tensor, gpu_ffn, layer_to_device, pack_bits, rel_l2,
                         slot_experts, unpack_bits)

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-3
TOL_F32 = 1e-5


def _tau(L, c, q, calib_tokens=None, per_expert=False):
    xc, lc = synth.make_tokens(c, 1)
    if calib_tokens:
        xc, lc = xc[:calib_tokens], lc[:calib_tokens]
    return oracle.calibrate(L, xc, lc, q, per_expert=per_expert)


# ---------------------------------------------------------------------------
# Tiny fp32 layer (H 256, E 8, I 512, top-2, 16 tokens, tau at the 80% quantile)
# ---------------------------------------------------------------------------
def test_tiny_fp32_sparse_and_dense():
    c, L = cached_layer(1)
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2)
    tau = _tau(L, c, 0.80)
    s = check_layer(L, DL, x, logits, tau, tol=TOL_F32)
    assert 0.05 < s["active"] < 0.5
    check_layer(L, DL, x, logits, None, mode=moe.MOE_DENSE, tol=TOL_F32)


@pytest.mark.parametrize("cfg", [1, 4])
def test_tau_zero_is_dense_bitwise(cfg):
    c, L = cached_layer(cfg, (("E", 16), ("I", 256)) if cfg == 4 else ())
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2)
    x, logits = x[:13], logits[:13]
    sp = gpu_ffn(DL, x, logits, 0.0)
    de = gpu_ffn(DL, x, logits, None, mode=moe.MOE_DENSE)
    assert np.array_equal(sp["y"], de["y"])
    Imax = max(L["I"], L["I_shared"])
    m = unpack_bits(sp["mask_bits"], Imax)
    assert m[:, :L["K"], :L["I"]].all() and not m[:, :L["K"], L["I"]:].any()
    assert m[:, L["K"]:, :L["I_shared"]].all()
    rows = np.where(np.arange(L["E"] + L["S"]) < L["E"], L["I"], L["I_shared"])
    touched = np.isin(np.arange(L["E"] + L["S"]), np.r_[sp["topk_ids"].ravel(), L["E"] + np.arange(L["S"])])
    np.testing.assert_array_equal(sp["union_cnt"], np.where(touched, rows, 0))


def test_tau_infinite_gives_zero():
    c, L = cached_layer(4, (("E", 16), ("I", 256)))
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2)
    g = gpu_ffn(DL, x[:9], logits[:9], np.inf)
    assert (g["y"] == 0).all() and (g["mask_bits"] == 0).all() and (g["union_cnt"] == 0).all()


# ---------------------------------------------------------------------------
# Qwen-MoE-style decode layer (H 2048, E 128, I 768, top-8, q = 0.85)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 8, 32, 64])
def test_qwen_decode(T):
    c, L = cached_layer(2)
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, T)
    tau = _tau(L, c, 0.85)
    s = check_layer(L, DL, x, logits, tau, tol=TOL_BF16)
    print(f"T={T} err={s['err']:.2e} band={s['band']} flips={s['flips']} active={s['active']:.3f}")
    assert 0.05 < s["active"] < 0.3


def test_qwen_decode_dense():
    c, L = cached_layer(2)
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, 8)
    check_layer(L, DL, x, logits, None, mode=moe.MOE_DENSE, tol=TOL_BF16)


# ---------------------------------------------------------------------------
# DeepSeek-V2-Lite-style layer: 64 routed (top-6, no renormalisation) + 2
# shared experts on the sparse path, Zipf-skewed routing
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,q", [(1, 0.85), (8, 0.85), (32, 0.85), (64, 0.85), (1, 0.70), (8, 0.70), (32, 0.70),
                                 (64, 0.70)])
def test_deepseek_shared(T, q):
    c, L = cached_layer(4)
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, T)
    tau = _tau(L, c, q)
    assert tau[-1] != tau[0]  # the shared experts have their own threshold
    s = check_layer(L, DL, x, logits, tau, tol=TOL_BF16)
    print(f"T={T} q={q} err={s['err']:.2e} band={s['band']} flips={s['flips']}")


@pytest.mark.parametrize("T", [400, 700])
def test_deepseek_block_grouping(T):
    # more than 2048 routed pairs: grouped in blocks (per-block expert counts,
    # then a stable scatter per block), with the shared experts' pairs after
    # them; hot experts take the MFMA path (pairs of token tiles, odd counts)
    c, L = cached_layer(4, (("E", 16), ("I", 256)))
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, T)
    assert T * L["K"] > 2048
    tau = _tau(L, c, 0.85)
    rows = np.unique(np.r_[0, 1, T // 3, T // 2, T - 2, T - 1])
    s = check_layer(L, DL, x, logits, tau, tol=TOL_BF16, rows_idx=rows)
    print(f"T={T} err={s['err']:.2e} band={s['band']} flips={s['flips']}")


# ---------------------------------------------------------------------------
# MFMA down split into neuron-tile segments, with experts of two widths: a
# DeepSeek-style layer cut to H 512, 8 routed experts of I 1024 (16 neuron
# tiles, so the plan splits them into 2 segments) and 2 shared experts of
# I 512 (8 tiles), T 40 / 64 / 100 (every expert on the MFMA path; at 64 and
# 100 some take two token tiles).  Segment k of a pair is partial output k,
# added by the combine; every row is checked against the oracle.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T", [40, 64, 100])
def test_mfma_down_segments_mixed_widths(T):
    c, L = cached_layer(4, (("H", 512), ("E", 8), ("I", 1024), ("I_shared", 512)))
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, 100)
    x, logits = x[:T], logits[:T]
    tau = _tau(L, c, 0.8)
    s = check_layer(L, DL, x, logits, tau, tol=TOL_BF16)
    assert 0.05 < s["active"] < 0.5
    check_layer(L, DL, x, logits, None, mode=moe.MOE_DENSE, tol=TOL_BF16)
    sp = gpu_ffn(DL, x, logits, 0.0)
    de = gpu_ffn(DL, x, logits, None, mode=moe.MOE_DENSE)
    assert np.array_equal(sp["y"], de["y"])


@pytest.mark.parametrize("T", [1, 8, 40])
def test_deepseek_shared_kept_dense(T):
    # the policy of keeping the shared experts dense (their neurons matter
    # more): tau_shared = 0 with the routed experts at their calibrated tau.
    # Every shared-slot mask bit is set, the routed slots stay sparse, and y
    # matches the oracle.  T 1 and 8 take the one-launch path, 40 the grouped
    # path with the shared experts on the MFMA body.
    c, L = cached_layer(4)
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, T)
    tau = _tau(L, c, 0.85, calib_tokens=16).copy()
    tau[L["E"]:] = 0.0
    s = check_layer(L, DL, x, logits, tau, tol=TOL_BF16)
    m = unpack_bits(s["gpu"]["mask_bits"], max(L["I"], L["I_shared"]))
    K = L["K"]
    assert m[:, K:, :L["I_shared"]].all()
    assert m[:, :K, :L["I"]].mean() < 0.3
    assert (s["gpu"]["union_cnt"][L["E"]:] == L["I_shared"]).all()


def test_deepseek_per_expert_tau():
    c, L = cached_layer(4)
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, 32)
    tau = _tau(L, c, 0.85, per_expert=True)
    check_layer(L, DL, x, logits, tau, tol=TOL_BF16)


# ---------------------------------------------------------------------------
# Mixtral-style layer (H 4096, E 8, I 14336, top-2)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,q", [(16, 0.9), (40, 0.7), (128, 0.9), (256, 0.7)])
def test_mixtral_reduced_ragged(T, q):
    # full H and E with I cut to 1056 (33 words: ragged row chunks) so the
    # oracle checks every token
    c, L = cached_layer(3, (("I", 1056),))
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, T)
    tau = _tau(L, c, q)
    check_layer(L, DL, x, logits, tau, tol=TOL_BF16)


@pytest.mark.parametrize("T,q", [(1, 0.9), (16, 0.9), (128, 0.9), (256, 0.9), (16, 0.7), (128, 0.7)])
def test_mixtral_full_sampled(T, q):
    # full I = 14336: T 128 and 256 put every expert on the MFMA path
    c, L = cached_layer(3)
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, T)
    tau = _tau(L, c, q, calib_tokens=8)
    rows = np.unique(np.r_[0, T - 1, T // 2])
    s = check_layer(L, DL, x, logits, tau, tol=TOL_BF16, rows_idx=rows)
    print(f"T={T} q={q} err={s['err']:.2e}")


# ---------------------------------------------------------------------------
# Qwen-MoE-style prefill (4096 tokens): every output row the oracle checks is
# sampled; unions are checked against the GPU's own masks at full size
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("q,mode", [(0.5, moe.MOE_SPARSE), (0.7, moe.MOE_SPARSE), (0.9, moe.MOE_SPARSE),
                                    (None, moe.MOE_DENSE)])
def test_qwen_prefill_sampled(q, mode):
    # every expert has ~256 pairs here: the MFMA path
    c, L = cached_layer(5)
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2)
    tau = _tau(L, c, q, calib_tokens=16) if q is not None else None
    rows = np.random.default_rng(7).choice(x.shape[0], 6, replace=False)
    s = check_layer(L, DL, x, logits, tau, mode=mode, tol=TOL_BF16, rows_idx=np.sort(rows))
    print(f"q={q} err={s['err']:.2e}")


def test_mfma_and_gemv_paths_agree_at_threshold():
    # a DeepSeek-style batch of 40 tokens (MFMA from 16 pairs): the 2
    # shared experts (40 pairs) and the hottest routed experts take the MFMA
    # path, the rest the GEMV path; rows of both are checked against the oracle
    c, L = cached_layer(4)
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, 40)
    tau = _tau(L, c, 0.85, calib_tokens=16)
    ids = np.argsort(-logits, axis=1, kind="stable")[:, :L["K"]]
    counts = np.bincount(ids.ravel(), minlength=L["E"])
    assert counts.max() >= 16 > counts.min()
    check_layer(L, DL, x, logits, tau, tol=TOL_BF16)


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------
# batches of more than 8 tokens: the grouped path (smaller ones are covered
# by the one-launch tests below)
@pytest.mark.parametrize("over,T", [
    ((("E", 4), ("K", 4)), 11),                                     # K = E
    ((("E", 300), ("K", 3), ("I", 64)), 50),                        # many experts
    ((("H", 512), ("E", 6), ("I", 96), ("K", 2)), 13),              # H = 512 (one vector per lane)
    ((("H", 8192), ("E", 4), ("I", 64), ("K", 2)), 9),              # H = 8192 (16 vectors per lane)
    ((("H", 512), ("E", 2), ("I", 16384), ("K", 1)), 10),           # I = 16384 (the largest), KMAX pieces
])
def test_edge_shapes_bf16(over, T):
    c, L = cached_layer(2, over)
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, T)
    tau = _tau(L, c, 0.85, calib_tokens=8)
    check_layer(L, DL, x, logits, tau, tol=TOL_BF16)


def test_shared_wider_than_routed():
    c, L = cached_layer(4, (("E", 12), ("I", 128), ("I_shared", 320), ("S", 1)))
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, 11)
    tau = _tau(L, c, 0.7, calib_tokens=8)
    check_layer(L, DL, x, logits, tau, tol=TOL_BF16)


def test_fp32_two_vectors_per_lane():
    c, L = cached_layer(1, (("H", 512), ("I", 160), ("E", 5)))
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, 16)
    tau = _tau(L, c, 0.6)
    check_layer(L, DL, x, logits, tau, tol=TOL_F32)


def test_empty_batch():
    c, L = cached_layer(1)
    DL = layer_to_device(L)
    x = torch.empty((0, L["H"]), dtype=torch.float32, device="cuda")
    lg = torch.empty((0, L["E"]), dtype=torch.float32, device="cuda")
    out = moe.sparse_expert_ffn(x, lg, DL["w_gate"], DL["w_up"], DL["w_down"],
                                torch.zeros(L["E"], device="cuda"), K=L["K"], want_masks=False)
    torch.cuda.synchronize()
    assert out["y"].shape == (0, L["H"])


def test_nan_input_is_active_and_propagates():
    c, L = cached_layer(1)
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2)
    x = x.copy()
    x[3, 17] = np.nan
    tau = _tau(L, c, 0.8)
    g = gpu_ffn(DL, x, logits, tau)
    assert np.isnan(g["y"][3]).all()
    assert np.isfinite(np.delete(g["y"], 3, axis=0)).all()
    assert unpack_bits(g["mask_bits"][3], L["I"]).all()


def test_deterministic():
    c, L = cached_layer(4)
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, 64)
    tau = _tau(L, c, 0.85, calib_tokens=16)
    a = gpu_ffn(DL, x, logits, tau)
    b = gpu_ffn(DL, x, logits, tau)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("T", [1, 64])
def test_profiled_call_matches_plain(T):
    # the measurement entry point (events around the dominant kernel) computes
    # the same outputs bit for bit, and its events bracket a positive time
    c, L = cached_layer(2)
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, T)
    tau = _tau(L, c, 0.85, calib_tokens=16)
    a = gpu_ffn(DL, x, logits, tau)
    timer = moe.Timer()
    try:
        b = gpu_ffn(DL, x, logits, tau, prof_events=timer.events)
        ms = timer.elapsed_ms()
    finally:
        timer.close()
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert 0.0 < ms < 1000.0


@pytest.mark.parametrize("cfg,T,mode", [(2, 64, moe.MOE_SPARSE), (4, 64, moe.MOE_SPARSE), (2, 1, moe.MOE_SPARSE),
                                        (4, 1, moe.MOE_SPARSE), (4, 8, moe.MOE_SPARSE), (2, 64, moe.MOE_TOPK)])
def test_graph_replay_matches_eager(cfg, T, mode):
    # the benchmark's launch configuration: calls captured in one HIP graph
    # (one per batch, in order, sharing a workspace) and replayed several times
    # with eager work between the replays; every replay must reproduce the
    # eager calls bit for bit
    c, L = cached_layer(cfg)
    DL = layer_to_device(L)
    tau = torch.from_numpy(np.broadcast_to(np.asarray(_tau(L, c, 0.85, calib_tokens=16), np.float32),
                                           (L["E"] + L["S"],)).copy()).cuda()
    shared = (DL["ws_gate"], DL["ws_up"], DL["ws_down"]) if L["S"] else None
    batches = []
    for r in range(3):
        x, lg = synth.make_tokens(c, 2, (r + 1) * T)
        batches.append((dev_tensor(x[r * T:], DL["dtype"]), torch.from_numpy(np.ascontiguousarray(lg[r * T:])).cuda()))
    shape = moe.layer_shape(batches[0][0], DL["w_gate"], L["K"], bool(L["renormalize"]), shared[0] if shared else None)
    ws = moe.alloc_workspace(moe.workspace_size(shape, mode), "cuda")

    def call(r, out=None):
        x, lg = batches[r]
        return moe.sparse_expert_ffn(x, lg, DL["w_gate"], DL["w_up"], DL["w_down"], tau, K=L["K"],
                                     renormalize=bool(L["renormalize"]), shared=shared, out=out, workspace=ws,
                                     mode=mode, neuron_budget=115)

    eager = [{k: v.clone() for k, v in call(r).items()} for r in range(3)]
    outs = [{k: torch.empty_like(v) for k, v in e.items()} for e in eager]
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for r in range(3):
                call(r, outs[r])
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            for v in o.values():
                v.fill_(-1)
        call(rep % 3)  # eager work on the same workspace between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r in range(3):
            for k in ("y", "mask_bits", "topk_ids", "topk_w", "union_cnt"):
                assert torch.equal(outs[r][k], eager[r][k]), (rep, r, k)


# ---------------------------------------------------------------------------
# Single-token batches: the one-launch path (routing, gate, mask, up and down
# in one workgroup per (slot, 32-row chunk), then the combine launch)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,over,q", [
    (1, (), 0.8),                                                   # fp32, H 256 (one wavefront)
    (1, (("H", 512), ("I", 160), ("E", 5)), 0.6),                   # fp32, two wavefronts
    (2, (), 0.85),                                                  # Qwen-style
    (2, (("H", 8192), ("E", 4), ("I", 64), ("K", 2)), 0.85),         # 16 vectors per lane
    (2, (("H", 512), ("E", 2), ("I", 16384), ("K", 1)), 0.85),       # 512 chunks per slot
    (2, (("E", 4), ("K", 4)), 0.85),                                # K = E
    (3, (("I", 1024),), 0.9),                                       # Mixtral-style H 4096
    (4, (), 0.85),                                                  # DeepSeek-style, shared experts
    (4, (("E", 12), ("I", 128), ("I_shared", 320), ("S", 1)), 0.7),  # shared wider than routed
])
def test_single_token_path(cfg, over, q):
    c, L = cached_layer(cfg, over)
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, 6)
    tau = _tau(L, c, q, calib_tokens=8)
    tol = TOL_F32 if L["dtype"] == "f32" else TOL_BF16
    for t in range(x.shape[0]):  # six tokens, one call each
        check_layer(L, DL, x[t:t + 1], logits[t:t + 1], tau, tol=tol)
    check_layer(L, DL, x[:1], logits[:1], None, mode=moe.MOE_DENSE, tol=tol)


@pytest.mark.parametrize("cfg,T,q", [(2, 2, 0.85), (2, 4, 0.85), (2, 8, 0.70), (2, 12, 0.85), (2, 16, 0.85),
                                     (4, 3, 0.85), (4, 8, 0.85), (1, 5, 0.8), (3, 2, 0.9)])
def test_few_token_batches(cfg, T, q):
    # up to 8 tokens of small-expert layers (16 without shared experts and
    # with T * K <= E) take the one-launch path (an expert chosen by several
    # tokens, and the shared experts, have several pairs whose masks form its
    # union); the Mixtral-style layer's 2 tokens take the grouped path
    c, L = cached_layer(cfg, (("I", 4096),) if cfg == 3 else ())  # 32 MiB of gate per expert
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, 3 * T)
    tau = _tau(L, c, q, calib_tokens=8)
    tol = TOL_F32 if L["dtype"] == "f32" else TOL_BF16
    for r in range(3):
        check_layer(L, DL, x[r * T:(r + 1) * T], logits[r * T:(r + 1) * T], tau, tol=tol)


def test_single_token_edge_cases():
    c, L = cached_layer(4, (("E", 16), ("I", 256)))
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, 4)
    x1, l1 = x[2:3], logits[2:3]
    # tau = 0 keeps every neuron: bitwise the dense layer
    sp, de = gpu_ffn(DL, x1, l1, 0.0), gpu_ffn(DL, x1, l1, None, mode=moe.MOE_DENSE)
    assert np.array_equal(sp["y"], de["y"]) and np.array_equal(sp["mask_bits"], de["mask_bits"])
    # tau = inf keeps none
    g = gpu_ffn(DL, x1, l1, np.inf)
    assert (g["y"] == 0).all() and (g["mask_bits"] == 0).all() and (g["union_cnt"] == 0).all()
    # a NaN hidden state is active and propagates
    tau = _tau(L, c, 0.8, calib_tokens=8)
    xn = x1.copy()
    xn[0, 5] = 0x7FC0  # a bf16 NaN (the layer's hidden states are bf16 bit patterns)
    g = gpu_ffn(DL, xn, l1, tau)
    assert np.isnan(g["y"]).all() and unpack_bits(g["mask_bits"], L["I"]).all()
    # without the optional outputs (routing kept in the workspace, no unions)
    full = gpu_ffn(DL, x1, l1, tau)
    bare = gpu_ffn(DL, x1, l1, tau, want_masks=False)
    assert np.array_equal(full["y"], bare["y"])
    # repeated calls are bitwise identical
    again = gpu_ffn(DL, x1, l1, tau)
    for k in full:
        assert np.array_equal(full[k], again[k]), k


# ---------------------------------------------------------------------------
# The top-k alternative (MOE_TOPK): for every (token, slot) pair the budget
# neurons with the largest |a| are active
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,T,frac", [(1, 16, 0.2), (2, 64, 0.15), (2, 5, 0.15), (4, 32, 0.15), (2, 40, 1.0),
                                        (4, 3, 0.02)])
def test_topk_variant(cfg, T, frac):
    c, L = cached_layer(cfg)
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, T)
    E, S, K = L["E"], L["S"], L["K"]
    budget = max(1, int(round(frac * L["I"])))
    g = gpu_ffn(DL, x, logits, None, mode=moe.MOE_TOPK, neuron_budget=budget)
    o = oracle.moe_topk(L, x, logits, budget)
    np.testing.assert_array_equal(g["topk_ids"], o.ids)
    Imax = max(L["I"], L["I_shared"]) if S else L["I"]
    W = Imax // 32
    exp = slot_experts(o.ids, E, S)
    rows = np.where(exp < E, L["I"], L["I_shared"] if S else 0)
    gm = unpack_bits(g["mask_bits"], W * 32)
    om = unpack_bits(o.mask_bits, W * 32)
    # exactly the budget (or every row) per pair, none past the expert's rows
    assert (gm.sum(axis=-1) == np.minimum(budget, rows)).all()
    assert not (gm & ~(np.arange(W * 32)[None, None, :] < rows[..., None])).any()
    # the selections differ only at the boundary: scores within 1e-3 of the
    # pair's budget-th largest |a| (the GPU ranks fp32 scores)
    mag = np.abs(np.nan_to_num(o.scores, nan=np.inf))
    kth = np.zeros(rows.shape)
    for idx in np.ndindex(rows.shape):
        srt = -np.sort(-mag[idx][:rows[idx]])
        kth[idx] = srt[min(budget, rows[idx]) - 1]
    band = np.zeros_like(gm)
    band[..., :Imax] = np.abs(mag - kth[..., None]) <= 1e-3 * kth[..., None]
    assert not ((gm != om) & ~band).any(), int(((gm != om) & ~band).sum())
    # the layer under the GPU's own masks
    o2 = oracle.moe(L, x, logits, 0.0, force_mask=pack_bits(gm[..., :Imax], W))
    tol = TOL_F32 if L["dtype"] == "f32" else TOL_BF16
    assert rel_l2(g["y"], o2.y) <= tol
    # unions: the OR of the GPU's masks over each expert's pairs
    for e in range(E + S):
        sel = exp == e
        r = L["I"] if e < E else L["I_shared"]
        want = np.flatnonzero(gm[sel].any(axis=0)[:r]) if sel.any() else np.array([], int)
        assert g["union_cnt"][e] == len(want)
        np.testing.assert_array_equal(g["union_idx"][e, :len(want)], want)


def test_topk_variant_edge_cases():
    c, L = cached_layer(4, (("E", 16), ("I", 256)))
    DL = layer_to_device(L)
    x, logits = synth.make_tokens(c, 2, 12)
    W = max(L["I"], L["I_shared"]) // 32
    # budget 0: nothing active; a budget of every row: the dense layer
    g0 = gpu_ffn(DL, x, logits, None, mode=moe.MOE_TOPK, neuron_budget=0)
    assert (g0["y"] == 0).all() and (g0["mask_bits"] == 0).all() and (g0["union_cnt"] == 0).all()
    gall = gpu_ffn(DL, x, logits, None, mode=moe.MOE_TOPK, neuron_budget=10_000)
    de = oracle.moe(L, x, logits, 0.0, dense=True)
    assert rel_l2(gall["y"], de.y) <= TOL_BF16
    rows = np.where(slot_experts(gall["topk_ids"], L["E"], L["S"]) < L["E"], L["I"], L["I_shared"])
    assert (unpack_bits(gall["mask_bits"], W * 32).sum(axis=-1) == rows).all()
    # a NaN hidden state makes every score of that token NaN: NaN ranks first and
    # equal keys go to the lower rows, so its pairs keep rows 0 .. budget - 1
    xn = x.copy()
    xn[4, 7] = 0x7FC0  # bf16 NaN
    g = gpu_ffn(DL, xn, logits, None, mode=moe.MOE_TOPK, neuron_budget=37)
    on = unpack_bits(g["mask_bits"][4], W * 32)
    assert (on[:, :37].all() and not on[:, 37:].any())
    assert np.isnan(g["y"][4]).all() and np.isfinite(np.delete(g["y"], 4, axis=0)).all()
    o = oracle.moe_topk(L, xn, logits, 37)
    np.testing.assert_array_equal(unpack_bits(o.mask_bits[4], W * 32), on)


# ---------------------------------------------------------------------------
# Routing alone
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,K,renorm", [(1, 8, 2, 1), (64, 128, 8, 1), (33, 64, 6, 0), (4096, 128, 8, 1),
                                          (7, 512, 32, 1), (5, 3, 3, 0)])
def test_route_topk(T, E, K, renorm):
    rng = np.random.default_rng([T, E, K])
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[: T // 2, 1] = logits[: T // 2, 0]  # ties: the lower id first
    ids, w = moe.route_topk(torch.from_numpy(logits).cuda(), K, bool(renorm))
    torch.cuda.synchronize()
    oids, ow = oracle.route(logits, K, renorm)
    np.testing.assert_array_equal(ids.cpu().numpy(), oids)
    np.testing.assert_allclose(w.cpu().numpy(), ow, rtol=2e-6, atol=1e-8)


# Routing inside the layer call, for E from 3 to 512 and K up to 32.  Ties go
# to the lower id; a NaN logit ranks last and makes its token's softmax
# denominator, so every weight of that token, NaN (renormalised or not).
@pytest.mark.parametrize("T,E,K,renorm", [(1, 8, 2, 1), (9, 3, 3, 0), (64, 16, 4, 1), (40, 32, 8, 1),
                                          (64, 64, 6, 0), (64, 128, 8, 1), (256, 128, 8, 1), (20, 256, 32, 1),
                                          (7, 512, 32, 0), (300, 128, 8, 1), (1500, 8, 2, 1)])
def test_layer_routing(T, E, K, renorm):
    c, L = cached_layer(2, (("H", 512), ("E", E), ("K", K), ("I", 64), ("renormalize", renorm)))
    DL = layer_to_device(L)
    rng = np.random.default_rng([T, E, K, 7])
    x, _ = synth.make_tokens(c, 2, T)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[: (T + 1) // 2, 1] = logits[: (T + 1) // 2, 0]  # ties: the lower id first
    if E > 2:
        logits[T - 1, 2] = np.nan
    out = gpu_ffn(DL, x, logits, 0.0)
    oids, ow = oracle.route(logits, K, renorm)
    np.testing.assert_array_equal(out["topk_ids"], oids)
    np.testing.assert_allclose(out["topk_w"], ow, rtol=2e-6, atol=1e-8, equal_nan=True)


# ---------------------------------------------------------------------------
# Calibration on the GPU
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,q,per_expert", [(1, 0.8, False), (2, 0.85, False), (4, 0.85, False),
                                              (4, 0.7, True), (1, 0.0, False), (1, 1.0, False)])
def test_calibrate(cfg, q, per_expert):
    c, L = cached_layer(cfg)
    DL = layer_to_device(L)
    xc, lc = synth.make_tokens(c, 1)
    dt = L["dtype"]
    from parity_util import dev_tensor
    tau_g = moe.calibrate_threshold(dev_tensor(xc, dt), torch.from_numpy(lc).cuda(), DL["w_gate"], q,
                                    K=L["K"], shared_gate=DL.get("ws_gate"), per_expert=per_expert)
    torch.cuda.synchronize()
    tau_g = tau_g.cpu().numpy().astype(np.float64)
    tau_o = oracle.calibrate(L, xc, lc, q, per_expert=per_expert)
    # the order statistic moves by at most the largest score error (fp32 vs fp64)
    finite = np.isfinite(tau_o)
    np.testing.assert_array_equal(np.isfinite(tau_g), finite)
    np.testing.assert_allclose(tau_g[finite], tau_o[finite], rtol=1e-4, atol=2e-6)
    if q in (0.0, 1.0):
        return
    # realised sparsity: the FFN's masks on the calibration tokens leave
    # floor(q*N) scores of each population below its tau, up to the scores that
    # fp32 rounding of a different summation order (GEMV vs MFMA path) can move
    # across tau: those within 1e-5*tau of it.  With per_expert every expert
    # with calibration pairs is its own population.
    g = gpu_ffn(DL, xc, lc, tau_g.astype(np.float32))
    o = oracle.moe(L, xc, lc, np.inf, want_scores=True)
    m = unpack_bits(g["mask_bits"], max(L["I"], L["I_shared"]))
    K, S, E = L["K"], L["S"], L["E"]
    exp = slot_experts(o.ids, E, S)
    pops = []  # (selector over [t, slot], rows, tau)
    if per_expert:
        for e in range(E + S):
            sel = exp == e
            if sel.any():
                pops.append((sel, L["I"] if e < E else L["I_shared"], tau_g[e]))
    else:
        pops.append((exp < E, L["I"], tau_g[0]))
        if S:
            pops.append((exp >= E, L["I_shared"], tau_g[-1]))
    for sel, rows, t in pops:
        inactive = int((~m[sel][:, :rows]).sum())
        v = np.abs(o.scores[sel][:, :rows]).ravel()
        kappa = int(np.floor(float(np.float32(q)) * v.size))
        slack = int((np.abs(v - t) <= 1e-5 * t).sum())
        assert kappa - slack <= inactive <= kappa + slack, (inactive, kappa, slack)


@pytest.mark.parametrize("per_expert", [False, True])
def test_calibrate_nan_scores(per_expert):
    # a NaN hidden state makes every score of its token NaN; NaN orders after
    # +inf, so a high q selects NaN for the populations it reaches, and an
    # expert's own NaN order statistic is kept (only an expert with no
    # calibration pair falls back to the routed value)
    c, L = cached_layer(1)
    DL = layer_to_device(L)
    xc, lc = synth.make_tokens(c, 1)
    xc = xc.copy()
    xc[5, 3] = np.nan
    for q in (0.8, 0.97, 0.99):
        tau_g = moe.calibrate_threshold(dev_tensor(xc, L["dtype"]), torch.from_numpy(lc).cuda(), DL["w_gate"], q,
                                        K=L["K"], per_expert=per_expert).cpu().numpy().astype(np.float64)
        tau_o = oracle.calibrate(L, xc, lc, q, per_expert=per_expert)
        np.testing.assert_array_equal(np.isnan(tau_g), np.isnan(tau_o))
        fin = np.isfinite(tau_o)
        np.testing.assert_allclose(tau_g[fin], tau_o[fin], rtol=1e-4, atol=2e-6)
        if q == 0.97:
            # the routed population's value is finite; with per_expert the NaN
            # token's own experts select NaN (the old sentinel would have
            # replaced it by the routed value)
            assert np.isfinite(tau_o).all() if not per_expert else (np.isnan(tau_o).any() and np.isfinite(tau_o).any())
        if q == 0.99:
            assert np.isnan(tau_o).any()  # the case is exercised

"""The allocation-free entry point (moe_sparse_expert_ffn_noalloc) against the
workspace entry point (moe_sparse_expert_ffn): both run the same kernels, so
every output must be bitwise identical.  Calls come in a row on the shared
per-device scratch, the later ones with smaller batches (the scratch keeps
the earlier call's contents), then a larger batch again."""
import ctypes

import numpy as np
import pytest
import torch

from intra_expert_activation_amd import moe, synth

from parity_util import cached_layer, dev_tensor, layer_to_device

pytestmark = pytest.mark.gpu


def _tau(L, c, q):
    import oracle
    xc, lc = synth.make_tokens(c, 1)
    return oracle.calibrate(L, xc[:16], lc[:16], q)


def _call(DL, L, x, lg, tau, noalloc):
    shared = (DL["ws_gate"], DL["ws_up"], DL["ws_down"]) if L["S"] else None
    out = moe.sparse_expert_ffn(x, lg, DL["w_gate"], DL["w_up"], DL["w_down"], tau, K=L["K"],
                                renormalize=bool(L["renormalize"]), shared=shared, noalloc=noalloc)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("cfg,sizes", [(2, (64, 8, 64)), (4, (64, 16, 1))])
def test_noalloc_matches_workspace_call(cfg, sizes):
    # Qwen-style: the grouped path at 64 tokens, the one-launch path at 8;
    # DeepSeek-style (shared experts; the hot experts and the shared ones on
    # the MFMA body at 64 and 16 tokens), then a single token
    c, L = cached_layer(cfg)
    DL = layer_to_device(L)
    x_all, l_all = synth.make_tokens(c, 2, max(sizes))
    tau = torch.from_numpy(np.broadcast_to(np.asarray(_tau(L, c, 0.85), np.float32),
                                           (L["E"] + L["S"],)).copy()).cuda()
    batches = [(dev_tensor(x_all[:T], L["dtype"]), torch.from_numpy(np.ascontiguousarray(l_all[:T])).cuda())
               for T in sizes]
    refs = [_call(DL, L, x, lg, tau, noalloc=False) for x, lg in batches]
    gots = [_call(DL, L, x, lg, tau, noalloc=True) for x, lg in batches]
    for T, ref, got in zip(sizes, refs, gots):
        assert set(ref) == set(got)
        for k in ref:
            assert np.array_equal(ref[k], got[k]), (T, k)
        assert np.isfinite(got["y"]).all() and np.abs(got["y"]).max() > 0


def test_noalloc_rejects_shapes_beyond_the_scratch():
    # the prefill batch needs a workspace larger than the fixed scratch: the
    # call returns MOE_ERR_WORKSPACE before any HIP call
    shape = moe.make_shape(T=4096, H=2048, E=128, I=768, K=8, dtype=moe.MOE_BF16, renormalize=1)
    assert moe.workspace_size(shape) > moe.NOALLOC_SCRATCH_BYTES
    a = moe.MoeFfnArgs()
    for k, v in dict(x=0x10000, router_logits=0x20000, w_gate=0x30000, w_up=0x40000, w_down=0x50000,
                     tau=0x60000, y=0x70000).items():
        setattr(a, k, v)
    rc = moe.lib().moe_sparse_expert_ffn_noalloc(ctypes.byref(shape), moe.MOE_SPARSE, ctypes.byref(a), None)
    assert rc == moe.MOE_ERR_WORKSPACE
    small = moe.make_shape(T=64, H=2048, E=128, I=768, K=8, dtype=moe.MOE_BF16, renormalize=1)
    assert moe.workspace_size(small) <= moe.NOALLOC_SCRATCH_BYTES

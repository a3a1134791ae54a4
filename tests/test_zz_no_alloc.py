"""The no-allocation expert FFN (moe_expert_ffn_noalloc: the SwiGLU intermediate lives in the
library's fixed per-GPU scratch array) against moe_expert_ffn with a caller workspace, through
the C ABI."""
import numpy as np
import pytest
import torch

import gen
from gen import configs
from gen.arena import device_arena_all_experts
import oracle
import expert_ffn_cache_amd as moe
from expert_ffn_cache_amd.layer import MoeLayer
from tests._helpers import assert_close, bf16_tol, dev, oracle_table, x_device

pytestmark = pytest.mark.gpu


def _ffn_both_ways(w, x, lg, arena, y_dtype):
    """Route and group once, then the expert FFN through both entry points."""
    L = MoeLayer(w.T, w.E, w.k, w.d, w.f, y_dtype=y_dtype, w_dtype=w.dtype)
    xd = x_device(w, x)
    L.route_permute(dev(lg))
    y_ws = torch.full_like(L.y_perm, 3.0)
    y_na = torch.full_like(L.y_perm, 5.0)
    moe.moe_expert_ffn(xd, w.act_dtype, L.perm, L.offsets, w.T, w.k, w.E, w.d, w.f, None, arena,
                       w.entry_bytes, w.dtype, None, None, 0, L.ffn_ws, L.ffn_ws_bytes, y_ws,
                       y_dtype, status=L.status)
    moe.moe_expert_ffn_noalloc(xd, w.act_dtype, L.perm, L.offsets, w.T, w.k, w.E, w.d, w.f, None,
                               arena, w.entry_bytes, w.dtype, None, None, 0, y_na, y_dtype,
                               status=L.status)
    torch.cuda.synchronize()
    assert int(L.status.item()) == 0
    return L, y_ws, y_na


@pytest.mark.parametrize("dtype", [gen.BF16, gen.MXFP4])
def test_noalloc_ffn_equals_workspace_ffn_on_consecutive_calls(dtype):
    """Two calls in a row on one GPU, the second with fewer tokens, so it rewrites only the
    start of the scratch array the first call filled: T=200 (grouped GEMMs; 1.2 MB of
    intermediate), then T=8 (weight-streaming kernels).  Each y_perm equals moe_expert_ffn's
    with a caller workspace bit for bit, and is within the bf16 rule of the oracle."""
    for T, y_dtype in ((200, moe.MOE_F32), (8, moe.MOE_BF16)):
        w = configs.Workload("noalloc", seed=61 + T, T=T, d=1024, E=64, k=6, f=512, dtype=dtype,
                             alpha=0.5)
        x, lg = configs.gen_x(w), configs.gen_logits(w)
        arena = device_arena_all_experts(w)
        L, y_ws, y_na = _ffn_both_ways(w, x, lg, arena, y_dtype)
        assert moe.moe_expert_ffn_workspace_bytes(T, w.k, w.f, w.act_dtype) <= \
            moe.moe_expert_ffn_noalloc_max_bytes()
        assert torch.equal(y_na.view(torch.int16) if y_na.dtype == torch.bfloat16 else y_na,
                           y_ws.view(torch.int16) if y_ws.dtype == torch.bfloat16 else y_ws), T
        ids, _ = oracle.route(lg, w.k)
        counts, offsets, perm, inv = oracle.permute(ids, w.E)
        ref = oracle.expert_ffn(x, ids, oracle_table(w, sorted(set(ids.ravel().tolist()))), perm)
        got = y_na.float().cpu().numpy()
        assert_close(got, ref, bf16_tol(ref), f"noalloc T={T}")
        del arena


def test_noalloc_ffn_one_launch_mxfp4_equals_workspace_ffn():
    """MXFP4 decode calls whose tagged h entries fit the array (T=8 and then T=6, f=2048) run
    both projections in one launch inside the array, as moe_expert_ffn does with a workspace
    of moe_expert_ffn_workspace_bytes: the same bits, within the bf16 rule of the oracle."""
    for T in (8, 6):
        w = configs.Workload("noalloc_one", seed=91 + T, T=T, d=512, E=64, k=6, f=2048,
                             dtype=gen.MXFP4, alpha=0.5)
        assert min(w.E, w.T * w.k) * w.f >= 65536
        assert w.T * w.k * w.f * 4 <= moe.moe_expert_ffn_noalloc_max_bytes()
        x, lg = configs.gen_x(w), configs.gen_logits(w)
        arena = device_arena_all_experts(w)
        L, y_ws, y_na = _ffn_both_ways(w, x, lg, arena, moe.MOE_F32)
        assert torch.equal(y_na, y_ws), T
        ids, _ = oracle.route(lg, w.k)
        counts, offsets, perm, inv = oracle.permute(ids, w.E)
        ref = oracle.expert_ffn(x, ids, oracle_table(w, sorted(set(ids.ravel().tolist()))), perm)
        assert_close(y_na.cpu().numpy(), ref, bf16_tol(ref), f"noalloc one launch T={T}")
        del arena


def test_noalloc_ffn_refuses_an_intermediate_beyond_its_array():
    """T*k*f past the fixed array: MOE_ETOOBIG before anything is enqueued (y untouched)."""
    w = configs.Workload("noalloc_big", seed=67, T=2048, d=256, E=16, k=4, f=1024,
                         dtype=gen.BF16)
    assert moe.moe_expert_ffn_workspace_bytes(w.T, w.k, w.f, w.act_dtype) > \
        moe.moe_expert_ffn_noalloc_max_bytes()
    y = torch.full((w.T * w.k, w.d), 7.0, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_expert_ffn_noalloc(None, w.act_dtype, None, None, w.T, w.k, w.E, w.d, w.f, None,
                                   None, w.entry_bytes, w.dtype, None, None, 0, y, moe.MOE_F32)
    assert ei.value.status == moe.MOE_ETOOBIG
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())

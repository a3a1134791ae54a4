"""GPU parity of each entry point against the oracle on seeded inputs (small-to-medium sizes)."""
import numpy as np
import pytest
import torch

import gen
from gen import configs
from gen.arena import device_arena_all_experts
import oracle
import expert_ffn_cache_amd as moe
from tests._helpers import (assert_close, f32_tol, bf16_tol, np_of, dev, x_device, oracle_table)

pytestmark = pytest.mark.gpu


def _i32(n):
    return torch.empty(n, dtype=torch.int32, device="cuda")


# ---------------------------------------------------------------- routing
ROUTE_CASES = [  # (T, E, k, kind)
    (16, 8, 2, "normal"), (1, 256, 6, "zipf"), (8, 256, 6, "zipf"), (8192, 256, 6, "zipf"),
    (2047, 128, 8, "zipf"), (333, 1024, 16, "normal"), (61, 16, 16, "normal"),
    (100, 300, 5, "ties"), (37, 65, 3, "zeros"), (5, 1, 1, "normal"),
]


def _route_logits(T, E, k, kind, seed):
    if kind == "zipf":
        w = configs.with_(configs.DECODE, T=T, E=E, k=k, seed=seed)
        return configs.gen_logits(w)
    if kind == "normal":
        return gen.routing_logits(seed, gen.TAG_LOGIT, T, E, k)
    r = np.random.default_rng(seed)
    if kind == "ties":
        return (r.integers(-2, 3, size=(T, E)) * 0.5).astype(np.float32)
    lg = r.choice(np.array([0.0, -0.0, 1.0, -1.0], dtype=np.float32), size=(T, E))
    return lg


@pytest.mark.parametrize("T,E,k,kind", ROUTE_CASES)
def test_route_parity(T, E, k, kind):
    lg = _route_logits(T, E, k, kind, seed=T + E + k)
    ids = _i32((T, k))
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route(dev(lg), T, E, k, ids, w)
    torch.cuda.synchronize()
    ref_ids, ref_w = oracle.route(lg, k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    assert_close(w.cpu().numpy(), ref_w, 1e-5 * float(np.abs(ref_w).max()), "topk_w")


@pytest.mark.parametrize("T,d,E", [(1, 1, 1), (3, 7, 65), (300, 256, 8), (17, 512, 1024)])
def test_router_logits_parity(T, d, E):
    """Router logits (fp32) against the oracle's double-precision product, element by element,
    on ragged shapes (one element, d not a multiple of anything, the largest E)."""
    r = np.random.default_rng(T * 31 + d + E)
    x = r.standard_normal((T, d)).astype(np.float32)
    wr = (r.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    out = torch.full((T + 1, E), 7.0, dtype=torch.float32, device="cuda")
    moe.moe_router_logits(dev(x), dev(wr), moe.MOE_F32, T, d, E, out)
    torch.cuda.synchronize()
    ref = oracle.router_logits(x, wr)
    got = out.cpu().numpy()
    assert_close(got[:T], ref, 1e-5 * float(np.abs(ref).max()), "router logits")
    assert (got[T:] == 7.0).all()
    moe.moe_router_logits(dev(x), dev(wr), moe.MOE_F32, 0, d, E, out)  # T = 0: no work
    torch.cuda.synchronize()
    assert (out.cpu().numpy()[T:] == 7.0).all()


def test_route_empty_and_invalid_args():
    moe.moe_route(None, 0, 8, 2, None, None)  # T = 0 is a no-op
    with pytest.raises(moe.MoeError):
        moe.moe_route(None, 4, 8, 2, None, None)
    x = torch.zeros((4, 8), device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_route(x, 4, 8, 9, _i32(36), torch.zeros(36, device="cuda"))  # k > E


# ---------------------------------------------------------------- grouping
PERM_CASES = [(1, 1, 1), (8, 6, 256), (64, 6, 256), (170, 6, 256), (171, 6, 256), (8192, 6, 256),
              (2048, 8, 128), (3001, 16, 1024), (16, 2, 8), (500, 3, 7)]


@pytest.mark.parametrize("T,k,E", PERM_CASES)
def test_permute_parity(T, k, E):
    r = np.random.default_rng(T * 31 + k * 7 + E)
    p = np.exp(-0.01 * np.arange(E)) if E > 1 else np.ones(1)
    ids = np.stack([r.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv, status = _i32(E), _i32(E + 1), _i32(T * k), _i32(T * k), torch.zeros(1, dtype=torch.int32, device="cuda")
    nws = moe.moe_permute_workspace_bytes(T, k, E)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    for _ in range(2):  # run twice: results must be identical (deterministic)
        moe.moe_permute(dev(ids), T, k, E, counts, offsets, perm, inv, ws, nws, status)
        torch.cuda.synchronize()
        rc, ro, rp, ri = oracle.permute(ids, E)
        np.testing.assert_array_equal(counts.cpu().numpy(), rc)
        np.testing.assert_array_equal(offsets.cpu().numpy(), ro)
        np.testing.assert_array_equal(perm.cpu().numpy(), rp)
        np.testing.assert_array_equal(inv.cpu().numpy(), ri)
    assert int(status.item()) == 0


def test_permute_out_of_range_id_sets_status():
    T, k, E = 300, 4, 16
    ids = np.tile(np.arange(k, dtype=np.int32), (T, 1))
    ids[123, 2] = E  # invalid
    counts, offsets, perm, inv = _i32(E), _i32(E + 1), _i32(T * k), _i32(T * k)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    nws = moe.moe_permute_workspace_bytes(T, k, E)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    moe.moe_permute(dev(ids), T, k, E, counts, offsets, perm, inv, ws, nws, status)
    torch.cuda.synchronize()
    assert int(status.item()) == moe.MOE_ERANGE


ROUTE_PERMUTE_CASES = [  # (T, E, k, kind): one-launch form up to T = 16, two calls above
    (1, 256, 6, "zipf"), (8, 256, 6, "zipf"), (5, 8, 2, "normal"), (16, 1024, 16, "normal"),
    (13, 65, 3, "zeros"), (16, 300, 5, "ties"), (1, 1, 1, "normal"), (17, 256, 6, "zipf"),
    (64, 128, 8, "zipf"), (0, 256, 6, "zipf")]


@pytest.mark.parametrize("T,E,k,kind", ROUTE_PERMUTE_CASES)
def test_route_permute_equals_route_then_permute(T, E, k, kind):
    """The combined entry point gives what moe_route and moe_permute give, bit for bit, and
    the oracle's routing and grouping."""
    lg = _route_logits(max(T, 1), E, k, kind, seed=T + 3 * E + k)[:T]
    outs = []
    for combined in (False, True):
        ids, w = _i32((max(T, 1), k)), torch.full((max(T, 1), k), -1.0, device="cuda")
        counts, offsets = _i32(E), _i32(E + 1)
        perm, inv = _i32(max(T * k, 1)), _i32(max(T * k, 1))
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        nws = moe.moe_permute_workspace_bytes(T, k, E)
        ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
        lg_d = dev(lg) if T else torch.empty((1, E), device="cuda")
        if combined:
            moe.moe_route_permute(lg_d, T, E, k, ids, w, counts, offsets, perm, inv, ws, nws, status)
        else:
            moe.moe_route(lg_d, T, E, k, ids, w)
            moe.moe_permute(ids, T, k, E, counts, offsets, perm, inv, ws, nws, status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        outs.append([a.cpu().numpy()[:n] if n is not None else a.cpu().numpy()
                     for a, n in ((ids.view(-1), T * k), (w.view(-1), T * k), (counts, None),
                                  (offsets, None), (perm, T * k), (inv, T * k))])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)
    if T:
        ref_ids, ref_w = oracle.route(lg, k)
        np.testing.assert_array_equal(outs[1][0].reshape(T, k), ref_ids)
        rc, ro, rp, ri = oracle.permute(ref_ids, E)
        for got, want in zip(outs[1][2:], (rc, ro, rp, ri)):
            np.testing.assert_array_equal(got, want)
    else:
        assert not outs[1][2].any() and not outs[1][3].any()


# ---------------------------------------------------------------- combine
@pytest.mark.parametrize("ydt", [moe.MOE_F32, moe.MOE_BF16])
@pytest.mark.parametrize("T,k,d", [(16, 2, 256), (8, 6, 4096), (777, 8, 2048), (1, 1, 64),
                                   (5, 16, 192), (33, 9, 2112)])
def test_combine_parity(T, k, d, ydt):
    r = np.random.default_rng(T + k + d)
    y32 = gen.normal(11, gen.TAG_MISC, 0, (T * k, d))
    if ydt == moe.MOE_BF16:
        ybits = gen.normal(11, gen.TAG_MISC, 0, (T * k, d), 1.0, gen.BF16)
        y_dev = torch.from_numpy(ybits.view(np.int16)).view(torch.bfloat16).cuda()
        y_ref = gen.bf16_bits_to_f32(ybits)
    else:
        y_dev, y_ref = dev(y32), y32
    inv = r.permutation(T * k).astype(np.int32)
    w = r.random((T, k)).astype(np.float32)
    out = torch.empty((T, d), dtype=torch.float32, device="cuda")
    moe.moe_combine(y_dev, ydt, dev(inv), dev(w), T, k, d, out)
    torch.cuda.synchronize()
    ref = oracle.combine(y_ref.astype(np.float64), inv, w.astype(np.float64))
    assert_close(out.cpu().numpy(), ref, f32_tol(ref), "combine")


# ---------------------------------------------------------------- expert FFN
def _ffn_case(w, path, ydt=moe.MOE_F32):
    """Route, group (oracle) and run the GPU FFN over all-resident experts; compare y_perm."""
    x = configs.gen_x(w)
    lg = configs.gen_logits(w) if w.alpha else gen.routing_logits(w.seed, gen.TAG_LOGIT, w.T, w.E, w.k)
    ids, _ = oracle.route(lg, w.k)
    counts, offsets, perm, inv = oracle.permute(ids, w.E)
    arena = device_arena_all_experts(w)
    A = w.T * w.k
    nws = moe.moe_expert_ffn_workspace_bytes(w.T, w.k, w.f, w.act_dtype)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    ytd = torch.float32 if ydt == moe.MOE_F32 else torch.bfloat16
    y = torch.full((A, w.d), float("nan"), dtype=ytd, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert w.entry_bytes == moe.moe_entry_bytes(w.d, w.f, w.dtype)
    moe.moe_expert_ffn(x_device(w, x), w.act_dtype, dev(perm), dev(offsets), w.T, w.k, w.E, w.d,
                       w.f, None, arena, w.entry_bytes, w.dtype, None, None, 0, ws, nws, y, ydt,
                       path, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    table = oracle_table(w, sorted(set(ids.ravel().tolist())))
    ref = oracle.expert_ffn(x, ids, table, perm)
    return np_of(y), ref


def test_ffn_fp32_tiny_parity():
    w = configs.TINY
    y, ref = _ffn_case(w, moe.MOE_PATH_AUTO)
    assert_close(y, ref, f32_tol(ref), "y_perm fp32")


SMALL_BF16 = configs.Workload("small_bf16", seed=21, T=150, d=256, E=12, k=3, f=320,
                              dtype=gen.BF16, alpha=0.5)


@pytest.mark.parametrize("path", [moe.MOE_PATH_GEMV, moe.MOE_PATH_GEMM])
@pytest.mark.parametrize("ydt", [moe.MOE_F32, moe.MOE_BF16])
def test_ffn_bf16_paths_parity(path, ydt):
    """Several tiles in every direction and ragged m-tiles (counts not multiples of 16/128)."""
    y, ref = _ffn_case(SMALL_BF16, path, ydt)
    assert_close(y, ref, bf16_tol(ref), f"y_perm path={path}")


@pytest.mark.parametrize("T", [1, 8, 40])
def test_ffn_gemv_decode_shapes(T):
    w = configs.with_(configs.DECODE, T=T, E=16, d=512, f=256)
    y, ref = _ffn_case(w, moe.MOE_PATH_GEMV)
    assert_close(y, ref, bf16_tol(ref), "y_perm gemv")


@pytest.mark.parametrize("T,E,k,d,f", [(8, 4, 2, 320, 192), (8, 6, 3, 1088, 448), (5, 16, 4, 4160, 64),
                                       (1, 8, 8, 512, 2048), (7, 64, 6, 2048, 960),
                                       (24, 32, 4, 512, 256), (64, 64, 6, 384, 320),
                                       (48, 256, 6, 512, 256)])
@pytest.mark.parametrize("ydt", [moe.MOE_F32, moe.MOE_BF16])
def test_ffn_decode_dot_and_mfma_split(T, E, k, d, f, ydt):
    """Weight-streaming calls: up to 8 tokens every expert takes the dot-product kernels
    (any number of rows, staged two at a time); up to 64 tokens experts are split on the
    device by rows between the dot-product and the MFMA kernels.  Row lengths that are not
    multiples of 512 elements (partial last chunk per lane), few experts with many rows,
    many experts with one row each; more (expert, row block) items than the split launch's
    workgroups, so each workgroup loops over several."""
    w = configs.Workload("dot_split", seed=23, T=T, d=d, E=E, k=k, f=f, dtype=gen.BF16, alpha=0.5)
    y, ref = _ffn_case(w, moe.MOE_PATH_GEMV, ydt)
    assert_close(y, ref, bf16_tol(ref), f"y_perm T={T} E={E} d={d} f={f}")


def _ids_with_counts(counts, T, k):
    """ids [T][k] in which expert e is picked by exactly counts[e] tokens (k distinct experts
    per token: the sorted pick list is dealt column by column, and no expert has T or more
    rows, so no token gets one expert twice)."""
    picks = np.repeat(np.arange(len(counts)), counts).astype(np.int32)
    assert picks.size == T * k and max(counts) < T
    ids = picks.reshape(k, T).T.copy()
    assert all(len(set(r)) == k for r in ids.tolist())
    return ids


@pytest.mark.parametrize("T,counts", [
    (130, [3, 5, 16, 17, 32, 33, 48, 64, 42, 0, 0, 0]),
    (130, [3, 5, 16, 17, 33, 65, 97, 24, 0, 0, 0, 0]),
    (30, [1, 4, 5, 16, 17, 0, 15, 2]),
])
@pytest.mark.parametrize("ydt", [moe.MOE_F32, moe.MOE_BF16])
def test_ffn_gemv_row_counts_at_chunk_boundaries(T, counts, ydt):
    """The MFMA weight-streaming kernels take 16, 32 or 64 token rows per pass (the fewest
    16-row chunks a pass needs, up to the call's limit); experts with rows on both sides of
    each boundary and with several passes (65, 97 rows) against the oracle; experts with up
    to 4 rows take the dot-product kernels of the same call."""
    k = 2
    w = configs.Workload("gemv_rows", seed=29, T=T, d=512, E=len(counts), k=k, f=256,
                         dtype=gen.BF16, alpha=0.0)
    ids = _ids_with_counts(counts, T, k)
    x = configs.gen_x(w)
    counts_o, offsets, perm, inv = oracle.permute(ids, w.E)
    np.testing.assert_array_equal(counts_o, counts)
    arena = device_arena_all_experts(w)
    nws = moe.moe_expert_ffn_workspace_bytes(T, k, w.f, w.act_dtype)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    ytd = torch.float32 if ydt == moe.MOE_F32 else torch.bfloat16
    y = torch.full((T * k, w.d), float("nan"), dtype=ytd, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_expert_ffn(x_device(w, x), w.act_dtype, dev(perm), dev(offsets), T, k, w.E, w.d, w.f,
                       None, arena, w.entry_bytes, w.dtype, None, None, 0, ws, nws, y, ydt,
                       moe.MOE_PATH_GEMV, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    table = oracle_table(w, sorted(set(ids.ravel().tolist())))
    ref = oracle.expert_ffn(x, ids, table, perm)
    assert_close(np_of(y), ref, bf16_tol(ref), f"y_perm T={T} counts={counts}")



@pytest.mark.parametrize("T,k,d,f,counts", [
    (12, 4, 512, 4096, [1, 2, 3, 4, 5, 6, 7, 8, 11, 1, 0, 0, 0, 0, 0, 0]),  # one launch
    (9, 2, 256, 128, [8, 6, 1, 2, 1, 0]),                                   # two launches
    (40, 3, 320, 192, [1, 5, 6, 7, 11, 12, 13, 16, 17, 32, 0, 0, 0, 0, 0, 0]),  # + grouped GEMM
    (32, 2, 256, 256, [31, 17, 16, 0, 0, 0, 0, 0]),                          # 2 blocks, no GEMM
    (24, 4, 512, 1024, [6, 12, 13, 16, 1, 7, 18, 23, 0, 0, 0, 0]),           # 2 blocks of 16
    (12, 2, 7936, 64, [11, 9, 4]),    # K = 7936: at most 2 slices; 4 waves per strip
])
@pytest.mark.parametrize("ydt", [moe.MOE_F32, moe.MOE_BF16])
def test_ffn_mxfp4_row_counts_at_pass_boundaries(T, k, d, f, counts, ydt):
    """The MXFP4 weight-streaming kernels stage an expert's rows in blocks over slices of the
    contraction (up to 4 rows over all of K, 8 over each half, 16 over each quarter, fewer
    slices where the block would not fit the LDS, as at K = 7936): experts with 1 to 16 rows
    on both sides of each block size, a short last tile inside a slice (K = 320, 192, 64),
    through the one-launch form (h exchanged as tagged entries), the two-launch form with one
    or four waves per strip (up to 32 tokens every expert, 17 to 31 rows in two blocks of 16)
    and, above 32 tokens, beside the grouped GEMM that takes the experts with more than 16
    rows; every row against the oracle on the exactly dequantised weights."""
    w = configs.Workload("mx_rows", seed=31, T=T, d=d, E=len(counts), k=k, f=f,
                         dtype=gen.MXFP4, alpha=0.0)
    ids = _ids_with_counts(counts, T, k)
    x = configs.gen_x(w)
    counts_o, offsets, perm, inv = oracle.permute(ids, w.E)
    np.testing.assert_array_equal(counts_o, counts)
    arena = device_arena_all_experts(w)
    nws = moe.moe_expert_ffn_workspace_bytes(T, k, w.f, w.act_dtype)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    ytd = torch.float32 if ydt == moe.MOE_F32 else torch.bfloat16
    y = torch.full((T * k, w.d), float("nan"), dtype=ytd, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_expert_ffn(x_device(w, x), w.act_dtype, dev(perm), dev(offsets), T, k, w.E, w.d, w.f,
                       None, arena, w.entry_bytes, w.dtype, None, None, 0, ws, nws, y, ydt,
                       moe.MOE_PATH_AUTO, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    table = oracle_table(w, sorted(set(ids.ravel().tolist())))
    ref = oracle.expert_ffn(x, ids, table, perm)
    assert_close(np_of(y), ref, bf16_tol(ref), f"y_perm mxfp4 T={T} counts={counts}")

@pytest.mark.parametrize("ydt", [moe.MOE_F32, moe.MOE_BF16])
def test_ffn_split_stale_slot_skips_only_that_expert(ydt):
    """Key-checked slots on the row-split path (T=48: more items than the looping launches'
    workgroups): a stale slot of one few-row expert and of one many-row expert sets
    MOE_ERANGE and leaves exactly those experts' rows unwritten; the looping workgroups go on
    to the items after them, so every other row still equals the oracle."""
    w = configs.Workload("split_stale", seed=29, T=48, d=512, E=256, k=6, f=256,
                         dtype=gen.BF16, alpha=0.5)
    x = configs.gen_x(w)
    lg = configs.gen_logits(w)
    ids, _ = oracle.route(lg, w.k)
    counts, offsets, perm, inv = oracle.permute(ids, w.E)
    few = [e for e in range(w.E) if 1 <= counts[e] <= 4]
    many = [e for e in range(w.E) if counts[e] > 4]
    assert few and many
    stale = {few[len(few) // 2], many[0]}
    arena = device_arena_all_experts(w)
    slots = dev(np.arange(w.E, dtype=np.int32))
    keys = np.arange(w.E, dtype=np.int32)
    for e in stale:
        keys[e] = -7
    A = w.T * w.k
    nws = moe.moe_expert_ffn_workspace_bytes(w.T, w.k, w.f, w.act_dtype)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    ytd = torch.float32 if ydt == moe.MOE_F32 else torch.bfloat16
    y = torch.full((A, w.d), float("nan"), dtype=ytd, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_expert_ffn(x_device(w, x), w.act_dtype, dev(perm), dev(offsets), w.T, w.k, w.E, w.d,
                       w.f, slots, arena, w.entry_bytes, w.dtype, None, dev(keys), 0, ws, nws, y,
                       ydt, moe.MOE_PATH_AUTO, status)
    torch.cuda.synchronize()
    assert int(status.item()) == moe.MOE_ERANGE
    yv = np_of(y)
    bad = np.zeros(A, dtype=bool)
    for e in stale:
        bad[offsets[e]:offsets[e + 1]] = True
    assert np.isnan(yv[bad]).all()
    table = oracle_table(w, sorted(set(ids.ravel().tolist())))
    ref = oracle.expert_ffn(x, ids, table, perm)
    assert_close(yv[~bad], ref[~bad], bf16_tol(ref), "rows of the other experts")


@pytest.mark.parametrize("T,E,k,d,f", [(8, 16, 6, 512, 256), (1, 8, 4, 4096, 2048), (8, 4, 2, 320, 192),
                                       (40, 6, 3, 1088, 448), (5, 64, 6, 2048, 4096),
                                       (32, 128, 8, 1088, 576),
                                       (4, 4, 2, 8128, 64),     # longest rows the streaming kernels stage
                                       (4, 4, 2, 64, 8192)])    # beyond it: the GEMM takes decode too
@pytest.mark.parametrize("ydt", [moe.MOE_F32, moe.MOE_BF16])
def test_ffn_mxfp4_parity(T, E, k, d, f, ydt):
    """MXFP4 expert weights (OCP MX: E2M1 codes, E8M0 scale per 32) against the oracle on the
    exactly dequantised weights: decode shapes, row lengths that leave a short last tile,
    experts with many rows (several staging passes), the full decode row lengths; strips
    streamed by one wave (many experts) and split over 2 or 4 waves (few experts)."""
    w = configs.Workload("mx", seed=25, T=T, d=d, E=E, k=k, f=f, dtype=gen.MXFP4, alpha=0.5)
    y, ref = _ffn_case(w, moe.MOE_PATH_AUTO, ydt)
    assert_close(y, ref, bf16_tol(ref), f"y_perm mxfp4 T={T} d={d} f={f}")


@pytest.mark.parametrize("T,E,k,d,f,alpha", [(64, 64, 4, 512, 256, 1.0), (48, 256, 6, 1088, 320, 1.0),
                                             (40, 32, 4, 320, 192, 0.5)])
@pytest.mark.parametrize("ydt", [moe.MOE_F32, moe.MOE_BF16])
def test_ffn_mxfp4_row_split_parity(T, E, k, d, f, alpha, ydt):
    """MXFP4 decode-shaped calls above 32 tokens: experts with at most 16 rows stay on the
    weight-streaming kernels, the others go to the grouped GEMM; both groups are present and
    every row equals the oracle."""
    w = configs.Workload("mx_split", seed=27, T=T, d=d, E=E, k=k, f=f, dtype=gen.MXFP4, alpha=alpha)
    ids, _ = oracle.route(configs.gen_logits(w), w.k)
    counts = np.bincount(ids.ravel(), minlength=w.E)
    assert (counts > 16).any() and ((counts > 0) & (counts <= 16)).any()
    y, ref = _ffn_case(w, moe.MOE_PATH_AUTO, ydt)
    assert_close(y, ref, bf16_tol(ref), f"y_perm mxfp4 split T={T} E={E}")


@pytest.mark.parametrize("T,E,k,d,f,alpha,path", [
    (300, 8, 2, 512, 256, 0.5, moe.MOE_PATH_AUTO),     # several 64-row blocks per expert
    (200, 6, 3, 320, 192, 0.5, moe.MOE_PATH_AUTO),     # short last tiles, partial weight blocks
    (512, 16, 4, 256, 384, 1.0, moe.MOE_PATH_AUTO),    # skewed: empty and crowded experts
    (64, 4, 2, 4096, 2048, 0.5, moe.MOE_PATH_GEMM),    # full row lengths, partial row blocks
    (1, 4, 2, 256, 128, 0.5, moe.MOE_PATH_GEMM)])      # a single token
@pytest.mark.parametrize("ydt", [moe.MOE_F32, moe.MOE_BF16])
def test_ffn_mxfp4_gemm_parity(T, E, k, d, f, alpha, path, ydt):
    """MXFP4 weights on the grouped-GEMM path (prefill-shaped counts) against the oracle on
    the exactly dequantised weights."""
    w = configs.Workload("mxg", seed=27, T=T, d=d, E=E, k=k, f=f, dtype=gen.MXFP4, alpha=alpha)
    y, ref = _ffn_case(w, path, ydt)
    assert_close(y, ref, bf16_tol(ref), f"y_perm mxfp4 gemm T={T} d={d} f={f}")


def _mx_ffn_call(w, x, perm, offsets, arena, ws, nws, ydt, slots=None, keys=None):
    """One MXFP4 moe_expert_ffn call on the weight-streaming path with nws workspace bytes;
    returns (y_perm as numpy, status)."""
    ytd = torch.float32 if ydt == moe.MOE_F32 else torch.bfloat16
    y = torch.full((w.T * w.k, w.d), float("nan"), dtype=ytd, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_expert_ffn(x_device(w, x), w.act_dtype, dev(perm), dev(offsets), w.T, w.k, w.E, w.d,
                       w.f, slots, arena, w.entry_bytes, w.dtype, None, keys, 0, ws, nws, y, ydt,
                       moe.MOE_PATH_AUTO, status)
    torch.cuda.synchronize()
    return np_of(y), int(status.item())


@pytest.mark.parametrize("T,E,k,d,f,alpha", [
    (8, 256, 6, 4096, 2048, 0.2),   # the decode layer: a wave per strip on both projections
    (8, 256, 6, 4096, 2048, 1.0),
    (8, 256, 6, 1024, 2048, 1.0),   # down strips split over 2 waves
    (8, 256, 6, 320, 1472, 0.5),    # over 4 waves; short last tiles on both projections
    (13, 256, 4, 1088, 1536, 0.5),  # experts with more than 4 rows: several staging passes
    (16, 128, 8, 512, 2048, 1.0),
    (2, 64, 6, 1024, 512, 0.5),     # too few gate/up strips: both calls take two launches
    (1, 16, 6, 512, 256, 0.5)])
@pytest.mark.parametrize("ydt", [moe.MOE_F32, moe.MOE_BF16])
def test_ffn_mxfp4_one_launch_matches_two_launches(T, E, k, d, f, alpha, ydt):
    """MXFP4 calls of up to 16 tokens whose workspace holds h as tagged entries run gate/up
    and down in one launch when gate/up has a wave per strip (min(E, T*k)*f >= 65536); with
    only the plain intermediate they take two launches.  Both give the same bits and equal the
    oracle within the bf16 rule.  A second one-launch call on the same workspace with other
    token rows (same routing) is checked too: the first call's entries carry the same tag, so
    only the clearing before each launch keeps them out."""
    w = configs.Workload("mx_one", seed=71 + T, T=T, d=d, E=E, k=k, f=f, dtype=gen.MXFP4,
                         alpha=alpha)
    lg = configs.gen_logits(w)
    ids, _ = oracle.route(lg, w.k)
    counts, offsets, perm, inv = oracle.permute(ids, w.E)
    arena = device_arena_all_experts(w)
    A = w.T * w.k
    nws = moe.moe_expert_ffn_workspace_bytes(w.T, w.k, w.f, w.act_dtype)
    assert nws >= A * w.f * 4
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    table = oracle_table(w, sorted(set(ids.ravel().tolist())))
    for call in range(2):
        x = configs.gen_x(configs.with_(w, seed=w.seed + 1000 * call))
        y1, st1 = _mx_ffn_call(w, x, perm, offsets, arena, ws, nws, ydt)
        y2, st2 = _mx_ffn_call(w, x, perm, offsets, arena, ws, A * w.f * 2, ydt)
        assert st1 == 0 and st2 == 0
        assert np.array_equal(y1.view(np.uint8), y2.view(np.uint8)), f"call {call}"
        ref = oracle.expert_ffn(x, ids, table, perm)
        assert_close(y1, ref, bf16_tol(ref), f"one launch T={T} call {call}")
    del arena


@pytest.mark.parametrize("T", [8, 16])
def test_ffn_mxfp4_one_launch_stale_slot_skips_only_that_expert(T):
    """Key-checked slots on the one-launch path: a stale slot sets MOE_ERANGE and leaves that
    expert's rows unwritten, and its down workgroups return without waiting for entries that
    no gate/up workgroup writes; every other row equals the oracle."""
    w = configs.Workload("mx_one_stale", seed=83 + T, T=T, d=1024, E=64, k=6, f=2048,
                         dtype=gen.MXFP4, alpha=0.5)
    x = configs.gen_x(w)
    ids, _ = oracle.route(configs.gen_logits(w), w.k)
    counts, offsets, perm, inv = oracle.permute(ids, w.E)
    used = [e for e in range(w.E) if counts[e] > 0]
    stale = {used[0], used[len(used) // 2]}
    keys = np.arange(w.E, dtype=np.int32)
    for e in stale:
        keys[e] = -7
    arena = device_arena_all_experts(w)
    A = w.T * w.k
    nws = moe.moe_expert_ffn_workspace_bytes(w.T, w.k, w.f, w.act_dtype)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    yv, st = _mx_ffn_call(w, x, perm, offsets, arena, ws, nws, moe.MOE_F32,
                          slots=dev(np.arange(w.E, dtype=np.int32)), keys=dev(keys))
    assert st == moe.MOE_ERANGE
    bad = np.zeros(A, dtype=bool)
    for e in stale:
        bad[offsets[e]:offsets[e + 1]] = True
    assert bad.any() and (~bad).any() and np.isnan(yv[bad]).all()
    ref = oracle.expert_ffn(x, ids, oracle_table(w, sorted(set(ids.ravel().tolist()))), perm)
    assert_close(yv[~bad], ref[~bad], bf16_tol(ref), "rows of the other experts")
    del arena


def test_ffn_gemm_wide_n_tiles():
    w = configs.Workload("gemm_wide", seed=22, T=400, d=384, E=6, k=2, f=448, dtype=gen.BF16,
                         alpha=1.0)
    y, ref = _ffn_case(w, moe.MOE_PATH_GEMM)
    assert_close(y, ref, bf16_tol(ref), "y_perm gemm")


# ---------------------------------------------------------------- degenerate FFN calls
def _ffn_masked(w, path, mask=None, ydt=moe.MOE_F32):
    """As _ffn_case with an optional expert mask; returns (y, ref, offsets) with y NaN-filled
    where nothing was written."""
    x = configs.gen_x(w)
    lg = configs.gen_logits(w)
    ids, _ = oracle.route(lg, w.k)
    counts, offsets, perm, inv = oracle.permute(ids, w.E)
    arena = device_arena_all_experts(w)
    A = w.T * w.k
    nws = moe.moe_expert_ffn_workspace_bytes(w.T, w.k, w.f, w.act_dtype)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    ytd = torch.float32 if ydt == moe.MOE_F32 else torch.bfloat16
    y = torch.full((A, w.d), float("nan"), dtype=ytd, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    moe.moe_expert_ffn(x_device(w, x), w.act_dtype, dev(perm), dev(offsets), w.T, w.k, w.E, w.d,
                       w.f, None, arena, w.entry_bytes, w.dtype,
                       None if mask is None else dev(mask.astype(np.uint8)), None, 0, ws, nws,
                       y, ydt, path, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    table = oracle_table(w, sorted(set(ids.ravel().tolist())))
    return np_of(y), oracle.expert_ffn(x, ids, table, perm), offsets


_PATHS = [moe.MOE_PATH_AUTO, moe.MOE_PATH_GEMV, moe.MOE_PATH_GEMM]


@pytest.mark.parametrize("dtype", [gen.BF16, gen.MXFP4])
@pytest.mark.parametrize("path", _PATHS)
@pytest.mark.parametrize("T,E,k", [(5, 1, 1), (6, 4, 4), (24, 3, 3)])
def test_ffn_single_expert_and_all_experts(T, E, k, path, dtype):
    """E = 1 (every token to the one expert: a dense SwiGLU FFN) and k = E (every token to
    every expert), on each path, bf16 and MXFP4 weights."""
    w = configs.Workload("degenerate", seed=41 + T + E, T=T, d=192, E=E, k=k, f=128,
                         dtype=dtype, alpha=0.5)
    y, ref, _ = _ffn_masked(w, path)
    assert_close(y, ref, bf16_tol(ref), f"E={E} k={k} path={path}")


@pytest.mark.parametrize("dtype", [gen.BF16, gen.MXFP4])
@pytest.mark.parametrize("path", _PATHS)
def test_ffn_zero_tokens_writes_nothing(path, dtype):
    w = configs.Workload("empty", seed=43, T=1, d=128, E=8, k=2, f=64, dtype=dtype, alpha=0.5)
    arena = device_arena_all_experts(w)
    y = torch.full((1, w.d), float("nan"), device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    one = dev(np.zeros(w.E + 1, dtype=np.int32))
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    xb = torch.zeros((1, w.d), dtype=torch.bfloat16, device="cuda")
    moe.moe_expert_ffn(xb, w.act_dtype, one, one, 0, w.k, w.E, w.d, w.f, None, arena,
                       w.entry_bytes, w.dtype, None, None, 0, ws, 256, y, moe.MOE_F32, path, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and torch.isnan(y).all()


def test_ffn_mxfp4_one_launch_expert_mask_selects_experts():
    """expert_mask on the one-launch MXFP4 path (T=8, f=2048: a wave per gate/up strip):
    the flagged experts' rows equal the oracle, every other row is left as it was, and the
    masked experts' down workgroups wait for nothing."""
    w = configs.Workload("masked_one", seed=59, T=8, d=512, E=256, k=6, f=2048,
                         dtype=gen.MXFP4, alpha=0.5)
    assert min(w.E, w.T * w.k) * w.f >= 65536
    mask = np.zeros(w.E, dtype=bool)
    mask[np.random.default_rng(7).permutation(w.E)[: w.E // 3]] = True
    y, ref, offsets = _ffn_masked(w, moe.MOE_PATH_AUTO, mask)
    on = np.zeros(w.T * w.k, dtype=bool)
    for e in np.flatnonzero(mask):
        on[offsets[e]:offsets[e + 1]] = True
    assert on.any() and (~on).any()
    assert np.isnan(y[~on]).all()
    assert_close(y[on], ref[on], bf16_tol(ref), "masked experts, one launch")


@pytest.mark.parametrize("dtype", [gen.BF16, gen.MXFP4])
@pytest.mark.parametrize("T,path", [(8, moe.MOE_PATH_GEMV), (48, moe.MOE_PATH_GEMV),
                                    (100, moe.MOE_PATH_GEMV), (300, moe.MOE_PATH_GEMM)])
def test_ffn_expert_mask_selects_experts(T, path, dtype):
    """expert_mask runs only the flagged experts: their rows equal the oracle, every other
    row is left as it was (one-item, looping row-split and grouped-GEMM launches)."""
    w = configs.Workload("masked", seed=47 + T, T=T, d=512, E=256, k=6, f=256, dtype=dtype,
                         alpha=0.5)
    mask = np.zeros(w.E, dtype=bool)
    mask[np.random.default_rng(T).permutation(w.E)[: w.E // 3]] = True
    y, ref, offsets = _ffn_masked(w, path, mask)
    on = np.zeros(w.T * w.k, dtype=bool)
    for e in np.flatnonzero(mask):
        on[offsets[e]:offsets[e + 1]] = True
    assert on.any() and (~on).any()
    assert np.isnan(y[~on]).all()
    assert_close(y[on], ref[on], bf16_tol(ref), f"masked rows T={T} path={path}")


# ---------------------------------------------------------------- measurement probes
@pytest.mark.parametrize("nbytes", [16, 2048 * 16 + 16, 3 * (1 << 20) + 48, (200 << 20) + 16])
def test_probes_read_and_copy_every_byte_once(nbytes):
    """The read probe's per-workgroup words XOR to the XOR of every 32-bit word of the source
    (a word read twice or skipped would change it), and the copy probe's destination equals
    the source with nothing past it written; sizes leave partial chunks, and the largest takes
    the read probe's grid-stride loop twice."""
    r = np.random.default_rng(nbytes)
    src_np = r.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    src = dev(src_np.view(np.int32))
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    moe.moe_hbm_read_probe(src, nbytes, sink)
    dst = torch.full((nbytes // 4 + 16,), -1, dtype=torch.int32, device="cuda")
    moe.moe_copy_probe(src, dst, nbytes)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(src_np)
    got = dst.cpu().numpy()
    np.testing.assert_array_equal(got[:nbytes // 4].view(np.uint32), src_np)
    assert (got[nbytes // 4:] == -1).all()

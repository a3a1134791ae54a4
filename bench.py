"""Benchmark of the routed-MoE layer hot path on one MI355X.

Primary line: one decode-shaped MoE layer forward (E=256 experts, top-6,
d=4096, f=2048, bf16 weights, T=8 tokens, all experts resident in HBM):
route -> permute -> expert FFN (weight-streaming path) -> combine, replayed
from captured HIP graphs over 16 pre-drawn routing sets.  value = tokens/s.

Extra measurements in the same JSON line ("extra"): the decode layer at
T = 1, 64 and 128 and at Zipf alpha 1, the T=8192 prefill layer (grouped-GEMM path), the 16-layer decode loop through the bounded LRU
expert cache with PCIe miss fills, and the 8-layer prefill with full-layer
double-buffered streaming.  All inputs are seeded synthetic tensors shaped
like the FreeToken pages' models; weights are random.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|decode|prefill|lru|stream]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def _mk_event(torch, stream, timing=False):
    """A torch event whose HIP handle exists (recorded once), so it can be passed to the C ABI."""
    ev = torch.cuda.Event(enable_timing=timing)
    ev.record(stream)
    return ev


def _ffn_bytes(w, U, y_bytes=4):
    """Algorithmic HBM bytes of one expert-FFN call: every used expert entry once, token rows
    gathered once per assignment, h written and read once (bf16), y written once (fp32, or
    y_bytes per element)."""
    A = w.T * w.k
    return U * w.entry_bytes + A * w.d * 2 + 2 * A * w.f * 2 + A * w.d * y_bytes


def _token_bytes(w, U):
    """Algorithmic HBM bytes of one single-token one-launch layer: every used expert entry
    once, the logits and x read, h written and read once (bf16), out written (fp32)."""
    return U * w.entry_bytes + w.E * 4 + w.d * 2 + 2 * w.k * w.f * 2 + w.d * 4


_STREAMS = {}


def _stream(torch, role):
    """The stream of a role ("comp", "copy", "side"), created once per process.  HIP maps
    streams onto a few hardware queues (GPU_MAX_HW_QUEUES, 4 here); streams that share a
    queue run in queue order, so a fresh pair of streams per measurement can serialise a
    copy with unrelated compute.  One stream per role, created together at start-up, keeps
    the roles on distinct queues for every measurement."""
    if not _STREAMS:
        for r in ("comp", "copy", "side"):
            _STREAMS[r] = torch.cuda.Stream()
    return _STREAMS[role]


def _ffn_flops(w):
    return 2.0 * w.T * w.k * 3 * w.d * w.f


CSRC = os.path.join(ROOT, "expert_ffn_cache_amd", "csrc")
# sources of the decode expert-FFN kernels (dot-product kernels and the headers they
# include), which the committed counter summary was taken on
DECODE_FFN_SOURCES = [os.path.join(CSRC, n) for n in ("common.h", "ffn_args.h", "wave.h", "ffn_dot.hip")]
# the same for MXFP4 weights (FP4-expanding MFMA kernels)
MXFP4_FFN_SOURCES = [os.path.join(CSRC, n) for n in ("common.h", "ffn_args.h", "mx_dev.h", "ffn_mx.hip")]


def sources_sha256(paths):
    """sha256 over the concatenated bytes of the given kernel sources, in order."""
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


# sources of the prefill grouped GEMMs (bf16, MXFP4) and the headers they include
PREFILL_GEMM_SOURCES = [os.path.join(CSRC, n) for n in ("common.h", "ffn_args.h", "ffn_gemm.hip")]
MXFP4_GEMM_SOURCES = [os.path.join(CSRC, n) for n in ("common.h", "ffn_args.h", "ffn_mx_gemm.hip")]
PREFILL_TRAFFIC = "gemm_prefill_e256_k6_d4096_f2048_T8192_traffic.txt"


def _prefill_traffic(dtype, alpha):
    """HBM bytes per prefill FFN call at Zipf alpha from the committed counter summary, if it
    was taken on the current GEMM sources; else None."""
    import gen
    mx = dtype == gen.MXFP4
    key = f"{'mxfp4' if mx else 'bf16'}_alpha_{alpha}_hbm_bytes_per_call"
    return _counter_traffic(MXFP4_GEMM_SOURCES if mx else PREFILL_GEMM_SOURCES, PREFILL_TRAFFIC,
                            key=key, sha_key=f"{'mxfp4' if mx else 'bf16'}_kernel_source_sha256")


def _counter_traffic(kernel_srcs, name, key="hbm_bytes_per_call", sha_key="kernel_source_sha256"):
    """HBM bytes per FFN call from the committed rocprofv3 counter summary, if it was taken
    on the current kernel sources (sha256 match); else None."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    sha = sources_sha256(kernel_srcs)
    vals = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get(sha_key) != sha or key not in vals:
        return None
    return float(vals[key])


# ------------------------------------------------------------------------ decode layer
def decode_arena(torch, dtype=None):
    """All 256 experts of the decode layer, resident (shared by every decode measurement of
    one weight format)."""
    from gen import configs
    from gen.arena import device_arena_all_experts
    w = configs.DECODE if dtype is None else configs.with_(configs.DECODE, dtype=dtype)
    t0 = time.time()
    arena = device_arena_all_experts(w)
    log(f"[decode] arena {w.E} x {w.entry_bytes / 1e6:.1f} MB generated in {time.time() - t0:.1f}s")
    return arena


def bench_decode(args, torch, moe, T, alpha, arena, dtype=None):
    import gen
    from gen import configs
    from expert_ffn_cache_amd.layer import MoeLayer

    w = configs.with_(configs.DECODE, T=T, alpha=alpha)
    if dtype is not None:
        w = configs.with_(w, dtype=dtype)
    path = {"auto": moe.MOE_PATH_AUTO, "gemv": moe.MOE_PATH_GEMV, "gemm": moe.MOE_PATH_GEMM}[args.ffn_path]
    R = 16
    x = torch.from_numpy(configs.gen_x(w).view(np.int16)).view(torch.bfloat16).cuda()
    logits = [torch.from_numpy(configs.gen_logits(w, rotation=r)).cuda() for r in range(R)]
    layers = [MoeLayer(w.T, w.E, w.k, w.d, w.f, w_dtype=w.dtype) for _ in range(R)]
    s = _stream(torch, "comp")
    graphs = []
    with torch.cuda.stream(s):
        for r in range(R):
            layers[r].forward(x, logits[r], arena, w.entry_bytes, path=path, stream=s)
        s.synchronize()
        # experts each layer reads (from the routed ids: the one-launch single-token path
        # leaves counts untouched)
        U = [int(torch.unique(layers[r].ids).numel()) for r in range(R)]
        fused = [layers[r].fusable and path == moe.MOE_PATH_AUTO for r in range(R)]
        if not args.no_graph:
            for r in range(R):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    layers[r].forward(x, logits[r], arena, w.entry_bytes, path=path, stream=s)
                graphs.append(g)

        def run(i):
            if args.no_graph:
                layers[i % R].forward(x, logits[i % R], arena, w.entry_bytes, path=path, stream=s)
            else:
                graphs[i % R].replay()
        for i in range(args.warmup):
            run(i)
        s.synchronize()
        e0, e1 = _events(torch, 2)
        torch.cuda.synchronize()
        e0.record(s)
        for i in range(args.steps):
            run(i)
        e1.record(s)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # the same R layer forwards captured back to back in one graph (as a serving step runs
    # its layers): per-layer time without the launch gap between single-layer replays
    ms_multi = None
    if not args.no_graph:
        with torch.cuda.stream(s):
            gm = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gm, stream=s):
                for r in range(R):
                    layers[r].forward(x, logits[r], arena, w.entry_bytes, path=path, stream=s)
            gm.replay()
            s.synchronize()
            reps = max(1, args.steps // R)
            e2, e3 = _events(torch, 2)
            torch.cuda.synchronize()
            e2.record(s)
            for _ in range(reps):
                gm.replay()
            e3.record(s)
            torch.cuda.synchronize()
            ms_multi = e2.elapsed_time(e3) / (reps * R)
            del gm
    # the dominant entry point, timed per call with events on its stream: the expert FFN
    # (gate/up + down weight-streaming kernels), or for one token the one-launch layer
    ffn_ms = []
    with torch.cuda.stream(s):
        n = max(args.steps, 2 * R)
        starts, ends = _events(torch, n), _events(torch, n)
        for i in range(n):
            r = i % R
            starts[i].record(s)
            if fused[r]:
                layers[r].decode_token(x, logits[r], arena, w.entry_bytes, stream=s)
            else:
                layers[r].ffn(x, arena, w.entry_bytes, path=path, stream=s)
            ends[i].record(s)
        torch.cuda.synchronize()
        ffn_ms = [starts[i].elapsed_time(ends[i]) for i in range(n)]
        byts = [(_token_bytes if fused[i % R] else _ffn_bytes)(w, U[i % R]) for i in range(n)]
    status = max(int(layers[r].status.item()) for r in range(R))
    if status != 0:
        raise RuntimeError(f"decode: device status {status}")
    ffn_avg_ms = float(np.mean(ffn_ms))
    achieved = float(np.sum(byts) / (np.sum(ffn_ms) * 1e-3) / 1e9)
    A = w.T * w.k
    if all(fused):
        step_bytes = float(np.mean(byts))  # the launch is the whole step
    else:
        step_bytes = float(np.mean(byts)) + w.T * w.E * 4 + A * w.d * 4 + w.T * w.d * 4
    traffic = None
    if T == 8 and alpha == 0.2:  # what the committed counter summaries cover
        if dtype is None:
            traffic = _counter_traffic(DECODE_FFN_SOURCES, "ffn_dot_decode_e256_k6_d4096_f2048_T8_counters.txt")
        elif dtype == gen.MXFP4:
            traffic = _counter_traffic(MXFP4_FFN_SOURCES, "ffn_mx_decode_e256_k6_d4096_f2048_T8_counters.txt")
    del graphs
    torch.cuda.empty_cache()
    return dict(
        workload=w.name, T=w.T, ms_per_step=ms, tok_s=w.T / (ms * 1e-3), U_mean=float(np.mean(U)),
        dominant="moe_decode_token" if all(fused) else "moe_expert_ffn",
        ffn_ms=ffn_avg_ms,
        ms_per_layer_in_16_layer_graph=ms_multi,
        tok_s_16_layer_graph=None if ms_multi is None else w.T / (ms_multi * 1e-3),
        roofline=dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=achieved / HBM_PEAK_GBS,
                      traffic=None if traffic is None else traffic),
        algorithmic_bytes_per_call=float(np.mean(byts)),
        # the whole step (route + group + FFN + combine) against the same roof: the FFN's
        # bytes plus the logits read, y read back by the combine and out written
        step_bytes=step_bytes, step_hbm_frac=step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)


def _sweep_entry(r):
    """One decode-sweep record: single-layer graph replays, the same layers captured 16 to a
    graph, and the dominant entry point (the expert FFN, or for one token the one-launch
    layer) against the HBM roof."""
    us16 = r["ms_per_layer_in_16_layer_graph"]
    return dict(tok_s=r["tok_s"], us_per_layer=r["ms_per_step"] * 1e3,
                tok_s_16_layer_graph=r["tok_s_16_layer_graph"],
                us_per_layer_16_layer_graph=None if us16 is None else us16 * 1e3,
                dominant=r["dominant"], ffn_us=r["ffn_ms"] * 1e3, unique_experts=r["U_mean"],
                ffn_gbs=r["roofline"]["achieved"], hbm_frac=r["roofline"]["frac"])


# ------------------------------------------------------------------------ prefill layer
def bench_prefill(args, torch, moe, dtype=None):
    from gen import configs
    from gen.arena import device_arena_all_experts
    from expert_ffn_cache_amd.layer import MoeLayer

    out = {}
    t0 = time.time()
    base = configs.PREFILL if dtype is None else configs.with_(configs.PREFILL, dtype=dtype)
    arena = device_arena_all_experts(base)
    log(f"[prefill] arena generated in {time.time() - t0:.1f}s")
    x = torch.from_numpy(configs.gen_x(base).view(np.int16)).view(torch.bfloat16).cuda()
    alphas = (0.2, 1.0) if args.prefill_alpha is None else (args.prefill_alpha,)
    for alpha in alphas:
        w = configs.with_(base, alpha=alpha)
        R = 2
        logits = [torch.from_numpy(configs.gen_logits(w, rotation=r)).cuda() for r in range(R)]
        layers = [MoeLayer(w.T, w.E, w.k, w.d, w.f, y_dtype=moe.MOE_BF16, w_dtype=w.dtype)
                  for _ in range(R)]
        s = _stream(torch, "comp")
        steps = max(4, args.steps // 5)
        with torch.cuda.stream(s):
            for r in range(R):
                layers[r].forward(x, logits[r], arena, w.entry_bytes, stream=s)
            s.synchronize()
            U = [int((layers[r].counts > 0).sum().item()) for r in range(R)]
            maxc = [int(layers[r].counts.max().item()) for r in range(R)]
            graphs = []
            for r in range(R):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    layers[r].forward(x, logits[r], arena, w.entry_bytes, stream=s)
                graphs.append(g)
            for i in range(2):
                graphs[i % R].replay()
            e0, e1 = _events(torch, 2)
            torch.cuda.synchronize()
            e0.record(s)
            for i in range(steps):
                graphs[i % R].replay()
            e1.record(s)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            starts, ends = _events(torch, steps), _events(torch, steps)
            for i in range(steps):
                starts[i].record(s)
                layers[i % R].ffn(x, arena, w.entry_bytes, stream=s)
                ends[i].record(s)
            torch.cuda.synchronize()
        ffn_ms = float(np.mean([starts[i].elapsed_time(ends[i]) for i in range(steps)]))
        status = max(int(l.status.item()) for l in layers)
        if status != 0:
            raise RuntimeError(f"prefill: device status {status}")
        fl = _ffn_flops(w)
        byts = float(np.mean([_ffn_bytes(w, u, y_bytes=2) for u in U]))
        # the binding roof: the larger of the MFMA-peak and HBM-peak times of the call
        t_mfma, t_hbm = fl / (BF16_PEAK_TFLOPS * 1e12) * 1e3, byts / (HBM_PEAK_GBS * 1e9) * 1e3
        out[f"alpha_{alpha}"] = dict(
            T=w.T, ms_per_step=ms, tok_s=w.T / (ms * 1e-3), ffn_ms=ffn_ms, U_mean=float(np.mean(U)),
            max_tokens_per_expert=int(np.max(maxc)),
            ffn_tflops=fl / (ffn_ms * 1e-3) / 1e12, mfma_frac=fl / (ffn_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            ffn_weight_gbs=byts / (ffn_ms * 1e-3) / 1e9,
            hbm_frac=byts / (ffn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            roofline_bound="hbm" if t_hbm >= t_mfma else "mfma",
            roofline_floor_ms=max(t_mfma, t_hbm), roofline_frac=max(t_mfma, t_hbm) / ffn_ms)
        traffic = _prefill_traffic(dtype, alpha)
        if traffic is not None:  # HBM bytes of the call from the committed counter summary
            out[f"alpha_{alpha}"].update(traffic_bytes=traffic, algorithmic_bytes=byts,
                                         traffic_over_algorithmic=traffic / byts)
        del graphs, layers
    out["workload"] = base.name
    del arena
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------------ multi-layer LRU decode
def bench_lru(args, torch, moe, dtype=None, with_resize=True):
    import ctypes
    from gen import configs
    import gen
    from gen.arena import host_pool, torch_dtype
    from expert_ffn_cache_amd.layer import MoeLayer

    w = configs.LRU_DECODE if dtype is None else configs.with_(configs.LRU_DECODE, dtype=dtype)
    steps = args.lru_steps
    t0 = time.time()
    pool = host_pool(w)
    log(f"[lru] pinned pool {pool.nbytes / 1e9:.1f} GB in {time.time() - t0:.1f}s")
    _, lg = gen.markov_routing(w.seed, steps, w.L, w.T, w.E, w.k, w.p_stay, w.zipf_s)
    logits = torch.from_numpy(lg).cuda()
    xs = [torch.from_numpy(configs.gen_x(w, l).view(np.int16)).view(torch.bfloat16).cuda()
          for l in range(w.L)]
    arena = torch.empty((w.S, w.entry_elems), dtype=torch_dtype(w), device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    i64 = dict(dtype=torch.int64, device="cuda")
    slot_of, key_of = torch.empty(w.L * w.E, **i32), torch.empty(w.S, **i32)
    stamp, clock, stats = torch.empty(w.S, **i64), torch.empty(1, **i64), torch.empty(4, **i64)
    status = torch.zeros(1, **i32)
    desc = moe.moe_cache_t(w.L, w.E, w.S, w.L * w.E, w.entry_bytes, slot_of.data_ptr(), key_of.data_ptr(),
                           stamp.data_ptr(), clock.data_ptr(), stats.data_ptr(), status.data_ptr(),
                           arena.data_ptr(), pool.data_ptr())
    expert_slot = torch.empty(w.E, **i32)
    fills_dev = torch.empty((w.E + 1) * 4, **i32)  # records, then n_fills in the last word
    n_fills_dev = fills_dev[w.E * 4:]
    mirror = torch.empty((w.E + 1) * 4, dtype=torch.int32, pin_memory=True)
    masks = torch.zeros((2, 2, w.E), dtype=torch.uint8, pin_memory=True)
    masks_dev = torch.zeros((w.L, 2, w.E), dtype=torch.uint8, device="cuda")
    lay = MoeLayer(w.T, w.E, w.k, w.d, w.f, w_dtype=w.dtype)
    comp, copy = _stream(torch, "comp"), _stream(torch, "copy")
    # pinned H2D bandwidth for these entries: 64 pool entries into the arena (overwritten
    # by the fills later; the cache starts cold)
    nb = min(64, w.S) * w.entry_bytes
    with torch.cuda.stream(copy):
        moe.layer_stream_prefetch(pool.entry_ptr(0), arena, nb, 1, copy, None, None)
        ha, hb = _events(torch, 2)
        torch.cuda.synchronize()
        ha.record(copy)
        for _ in range(3):
            moe.layer_stream_prefetch(pool.entry_ptr(0), arena, nb, 1, copy, None, None)
        hb.record(copy)
        torch.cuda.synchronize()
    h2d_gbs = 3 * nb / (ha.elapsed_time(hb) * 1e-3) / 1e9
    last_ffn = _mk_event(torch, comp)
    fill_done = _mk_event(torch, copy)
    got = torch.cuda.Event()
    with torch.cuda.stream(comp):
        moe.cache_init(desc, comp)
        torch.cuda.synchronize()
        t_start = time.time()
        for s in range(steps):
            for l in range(w.L):
                lay.route(logits[s, l], comp)
                moe.cache_lookup_update(desc, l, lay.ids, w.T, w.k, expert_slot, fills_dev,
                                        n_fills_dev, comp)
                mirror.copy_(fills_dev, non_blocking=True)
                got.record(comp)
                lay.permute(comp)
                got.synchronize()  # the one host read per layer: the fill list
                n = int(mirror[w.E * 4])
                miss = mirror[:n * 4].view(n, 4).numpy()[:, 2] if n else np.zeros(0, np.int64)
                mk = masks[l % 2].numpy()
                mk[0, :] = 1
                mk[0, miss] = 0     # hits (experts with no tokens are skipped anyway)
                mk[1, :] = 0
                mk[1, miss] = 1     # misses
                masks_dev[l].copy_(masks[l % 2], non_blocking=True)
                if n:
                    copy.wait_event(last_ffn)  # WAR: earlier readers of the victim slots
                    moe.cache_fill(desc, mirror.data_ptr(), n, copy)
                    fill_done.record(copy)
                lay.ffn(xs[l], arena, w.entry_bytes, expert_slot, mask=masks_dev[l, 0],
                        slot_key=key_of, key_base=l * w.E, stream=comp)
                if n:
                    comp.wait_event(fill_done)
                    lay.ffn(xs[l], arena, w.entry_bytes, expert_slot, mask=masks_dev[l, 1],
                            slot_key=key_of, key_base=l * w.E, stream=comp)
                lay.combine(comp)
                last_ffn.record(comp)
        torch.cuda.synchronize()
        wall = time.time() - t_start
    st = stats.cpu().numpy()
    if int(status.item()) != 0 or int(lay.status.item()) != 0:
        raise RuntimeError(f"lru: status {int(status.item())} / {int(lay.status.item())}")
    out_host = lay.out.clone()

    # the same loop with device-driven fills: one decode step (all layers, misses included)
    # captured once as a graph and replayed per step; no host reads.  With overlap the graph
    # forks after each lookup: the fill kernel runs on a side branch while the FFN of the
    # hits runs, and the FFN of the misses follows the join.
    lg_static = torch.empty((w.L, w.T, w.E), dtype=torch.float32, device="cuda")
    side = _stream(torch, "side")
    walls = {}
    for overlap in (False, True):
        with torch.cuda.stream(comp):
            moe.cache_init(desc, comp)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=comp):
                for l in range(w.L):
                    lay.route(lg_static[l], comp)
                    moe.cache_lookup_update(desc, l, lay.ids, w.T, w.k, expert_slot, fills_dev,
                                            n_fills_dev, comp)
                    key = dict(slot_key=key_of, key_base=l * w.E, stream=comp)
                    if overlap:
                        hit, miss = masks_dev[l, 0], masks_dev[l, 1]
                        moe.cache_fill_masks(expert_slot, fills_dev, n_fills_dev, w.E, hit, miss,
                                             status, comp)
                        side.wait_stream(comp)
                        moe.cache_fill_device(desc, fills_dev, n_fills_dev, w.E, side)
                        lay.permute(comp)
                        lay.ffn(xs[l], arena, w.entry_bytes, expert_slot, mask=hit, **key)
                        comp.wait_stream(side)
                        lay.ffn(xs[l], arena, w.entry_bytes, expert_slot, mask=miss, **key)
                    else:
                        moe.cache_fill_device(desc, fills_dev, n_fills_dev, w.E, comp)
                        lay.permute(comp)
                        lay.ffn(xs[l], arena, w.entry_bytes, expert_slot, **key)
                    lay.combine(comp)
            torch.cuda.synchronize()
            t_start = time.time()
            for s in range(steps):
                lg_static.copy_(logits[s])
                g.replay()
            torch.cuda.synchronize()
            walls[overlap] = time.time() - t_start
        st_g = stats.cpu().numpy()
        if int(status.item()) != 0 or int(lay.status.item()) != 0:
            raise RuntimeError(f"lru graph: status {int(status.item())} / {int(lay.status.item())}")
        if not np.array_equal(st, st_g) or not torch.equal(out_host, lay.out):
            raise RuntimeError("lru graph path disagrees with the host-driven path")
        del g
    wall_g = walls[False]

    # elastic resize at a safe point: 1024 -> 512 slots (keeps the 512 most recent entries,
    # copied arena to arena), then 512 -> 1536
    def make_cache(S2):
        t = dict(slot_of=torch.empty(w.L * w.E, **i32), key_of=torch.empty(S2, **i32),
                 stamp=torch.empty(S2, **i64), clock=torch.empty(1, **i64),
                 stats=torch.empty(4, **i64), status=torch.zeros(1, **i32),
                 arena=torch.empty((S2, w.entry_elems), dtype=torch_dtype(w), device="cuda"))
        d = moe.moe_cache_t(w.L, w.E, S2, w.L * w.E, w.entry_bytes, *(t[n].data_ptr() for n in (
            "slot_of", "key_of", "stamp", "clock", "stats", "status", "arena")), pool.data_ptr())
        return d, t
    resize = {}
    cur, keep_alive = desc, None
    for S2 in ((w.S // 2, w.S * 3 // 2) if with_resize else ()):
        d2, t2 = make_cache(S2)
        e0, e1 = _events(torch, 2)
        with torch.cuda.stream(comp):
            torch.cuda.synchronize()
            e0.record(comp)
            moe.cache_resize(cur, d2, comp)
            e1.record(comp)
            torch.cuda.synchronize()
        kept = int((t2["key_of"] >= 0).sum().item())
        ms = e0.elapsed_time(e1)
        resize[f"{cur.S}_to_{S2}"] = dict(ms=ms, kept=kept,
                                          copy_gbs=2 * kept * w.entry_bytes / (ms * 1e-3) / 1e9)
        cur, keep_alive = d2, t2
    keep_alive = None
    pool.close()
    del arena
    torch.cuda.empty_cache()
    return dict(workload=w.name, weights="mxfp4" if w.dtype == gen.MXFP4 else "bf16",
                entry_bytes=w.entry_bytes, steps=steps, tok_s=steps * w.T / wall, wall_s=wall,
                graph_device_fill_tok_s=steps * w.T / wall_g, graph_wall_s=wall_g,
                graph_overlap_tok_s=steps * w.T / walls[True], graph_overlap_wall_s=walls[True],
                graph_overlap_fill_gbs=float(st[3]) / walls[True] / 1e9, resize=resize,
                miss_rate=float(st[2] / st[0]), hits=int(st[1]), misses=int(st[2]),
                fill_gb=float(st[3] / 1e9), fill_gb_per_step=float(st[3] / 1e9 / steps),
                h2d_gbs=h2d_gbs, fill_time_s=float(st[3]) / (h2d_gbs * 1e9),
                fill_time_over_wall=float(st[3]) / (h2d_gbs * 1e9) / wall,
                fill_time_over_graph_overlap_wall=float(st[3]) / (h2d_gbs * 1e9) / walls[True])


# ------------------------------------------------------------------------ streamed prefill
def bench_stream(args, torch, moe, dtype=None):
    import gen
    from gen import configs
    from gen.arena import host_pool, torch_dtype
    from expert_ffn_cache_amd.layer import MoeLayer

    w = configs.STREAM_PREFILL if dtype is None else configs.with_(configs.STREAM_PREFILL, dtype=dtype)
    t0 = time.time()
    pool = host_pool(w)
    log(f"[stream] pinned pool {pool.nbytes / 1e9:.2f} GB in {time.time() - t0:.1f}s")
    layer_bytes = w.E * w.entry_bytes
    bufs = [torch.empty((w.E, w.entry_elems), dtype=torch_dtype(w), device="cuda") for _ in range(2)]
    xs = [torch.from_numpy(configs.gen_x(w, l).view(np.int16)).view(torch.bfloat16).cuda()
          for l in range(w.L)]
    lgs = [torch.from_numpy(configs.gen_logits(w, layer=l)).cuda() for l in range(w.L)]
    layers = [MoeLayer(w.T, w.E, w.k, w.d, w.f, y_dtype=moe.MOE_BF16, w_dtype=w.dtype)
              for _ in range(w.L)]
    comp, copy = _stream(torch, "comp"), _stream(torch, "copy")
    # measured pinned H2D bandwidth (one layer block through the same copy entry point)
    with torch.cuda.stream(copy):
        a, b = _events(torch, 2)
        moe.layer_stream_prefetch(pool.entry_ptr(0), bufs[0], layer_bytes, 1, copy, None, None)
        torch.cuda.synchronize()
        a.record(copy)
        for _ in range(3):
            moe.layer_stream_prefetch(pool.entry_ptr(0), bufs[0], layer_bytes, 1, copy, None, None)
        b.record(copy)
        torch.cuda.synchronize()
    h2d_gbs = 3 * layer_bytes / (a.elapsed_time(b) * 1e-3) / 1e9
    runs = []
    for rep in range(3):
        ready = [_mk_event(torch, copy, timing=True) for _ in range(w.L)]
        cstart = _events(torch, w.L)
        cend = _events(torch, w.L)
        pstart = _events(torch, w.L)
        free = [_mk_event(torch, comp) for _ in range(2)]
        torch.cuda.synchronize()
        t_start = _events(torch, 1)[0]
        t_start.record(copy)
        pstart[0].record(copy)
        moe.layer_stream_prefetch(pool.entry_ptr(0), bufs[0], layer_bytes, 1, copy, None, ready[0])
        for l in range(w.L):
            if l + 1 < w.L:
                nb = (l + 1) % 2
                if l >= 1:
                    copy.wait_event(free[nb])  # compute of layer l-1 released this buffer
                pstart[l + 1].record(copy)
                moe.layer_stream_prefetch(pool.entry_ptr((l + 1) * w.E), bufs[nb], layer_bytes,
                                          1, copy, None, ready[l + 1])
            comp.wait_event(ready[l])
            cstart[l].record(comp)
            layers[l].forward(xs[l], lgs[l], bufs[l % 2], w.entry_bytes, stream=comp)
            cend[l].record(comp)
            free[l % 2].record(comp)
        torch.cuda.synchronize()
        wall_ms = t_start.elapsed_time(cend[-1])
        copies = [(t_start.elapsed_time(pstart[l]), t_start.elapsed_time(ready[l])) for l in range(w.L)]
        comps = [(t_start.elapsed_time(cstart[l]), t_start.elapsed_time(cend[l])) for l in range(w.L)]
        ov = 0.0
        for c0, c1 in comps:
            for p0, p1 in copies:
                ov += max(0.0, min(c1, p1) - max(c0, p0))
        runs.append((wall_ms, copies, comps, ov / sum(c1 - c0 for c0, c1 in comps)))
    wall_ms, copies, comps, overlap = min(runs, key=lambda r: r[0])
    status = max(int(l.status.item()) for l in layers)
    if status != 0:
        raise RuntimeError(f"stream: device status {status}")
    ideal_ms = w.L * layer_bytes / (h2d_gbs * 1e9) * 1e3
    # closed-form double-buffer timing from the measured per-layer copy (c) and compute (k)
    # times: the first copy, then each step waits for the longer of the next copy and the
    # current compute, then the last compute
    c = [b - a for a, b in copies]
    k = [b - a for a, b in comps]
    model_ms = c[0] + sum(max(c[l + 1], k[l]) for l in range(w.L - 1)) + k[-1]
    pool.close()
    del bufs
    torch.cuda.empty_cache()
    return dict(workload=w.name, weights="mxfp4" if w.dtype == gen.MXFP4 else "bf16",
                layer_bytes=layer_bytes, tok_s=w.T / (wall_ms * 1e-3), wall_ms=wall_ms,
                h2d_gbs=h2d_gbs, ideal_ms=ideal_ms, efficiency=ideal_ms / wall_ms,
                model_ms=model_ms, wall_over_model=wall_ms / model_ms,
                overlap=overlap, copy_ms_per_layer=float(np.mean([b - a for a, b in copies])),
                compute_ms_per_layer=float(np.mean([b - a for a, b in comps])))


# ------------------------------------------------------------------------ calibration probes
def bench_probe(args, torch, moe):
    """Achievable HBM read bandwidth (read probe) and a plain copy of known size (the
    reference for scaling hardware byte counters: 1 GiB read + 1 GiB written per copy)."""
    n = 1 << 30
    nr = 4 << 30  # read probe: 4 GiB, far beyond the 256 MB last-level cache
    big = torch.empty(nr, dtype=torch.uint8, device="cuda")
    big.fill_(1)
    src = big[:n]
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    s = _stream(torch, "comp")
    reps = 10
    with torch.cuda.stream(s):
        moe.moe_hbm_read_probe(big, nr, sink, s)
        moe.moe_copy_probe(src, dst, n, s)
        a, b, c = _events(torch, 3)
        torch.cuda.synchronize()
        a.record(s)
        for _ in range(reps):
            moe.moe_hbm_read_probe(big, nr, sink, s)
        b.record(s)
        for _ in range(reps):
            moe.moe_copy_probe(src, dst, n, s)
        c.record(s)
        torch.cuda.synchronize()
    read_gbs = reps * nr / (a.elapsed_time(b) * 1e-3) / 1e9
    copy_gbs = reps * 2 * n / (b.elapsed_time(c) * 1e-3) / 1e9
    del big
    return dict(read_bytes=nr, copy_bytes=n, read_gbs=read_gbs, copy_gbs=copy_gbs,
                read_frac=read_gbs / HBM_PEAK_GBS)


# ------------------------------------------------------------------------ CPU baseline
def _oracle_rate(layer_fn, tokens_per_call, seconds, max_calls=4096):
    spent, tokens, calls = 0.0, 0, 0
    while spent < seconds and calls < max_calls:
        t0 = time.perf_counter()
        layer_fn(calls)
        spent += time.perf_counter() - t0
        tokens += tokens_per_call
        calls += 1
    return tokens / spent, calls, spent


def cpu_baseline(args):
    """The oracle (plain double-precision C; OpenMP over the (token, expert) FFNs of a layer,
    the same arithmetic at any thread count) on whole decode layers, timed on the host cores,
    cycling over 16 rotated routing sets until about args.cpu_seconds of time has been spent
    (weights generated once, untimed).  Also on one core: the same decode layer and the tiny
    fp32 layer, a few seconds each."""
    from gen import configs
    import oracle

    w = configs.with_(configs.DECODE, T=args.decode_T, alpha=args.alpha)
    x = configs.gen_x(w)
    lgs = [configs.gen_logits(w, rotation=r) for r in range(16)]
    used = sorted(set(int(e) for lg in lgs for e in oracle.route(lg, w.k)[0].ravel()))
    table = oracle.ExpertTable(w.E, {e: configs.gen_expert(w, 0, e) for e in used})
    threads = oracle.max_threads()
    rate, layers, spent = _oracle_rate(lambda i: oracle.moe_layer(x, lgs[i % 16], w.k, table),
                                       w.T, args.cpu_seconds)
    tw = configs.TINY
    tx, tlg = configs.gen_x(tw), configs.gen_logits(tw)
    ttab = oracle.ExpertTable(tw.E, {e: configs.gen_expert(tw, 0, e) for e in range(tw.E)})
    oracle.set_threads(1)
    one_dec, n1, s1 = _oracle_rate(lambda i: oracle.moe_layer(x, lgs[i % 16], w.k, table), w.T,
                                   max(2.0, args.cpu_seconds / 4))
    one_tiny, n2, s2 = _oracle_rate(lambda i: oracle.moe_layer(tx, tlg, tw.k, ttab), tw.T, 2.0)
    oracle.set_threads(threads)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return dict(value=rate, unit="tokens/s", cores=min(w.T * w.k, threads), kind="oracle",
                sample=f"{layers} whole decode layers (T={w.T}, E={w.E}, k={w.k}, d={w.d}, "
                       f"f={w.f}, bf16 weights) cycling 16 routing sets, {spent:.1f} s of oracle "
                       f"time on {threads} threads",
                nproc=os.cpu_count(), affinity_cpus=affinity, omp_threads=threads,
                one_core=dict(decode_tok_s=one_dec, decode_layers=n1,
                              tiny_fp32_tok_s=one_tiny, tiny_layers=n2))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    choices=["all", "decode", "prefill", "lru", "stream", "probe"])
    ap.add_argument("--no-graph", action="store_true", help="eager launches instead of graph replay")
    ap.add_argument("--decode-T", type=int, default=8)
    ap.add_argument("--alpha", type=float, default=0.2)
    ap.add_argument("--ffn-path", choices=["auto", "gemv", "gemm"], default="auto",
                    help="expert-FFN path of the decode workload (auto: chosen by the library)")
    ap.add_argument("--lru-steps", type=int, default=512)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="primary lines only: no decode T/alpha sweep and no MXFP4 extras")
    ap.add_argument("--prefill-alpha", type=float, default=None,
                    help="run the prefill workload at this Zipf alpha only (default: 0.2 and 1)")
    ap.add_argument("--weights", choices=["bf16", "mxfp4"], default="bf16",
                    help="expert weight format of the primary decode line (--workload decode)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no "
              "multi-GPU path (expert-parallel sharding is a design note, not code).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import expert_ffn_cache_amd as moe
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    moe.lib()
    wl = args.workload
    extra = {}
    dec = None
    if wl in ("all", "decode"):
        import gen
        wfmt = gen.MXFP4 if args.weights == "mxfp4" else None
        arena = decode_arena(torch, wfmt)
        dec = bench_decode(args, torch, moe, args.decode_T, args.alpha, arena, wfmt)
        log(f"[decode] {dec['tok_s']:.0f} tok/s, {dec['ms_per_step'] * 1e3:.1f} us/layer, "
            f"ffn {dec['ffn_ms'] * 1e3:.1f} us, {dec['roofline']['achieved']:.0f} GB/s")
        if dec["ms_per_layer_in_16_layer_graph"] is not None:
            log(f"[decode] 16 layers per graph: {dec['tok_s_16_layer_graph']:.0f} tok/s, "
                f"{dec['ms_per_layer_in_16_layer_graph'] * 1e3:.1f} us/layer")
        if not args.no_sweep and wfmt is None:
            sweep = {}
            for T, alpha in ((1, 0.2), (64, 0.2), (8, 1.0), (64, 1.0), (128, 0.2), (128, 1.0)):
                r = bench_decode(args, torch, moe, T, alpha, arena)
                sweep[f"T{T}_alpha{alpha}"] = _sweep_entry(r)
                log(f"[decode T={T} alpha={alpha}] {json.dumps(sweep[f'T{T}_alpha{alpha}'])}")
            extra["decode_sweep"] = sweep
        del arena
        torch.cuda.empty_cache()
        if not args.no_sweep and wfmt is None:
            # MXFP4 routed experts (the pages' DeepSeek-V4-Flash deployment format)
            arena = decode_arena(torch, gen.MXFP4)
            mx = {}
            for T, alpha in ((8, 0.2), (1, 0.2), (64, 0.2), (8, 1.0), (64, 1.0)):
                r = bench_decode(args, torch, moe, T, alpha, arena, gen.MXFP4)
                mx[f"T{T}_alpha{alpha}"] = _sweep_entry(r)
                log(f"[decode mxfp4 T={T} alpha={alpha}] {json.dumps(mx[f'T{T}_alpha{alpha}'])}")
            extra["decode_mxfp4"] = mx
            del arena
            torch.cuda.empty_cache()
    if wl in ("all", "prefill"):
        extra["prefill"] = bench_prefill(args, torch, moe)
        log(f"[prefill] {json.dumps(extra['prefill'])}")
        if not args.no_sweep or args.weights == "mxfp4":
            import gen
            extra["prefill_mxfp4"] = bench_prefill(args, torch, moe, gen.MXFP4)
            log(f"[prefill mxfp4] {json.dumps(extra['prefill_mxfp4'])}")
    if wl in ("all", "stream"):
        extra["stream_prefill"] = bench_stream(args, torch, moe)
        log(f"[stream] {json.dumps(extra['stream_prefill'])}")
        if not args.no_sweep:
            import gen
            extra["stream_prefill_mxfp4"] = bench_stream(args, torch, moe, gen.MXFP4)
            log(f"[stream mxfp4] {json.dumps(extra['stream_prefill_mxfp4'])}")
    if wl in ("all", "probe"):
        extra["hbm_probe"] = bench_probe(args, torch, moe)
        log(f"[probe] {json.dumps(extra['hbm_probe'])}")
    if wl in ("all", "lru"):
        extra["lru_decode"] = bench_lru(args, torch, moe)
        log(f"[lru] {json.dumps(extra['lru_decode'])}")
        if not args.no_sweep:
            import gen
            extra["lru_decode_mxfp4"] = bench_lru(args, torch, moe, gen.MXFP4, with_resize=False)
            log(f"[lru mxfp4] {json.dumps(extra['lru_decode_mxfp4'])}")
    cpu = None
    if dec and not args.no_cpu_baseline:
        cpu = cpu_baseline(args)
        log(f"[cpu] {json.dumps(cpu)}")
    if dec is None:
        print(json.dumps(extra))
        return
    line = {
        "metric": "MoE-layer tokens/s at decode T=8 & prefill T=8192; % HBM/MFMA peak",
        "value": dec["tok_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": dec["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": dec["workload"], "T": dec["T"], "E": 256, "k": 6, "d": 4096,
                   "f": 2048, "zipf_alpha": args.alpha, "experts_resident": 256,
                   "graph_replay": not args.no_graph},
        "roofline": dec["roofline"],
        "cpu_baseline": cpu,
        "extra": dict(decode_ffn_ms=dec["ffn_ms"], decode_unique_experts=dec["U_mean"],
                      decode_algorithmic_bytes_per_ffn=dec["algorithmic_bytes_per_call"],
                      decode_tok_s_16_layer_graph=dec["tok_s_16_layer_graph"],
                      decode_step_bytes=dec["step_bytes"],
                      decode_step_hbm_frac=dec["step_hbm_frac"], **extra),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()

"""The five synthetic workloads: shapes, seeds and input recipes.

Shapes follow the MoE models the FreeToken pages evaluate (DeepSeek-V4-Flash:
6 of 256 routed experts per layer, "How the MoE memory hierarchy works" on the
RTX-4090 page; Qwen3.6-35B-A3B on the benchmark page's model table).  Every
input is synthetic; weights are random (no trained checkpoints).
"""
from dataclasses import dataclass, field
import math

import numpy as np

from . import (F32, BF16, MXFP4, mxfp4_rows, TAG_X, TAG_WG, TAG_WU, TAG_WD, TAG_WR, TAG_LOGIT, TAG_RANK,
               normal, zipf_bias, routing_logits)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    T: int
    d: int
    E: int
    k: int
    f: int
    dtype: int            # F32 or BF16 for x and all weights; MXFP4: bf16 x, MXFP4 weights
    L: int = 1            # layers
    S: int = 0            # cache slots (0 = all experts resident, identity slots)
    alpha: float = 0.2    # Zipf(1.1) bias strength on router logits
    zipf_s: float = 1.1
    steps: int = 1        # decode steps (multi-layer LRU workload)
    p_stay: float = 0.7   # Markov re-pick probability (multi-layer LRU workload)

    @property
    def w_sd(self):
        return 1.0 / math.sqrt(self.d)

    @property
    def act_dtype(self):
        """Data type of the activations x (MXFP4 applies to the expert weights only)."""
        return BF16 if self.dtype == MXFP4 else self.dtype

    @property
    def elem(self):
        """Bytes per storage unit of an entry (MXFP4 entries are counted in bytes)."""
        return 4 if self.dtype == F32 else 1 if self.dtype == MXFP4 else 2

    @property
    def entry_elems(self):
        """Storage units per (layer, expert) entry: 3*d*f weights, or the MXFP4 bytes."""
        if self.dtype == MXFP4:
            return 3 * self.d * self.f // 2 + 3 * self.d * self.f // 32
        return 3 * self.d * self.f

    @property
    def entry_bytes(self):
        return self.entry_elems * self.elem


TINY = Workload("tiny_fp32", seed=1, T=16, d=256, E=8, k=2, f=512, dtype=F32, S=8, alpha=0.0)
DECODE = Workload("decode_e256_k6_d4096_f2048", seed=2, T=8, d=4096, E=256, k=6, f=2048,
                  dtype=BF16)
PREFILL = Workload("prefill_e256_k6_d4096_f2048", seed=3, T=8192, d=4096, E=256, k=6, f=2048,
                   dtype=BF16)
LRU_DECODE = Workload("lru_decode_l16_e256_k6_d2048_f1024", seed=4, T=8, d=2048, E=256, k=6,
                      f=1024, dtype=BF16, L=16, S=1024, steps=512)
STREAM_PREFILL = Workload("stream_prefill_l8_e128_k8_d2048_f768", seed=5, T=2048, d=2048, E=128,
                          k=8, f=768, dtype=BF16, L=8)

ALL = [TINY, DECODE, PREFILL, LRU_DECODE, STREAM_PREFILL]


def with_(w, **kw):
    """A copy of workload w with some fields replaced (e.g. T, alpha)."""
    d = dict(w.__dict__)
    d.update(kw)
    return Workload(**d)


# ---- logical-tensor index maps (row-major, out-major weights) -------------------------
def wg_index(w, layer, e):
    """First logical index of W_gate[layer, e], stored [f, d] (row i = gate unit i)."""
    return ((layer * w.E + e) * w.f) * w.d


def wd_index(w, layer, e):
    """First logical index of W_down[layer, e], stored [d, f] (row o = output channel o)."""
    return ((layer * w.E + e) * w.d) * w.f


def x_index(w, layer, attempt=0):
    return ((attempt * w.L + layer) * w.T) * w.d


def gen_x(w, layer=0, attempt=0):
    return normal(w.seed, TAG_X, x_index(w, layer, attempt), (w.T, w.d), 1.0, w.act_dtype)


def gen_expert(w, layer, e, dtype=None):
    """(W_gate [f,d], W_up [f,d], W_down [d,f]) of one (layer, expert) entry.  For MXFP4
    workloads each matrix is (codes [rows, K/2] uint8, scales [rows, K/32] uint8)."""
    dt = w.dtype if dtype is None else dtype
    if dt == MXFP4:
        return (mxfp4_rows(w.seed, TAG_WG, wg_index(w, layer, e), w.f, w.d, w.w_sd),
                mxfp4_rows(w.seed, TAG_WU, wg_index(w, layer, e), w.f, w.d, w.w_sd),
                mxfp4_rows(w.seed, TAG_WD, wd_index(w, layer, e), w.d, w.f, w.w_sd))
    wg = normal(w.seed, TAG_WG, wg_index(w, layer, e), (w.f, w.d), w.w_sd, dt)
    wu = normal(w.seed, TAG_WU, wg_index(w, layer, e), (w.f, w.d), w.w_sd, dt)
    wd = normal(w.seed, TAG_WD, wd_index(w, layer, e), (w.d, w.f), w.w_sd, dt)
    return wg, wu, wd


def gen_router_weight(w):
    return normal(w.seed, TAG_WR, 0, (w.E, w.d), w.w_sd, F32)


def gen_bias(w, layer=0):
    if w.alpha == 0.0:
        return np.zeros(w.E, dtype=np.float32)
    return zipf_bias(w.seed, TAG_RANK + layer * 0x10000, w.E, w.alpha, w.zipf_s)


def gen_logits(w, layer=0, rotation=0):
    """Zipf-biased N(0,1) router logits with the top-k margin guard (1e-3)."""
    tag = TAG_LOGIT + layer * 0x10000 + rotation * 0x100
    return routing_logits(w.seed, tag, w.T, w.E, w.k, gen_bias(w, layer))

"""One routed-MoE layer forward as a sequence of library calls on caller-owned buffers.

route + permute (one launch for small T) -> expert FFN -> combine, each a libmoecache.so
entry point; a single token takes moe_decode_token instead where it applies, which does all
of it in one launch.
Device memory comes from torch; this class only allocates the intermediate
buffers once and forwards pointers.
"""
import torch

from . import (MOE_F32, MOE_BF16, MOE_MXFP4, MOE_PATH_AUTO, moe_route, moe_permute, moe_route_permute,
               moe_permute_workspace_bytes, moe_expert_ffn, moe_expert_ffn_workspace_bytes,
               moe_combine, moe_decode_token, moe_decode_token_workspace_bytes)


def decode_token_supported(T, k, d, f, dtype, w_dtype, y_dtype):
    """Shapes and types moe_decode_token takes (one token, bf16 activations, bf16 or MXFP4
    weights, fp32 expert outputs, x and h within 64 KB of LDS; MXFP4 strips held whole in
    registers: d <= 4096, f <= 2048, k <= 8)."""
    if T != 1 or dtype != MOE_BF16 or y_dtype != MOE_F32:
        return False
    if d > 8192 or f > 8192 or (d + k * f) * 2 > 65536:
        return False
    if w_dtype == MOE_MXFP4:
        return d <= 4096 and f <= 2048 and k <= 8
    return w_dtype == MOE_BF16


def _tdtype(code):
    return torch.float32 if code == MOE_F32 else torch.bfloat16


class MoeLayer:
    def __init__(self, T, E, k, d, f, dtype=MOE_BF16, y_dtype=MOE_F32, device="cuda",
                 w_dtype=None):
        """dtype: activations (and weights unless w_dtype is given, e.g. MOE_MXFP4)."""
        self.T, self.E, self.k, self.d, self.f = T, E, k, d, f
        self.dtype, self.y_dtype = dtype, y_dtype
        self.w_dtype = dtype if w_dtype is None else w_dtype
        A = T * k
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.ids = torch.empty((T, k), **i32)
        self.w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.perm = torch.empty(max(A, 1), **i32)
        self.inv = torch.empty(max(A, 1), **i32)
        self.status = torch.zeros(1, **i32)
        self.perm_ws_bytes = moe_permute_workspace_bytes(T, k, E)
        self.perm_ws = torch.empty(self.perm_ws_bytes, dtype=torch.uint8, device=dev)
        self.ffn_ws_bytes = moe_expert_ffn_workspace_bytes(T, k, f, dtype)
        self.ffn_ws = torch.empty(self.ffn_ws_bytes, dtype=torch.uint8, device=dev)
        self.y_perm = torch.empty((max(A, 1), d), dtype=_tdtype(y_dtype), device=dev)
        self.out = torch.empty((T, d), dtype=torch.float32, device=dev)
        self.fusable = decode_token_supported(T, k, d, f, dtype, self.w_dtype, y_dtype)
        if self.fusable:
            # counters of the one-launch path: zero before the first call, zero after each
            self.tok_ws_bytes = moe_decode_token_workspace_bytes(k, f)
            self.tok_ws = torch.zeros(self.tok_ws_bytes, dtype=torch.uint8, device=dev)

    def route(self, logits, stream=None):
        moe_route(logits, self.T, self.E, self.k, self.ids, self.w, stream)

    def permute(self, stream=None):
        moe_permute(self.ids, self.T, self.k, self.E, self.counts, self.offsets, self.perm,
                    self.inv, self.perm_ws, self.perm_ws_bytes, self.status, stream)

    def route_permute(self, logits, stream=None):
        """route() then permute(), in one launch for small T."""
        moe_route_permute(logits, self.T, self.E, self.k, self.ids, self.w, self.counts,
                          self.offsets, self.perm, self.inv, self.perm_ws, self.perm_ws_bytes,
                          self.status, stream)

    def ffn(self, x, arena, entry_stride, expert_slot=None, mask=None, slot_key=None, key_base=0,
            path=MOE_PATH_AUTO, stream=None):
        moe_expert_ffn(x, self.dtype, self.perm, self.offsets, self.T, self.k, self.E, self.d,
                       self.f, expert_slot, arena, entry_stride, self.w_dtype, mask, slot_key,
                       key_base, self.ffn_ws, self.ffn_ws_bytes, self.y_perm, self.y_dtype, path,
                       self.status, stream)

    def combine(self, stream=None):
        moe_combine(self.y_perm, self.y_dtype, self.inv, self.w, self.T, self.k, self.d,
                    self.out, stream)

    def decode_token(self, x, logits, arena, entry_stride, expert_slot=None, slot_key=None,
                     key_base=0, stream=None):
        """The whole layer for one token in one launch (logits None: route with self.ids and
        self.w as they stand).  Leaves counts/offsets/perm/inv untouched."""
        moe_decode_token(logits, x, self.E, self.k, self.d, self.f, expert_slot, arena,
                         entry_stride, self.w_dtype, slot_key, key_base, self.ids, self.w,
                         self.tok_ws, self.tok_ws_bytes, self.out, self.status, stream)
        return self.out

    def forward(self, x, logits, arena, entry_stride, expert_slot=None, path=MOE_PATH_AUTO,
                stream=None, fused=None):
        """fused: None = the one-launch path where it applies (path AUTO), True = require it,
        False = separate launches."""
        if fused is None:
            fused = self.fusable and path == MOE_PATH_AUTO
        if fused:
            return self.decode_token(x, logits, arena, entry_stride, expert_slot, stream=stream)
        self.route_permute(logits, stream)
        self.ffn(x, arena, entry_stride, expert_slot, path=path, stream=stream)
        self.combine(stream)
        return self.out

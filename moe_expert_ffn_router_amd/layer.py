"""MoELayer: buffers + the call sequence of one layer forward.

Owns the device buffers of one layer (routing results, permutation,
workspaces, outputs) and issues route -> permute -> expert_ffn -> combine on
one stream through the C ABI.  With an expert cache, the slot-table path is
route -> permute -> counts to host -> expert_cache_lookup -> expert_cache_fill
-> expert_ffn (through the slot table) -> combine; the streamed variant hands
the whole step to moe_expert_ffn_streamed (waves, grouped fills on a side
stream, the FFN behind them).  No arithmetic happens here; it only sequences
library calls.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (Experts, experts, moe_combine, moe_expert_ffn, moe_expert_ffn_workspace,
               moe_expert_ffn_hybrid_host_bytes, moe_expert_ffn_streamed_workspace,
               moe_forward_decode, moe_forward_decode_supported, moe_forward_decode_workspace,
               moe_shared_ffn, moe_shared_ffn_workspace,
               moe_permute, moe_permute_workspace, moe_route, moe_route_permute)


def _i32(n, dev):
    return torch.empty(max(int(n), 1), dtype=torch.int32, device=dev)


class MoELayer:
    def __init__(self, fmt: str, E: int, H: int, I: int, k: int, T_max: int, stride: int,
                 shared_I: int = 0, shared_stride: int = 0, renorm: bool = True,
                 device: str | torch.device = "cuda"):
        self.fmt, self.E, self.H, self.I, self.k = fmt, E, H, I, k
        self.T_max, self.stride, self.renorm = T_max, stride, renorm
        dev = torch.device(device)
        self.device = dev
        A = T_max * k
        self.ids = _i32(A, dev)
        self.w = torch.empty(max(A, 1), dtype=torch.float32, device=dev)
        self.counts = _i32(E, dev)
        self.offsets = _i32(E + 1, dev)
        self.sorted_idx = _i32(A, dev)
        self.inv_idx = _i32(A, dev)
        self.perm_ws = torch.empty(max(moe_permute_workspace(T_max, k, E), 256), dtype=torch.uint8,
                                   device=dev)
        probe = Experts(0, E, H, I, None, stride)
        from . import FMT
        probe.fmt = FMT[fmt]
        self.ffn_ws = torch.empty(max(moe_expert_ffn_workspace(probe, T_max, k), 256),
                                  dtype=torch.uint8, device=dev)
        self._probe = probe
        self.stream_ws = None                 # streamed cache path: made on first use
        self.counts_host = torch.zeros(E, dtype=torch.int32).pin_memory()
        self.plan_out = tuple(torch.zeros(E, dtype=torch.int32) for _ in range(3))
        self.hybrid_out = tuple(torch.zeros(E, dtype=torch.int32) for _ in range(4))
        self.host_stage = None                # hybrid path: pinned staging, made on first use
        self.y_perm = torch.empty((max(A, 1), H), dtype=torch.bfloat16, device=dev)
        self.y = torch.empty((max(T_max, 1), H), dtype=torch.bfloat16, device=dev)
        self.shared_I = shared_I
        if shared_I:
            self.shared_stride = shared_stride
            sp = Experts(FMT["bf16"], 1, H, shared_I, None, shared_stride)
            self.s_ws = torch.empty(max(moe_shared_ffn_workspace(sp, T_max), 256),
                                    dtype=torch.uint8, device=dev)
            self.y_shared = torch.empty((T_max, H), dtype=torch.bfloat16, device=dev)
        # decode-sized batches: the two-launch whole-layer path
        self.decode_ws = None
        if moe_forward_decode_supported(H, I, T_max, k):
            self.decode_ws = torch.empty(max(moe_forward_decode_workspace(probe, T_max, k), 256),
                                         dtype=torch.uint8, device=dev)

    # -- individual steps ---------------------------------------------------
    def route(self, logits: torch.Tensor, stream=None):
        T = logits.shape[0]
        moe_route(logits, self.k, self.ids, self.w, self.renorm, stream)
        return T

    def permute(self, T: int, stream=None):
        moe_permute(self.ids, T, self.k, self.E, self.counts, self.offsets, self.sorted_idx,
                    self.inv_idx, self.perm_ws, stream)

    def expert_ffn(self, W: Experts, x: torch.Tensor, T: int, slot_of_expert=None,
                   variant="auto", stream=None):
        moe_expert_ffn(W, slot_of_expert, x, T, self.k, self.counts, self.offsets, self.sorted_idx,
                       self.y_perm, self.ffn_ws, variant, stream)

    def shared_ffn(self, Ws: Experts, x: torch.Tensor, T: int, variant="auto", stream=None):
        """The always-on shared expert (bf16 record): dense, every token (moe_shared_ffn)."""
        moe_shared_ffn(Ws, x, T, self.y_shared, self.s_ws, stream)

    def combine(self, T: int, with_shared: bool, stream=None):
        moe_combine(self.y_perm, self.inv_idx, self.w, T, self.k, self.H,
                    self.y_shared if with_shared else None, self.y, stream)

    def route_permute(self, logits: torch.Tensor, stream=None):
        moe_route_permute(logits, self.k, self.ids, self.w, self.counts, self.offsets,
                          self.sorted_idx, self.inv_idx, self.perm_ws, self.renorm, stream)
        return logits.shape[0]

    # -- whole layer ----------------------------------------------------------
    def weights(self, base) -> Experts:
        return experts(self.fmt, self.E, self.H, self.I, base, self.stride)

    def forward_decode(self, logits: torch.Tensor, x: torch.Tensor, W: Experts,
                       slot_of_expert=None, y_shared=None, stream=None) -> torch.Tensor:
        """Whole layer in two launches (decode-sized batches)."""
        T = logits.shape[0]
        moe_forward_decode(W, slot_of_expert, logits, x, self.k, self.ids, self.w, self.counts,
                           self.offsets, self.sorted_idx, self.inv_idx, y_shared, self.y,
                           self.decode_ws, self.renorm, stream)
        return self.y[:T]

    def forward(self, logits: torch.Tensor, x: torch.Tensor, W: Experts, Ws: Experts | None = None,
                slot_of_expert=None, variant="auto", stream=None) -> torch.Tensor:
        T = logits.shape[0]
        assert T <= self.T_max and x.shape == (T, self.H)
        if self.decode_ws is not None and Ws is None and variant == "auto":
            return self.forward_decode(logits, x, W, slot_of_expert, None, stream)
        self.route_permute(logits, stream)
        self.expert_ffn(W, x, T, slot_of_expert, variant, stream)
        if Ws is not None:
            self.shared_ffn(Ws, x, T, variant, stream)
        self.combine(T, Ws is not None, stream)
        return self.y[:T]

    def forward_cached(self, logits: torch.Tensor, x: torch.Tensor, layer: int, cache,
                       pool_W: Experts, slot_table: torch.Tensor, side=None, variant="auto",
                       stream=None) -> tuple[torch.Tensor, dict]:
        """Slot-table path: misses are filled from the pinned bank before the FFN."""
        T = logits.shape[0]
        self.route_permute(logits, stream)
        counts_host = self.counts[:self.E].to("cpu")          # the one host sync of the step
        me, ms, n_miss, n_hit, _ = cache.expert_cache_lookup(layer, counts_host)
        cache.expert_cache_fill(layer, me, ms, side=side, compute=stream)
        row = slot_table[layer * self.E:(layer + 1) * self.E]
        self.expert_ffn(pool_W, x, T, row, variant, stream)
        self.combine(T, False, stream)
        return self.y[:T], {"misses": n_miss, "hits": n_hit, "fills": list(zip(me.tolist(), ms.tolist()))}

    def forward_streamed(self, logits: torch.Tensor, x: torch.Tensor, layer: int, cache,
                         pool_W: Experts, slot_table: torch.Tensor, side=None, groups: int = 4,
                         variant="auto", stream=None) -> tuple[torch.Tensor, dict]:
        """Slot-table path with the FFN behind the fills (moe_expert_ffn_streamed): waves of
        at most S (or S/2 when the step needs more than S experts), each wave's misses in
        `groups` copy groups on `side`, the FFN over the hits at once and over each group as
        it lands.  y is bit-identical to forward_cached whenever that one fits."""
        T = logits.shape[0]
        E = self.E
        cs = stream if stream is not None else torch.cuda.current_stream()
        if self.stream_ws is None:
            self.stream_ws = torch.empty(
                max(moe_expert_ffn_streamed_workspace(self._probe, self.T_max, self.k), 256),
                dtype=torch.uint8, device=self.device)
        self.route_permute(logits, cs)
        with torch.cuda.stream(cs):
            self.counts_host.copy_(self.counts[:E], non_blocking=True)
        cs.synchronize()                                 # the one host sync of the step
        nw, nh = cache.moe_expert_ffn_streamed(layer, pool_W, x, T, self.k, self.counts_host,
                                               self.offsets, self.sorted_idx, self.y_perm,
                                               groups, self.stream_ws, side=side, compute=cs,
                                               out=self.plan_out)
        fe, fs, we = self.plan_out
        n_fill = int(we[nw - 1]) if nw else 0
        fills = list(zip(fe[:n_fill].tolist(), fs[:n_fill].tolist()))
        self.combine(T, False, cs)
        return self.y[:T], {"misses": n_fill, "hits": nh, "waves": nw, "fills": fills}

    def forward_hybrid(self, logits: torch.Tensor, x: torch.Tensor, layer: int, cache, pool_W: Experts,
                       slot_table: torch.Tensor, cpu_pool, fetch_fraction: float,
                       max_fetch: int = -1, side=None, groups: int = 4,
                       stream=None) -> tuple[torch.Tensor, dict]:
        """Hybrid step (moe_expert_ffn_hybrid): ceil(fetch_fraction * misses) of the misses
        (the most recently active) are fetched and computed on the GPU behind their copies,
        the others computed on the CPU from the bank while the GPU runs; then combine."""
        T = logits.shape[0]
        E = self.E
        cs = stream if stream is not None else torch.cuda.current_stream()
        if self.stream_ws is None:
            self.stream_ws = torch.empty(
                max(moe_expert_ffn_streamed_workspace(self._probe, self.T_max, self.k), 256),
                dtype=torch.uint8, device=self.device)
        if self.host_stage is None:
            self.host_stage = torch.empty(
                moe_expert_ffn_hybrid_host_bytes(self._probe, self.T_max, self.k),
                dtype=torch.uint8).pin_memory()
        self.route_permute(logits, cs)
        with torch.cuda.stream(cs):
            self.counts_host.copy_(self.counts[:E], non_blocking=True)
        cs.synchronize()                                 # the one host sync of the step
        nc, nw, nh = cache.moe_expert_ffn_hybrid(layer, pool_W, cpu_pool, x, T, self.k,
                                                 self.counts_host, self.offsets, self.sorted_idx,
                                                 self.y_perm, fetch_fraction, max_fetch, groups,
                                                 self.stream_ws, self.host_stage, side=side,
                                                 compute=cs, out=self.hybrid_out)
        ce, fe, fs, we = self.hybrid_out
        n_fill = int(we[nw - 1]) if nw else 0
        fills = list(zip(fe[:n_fill].tolist(), fs[:n_fill].tolist()))
        self.combine(T, False, cs)
        return self.y[:T], {"misses": n_fill + nc, "fetched": n_fill, "cpu": ce[:nc].tolist(),
                            "hits": nh, "waves": nw, "fills": fills}

"""Shared set-up for the GPU parity tests: seeded inputs on the device and
matching oracle views of the same bytes.  Test infrastructure only."""
from __future__ import annotations

import numpy as np
import torch

import synth
from oracle import layer as OL

TOL = 2e-2  # max |gpu - oracle| <= TOL * max |oracle|


def flush(msg: str) -> None:
    print(msg, flush=True)


class Case:
    """One layer's inputs, resident on the GPU, plus oracle accessors."""

    def __init__(self, wl: synth.Workload, gen_device: str = "cpu", batch: int = 0):
        self.wl = wl
        dev = torch.device("cuda")
        self.logits_np = synth.make_logits(wl, batch)
        self.x_np = synth.make_x(wl, batch)
        self.logits = torch.from_numpy(self.logits_np).to(dev)
        self.x = torch.from_numpy(self.x_np.view(np.int16)).to(dev).view(torch.bfloat16)
        self.layout = synth.record_layout(wl.fmt, wl.H, wl.I)
        self.stride = self.layout["stride"]
        recs = synth.make_expert_records(wl.fmt, wl.E, wl.H, wl.I, wl.seed, device=gen_device)
        self.records = recs.to(dev)
        del recs
        self.shared = None
        if wl.shared_I:
            self.shared = synth.make_shared_record(wl.seed, wl.H, wl.shared_I,
                                                   device=gen_device).to(dev)
        self._host_rec = {}

    def rec_host(self, e: int) -> np.ndarray:
        if e not in self._host_rec:
            self._host_rec[e] = self.records[e].cpu().numpy()
        return self._host_rec[e]

    def oracle_experts(self) -> OL.ExpertSet:
        return OL.ExpertSet(self.wl.fmt, self.wl.H, self.wl.I, self.rec_host)

    def oracle_shared(self):
        if self.shared is None:
            return None
        s = self.shared[0].cpu().numpy()
        return OL.ExpertSet("bf16", self.wl.H, self.wl.shared_I, lambda e: s)


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))

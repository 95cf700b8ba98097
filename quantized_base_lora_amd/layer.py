"""One decoder layer's LoRA linears as a training step, in the launch
configuration the benchmark times: the forward of every projection, then the
backward of every projection in reverse order, recorded once per packed
weight copy as a launch plan and enqueued by one library call per step.

Projections that read the same input in a decoder layer run as grouped calls
(q|k|v and gate|up); o and down stay alone, since in a real layer their
inputs depend on the earlier groups (attention, the gated activation).  Every
projection gets its own seeded inputs (synth.layer_tensors_torch), drawn on
the GPU.  Host orchestration only: every arithmetic step runs in the
library's kernels.
"""

import torch

from . import binding as B, synth

GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


class LayerStep:
    """Inputs, packed bases (`copies` identical packed copies, rotated step by
    step so that weight reads come from HBM rather than the last-level cache),
    preallocated outputs and workspaces of one layer at m tokens.

    exclude: projection names left out; only: keep just this projection;
    keep_w: keep each fp32 base weight on the host (d["W"]) for the oracle."""

    def __init__(self, wl, m, copies=1, exclude=(), only=None, keep_w=False, device="cuda"):
        self.wl, self.m = wl, int(m)
        self.device = torch.device(device)
        self.projs = []
        for pi, p in enumerate(wl.projs):
            if p.name in exclude or (only is not None and p.name != only):
                continue
            t = synth.layer_tensors_torch(wl, pi, m=self.m, device=self.device)
            qw = B.quant_pack(wl.fmt, t["W"])
            d = {"pi": pi, "p": p, "qws": [qw], "x": t["x"], "dy": t["dY"], "a": t["A"], "b": t["B"]}
            if keep_w:
                d["W"] = t["W"].cpu()
            del t
            self._alloc_outputs(d)
            self.projs.append(d)
        self.copies = max(1, int(copies))
        if self.copies > 1:
            # all copies of a projection in one allocation (a small layer needs
            # thousands of them to fill the rotation)
            for d in self.projs:
                base = d["qws"][0]
                codes = base.codes.unsqueeze(0).repeat((self.copies,) + (1,) * base.codes.dim())
                scales = base.scales.unsqueeze(0).repeat((self.copies,) + (1,) * base.scales.dim())
                d["qws"] = [base] + [B.QWeight(base.fmt, base.n, base.k, codes[i], scales[i])
                                     for i in range(1, self.copies)]
                d["copies_storage"] = (codes, scales)
        by_name = {d["p"].name: d for d in self.projs}
        groups = [[by_name[n] for n in g if n in by_name] for g in GROUPS]
        self.groups = [g for g in groups if g]
        if sum(len(g) for g in self.groups) != len(self.projs):
            self.groups = [[d] for d in self.projs]
        self._plans = None

    def _alloc_outputs(self, d):
        wl, m, dev, p = self.wl, self.m, self.device, d["p"]
        d["y"] = torch.empty((m, p.n), dtype=torch.bfloat16, device=dev)
        d["u"] = torch.empty((m, wl.r), dtype=torch.float32, device=dev)
        d["dx"] = torch.empty((m, p.k), dtype=torch.bfloat16, device=dev)
        d["da"] = torch.empty((wl.r, p.k), dtype=torch.float32, device=dev)
        d["db"] = torch.empty((p.n, wl.r), dtype=torch.float32, device=dev)
        d["ws"] = torch.empty(max(256, B.workspace_bytes(B.OP_BWD, wl.fmt, p.n, p.k, m, wl.r)),
                              dtype=torch.uint8, device=dev)
        d["wsf"] = torch.empty(max(256, B.workspace_bytes(B.OP_FWD, wl.fmt, p.n, p.k, m, wl.r)),
                               dtype=torch.uint8, device=dev)

    def packed_bytes(self):
        """Bytes of one packed copy of the layer's bases."""
        return sum(d["qws"][0].nbytes() for d in self.projs)

    def fwd_items(self, g, i):
        a = self.wl.alpha
        return [(d["qws"][i % self.copies], d["x"], d["a"], d["b"], a, d["y"], d["u"], d["wsf"]) for d in g]

    def bwd_items(self, g, i):
        a = self.wl.alpha
        return [(d["qws"][i % self.copies], d["x"], d["dy"], d["u"], d["a"], d["b"], a, d["dx"], d["da"],
                 d["db"], d["ws"], False) for d in reversed(g)]

    def record(self, plan, i, phase="both"):
        """Append the step on weight copy i to `plan`: forward groups in order,
        then backward groups in reverse (phase "fwd" / "bwd": one pass only)."""
        if phase != "bwd":
            for g in self.groups:
                plan.add_fwd_group(self.fwd_items(g, i))
        if phase != "fwd":
            for g in reversed(self.groups):
                plan.add_bwd_group(self.bwd_items(g, i))

    def plans(self, phase="both"):
        if self._plans is None:
            self._plans = []
            for i in range(self.copies):
                pl = B.Plan()
                self.record(pl, i, phase)
                self._plans.append(pl)
        return self._plans

    def run(self, i=0, stream=None):
        """One step on weight copy i % copies (one library call)."""
        self.plans()[i % self.copies].run(stream)

    def fwd_launches_per_step(self):
        """GEMM launches of one step's forward: one per group of calls (with
        its reduction launch on the small-M path, or for the FP8 base above 64
        tokens after the group's activation splits and projections)."""
        return len(self.groups)

    def close(self):
        for pl in self._plans or []:
            pl.close()
        self._plans = None

"""A stack of decoder layers whose frozen bases are either resident in VRAM or
streamed from pinned host memory through the library's slot pool, one layer
ahead on a side stream (Soup page, opening paragraph).

Host orchestration only: every byte moves through the library (the pool's
copies) and every arithmetic step runs in its kernels.  Each layer's packed
projections are laid out in one contiguous image (codes then scales per
projection, each at a 256-byte aligned offset), so a layer moves with one
copy and the kernels see the same layout wherever the image lives.
"""

import torch

from . import binding as B, synth
from .layer import GROUPS

ALIGN = 256


def _up(v):
    return (v + ALIGN - 1) // ALIGN * ALIGN


def _sizes(fmt, n, k):
    if fmt == B.FMT_FP8:
        return n * k, 4
    if fmt == B.FMT_Q4_0:
        return n * k // 2, n * (k // 32) * 2
    if fmt == B.FMT_MXFP4:
        return n * k // 2, n * (k // 32)
    if fmt == B.FMT_Q8_0:
        return n * k, n * (k // 32) * 2
    if fmt == B.FMT_NVFP4:
        return n * k // 2, 16 + n * (k // 16)
    return n * k // 2, n * (k // 64) * 4


class LayerLayout:
    """Offsets of each projection's codes and scales inside a layer image."""

    def __init__(self, fmt, projs):
        self.fmt = fmt
        self.projs = [(int(p.n), int(p.k)) for p in projs]
        self.offsets = []
        off = 0
        for n, k in self.projs:
            cb, sb = _sizes(fmt, n, k)
            co = off
            off = _up(off + cb)
            so = off
            off = _up(off + sb)
            self.offsets.append((co, cb, so, sb))
        self.nbytes = off

    def weights_at(self, base_ptr, keepalive=None):
        """QWeight views of every projection for an image at device address base_ptr."""
        return [B.QWeight.view(self.fmt, n, k, base_ptr + co, base_ptr + so, keepalive)
                for (n, k), (co, _, so, _) in zip(self.projs, self.offsets)]

    def image_from(self, qweights, device="cuda"):
        """Device image holding the given packed weights at this layout's offsets."""
        img = torch.zeros(self.nbytes, dtype=torch.uint8, device=device)
        for qw, (co, cb, so, sb) in zip(qweights, self.offsets):
            img[co:co + cb].copy_(qw.codes.reshape(-1).view(torch.uint8))
            img[so:so + sb].copy_(qw.scales.reshape(-1).view(torch.uint8))
        return img


class Stack:
    """fwd over layers 0..L-1 then bwd over L-1..0, every layer's 7 (or fewer)
    projections with their own activations and adapters."""

    def __init__(self, layout, r, alpha, images_dev=None, images_host=None, n_slots=2):
        self.layout, self.r, self.alpha = layout, r, alpha
        self.resident = images_dev is not None
        if self.resident:
            self.images = images_dev
            self.n_layers = len(images_dev)
            self.views = [layout.weights_at(img.data_ptr(), img) for img in images_dev]
        else:
            self.images = images_host
            self.n_layers = len(images_host)
            self.slots = [torch.empty(layout.nbytes, dtype=torch.uint8, device="cuda") for _ in range(n_slots)]
            self.pool = B.Pool(self.slots, images_host)
            self.copy_stream = torch.cuda.Stream()

    def _weights(self, layer):
        if self.resident:
            return self.views[layer]
        ptr = self.pool.acquire(layer)
        return self.layout.weights_at(ptr, self.slots)

    def _done(self, layer):
        if not self.resident:
            self.pool.release(layer)

    def _ahead(self, layer):
        if not self.resident and 0 <= layer < self.n_layers:
            self.pool.prefetch(layer, self.copy_stream)

    def run(self, acts, outs, groups=None):
        """acts[l][p] = dict(x, dy, a, b) device tensors; outs[l][p] = dict of
        preallocated y, u, dx, da, db and ws (backward workspace) tensors,
        written in place, and optionally wsf (forward workspace; needed by
        grouped calls of at most 64 tokens).  groups: lists of projection
        indices whose calls are independent (q|k|v, gate|up of a decoder
        layer) and run as one grouped call each, in the order given (backward
        in reverse); default: one call per projection."""
        L = self.n_layers
        gs = groups or [[p] for p in range(len(self.layout.projs))]
        self._ahead(0)
        for l in range(L):
            self._ahead(l + 1)
            ws = self._weights(l)
            for g in gs:
                items = [(ws[p], acts[l][p]["x"], acts[l][p]["a"], acts[l][p]["b"], self.alpha,
                          outs[l][p]["y"], outs[l][p]["u"], outs[l][p].get("wsf")) for p in g]
                if len(items) == 1:
                    qw, x, a, b, alpha, y, u, wsf = items[0]
                    B.linear_fwd(qw, x, a, b, alpha, y=y, u=u, ws=wsf)
                else:
                    B.linear_fwd_group(items)
            self._done(l)
        for l in reversed(range(L)):
            self._ahead(l - 1)
            ws = self._weights(l)
            for g in reversed(gs):
                items = [(ws[p], acts[l][p]["x"], acts[l][p]["dy"], outs[l][p]["u"], acts[l][p]["a"],
                          acts[l][p]["b"], self.alpha, outs[l][p]["dx"], outs[l][p]["da"], outs[l][p]["db"],
                          outs[l][p]["ws"], False) for p in g]
                if len(items) == 1:
                    qw, x, dy, u, a, b, alpha, dx, da, db, wsb, _ = items[0]
                    B.linear_bwd(qw, x, dy, u, a, b, alpha, dx=dx, da=da, db=db, ws=wsb)
                else:
                    B.linear_bwd_group(items)
            self._done(l)

    def close(self):
        if not self.resident:
            self.pool.close()


# ----------------------------------------------------------------------------- a stack of model layers

def build_host_images(wl, n_layers, keep_w=(), device="cuda"):
    """Pinned host images of n_layers layers of workload wl: layer l's
    projection weights are drawn on the GPU (synth.layer_tensors_torch with
    layer=l), packed by the library, laid out in one image and copied to
    page-locked host memory.  Returns (layout, images, kept) with kept[(l, p)]
    the fp32 weight of projection p of each layer l in keep_w (host)."""
    layout = LayerLayout(wl.fmt, wl.projs)
    host, kept = [], {}
    for layer in range(n_layers):
        qws = []
        for pi in range(len(wl.projs)):
            w = synth.layer_tensors_torch(wl, pi, layer=layer, device=device, want=("W",))["W"]
            qws.append(B.quant_pack(wl.fmt, w))
            if layer in keep_w:
                kept[(layer, pi)] = w.cpu()
            del w
        img = layout.image_from(qws, device=device)
        h = torch.empty(layout.nbytes, dtype=torch.uint8, pin_memory=True)
        h.copy_(img)
        host.append(h)
        del img, qws
    torch.cuda.synchronize()
    return layout, host, kept


def layer_inputs(wl, m, n_layers, device="cuda"):
    """acts[l][p] = dict(x, dy, a, b): layer l's seeded inputs at m tokens."""
    acts = []
    for layer in range(n_layers):
        al = []
        for pi in range(len(wl.projs)):
            t = synth.layer_tensors_torch(wl, pi, m=m, layer=layer, device=device, want=("A", "B", "x", "dY"))
            al.append({"x": t["x"], "dy": t["dY"], "a": t["A"], "b": t["B"]})
        acts.append(al)
    return acts


def layer_outputs(wl, m, n_layers, device="cuda"):
    """outs[l][p]: preallocated y, u, dx, da, db and the workspaces ws, wsf."""
    outs = []
    for _ in range(n_layers):
        ol = []
        for p in wl.projs:
            ol.append({"y": torch.empty((m, p.n), dtype=torch.bfloat16, device=device),
                       "u": torch.empty((m, wl.r), dtype=torch.float32, device=device),
                       "dx": torch.empty((m, p.k), dtype=torch.bfloat16, device=device),
                       "da": torch.empty((wl.r, p.k), dtype=torch.float32, device=device),
                       "db": torch.empty((p.n, wl.r), dtype=torch.float32, device=device),
                       "ws": torch.empty(max(256, B.workspace_bytes(B.OP_BWD, wl.fmt, p.n, p.k, m, wl.r)),
                                         dtype=torch.uint8, device=device),
                       "wsf": torch.empty(max(256, B.workspace_bytes(B.OP_FWD, wl.fmt, p.n, p.k, m, wl.r)),
                                          dtype=torch.uint8, device=device)})
        outs.append(ol)
    return outs


def layer_groups(projs):
    """Indices of the calls that run grouped in a decoder layer (q|k|v, o,
    gate|up, down), or None when the projections are not those of one."""
    names = [p.name for p in projs]
    groups = [[names.index(n) for n in g if n in names] for g in GROUPS]
    groups = [g for g in groups if g]
    if sorted(i for g in groups for i in g) != list(range(len(names))):
        return None
    return groups


OUTPUT_KEYS = ("y", "u", "dx", "da", "db")


def compare_outputs(o1, o2):
    """Bitwise comparison of every output of every layer of two runs.
    Returns (equal, first mismatch (layer, projection, key) or None, max abs
    difference over all outputs as a float)."""
    equal, first, worst = True, None, 0.0
    for layer in range(len(o1)):
        for pi in range(len(o1[layer])):
            for key in OUTPUT_KEYS:
                a, b = o1[layer][pi][key], o2[layer][pi][key]
                ia = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32)
                ib = b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)
                if not torch.equal(ia, ib):
                    if equal:
                        first = (layer, pi, key)
                    equal = False
                    d = (a.float() - b.float()).abs().max().item()
                    worst = max(worst, d if d == d else float("inf"))
    return equal, first, worst

"""Streamed vs resident frozen base: bitwise equality (max abs difference 0.0)
of every output of every layer, with poisoned slots and delayed copies; a
negative control shows the check can fail; pool misuse returns QL_ESTATE.
(Soup page: "Correctness" paragraph -- bit-exactness against a resident run
with the same numerics, every output compared, not only a loss.)"""

import sys

import numpy as np
import pytest
import torch

import helpers as H
from oracle import formats as ofmt
from quantized_base_lora_amd import binding as B, stack, synth

pytestmark = pytest.mark.gpu

PROJS = [synth.Proj("a", 256, 512), synth.Proj("b", 512, 256), synth.Proj("c", 256, 256)]
L, M, R, ALPHA = 5, 96, 16, 32.0


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def build(fmt=ofmt.FMT_NF4):
    layout = stack.LayerLayout(fmt, PROJS)
    imgs, acts = [], []
    for l in range(L):
        qws, la = [], []
        for pi, p in enumerate(PROJS):
            c = H.make_case(M, p.k, p.n, R, seed=1000 * l + pi)
            qws.append(B.quant_pack(fmt, torch.from_numpy(c["W"]).cuda()))
            la.append({k2: H.bits_to_bf16_tensor(c[k1]) for k1, k2 in
                       (("x", "x"), ("dY", "dy"), ("A", "a"), ("B", "b"))})
        imgs.append(layout.image_from(qws))
        acts.append(la)
    torch.cuda.synchronize()
    return layout, imgs, acts


def new_outs():
    outs = []
    for l in range(L):
        lo = []
        for p in PROJS:
            lo.append({"y": torch.empty((M, p.n), dtype=torch.bfloat16, device="cuda"),
                       "u": torch.empty((M, R), dtype=torch.float32, device="cuda"),
                       "dx": torch.empty((M, p.k), dtype=torch.bfloat16, device="cuda"),
                       "da": torch.empty((R, p.k), dtype=torch.float32, device="cuda"),
                       "db": torch.empty((p.n, R), dtype=torch.float32, device="cuda"),
                       "ws": torch.empty(B.workspace_bytes(B.OP_BWD, B.FMT_NF4, p.n, p.k, M, R),
                                         dtype=torch.uint8, device="cuda")})
        outs.append(lo)
    return outs


def pinned(imgs):
    out = []
    for img in imgs:
        h = torch.empty(img.numel(), dtype=torch.uint8, pin_memory=True)
        h.copy_(img.cpu())
        out.append(h)
    return out


def same(o1, o2):
    for l in range(L):
        for p in range(len(PROJS)):
            for key in ("y", "u", "dx", "da", "db"):
                a, b = o1[l][p][key], o2[l][p][key]
                ia = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32)
                ib = b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)
                if not torch.equal(ia, ib):
                    return False, (l, p, key)
    return True, None


def test_streamed_equals_resident_bitwise(lib):
    layout, imgs, acts = build()
    res = stack.Stack(layout, R, ALPHA, images_dev=imgs)
    o_res = new_outs()
    res.run(acts, o_res)
    torch.cuda.synchronize()
    host = pinned(imgs)
    for delay_us, poison in ((0, False), (3000, True)):
        say(f"streamed run delay={delay_us}us poison={poison}")
        st = stack.Stack(layout, R, ALPHA, images_host=host, n_slots=2)
        st.pool.debug(delay_us=delay_us, poison=poison)
        o_st = new_outs()
        st.run(acts, o_st)
        torch.cuda.synchronize()
        ok, where = same(o_res, o_st)
        assert ok, where
        stats = st.pool.stats()
        assert stats["copies"] == 2 * L - 2, stats          # fwd L copies, bwd L-2 (two layers stay)
        assert stats["bytes"] == stats["copies"] * layout.nbytes
        st.close()
    # grouped calls (projections a and c in one call) over the streamed base give
    # the same bits as the resident one-call-per-projection run
    say("streamed run, grouped calls")
    st = stack.Stack(layout, R, ALPHA, images_host=host, n_slots=2)
    st.pool.debug(delay_us=3000, poison=True)
    o_st = new_outs()
    st.run(acts, o_st, groups=[[0, 2], [1]])
    torch.cuda.synchronize()
    ok, where = same(o_res, o_st)
    assert ok, where
    st.close()
    # the outputs are the real thing: max abs difference 0.0 and finite
    assert all(torch.isfinite(o_res[l][p]["y"].float()).all() for l in range(L) for p in range(len(PROJS)))


def test_negative_control_detects_skipped_wait(lib):
    """With the compute stream's wait removed and each copy delayed behind a
    poison fill, the first layer reads its slot before the copy lands; the
    bitwise check must catch it."""
    layout, imgs, acts = build()
    res = stack.Stack(layout, R, ALPHA, images_dev=imgs)
    o_res = new_outs()
    res.run(acts, o_res)
    torch.cuda.synchronize()
    st = stack.Stack(layout, R, ALPHA, images_host=pinned(imgs), n_slots=2)
    for slot in st.slots:                                    # every slot starts as NaN bytes
        slot.fill_(255)
    torch.cuda.synchronize()
    st.pool.debug(delay_us=200000, poison=True, skip_wait=True)
    o_st = new_outs()
    st.run(acts, o_st)
    torch.cuda.synchronize()
    ok, _ = same(o_res, o_st)
    assert not ok
    st.close()


def test_pool_misuse(lib):
    layout, imgs, _ = build()
    host = pinned(imgs)
    slots = [torch.empty(layout.nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    pool = B.Pool(slots, host)
    cs = torch.cuda.Stream()
    with pytest.raises(B.QLError) as e:
        pool.acquire(0)
    assert e.value.code == B.QL_ESTATE
    pool.prefetch(0, cs)
    pool.prefetch(1, cs)
    with pytest.raises(B.QLError) as e:
        pool.prefetch(2, cs)                                 # both slots pending
    assert e.value.code == B.QL_ESTATE
    pool.acquire(0)
    with pytest.raises(B.QLError) as e:
        pool.acquire(0)
    assert e.value.code == B.QL_ESTATE
    pool.release(0)
    with pytest.raises(B.QLError) as e:
        pool.release(0)
    assert e.value.code == B.QL_ESTATE
    pool.prefetch(2, cs)                                     # evicts layer 0
    with pytest.raises(B.QLError) as e:
        pool.acquire(0)
    assert e.value.code == B.QL_ESTATE
    with pytest.raises(B.QLError) as e:
        pool.prefetch(L + 3, cs)
    assert e.value.code == B.QL_EINVAL
    torch.cuda.synchronize()
    pool.close()

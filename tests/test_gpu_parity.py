"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: packing, dequantization and the FP8 activation split bit-exact;
forward / backward max|err| / max|ref| <= 1e-2 (3e-2 on y and dX for the FP8
base); bitwise equality where the arithmetic is exact (integer data, B = 0)."""

import sys
import zlib

import numpy as np
import pytest
import torch

import helpers as H
from oracle import codecs, formats as ofmt, lora as olora
from quantized_base_lora_amd import synth

pytestmark = pytest.mark.gpu

FMTS = [ofmt.FMT_Q4_0, ofmt.FMT_NF4, ofmt.FMT_FP8, ofmt.FMT_MXFP4, ofmt.FMT_Q8_0, ofmt.FMT_NVFP4]
FNAME = {1: "q4_0", 2: "nf4", 3: "fp8", 4: "mxfp4", 5: "q8_0", 6: "nvfp4"}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def pack_gpu(lib, fmt, w_np):
    from quantized_base_lora_amd import binding as B
    return B.quant_pack(fmt, torch.from_numpy(w_np).cuda())


def special_weight(fmt, n, k, seed):
    """Random N(0, 0.02^2) with planted edge cases: a zero block, a tiny block,
    exact ties (Q4_0) or exact book levels (NF4), repeated values."""
    g = np.random.default_rng(seed)
    w = (g.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    blk = 64 if fmt == ofmt.FMT_NF4 else 32
    w[0, :blk] = 0.0
    w[1, :blk] = np.float32(3e-9) * g.standard_normal(blk, dtype=np.float32)
    if fmt == ofmt.FMT_Q4_0:
        d = np.float32(1638 * 2.0 ** -14)
        w[2, :32] = 0
        w[2, 0] = np.float32(0.7)
        w[2, 1:12] = (np.arange(1, 12, dtype=np.float32) - 6.5) * d      # half-integer multiples of d
    elif fmt == ofmt.FMT_NF4:
        w[2, :64] = np.tile(ofmt.nf4_codebook(), 4) * np.float32(0.031)
        w[3, :15] = ofmt.nf4_thresholds() * np.float32(1.0)
        w[3, 15] = 1.0
    elif fmt == ofmt.FMT_MXFP4:
        # block scale 2^-7 (largest magnitude 7.9 * 2^-7 lands in [4, 8)): every
        # E2M1 rounding tie, both signs, saturation above 6, negative zero and a
        # negative value that rounds to zero
        x = np.float32(2.0 ** -7)
        t = np.float32([7.9, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 6.5, 0.1, 0.0])
        w[2, :32] = 0
        w[2, :12] = t * x
        w[2, 12:23] = -t[1:] * x
        w[2, 23] = -0.0
        w[2, 24] = np.float32(-0.2) * x
        # fp32 subnormals and the smallest block scale: 2^-127 * {0.5, 1, 3, 6}
        w[3, :32] = 0
        w[3, :4] = np.float32([0.5, 1.0, 3.0, 6.0]) * np.float32(2.0 ** -64) * np.float32(2.0 ** -63)
        w[5, :32] = np.float32(1e30) * g.standard_normal(32, dtype=np.float32)
    elif fmt == ofmt.FMT_Q8_0:
        # scale exactly 2^-7: rounding ties on half-integers of d in both signs
        w[2, :32] = (np.arange(32, dtype=np.float32) - 15.5) * np.float32(2.0 ** -7)
        w[2, 0] = np.float32(127 * 2.0 ** -7)
        # a scale that rounds down to the smallest fp16 subnormal: the clamp acts
        w[3, :32] = np.float32(8.5e-8 * 127) * np.linspace(-1, 1, 32, dtype=np.float32)
    elif fmt == ofmt.FMT_NVFP4:
        # the tensor maximum 2688 * 2^-12 makes g = 2^-12; a block whose
        # largest element 6 * 8 g gives scale byte 8.0 (0x50) and X = 2^-9,
        # holding every E2M1 midpoint in both signs, saturation, negative zero
        # and a negative value that rounds to zero; a block whose scale is an
        # E4M3 tie (42 -> 40); a block whose scale rounds to zero
        g = np.float32(2.0 ** -12)
        w[5, 0] = np.float32(2688) * g
        x = np.float32(8.0) * g
        t = np.float32([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
        w[2, :32] = 0
        w[2, :8] = t * x
        w[2, 8:15] = -t[1:] * x
        w[2, 15] = -0.0
        w[2, 16:24] = -t * x
        w[2, 24] = np.float32(-0.2) * x
        w[2, 25] = np.float32(6.3) * x      # scale quotient 8.4 rounds down to 8: saturates at 6 X
        w[3, :32] = 0
        w[3, :16] = np.float32(42 * 6) * g * np.linspace(-1, 1, 16, dtype=np.float32)
        w[3, 16] = np.float32(2.0 ** -12) * g
    w[4, :blk] = np.float32(0.01)
    return w


# ----------------------------------------------------------------------------- pack / dequant

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(64, 256), (96, 1024), (32, 192)])
def test_pack_bitexact(lib, fmt, shape):
    n, k = shape
    if fmt == ofmt.FMT_NF4 and k % 64:
        pytest.skip("NF4 needs K % 64 == 0")
    say(f"pack {FNAME[fmt]} {shape}")
    w = special_weight(fmt, n, k, 100 + n + k)
    qw = pack_gpu(lib, fmt, w)
    torch.cuda.synchronize()
    c, s = ofmt.pack(fmt, w)
    assert np.array_equal(H.tensor_bytes(qw.codes), np.ascontiguousarray(c).ravel())
    assert np.array_equal(H.tensor_bytes(qw.scales), H.scales_bytes(fmt, s))


@pytest.mark.parametrize("fmt", FMTS)
def test_pack_rejects_nonfinite(lib, fmt):
    from quantized_base_lora_amd import binding as B
    for bad in (np.nan, np.inf, -np.inf):
        w = np.zeros((32, 64), np.float32)
        w[5, 17] = bad
        with pytest.raises(B.QLError) as e:
            pack_gpu(lib, fmt, w)
        assert e.value.code == B.QL_ENONFINITE


@pytest.mark.parametrize("fmt,big", [(ofmt.FMT_Q4_0, 1e6), (ofmt.FMT_Q8_0, 1e7)])
def test_pack_fp16_scale_overflow(lib, fmt, big):
    from quantized_base_lora_amd import binding as B
    w = np.full((32, 32), big, np.float32)
    with pytest.raises(B.QLError) as e:
        pack_gpu(lib, fmt, w)
    assert e.value.code == B.QL_EOVERFLOW


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_bitexact_random(lib, fmt):
    from quantized_base_lora_amd import binding as B
    w = special_weight(fmt, 64, 512, 7)
    qw = pack_gpu(lib, fmt, w)
    f, b = B.dequant(qw)
    torch.cuda.synchronize()
    c, s = ofmt.pack(fmt, w)
    ref = ofmt.dequant(fmt, c, s)
    assert np.array_equal(f.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(H.bf16_tensor_bits(b), codecs.bf16_encode(ref))


def test_dequant_all_codes_and_scales(lib):
    """Every 4-bit code against a grid of scales, and all 256 E4M3 codes."""
    from quantized_base_lora_amd import binding as B
    g = np.random.default_rng(3)
    # Q4_0: rows = fp16 scales (every 64th finite pattern plus extremes), all 16 codes
    d_bits = np.unique(np.concatenate([np.arange(0, 0x7C00, 61), [0x0001, 0x03FF, 0x0400, 0x7BFF]])).astype(np.uint16)
    n = (d_bits.size + 31) // 32 * 32
    d_bits = np.resize(d_bits, n)
    d_bits_q40 = d_bits
    q = np.tile(np.arange(16, dtype=np.uint8), (n, 2))
    codes = ofmt.nibbles_to_bytes(q)
    qw = B.QWeight(B.FMT_Q4_0, n, 32, torch.from_numpy(codes).cuda(),
                   torch.from_numpy(d_bits.view(np.int16).reshape(n, 1).copy()).cuda())
    f, b = B.dequant(qw)
    ref = ofmt.dequant_q4_0(codes, d_bits.reshape(n, 1))
    assert np.array_equal(f.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(H.bf16_tensor_bits(b), codecs.bf16_encode(ref))
    # NF4: scales include powers of two, random, subnormal-adjacent
    sc = np.concatenate([2.0 ** np.arange(-30, 2), g.uniform(1e-4, 0.3, 30), [1.1754944e-38, 3e-38]]).astype(np.float32)
    n = (sc.size + 31) // 32 * 32
    sc = np.resize(sc, n).reshape(n, 1)
    q = np.tile(np.arange(16, dtype=np.uint8), (n, 4))
    codes = ofmt.nibbles_to_bytes(q)
    qw = B.QWeight(B.FMT_NF4, n, 64, torch.from_numpy(codes).cuda(), torch.from_numpy(sc).cuda())
    f, b = B.dequant(qw)
    ref = ofmt.dequant_nf4(codes, sc)
    assert np.array_equal(f.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(H.bf16_tensor_bits(b), codecs.bf16_encode(ref))
    # Q8_0: all 256 code bytes against the same fp16 scale grid as Q4_0
    n = d_bits_q40.size
    codes = np.tile(np.arange(256, dtype=np.uint8), (n, 1))
    qw = B.QWeight(B.FMT_Q8_0, n, 256, torch.from_numpy(codes).cuda(),
                   torch.from_numpy(np.repeat(d_bits_q40.view(np.int16).reshape(n, 1), 8, axis=1).copy()).cuda())
    f, b = B.dequant(qw)
    ref = ofmt.dequant_q8_0(codes, np.repeat(d_bits_q40.reshape(n, 1), 8, axis=1))
    assert np.array_equal(f.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(H.bf16_tensor_bits(b), codecs.bf16_encode(ref))
    # MXFP4: all 16 codes against every E8M0 scale byte (255 is NaN)
    n = 256
    e8 = np.arange(256, dtype=np.uint8).reshape(n, 1)
    q = np.tile(np.arange(16, dtype=np.uint8), (n, 2))
    codes = ofmt.pairs_to_bytes(q)
    qw = B.QWeight(B.FMT_MXFP4, n, 32, torch.from_numpy(codes).cuda(), torch.from_numpy(e8.copy()).cuda())
    f, b = B.dequant(qw)
    ref = ofmt.dequant_mxfp4(codes, e8)
    got = f.cpu().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 32 and np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    gb = H.bf16_tensor_bits(b).reshape(n, 32)
    assert np.array_equal(gb[:255], codecs.bf16_encode(ref[:255]))
    # NVFP4: all 16 codes against every E4M3 scale byte (0x7F and 0xFF are NaN), a few tensor scales
    n = 256
    sb = np.stack([np.arange(256, dtype=np.uint8), np.arange(256, dtype=np.uint8)[::-1]], axis=1)
    q = np.tile(np.arange(16, dtype=np.uint8), (n, 2))
    codes = ofmt.nibbles_to_bytes(q)
    for gt in np.float32([1.0, 0.1, 3.7e-5]):
        image = ofmt.nvfp4_scale_image(gt, sb)
        qw = B.QWeight(B.FMT_NVFP4, n, 32, torch.from_numpy(codes).cuda(), torch.from_numpy(image).cuda())
        f, b = B.dequant(qw)
        ref = ofmt.dequant_nvfp4(codes, image)
        got = f.cpu().numpy()
        nan = np.isnan(ref)
        assert nan.sum() == 64 and np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
        gb = H.bf16_tensor_bits(b)
        rb = codecs.bf16_encode(ref)
        assert np.array_equal(gb[~nan], rb[~nan])
    # FP8: all 256 codes (two of them NaN) times a few scales
    for s in np.float32([1.0, 0.02 / 448, 7.77e-3]):
        codes = np.tile(np.arange(256, dtype=np.uint8), (32, 1))
        qw = B.QWeight(B.FMT_FP8, 32, 256, torch.from_numpy(codes).cuda(),
                       torch.tensor([s], dtype=torch.float32).cuda())
        f, b = B.dequant(qw)
        ref = ofmt.dequant_fp8(codes, s)
        got = f.cpu().numpy()
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


# the register-resident workgroup-per-row kernel in each of its shapes (rows
# of at most 1024, 2048, 4096, 8192, 12288 and 16384 elements, ragged ones
# included) and the two-pass kernel for longer rows
@pytest.mark.parametrize("shape", [(40, 320), (10, 1040), (37, 4096), (9, 2064), (6, 4608), (7, 12288),
                                   (6, 12304), (6, 16384), (6, 16400)])
def test_act_split_bitexact(lib, shape):
    from quantized_base_lora_amd import binding as B
    g = np.random.default_rng(5)
    x = g.standard_normal(shape, dtype=np.float32)
    x[3] = 0
    x[4, :7] = 1e-30
    x[5] *= 1e4
    bits = synth.to_bf16_bits(x)
    hi, lo, s = B.act_quant_e4m3(H.bits_to_bf16_tensor(bits))
    rh, rl, rs = olora.act_split_e4m3(synth.bf16_bits_to_f32(bits))
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(hi.cpu().numpy(), rh)
    assert np.array_equal(lo.cpu().numpy(), rl)


# ----------------------------------------------------------------------------- forward / backward

def run_layer(fmt, case, alpha, m, need_dx=True):
    from quantized_base_lora_amd import binding as B
    qw = B.quant_pack(fmt, torch.from_numpy(case["W"]).cuda())
    x = H.bits_to_bf16_tensor(case["x"])
    dy = H.bits_to_bf16_tensor(case["dY"])
    a = H.bits_to_bf16_tensor(case["A"])
    b = H.bits_to_bf16_tensor(case["B"])
    y, u = B.linear_fwd(qw, x, a, b, alpha)
    dx, da, db = B.linear_bwd(qw, x, dy, u, a, b, alpha, need_dx=need_dx)
    torch.cuda.synchronize()
    return qw, {"y": y, "U": u, "dX": dx, "dA": da, "dB": db}


def to_np(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


CASES = [
    # name,                fmt,            m,   k,   n,  r, alpha
    ("single256_q40", ofmt.FMT_Q4_0, 64, 256, 256, 8, 16.0),
    ("nf4_ragged_mn", ofmt.FMT_NF4, 300, 320, 160, 16, 32.0),
    ("q40_ragged_k_r32", ofmt.FMT_Q4_0, 257, 96, 224, 32, 64.0),
    ("fp8_r32", ofmt.FMT_FP8, 130, 256, 96, 32, 64.0),
    ("nf4_r8", ofmt.FMT_NF4, 64, 128, 64, 8, 16.0),
    ("nf4_m1", ofmt.FMT_NF4, 1, 128, 32, 16, 16.0),
    ("nf4_tiles_multi", ofmt.FMT_NF4, 512, 1024, 384, 16, 32.0),
    # FP8 base with more than 64 tokens: two-term E4M3 activations on fp8 matrix cores
    ("fp8_mfma_ragged", ofmt.FMT_FP8, 300, 160, 224, 16, 32.0),
    ("fp8_mfma_r8", ofmt.FMT_FP8, 520, 512, 384, 8, 16.0),
    # at most 64 tokens: contraction split across workgroups, fixed-order reduction
    ("small_q40_ragged_k", ofmt.FMT_Q4_0, 17, 1056, 224, 32, 64.0),
    ("small_nf4_splits", ofmt.FMT_NF4, 16, 2048, 320, 16, 32.0),
    ("small_fp8_m33", ofmt.FMT_FP8, 33, 512, 160, 8, 16.0),
    # 32 tokens: the largest count served by 32-row split tiles; ragged columns
    ("small_nf4_m32_r32", ofmt.FMT_NF4, 32, 640, 416, 32, 64.0),
    # FP8 base, rank 8, few tokens: dA and dB written by the dX reduction launch
    ("small_fp8_m20_r8", ofmt.FMT_FP8, 20, 256, 1216, 8, 16.0),
    # MXFP4 base (hardware E2M1 -> bf16 conversion): 128x128 and 256-row tiles with
    # ragged edges, the split path with 64, 33 and 17 tokens
    ("mxfp4_ragged_mn", ofmt.FMT_MXFP4, 300, 320, 160, 16, 32.0),
    ("mxfp4_tiles_r32", ofmt.FMT_MXFP4, 520, 1024, 416, 32, 64.0),
    ("small_mxfp4_m64_r8", ofmt.FMT_MXFP4, 64, 512, 384, 8, 16.0),
    ("small_mxfp4_m33", ofmt.FMT_MXFP4, 33, 1056, 224, 16, 32.0),
    ("small_mxfp4_m17_r32", ofmt.FMT_MXFP4, 17, 2048, 320, 32, 64.0),
    # MXFP4, 4 splits of 5 steps (K = 1152): slices whose scale bytes start at
    # odd 2-byte offsets, so the scale window is not used (it read the last
    # W row's last scales as zero: found by the shape sweep)
    ("small_mxfp4_m17_odd_slices", ofmt.FMT_MXFP4, 17, 1152, 160, 8, 16.0),
    ("small_mxfp4_m40_odd_slices", ofmt.FMT_MXFP4, 40, 1152, 32, 16, 32.0),
    # Q8_0 base (int8 codes, fp16 scale per 32): tiles with ragged edges, split path
    ("q80_ragged_mnk", ofmt.FMT_Q8_0, 300, 352, 160, 16, 32.0),
    ("q80_tiles_r8", ofmt.FMT_Q8_0, 520, 1024, 416, 8, 16.0),
    ("small_q80_m64_r32", ofmt.FMT_Q8_0, 64, 1056, 224, 32, 64.0),
    ("small_q80_m20", ofmt.FMT_Q8_0, 20, 2048, 320, 16, 32.0),
    # 8 tokens, a contraction slice of 12 steps of 128 per workgroup: longer
    # than the streaming kernel's LDS slice, so the staged 16-token kernel runs
    ("small_nf4_m8_long_slice", ofmt.FMT_NF4, 8, 6144, 13312, 16, 32.0),
    # NVFP4 base (E2M1 codes, E4M3 scale per 16, fp32 tensor scale): tiles with
    # ragged edges, the split path with 64, 33 and 17 tokens
    ("nvfp4_ragged_mn", ofmt.FMT_NVFP4, 300, 320, 160, 16, 32.0),
    ("nvfp4_tiles_r32", ofmt.FMT_NVFP4, 520, 1024, 416, 32, 64.0),
    ("small_nvfp4_m64_r8", ofmt.FMT_NVFP4, 64, 512, 384, 8, 16.0),
    ("small_nvfp4_m33", ofmt.FMT_NVFP4, 33, 1056, 224, 16, 32.0),
    ("small_nvfp4_m17_r32", ofmt.FMT_NVFP4, 17, 2048, 320, 32, 64.0),
    # 128x128 tiles, 10 row blocks x 16 column tiles = 160 tiles: the per-XCD
    # tile runs are active (tiles % 8 == 0) and the row blocks fall into
    # groups of 4 + 4 + 2; forward in the first case, dX in the second
    ("nf4_xcd_runs_fwd", ofmt.FMT_NF4, 1280, 256, 2048, 16, 32.0),
    ("nf4_xcd_runs_dx", ofmt.FMT_NF4, 1280, 2048, 256, 16, 32.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_layer_parity(lib, case):
    name, fmt, m, k, n, r, alpha = case
    say(f"layer parity {name}: fmt={FNAME[fmt]} m={m} k={k} n={n} r={r}")
    c = H.make_case(m, k, n, r, seed=zlib.crc32(name.encode()) % 1000)
    _, got = run_layer(fmt, c, alpha, m)
    _, _, wd = H.oracle_packed(fmt, c["W"])
    ref = H.oracle_layer(c, wd, alpha)
    tol = {"y": H.FWD_TOL, "U": H.FWD_TOL, "dX": H.FWD_TOL, "dA": H.FWD_TOL, "dB": H.FWD_TOL}
    for key in tol:
        e = H.rel(to_np(got[key]), ref[key])
        say(f"  {key}: rel err {e:.3e}")
        assert e <= tol[key], (key, e)


def test_m_zero_is_noop(lib):
    from quantized_base_lora_amd import binding as B
    c = H.make_case(4, 128, 64, 16, seed=9)
    qw = B.quant_pack(ofmt.FMT_NF4, torch.from_numpy(c["W"]).cuda())
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    a = H.bits_to_bf16_tensor(c["A"])
    b = H.bits_to_bf16_tensor(c["B"])
    y, u = B.linear_fwd(qw, x, a, b, 32.0)
    dy = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    dx, da, db = B.linear_bwd(qw, x, dy, u, a, b, 32.0)
    torch.cuda.synchronize()
    assert y.shape == (0, 64) and not da.any() and not db.any()


def test_no_dx_path(lib):
    c = H.make_case(96, 256, 128, 16, seed=12)
    _, got = run_layer(ofmt.FMT_NF4, c, 32.0, 96, need_dx=False)
    _, _, wd = H.oracle_packed(ofmt.FMT_NF4, c["W"])
    ref = H.oracle_layer(c, wd, 32.0)
    assert got["dX"] is None
    assert H.rel(to_np(got["dA"]), ref["dA"]) <= H.FWD_TOL
    assert H.rel(to_np(got["dB"]), ref["dB"]) <= H.FWD_TOL


# 128 tokens: separate adapter-gradient launch; 24: written by the dX reduction of the split path
@pytest.mark.parametrize("m", [128, 24])
def test_accumulate_adds(lib, m):
    from quantized_base_lora_amd import binding as B
    c = H.make_case(m, 128, 64, 16, seed=13)
    qw, got = run_layer(ofmt.FMT_NF4, c, 32.0, m)
    x = H.bits_to_bf16_tensor(c["x"])
    dy = H.bits_to_bf16_tensor(c["dY"])
    a = H.bits_to_bf16_tensor(c["A"])
    b = H.bits_to_bf16_tensor(c["B"])
    da0 = torch.full_like(got["dA"], 0.5)
    db0 = torch.full_like(got["dB"], -0.25)
    _, da, db = B.linear_bwd(qw, x, dy, got["U"], a, b, 32.0, accumulate=True, da=da0.clone(), db=db0.clone())
    torch.cuda.synchronize()
    assert torch.equal(da, got["dA"] + 0.5) and torch.equal(db, got["dB"] - 0.25)


# ----------------------------------------------------------------------------- exactness

def test_b_zero_and_a_zero_exact(lib):
    """B = 0: y and dX do not depend on A (bitwise), dA == 0 exactly.
    A = 0: y and dX do not depend on B, dB == 0 exactly, U == 0."""
    c = H.make_case(192, 256, 160, 16, seed=21)
    c0 = dict(c, B=np.zeros_like(c["B"]))
    c1 = dict(c0, A=synth.to_bf16_bits(synth.bf16_bits_to_f32(c["A"]) * 3.0))
    _, g0 = run_layer(ofmt.FMT_NF4, c0, 32.0, 192)
    _, g1 = run_layer(ofmt.FMT_NF4, c1, 32.0, 192)
    assert torch.equal(g0["y"].view(torch.int16), g1["y"].view(torch.int16))
    assert torch.equal(g0["dX"].view(torch.int16), g1["dX"].view(torch.int16))
    assert not g0["dA"].any()
    c2 = dict(c, A=np.zeros_like(c["A"]))
    c3 = dict(c2, B=synth.to_bf16_bits(synth.bf16_bits_to_f32(c["B"]) * 5.0))
    _, g2 = run_layer(ofmt.FMT_NF4, c2, 32.0, 192)
    _, g3 = run_layer(ofmt.FMT_NF4, c3, 32.0, 192)
    assert not g2["U"].any() and not g2["dB"].any()
    assert torch.equal(g2["y"].view(torch.int16), g3["y"].view(torch.int16))
    # with A = 0 the forward output is the base alone; with B = 0 too it is the same
    assert torch.equal(g2["y"].view(torch.int16), g0["y"].view(torch.int16))
    # and the LoRA path is live: B != 0 changes y
    _, gl = run_layer(ofmt.FMT_NF4, c, 32.0, 192)
    assert not torch.equal(gl["y"].view(torch.int16), g0["y"].view(torch.int16))


def test_integer_data_bitwise(lib):
    """Integer weights (Q4_0 with d = 1), sparse ternary x and dY, small integer
    adapters: every exact result is a small integer, so the GPU must match the
    oracle bit for bit whatever its summation order."""
    g = np.random.default_rng(31)
    m, k, n, r, alpha = 96, 128, 64, 8, 16.0
    w = g.integers(-7, 8, size=(n, k)).astype(np.float32)
    w[:, ::32] = 7.0                                         # every block has |w| = 7 -> d = 1
    x = np.zeros((m, k), np.float32)
    dy = np.zeros((m, n), np.float32)
    for i in range(m):
        x[i, g.choice(k, 3, replace=False)] = g.choice([-1.0, 1.0], 3)
        dy[i, g.choice(n, 3, replace=False)] = g.choice([-1.0, 1.0], 3)
    a = g.integers(-2, 3, size=(r, k)).astype(np.float32)
    b = g.integers(-2, 3, size=(n, r)).astype(np.float32)
    case = {"W": w, "x": synth.to_bf16_bits(x), "dY": synth.to_bf16_bits(dy),
            "A": synth.to_bf16_bits(a), "B": synth.to_bf16_bits(b)}
    _, got = run_layer(ofmt.FMT_Q4_0, case, alpha, m)
    c, s = ofmt.pack_q4_0(w)
    assert np.all(codecs.fp16_decode(s) == 1.0)
    wd = ofmt.dequant_q4_0(c, s)
    assert np.array_equal(wd, w)
    ref = H.oracle_layer(case, wd, alpha)
    assert np.abs(ref["y"]).max() < 256 and np.abs(ref["dX"]).max() < 256
    assert np.array_equal(to_np(got["y"]).astype(np.float64), ref["y"])
    assert np.array_equal(to_np(got["dX"]).astype(np.float64), ref["dX"])
    assert np.array_equal(to_np(got["U"]).astype(np.float64), ref["U"])
    assert np.array_equal(to_np(got["dA"]).astype(np.float64), ref["dA"])
    assert np.array_equal(to_np(got["dB"]).astype(np.float64), ref["dB"])


# every kernel path, run again on the same inputs: bitwise equal results
DET_CASES = [
    # name, fmt, m, k, n, r
    ("nf4_m384_128x128", ofmt.FMT_NF4, 384, 512, 256, 16),
    ("q40_m24_fused_grads", ofmt.FMT_Q4_0, 24, 512, 320, 32),
    ("nf4_m64_split", ofmt.FMT_NF4, 64, 1024, 512, 16),
    ("nf4_m2048_256rows", ofmt.FMT_NF4, 2048, 1024, 8192, 8),
    ("fp8_m300_fp8_mfma", ofmt.FMT_FP8, 300, 256, 512, 16),
    ("mxfp4_m640", ofmt.FMT_MXFP4, 640, 512, 768, 16),
    ("mxfp4_m24_fused_grads", ofmt.FMT_MXFP4, 24, 768, 256, 16),
    ("q80_m640", ofmt.FMT_Q8_0, 640, 512, 768, 16),
]


@pytest.mark.parametrize("case", DET_CASES, ids=[c[0] for c in DET_CASES])
def test_deterministic_and_base_untouched(lib, case):
    name, fmt, m, k, n, r = case
    c = H.make_case(m, k, n, r, seed=41)
    qw, g1 = run_layer(fmt, c, 32.0, m)
    before = (qw.codes.clone(), qw.scales.clone())
    from quantized_base_lora_amd import binding as B
    x = H.bits_to_bf16_tensor(c["x"])
    dy = H.bits_to_bf16_tensor(c["dY"])
    a = H.bits_to_bf16_tensor(c["A"])
    b = H.bits_to_bf16_tensor(c["B"])
    for _ in range(3):
        y, u = B.linear_fwd(qw, x, a, b, 32.0)
        dx, da, db = B.linear_bwd(qw, x, dy, u, a, b, 32.0)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), g1["y"].view(torch.int16)), name
        assert torch.equal(u.view(torch.int32), g1["U"].view(torch.int32)), name
        assert torch.equal(dx.view(torch.int16), g1["dX"].view(torch.int16)), name
        assert torch.equal(da.view(torch.int32), g1["dA"].view(torch.int32)), name
        assert torch.equal(db.view(torch.int32), g1["dB"].view(torch.int32)), name
    assert torch.equal(before[0], qw.codes) and torch.equal(before[1], qw.scales)


# at most 16 tokens the forward runs on 16x16x32 MFMAs over steps of 128:
# every format, ragged K (a step with live and dead groups), ragged N, one
# token; scale rows that do not start 4-byte aligned (Q4_0 at K = 1056, MXFP4
# at K = 4128) take the staged kernel, the others the streaming one
SMALL16 = [
    ("s16_nf4_k1088", ofmt.FMT_NF4, 16, 1088, 224, 16, 32.0),
    ("s16_q40_m5_k1056", ofmt.FMT_Q4_0, 5, 1056, 160, 32, 64.0),
    ("s16_fp8_m16", ofmt.FMT_FP8, 16, 768, 352, 8, 16.0),
    ("s16_mxfp4_m9_k4128", ofmt.FMT_MXFP4, 9, 4128, 96, 16, 32.0),
    ("s16_q80_m1", ofmt.FMT_Q8_0, 1, 2080, 416, 32, 64.0),
    # the streaming kernel (scale rows 4-byte aligned) with every 4-bit format
    ("s16_q40_m16_k1088", ofmt.FMT_Q4_0, 16, 1088, 288, 16, 32.0),
    ("s16_mxfp4_m7_k1152", ofmt.FMT_MXFP4, 7, 1152, 224, 8, 16.0),
    ("s16_nvfp4_m12_k1088", ofmt.FMT_NVFP4, 12, 1088, 160, 32, 64.0),
]


@pytest.mark.parametrize("case", SMALL16, ids=[c[0] for c in SMALL16])
def test_layer_parity_16_tokens(lib, case):
    name, fmt, m, k, n, r, alpha = case
    say(f"16-token parity {name}: fmt={FNAME[fmt]} m={m} k={k} n={n} r={r}")
    c = H.make_case(m, k, n, r, seed=zlib.crc32(name.encode()) % 1000)
    _, got = run_layer(fmt, c, alpha, m)
    _, _, wd = H.oracle_packed(fmt, c["W"])
    ref = H.oracle_layer(c, wd, alpha)
    for key in ("y", "U", "dX", "dA", "dB"):
        e = H.rel(to_np(got[key]), ref[key])
        say(f"  {key}: rel err {e:.3e}")
        assert e <= H.FWD_TOL, (key, e)

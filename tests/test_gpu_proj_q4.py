"""GPU parity of the projections with 4-bit weights (gdn_proj_q4_pack,
gdn_proj_q4), through the C ABI.

The 4-bit reading ("Kestrel_VLLM #24", sections 8 and 12): each weight is a
signed 4-bit value times the binary16 scale of its block of 32, exact in fp32.
Floating point: per element |y - r| <= max(1e-5 |r|, 1e-6 sum_c |W[o][c] x[c]|)
against the oracle's proj_q4 (a strict left fold of w x with w = n s; the
kernel forms the products n x on the fp16 matrix cores from x split exactly
into three binary16 parts, and scales each 32-column block's sum by s, so the
two differ by rounding only).
Bit-exact: every result when all partial sums are exact (integer-valued x,
power-of-two scales: any order gives the same bits), a row's result against
the same row in calls of every other row count, one launch of two products
against two launches, the two launch shapes (one or two workgroups per output
group) against each other, the packed order against its index definition in
include/gdn.h, and closed forms (all -8, all 7, one-hot columns).
"""
import numpy as np
import pytest
import torch

import gated_deltanet_recurrent_amd as gdn
import synth
from tests.helpers import assert_close, bits_equal, max_rel_pages

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "beta")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    gdn.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def say(*a):
    print(*a, flush=True)


def host(t):
    return np.ascontiguousarray(t.detach().cpu().numpy())


def decode_np(q, sc):
    """4-bit values (low nibble = even element, two's complement) times the
    block's binary16 scale, with numpy's float16."""
    q = np.asarray(q, np.uint8)
    n = np.empty((q.shape[0], 2 * q.shape[1]), np.int16)
    n[:, 0::2] = q & 15
    n[:, 1::2] = q >> 4
    n = np.where(n >= 8, n - 16, n).astype(np.float32)
    s = np.asarray(sc).view(np.float16).astype(np.float32)
    return np.ascontiguousarray(n * np.repeat(s, 32, axis=1))


def pack_q4_np(q, sc):
    """The packed order documented in include/gdn.h, by index arithmetic: per
    16-row column tile t and chunk m of 8 blocks of 32 columns (2304 bytes),
    dword 8 (16 d + o) + i = sum over k of (n + 8 of row 16 t + o, column
    256 m + 32 i + 8 d + k) << (4 (k >> 1) + 16 (k & 1)); then at 2048 + 16 o
    row 16 t + o's 8 scales of the chunk."""
    q = np.asarray(q, np.uint8)
    R, C = q.shape[0], 2 * q.shape[1]
    nib = np.empty((R, C), np.uint32)
    nib[:, 0::2] = q & 15
    nib[:, 1::2] = q >> 4
    u = (nib ^ 8).reshape(R // 16, 16, C // 256, 8, 4, 8)   # t, o, m, i, d, k
    shift = np.array([4 * (k >> 1) + 16 * (k & 1) for k in range(8)], np.uint32)
    dw = np.bitwise_or.reduce(u << shift, axis=5)             # t, o, m, i, d
    vals = np.ascontiguousarray(dw.transpose(0, 2, 4, 1, 3)).view(np.uint8)
    vals = vals.reshape(R // 16, C // 256, 2048)
    scl = np.asarray(sc).view(np.uint16).reshape(R // 16, 16, C // 256, 8)
    scl = np.ascontiguousarray(scl.transpose(0, 2, 1, 3)).view(np.uint8)
    scl = scl.reshape(R // 16, C // 256, 256)
    out = np.concatenate([vals, scl], axis=2)
    return np.ascontiguousarray(out.reshape(R // 64, 36 * C))


def q4_operands(seed, rows, R, C):
    gen = synth.make_gen(seed, "cuda")
    q, sc = synth.q4_weights(gen, R, C, device="cuda")
    x = torch.randn((rows, C), generator=gen, device="cuda")
    return x, q, sc


def ref_q4(orc, x, q, sc):
    y = np.zeros((x.shape[0], q.shape[0]), np.float32)
    orc.proj_q4(np.ascontiguousarray(x), host(q), host(sc).view(np.uint16), y)
    return y


def proj_floor(x, W):
    return 1e-6 * (np.abs(x.astype(np.float64)) @ np.abs(W.astype(np.float64)).T)


@pytest.mark.parametrize("R,C", [(64, 1024), (192, 2048), (10240, 5120), (5120, 6144)])
def test_q4_pack_layout(R, C):
    say(f"proj_q4_pack R={R} C={C}")
    _, q, sc = q4_operands(61, 1, R, C)
    Wq = gdn.proj_q4_pack(q, sc)
    assert Wq.numel() == gdn.proj_q4_bytes(R, C) == R * C * 9 // 16
    assert bits_equal(host(Wq), pack_q4_np(host(q), host(sc)))


@pytest.mark.parametrize("rows,R,C", [(1, 64, 1024), (3, 192, 2048), (8, 320, 3072),
                                      (16, 512, 5120), (1, 10240, 5120), (16, 5120, 6144),
                                      (5, 16384, 1024), (8, 5120, 1024), (6, 384, 2048)])
def test_q4_exact_when_every_partial_sum_is_exact(orc, rows, R, C):
    """Integer x in [-3, 3] and power-of-two scales 2^-2 .. 2^2: every product
    and partial sum is a multiple of 2^-2 below 2^22, so any summation order
    gives the oracle's bits; a dropped, repeated or misplaced term, a wrong
    nibble or a wrong scale shows as an exact mismatch."""
    say(f"proj_q4 exact sums rows={rows} R={R} C={C}")
    gen = synth.make_gen(70 + rows, "cuda")
    q = torch.randint(0, 256, (R, C // 2), generator=gen, device="cuda").to(torch.uint8)
    e = torch.randint(-2, 3, (R, C // 32), generator=gen, device="cuda").float()
    sc = torch.pow(2.0, e).to(torch.float16)
    x = torch.randint(-3, 4, (rows, C), generator=gen, device="cuda").float()
    y = host(gdn.proj_q4(x, gdn.proj_q4_pack(q, sc)))
    assert bits_equal(y, ref_q4(orc, host(x), q, sc))


@pytest.mark.parametrize("rows,R,C", [(2, 64, 131072), (1, 16384, 16384)])
def test_q4_large_sizes_exact(orc, rows, R, C):
    """Long quarters (C = 2^17: 128 chunks of x staged per workgroup, two
    workgroups per group) and a launch of 256 groups (one workgroup per
    group) with C = 2^14, whose one row of x just fills the up-front stage,
    on exactly summable operands (integer x, power-of-two scales): bit-exact
    against the oracle."""
    say(f"proj_q4 large rows={rows} R={R} C={C}")
    gen = synth.make_gen(151 + rows, "cuda")
    q = torch.randint(0, 256, (R, C // 2), generator=gen, device="cuda").to(torch.uint8)
    e = torch.randint(-2, 1, (R, C // 32), generator=gen, device="cuda").float()
    sc = torch.pow(2.0, e).to(torch.float16)
    x = torch.randint(-3, 4, (rows, C), generator=gen, device="cuda").float()
    y = host(gdn.proj_q4(x, gdn.proj_q4_pack(q, sc)))
    assert bits_equal(y, ref_q4(orc, host(x), q, sc))


@pytest.mark.parametrize("rows,R,C", [(1, 64, 1024), (5, 320, 3072), (11, 448, 2048),
                                      (16, 1024, 5120), (2, 16384, 1024)])
def test_q4_parity(orc, rows, R, C):
    say(f"proj_q4 parity rows={rows} R={R} C={C}")
    x, q, sc = q4_operands(80 + rows, rows, R, C)
    y = gdn.proj_q4(x, gdn.proj_q4_pack(q, sc))
    xh = host(x)
    Wd = decode_np(host(q), host(sc))
    assert_close(host(y), ref_q4(orc, xh, q, sc), f"proj_q4 {rows}x{R}x{C}", rel=1e-5,
                 floor=proj_floor(xh, Wd))


def test_q4_scales_of_every_kind(orc):
    """Scales drawn over every finite binary16 pattern of magnitude below 64
    (zero, subnormals, normals, both signs): the decoded weights stay exact, so
    the result stays within tolerance of the oracle."""
    say("proj_q4 any finite scale")
    rows, R, C = 4, 64, 2048
    gen = synth.make_gen(91, "cuda")
    q = torch.randint(0, 256, (R, C // 2), generator=gen, device="cuda").to(torch.uint8)
    mag = torch.randint(0, 0x5400, (R, C // 32), generator=gen, device="cuda")   # |s| < 64
    sign = torch.randint(0, 2, (R, C // 32), generator=gen, device="cuda") << 15
    sc = (mag | sign).to(torch.int32).to(torch.int16)
    x = torch.randn((rows, C), generator=gen, device="cuda")
    y4 = gdn.proj_q4(x, gdn.proj_q4_pack(q, sc))
    Wd = decode_np(host(q), host(sc))
    assert np.isfinite(Wd).all()
    xh = host(x)
    assert_close(host(y4), ref_q4(orc, xh, q, sc), "proj_q4 any scale", rel=1e-5,
                 floor=proj_floor(xh, Wd))


def test_q4_extreme_values_and_one_hot_columns():
    """All bytes 0x88 (every value -8) or 0x77 (every value 7) with scale 1
    and x = 1 give -8 C and 7 C exactly; one-hot rows select a decoded column
    exactly."""
    say("proj_q4 closed forms")
    R, C = 64, 1024
    one = torch.ones((R, C // 32), device="cuda").to(torch.float16)
    x1 = torch.ones((1, C), device="cuda")
    for byte, val in ((0x88, -8.0), (0x77, 7.0)):
        q = torch.full((R, C // 2), byte, dtype=torch.uint8, device="cuda")
        y = host(gdn.proj_q4(x1, gdn.proj_q4_pack(q, one)))
        assert (y == val * C).all(), (byte, y[0, :4])
    _, q, sc = q4_operands(97, 1, R, C)
    cols = [0, 1, 31, 32, 63, 64, 300, 511, 512, C - 1]
    x = torch.zeros((len(cols), C), device="cuda")
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    y = host(gdn.proj_q4(x, gdn.proj_q4_pack(q, sc)))
    Wd = decode_np(host(q), host(sc))
    for i, c in enumerate(cols):
        assert bits_equal(y[i], np.ascontiguousarray(Wd[:, c])), c


def test_q4_rows_are_independent_and_paired_launch_matches():
    """A row's bits do not depend on the other rows of the call: a 16-row call
    against calls over every row count 1..15 (each its own kernel instance);
    the paired launch (in_proj_qkv + in_proj_z) equals two single launches."""
    say("proj_q4 row independence, pairing")
    rows, C = 16, 1024
    x, q0, s0 = q4_operands(101, rows, 192, C)
    _, q1, s1 = q4_operands(103, 1, 64, C)
    W0, W1 = gdn.proj_q4_pack(q0, s0), gdn.proj_q4_pack(q1, s1)
    full0, full1 = gdn.proj_q4(x, W0, W1)
    full0, full1 = host(full0), host(full1)
    assert bits_equal(full0, host(gdn.proj_q4(x, W0)))
    assert bits_equal(full1, host(gdn.proj_q4(x, W1)))
    for n in range(1, 16):
        lo = (5 * n) % (17 - n)
        part = host(gdn.proj_q4(x[lo:lo + n].contiguous(), W0, W1)[0])
        assert bits_equal(part, np.ascontiguousarray(full0[lo:lo + n])), (lo, n)


@pytest.mark.parametrize("rows,R", [(1, 16384), (7, 192), (16, 192)])
def test_q4_nan_in_x_reaches_only_its_row(rows, R):
    """A NaN in x[r] makes exactly row r of y NaN (every weight is finite, a
    zero weight included: 0 x NaN is NaN); the other rows keep the bits of
    the NaN-free call, in both launch shapes (one and two workgroups per
    output group)."""
    say(f"proj_q4 NaN isolation rows={rows} R={R}")
    C = 2048
    x, q, sc = q4_operands(151, rows, R, C)
    Wq = gdn.proj_q4_pack(q, sc)
    clean = host(gdn.proj_q4(x, Wq))
    r = rows // 2
    xn = x.clone()
    xn[r, C - 3] = float("nan")
    y = host(gdn.proj_q4(xn, Wq))
    nan = np.zeros_like(clean, bool)
    nan[r, :] = True
    assert np.array_equal(np.isnan(y), nan)
    assert bits_equal(y[~nan], clean[~nan])


@pytest.mark.parametrize("rows,R", [(1, 16384), (1, 5120), (3, 192), (4, 192), (8, 256),
                                    (8, 16384), (16, 192)])
def test_q4_infinite_x_matches_oracle(orc, rows, R):
    """An infinite x (IEEE: w x is +-inf, NaN where w is 0, and +inf and -inf
    in one row give NaN) gives the oracle's class in every output of its row:
    +inf, -inf or NaN, with the row's other values scaled by the largest
    finite magnitude of their chunk (x of magnitude up to 12 here, which a
    scale set by the infinity would overflow in binary16).  Rows without one
    keep the bits of the call without infinities.  Every launch shape: one
    row with one or four tiles per workgroup, the up-front staging, one and
    two column tiles per wave, four row tiles."""
    say(f"proj_q4 infinite x rows={rows} R={R}")
    C = 2048
    x, q, sc = q4_operands(167, rows, R, C)
    x = x * 3.0
    Wq = gdn.proj_q4_pack(q, sc)
    clean = host(gdn.proj_q4(x, Wq))
    xi = x.clone()
    r = rows // 2
    xi[r, 5] = float("inf")
    if rows >= 3:
        xi[0, C - 7] = float("-inf")
        xi[rows - 1, 300] = float("inf")
        xi[rows - 1, 301] = float("-inf")
    y = host(gdn.proj_q4(xi, Wq))
    ref = ref_q4(orc, host(xi), q, sc)
    for cls in (np.isnan, np.isposinf, np.isneginf):
        assert np.array_equal(cls(y), cls(ref)), cls.__name__
    hit = ~np.isfinite(host(xi)).all(axis=1)
    assert (~np.isfinite(ref[hit])).all()
    assert bits_equal(np.ascontiguousarray(y[~hit]), np.ascontiguousarray(clean[~hit]))


@pytest.mark.parametrize("rows,R", [(1, 16384), (3, 192), (8, 256), (16, 192)])
def test_q4_extreme_magnitudes_of_x(orc, rows, R):
    """Rows of x near 1e30 and near 1e-30 (each 256-column chunk takes its
    own power-of-two scale, far from the usual k), and rows that mix 1e20 and
    1e-20 inside one chunk (the small values lie below 2^-15 of the chunk's
    largest and keep only what the three parts hold): within the projection
    tolerance of the oracle, in every launch shape."""
    say(f"proj_q4 extreme magnitudes rows={rows} R={R}")
    C = 2048
    x, q, sc = q4_operands(173, rows, R, C)
    scale = torch.ones((rows, C), device="cuda")
    for r in range(rows):
        kind = r % 3
        if kind == 0:
            scale[r] = 1e30
        elif kind == 1:
            scale[r] = 1e-30
        else:
            scale[r, 0::2] = 1e20
            scale[r, 1::2] = 1e-20
    xe = (x * scale).contiguous()
    y = host(gdn.proj_q4(xe, gdn.proj_q4_pack(q, sc)))
    xh = host(xe)
    assert np.isfinite(y).all()
    assert_close(y, ref_q4(orc, xh, q, sc), f"proj_q4 extreme {rows}x{R}", rel=1e-5,
                 floor=proj_floor(xh, decode_np(host(q), host(sc))))


def test_q4_staging_variants_agree_bit_for_bit():
    """At the layer's in_proj size (C = 5120, 16384 outputs) calls of 1-3 rows
    stage all of x up front and calls of 4-8 rows stage it chunk by chunk
    (5-8 rows with two column tiles per wave): every row of an 8-row call
    equals the same row in the calls of 1..7 rows, in either variant."""
    say("proj_q4 staging variants")
    C, R = 5120, 16384
    x, q, sc = q4_operands(157, 8, R, C)
    Wq = gdn.proj_q4_pack(q, sc)
    full = host(gdn.proj_q4(x, Wq))
    for n in range(1, 8):
        lo = 8 - n
        part = host(gdn.proj_q4(x[lo:].contiguous(), Wq))
        assert bits_equal(part, np.ascontiguousarray(full[lo:])), n


def test_q4_paired_tiles_agree_bit_for_bit():
    """At the layer's out_proj size (C = 6144, 5120 outputs: fewer 64-output
    groups than CUs) a call of 4-8 rows runs two workgroups per group of 4
    column tiles (one tile per wave: too few groups of 8 tiles to pair them),
    2-3 rows the up-front staging and 1 row one workgroup per tile: every row
    of an 8-row call equals the same row in the calls of 1..7 rows."""
    say("proj_q4 paired tiles")
    C, R = 6144, 5120
    x, q, sc = q4_operands(163, 8, R, C)
    Wq = gdn.proj_q4_pack(q, sc)
    full = host(gdn.proj_q4(x, Wq))
    for n in range(1, 8):
        lo = 8 - n
        part = host(gdn.proj_q4(x[lo:].contiguous(), Wq))
        assert bits_equal(part, np.ascontiguousarray(full[lo:])), n


def test_q4_launch_shapes_agree_bit_for_bit():
    """A launch with fewer 64-output groups than CUs takes two workgroups per
    group (half sums added into y); a larger one takes one.  The same matrix
    alone (192 outputs: split) and paired with a 16384-output matrix (one
    workgroup per group) gives the same bits, at 1, 7 and 16 rows; so does
    the large matrix alone (one workgroup per group) against its half-size
    slices (split)."""
    say("proj_q4 launch shapes")
    C = 2048
    _, q0, s0 = q4_operands(131, 1, 192, C)
    _, q1, s1 = q4_operands(137, 1, 16384, C)
    W0, W1 = gdn.proj_q4_pack(q0, s0), gdn.proj_q4_pack(q1, s1)
    W1a, W1b = gdn.proj_q4_pack(q1[:8192].contiguous(), s1[:8192].contiguous()), \
        gdn.proj_q4_pack(q1[8192:].contiguous(), s1[8192:].contiguous())
    for rows in (1, 7, 16):
        x = torch.randn((rows, C), generator=synth.make_gen(139 + rows, "cuda"), device="cuda")
        alone = host(gdn.proj_q4(x, W0))
        paired, big = gdn.proj_q4(x, W0, W1)
        assert bits_equal(alone, host(paired)), rows
        halves = np.concatenate([host(gdn.proj_q4(x, W1a)), host(gdn.proj_q4(x, W1b))], axis=1)
        assert bits_equal(host(big), halves), rows


def test_q4_binding_refuses_wrong_tensors():
    """The binding refuses a wrong dtype, a wrong shape or a wrong-size output
    before calling the C ABI, and the C ABI refuses shapes outside its limits."""
    say("proj_q4 binding refusals")
    x, q, sc = q4_operands(109, 2, 64, 1024)
    W = gdn.proj_q4_pack(q, sc)
    with pytest.raises(TypeError, match="q"):
        gdn.proj_q4_pack(q.to(torch.int32), sc)
    with pytest.raises(TypeError, match="scale"):
        gdn.proj_q4_pack(q, sc.float())
    with pytest.raises(ValueError, match="scale"):
        gdn.proj_q4_pack(q, sc[:, :-1].contiguous())
    with pytest.raises(gdn.GdnError) as e:
        gdn.proj_q4_pack(q[:, :256].contiguous(), sc[:, :16].contiguous())   # C = 512
    assert e.value.rc == gdn.GDN_EUNSUPPORTED
    with pytest.raises(ValueError, match="Wq0"):
        gdn.proj_q4(x, W.view(-1)[: W.numel() // 2].view(W.shape[0] // 2 or 1, -1))
    with pytest.raises(TypeError, match="Wq0"):
        gdn.proj_q4(x, W.view(torch.int8))
    with pytest.raises(ValueError, match="output"):
        gdn.proj_q4(x, W, y0=torch.empty((2, 63), device="cuda"))
    with pytest.raises(TypeError, match="x"):
        gdn.proj_q4(x.double(), W)


def test_q4_refuses_more_than_16_rows_and_accepts_none():
    say("proj_q4 row limits")
    x, q, sc = q4_operands(107, 17, 64, 1024)
    W = gdn.proj_q4_pack(q, sc)
    with pytest.raises(gdn.GdnError) as e:
        gdn.proj_q4(x, W)
    assert e.value.rc == gdn.GDN_EUNSUPPORTED
    y = torch.full((0, 64), 7.0, device="cuda")
    assert gdn.proj_q4(x[:0], W, y0=y).numel() == 0


@pytest.mark.parametrize("dims", [synth.DIMS128, synth.DIMS64])
def test_q4_layer_sizes_sampled(orc, dims):
    """The layer's full projection sizes with 4-bit weights at 1, 8 and 16
    rows, in the launches the benchmark times (8 rows: two column tiles per
    wave, in_proj_qkv and in_proj_z in one launch), on rows the oracle
    recomputes."""
    vh, kh, kd, vd = dims
    dim = synth.FE_DIM
    gen = synth.make_gen(113, "cuda")
    w = synth.proj_weights_q4(gen, dims, device="cuda")
    wq = {n: gdn.proj_q4_pack(*w[n]) for n in ("W_qkv", "W_z", "W_out")}
    for rows, pick in ((1, [0]), (8, [0, 5, 7]), (16, [0, 9, 15])):
        say(f"proj_q4 layer sizes dims={dims} rows={rows}")
        x = torch.randn((rows, dim), generator=gen, device="cuda")
        h = torch.randn((rows, vh * vd), generator=gen, device="cuda")
        xc, z = gdn.proj_q4(x, wq["W_qkv"], wq["W_z"])
        y = gdn.proj_q4(h, wq["W_out"])
        xh, hh = host(x)[pick], host(h)[pick]
        for name, got, inp in (("W_qkv", xc, xh), ("W_z", z, xh), ("W_out", y, hh)):
            q, sc = w[name]
            assert_close(host(got)[pick], ref_q4(orc, inp, q, sc), name, rel=1e-5,
                         floor=proj_floor(inp, decode_np(host(q), host(sc))))


def test_q4_layer_decode_chain(orc):
    """One GDN layer decoding two tokens with 4-bit projections, entirely
    through the C ABI: each projection matches the oracle's proj_q4 on the
    GPU's own inputs to it, and the chain matches the oracle's chain under the
    pages' layer criterion max|err| / max|ref| <= 1e-4 ("Kestrel_VLLM #24",
    section 6)."""
    dims = synth.DIMS128
    vh, kh, kd, vd = dims
    B, dim, T, eps = 2, 1024, 2, 1e-6
    cd = synth.conv_dim_of(dims)
    say(f"q4 layer chain B={B} dim={dim} T={T}")
    gen = synth.make_gen(127, "cuda")
    pw = synth.proj_weights_q4(gen, dims, dim=dim, device="cuda")
    fw = synth.frontend_weights(gen, dims, dim=dim, device="cuda")
    S = synth.state(gen, B, dims, device="cuda")
    hist = torch.randn((B, 3, cd), generator=gen, device="cuda")
    xs = torch.randn((T, B, dim), generator=gen, device="cuda")
    big = ("W_qkv", "W_z", "W_out")
    wq = {n: gdn.proj_q4_pack(*pw[n]) for n in big}
    W = {n: host(t) for n, t in fw.items()}
    qh = {n: (host(pw[n][0]), host(pw[n][1]).view(np.uint16)) for n in big}
    dec = {n: decode_np(*qh[n]) for n in big}
    S_r, hist_r = host(S), host(hist)

    def proj_r(x, n):
        y = np.zeros((x.shape[0], qh[n][0].shape[0]), np.float32)
        orc.proj_q4(np.ascontiguousarray(x), qh[n][0], qh[n][1], y)
        return y

    for t in range(T):
        xc, z = gdn.proj_q4(xs[t], wq["W_qkv"], wq["W_z"])
        fe = gdn.frontend(xs[t], fw["Wa"], fw["Wb"], fw["A_log"], fw["dt_bias"], xc, hist,
                          fw["conv_w"], dims)
        out = gdn.step_gated(S, *(fe[n].unsqueeze(0) for n in NAMES),
                             z.view(1, B, vh, vd), pw["norm_w"], eps)
        oh = host(out).reshape(B, vh * vd)
        y = host(gdn.proj_q4(out.view(B, vh * vd), wq["W_out"]))
        xh = host(xs[t])
        for name, got, inp in (("W_qkv", host(xc), xh), ("W_z", host(z), xh), ("W_out", y, oh)):
            assert_close(got, proj_r(inp, name), name, rel=1e-5, floor=proj_floor(inp, dec[name]))

        xc_r, z_r = proj_r(xh, "W_qkv"), proj_r(xh, "W_z")
        fr = {n: np.zeros(tuple(fe[n].shape), np.float32) for n in NAMES}
        orc.gdn_frontend(xh, W["Wa"], W["Wb"], W["A_log"], W["dt_bias"], xc_r, hist_r,
                         W["conv_w"], fr["q"], fr["k"], fr["v"], fr["g"], fr["beta"], dims)
        o_r = np.zeros((B, vh, vd), np.float32)
        orc.gdn_step(S_r, *(fr[n] for n in NAMES), o_r, dims)
        gn_r = np.zeros_like(o_r)
        orc.gated_norm(o_r, z_r.reshape(B, vh, vd), host(pw["norm_w"]), eps, gn_r)
        y_r = proj_r(gn_r.reshape(B, vh * vd), "W_out")
        for b in range(B):
            assert max_rel_pages(y[b], y_r[b]) <= 1e-4, (t, b)
    assert max_rel_pages(host(S), S_r) <= 1e-4


def test_q4_graph_replay_matches_eager(orc):
    """The layer's 4-bit projections captured as a HIP graph (in_proj: one
    workgroup per group; out_proj: two workgroups per group, whose fill
    kernel and atomic adds must run on every replay) replay bit-identically
    to eager calls, several times, with eager work and synchronisations in
    between and the outputs dirtied before each replay."""
    say("proj_q4 graph replay")
    dims = synth.DIMS128
    vh, kh, kd, vd = dims
    gen = synth.make_gen(157, "cuda")
    w = synth.proj_weights_q4(gen, dims, device="cuda")
    wq = {n: gdn.proj_q4_pack(*w[n]) for n in ("W_qkv", "W_z", "W_out")}
    rows = 3
    x = torch.randn((rows, synth.FE_DIM), generator=gen, device="cuda")
    h = torch.randn((rows, vh * vd), generator=gen, device="cuda")
    e_xc, e_z = gdn.proj_q4(x, wq["W_qkv"], wq["W_z"])
    e_y = gdn.proj_q4(h, wq["W_out"])
    torch.cuda.synchronize()
    # the eager results against the oracle (which the replays then equal)
    for got, xin, n in ((e_xc, x, "W_qkv"), (e_z, x, "W_z"), (e_y, h, "W_out")):
        xh = host(xin)
        assert_close(host(got), ref_q4(orc, xh, *w[n]), n,
                     floor=proj_floor(xh, decode_np(host(w[n][0]), host(w[n][1]))))
    xc, z, y = torch.empty_like(e_xc), torch.empty_like(e_z), torch.empty_like(e_y)

    def chain():
        gdn.proj_q4(x, wq["W_qkv"], wq["W_z"], y0=xc, y1=z)
        gdn.proj_q4(h, wq["W_out"], y0=y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                  # warm-up outside capture
        chain()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain()
    for rep in range(3):
        for t in (xc, z, y):
            t.fill_(float(rep + 1))                # dirty outputs: the fill must clear y
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in ((xc, e_xc), (z, e_z), (y, e_y)):
            assert bits_equal(host(got), host(want)), rep
        gdn.proj_q4(h, wq["W_out"])                 # eager work between replays
        torch.cuda.synchronize()
    del graph

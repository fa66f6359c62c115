"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

None of these re-types the oracle's own formulas.  Each pin compares the oracle
with something independent of it: numbers the pages print, a closed form, a
library routine (numpy), brute force on tiny inputs, or an invariant.  The
``check_*`` functions take the oracle module so that the mutation test can run
them against deliberately broken builds of the oracle.
"""
import json
import os

import numpy as np
import pytest

import tq_inputs as TI

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def pages():
    with open(os.path.join(GOLDEN, "pages_constants.json")) as f:
        return {k: v["value"] for k, v in json.load(f).items() if not k.startswith("_")}


# ----------------------------------------------------------------------------
# Independent decoders written in the tests (not the oracle's code).


def np_decode_pq2(W):
    """pq2_0 blocks -> (w, d) with numpy bit operations: field k&3 of byte k>>2."""
    codes = W[..., 2:].astype(np.int16)
    R, G, _ = codes.shape
    u = np.stack([(codes >> (2 * f)) & 3 for f in range(4)], axis=-1)  # [R, G, 32, 4]
    w = (u - 1).reshape(R, G * 128).astype(np.int64)
    d = np.ascontiguousarray(W[..., 0:2]).view("<f2")[..., 0].astype(np.float64)
    return w, d


def np_decode_ptq1(W):
    """ptq1_0 blocks -> (w, d) via the threshold form the pages give: trit = (v>=86)+(v>=171)."""
    P = pages()
    b = W[..., 2:].astype(np.int64)  # [R, G, 26]
    R, G, _ = b.shape
    trits = []
    for j in range(5):
        v = (b * 3**j) & 0xFF
        trits.append((v >= P["ptq1_threshold_low"]).astype(np.int64) + (v >= P["ptq1_threshold_high"]).astype(np.int64))
    t = np.stack(trits, axis=-1).reshape(R, G, 130)[:, :, :128]
    w = (t - 1).reshape(R, G * 128)
    d = np.ascontiguousarray(W[..., 0:2]).view("<f2")[..., 0].astype(np.float64)
    return w, d


def pack_pq2_from_w(w, d):
    """Encode int weights [R, K] in {-1,0,1} and fp16 scales [R, G] as pq2_0 blocks.

    Follows the pages' packer: code (w + 1) is or-ed in at bit 2*s."""
    R, K = w.shape
    G = K // 128
    u = (w + 1).astype(np.uint8).reshape(R, G, 32, 4)
    codes = np.zeros((R, G, 32), dtype=np.uint8)
    for s in range(4):
        codes |= (u[..., s] << (2 * s)).astype(np.uint8)
    return TI.assemble_pq2(codes, d.astype(np.float16))


def brute_y(w, dw, q, dx):
    """float64 brute force: (d_w * w) @ (d_x * q) per token."""
    Wf = w.astype(np.float64) * np.repeat(dw.astype(np.float64), 128, axis=1)
    Xf = q.astype(np.float64) * np.repeat(dx.astype(np.float64), 256, axis=1)
    return Xf @ Wf.T  # [T, R]


def rel_ok(y, ref, mag, rtol):
    y = y.astype(np.float64)
    err = np.abs(y - ref)
    bound = np.where(ref != 0, rtol * np.abs(ref), rtol * mag)
    # fp32 rounding of the result is allowed on top of the comparison tolerance
    bound = bound + np.abs(ref) * 2.0**-24 + 1e-300
    return err <= bound


# ----------------------------------------------------------------------------
# checks


def check_half(orc):
    """fp16 -> fp32 for all 65536 bit patterns against numpy's conversion."""
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([orc.half_to_float(int(h)) for h in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def check_pq2_decode(orc):
    g = TI.rng(99, 1)
    # fixed bytes: 0x55 -> all u=1 (w=0); 0xAA -> u=2 (w=+1); 0x00 -> w=-1;
    # 0x24 = 0b00100100 -> fields (low first) 0,1,2,0 -> w = -1, 0, +1, -1
    for byte, expect in ((0x55, [0, 0, 0, 0]), (0xAA, [1, 1, 1, 1]), (0x00, [-1] * 4), (0x24, [-1, 0, 1, -1])):
        blk = TI.assemble_pq2(np.full((1, 1, 32), byte, np.uint8), np.full((1, 1), 0.5, np.float16))
        w, d, bad = orc.decode("pq2_0", blk)
        assert bad == 0 and d[0, 0] == 0.5
        assert w[0].tolist() == expect * 32
    # code 3 is counted as invalid
    blk = TI.assemble_pq2(np.full((1, 1, 32), 0xE4, np.uint8), np.ones((1, 1), np.float16))
    w, _, bad = orc.decode("pq2_0", blk)
    assert bad == 32 and w[0, :4].tolist() == [-1, 0, 1, 2]
    # random weights through the test's own encoder round-trip exactly
    wr = g.integers(-1, 2, size=(7, 512))
    dr = g.uniform(0.01, 0.05, size=(7, 4)).astype(np.float16)
    blk = pack_pq2_from_w(wr, dr)
    w, d, bad = orc.decode("pq2_0", blk)
    assert bad == 0 and np.array_equal(w, wr) and np.array_equal(d, dr.astype(np.float32))
    # and the generator's blocks agree with the test's numpy decoder
    W = TI.pq2_matrix(g, 5, 1024)
    w, d, _ = orc.decode("pq2_0", W)
    wn, dn = np_decode_pq2(W)
    assert np.array_equal(w, wn) and np.array_equal(d.astype(np.float64), dn)


def check_ptq1_decode(orc):
    P = pages()
    # every byte value, every trit, against the pages' threshold form
    b = np.arange(256, dtype=np.uint8)
    codes = np.zeros((256, 1, 26), np.uint8)
    codes[:, 0, :] = b[:, None]
    blk = TI.assemble_ptq1(codes, np.ones((256, 1), np.float16))
    w, _, _ = orc.decode("ptq1_0", blk)
    wn, _ = np_decode_ptq1(blk)
    assert np.array_equal(w.astype(np.int64), wn)
    # the first v with trit 1 is 86 and the first with trit 2 is 171 (trit 0 of byte v is floor(3v/256))
    t0 = w[:, 0].astype(int) + 1
    assert int(np.argmax(t0 >= 1)) == P["ptq1_threshold_low"] and int(np.argmax(t0 >= 2)) == P["ptq1_threshold_high"]
    # closed-form encoder: byte ceil(256 n / 243) holds the base-3 digits of n, most significant first
    assert 3 ** P["trits_per_byte"] == P["three_pow_five"]
    for n in range(P["three_pow_five"]):
        byte = -(-256 * n // 243)
        digits = [(n // 3 ** (4 - j)) % 3 for j in range(5)]
        got = (w[byte, :5].astype(int) + 1).tolist()
        assert got == digits, (n, byte, got, digits)


def check_q8k(orc):
    P = pages()
    QB = P["q8k_block"]
    g = TI.rng(99, 2)
    xs = [
        TI.activations(g, 3, 1024),
        (g.standard_t(2, size=(2, 2048)) * 10).astype(np.float32),  # heavy tails
        (g.standard_normal((2, 512)) * 1e-40).astype(np.float32),  # subnormal range
        g.uniform(-1, 1, size=(1, 256)).astype(np.float32) * 3e38,
    ]
    for x in xs:
        q, d, bs = orc.quantize_q8k(x)
        T, K = x.shape
        assert bs.shape == (T, K // P["q8k_partial_sums"]) and d.shape == (T, K // QB)
        for t in range(T):
            for blk in range(K // QB):
                xb = x[t, blk * QB:(blk + 1) * QB].astype(np.float64)
                qb = q[t, blk * QB:(blk + 1) * QB].astype(np.int64)
                db = float(d[t, blk])
                amax = np.max(np.abs(xb))
                # d is max|x|/127 rounded once to fp32
                assert db == float(np.float32(np.float32(amax) / np.float32(127)))
                if db == 0:
                    assert not qb.any()
                else:
                    assert np.max(np.abs(qb)) == 127  # the block's largest value lands on +-127
                    assert np.all(np.abs(xb - db * qb) <= db * (0.5 + 127 * 2.0**-23))
                    assert np.all(np.sign(qb) * np.sign(xb) >= 0)
                sums = qb.reshape(QB // 16, 16).sum(axis=1)
                assert np.array_equal(bs[t, blk * 16:(blk + 1) * 16].astype(np.int64), sums)
    # an all-zero block gives d = 0, q = 0, bsums = 0
    x = np.zeros((1, 512), np.float32)
    x[0, 300] = 1.0
    q, d, bs = orc.quantize_q8k(x)
    assert d[0, 0] == 0 and not q[0, :256].any() and not bs[0, :16].any()
    assert q[0, 300] == 127 and d[0, 1] == np.float32(1.0) / np.float32(127)
    # hand-derived ties (golden file)
    rows = [l.split() for l in open(os.path.join(GOLDEN, "q8k_ties.txt")) if l.strip() and not l.startswith("#")]
    x = np.zeros((1, 256), np.float32)
    x[0, 0] = 254
    for i, (xv, _) in enumerate(rows[1:], start=1):
        x[0, i] = float(xv)
    q, d, _ = orc.quantize_q8k(x)
    assert d[0, 0] == 2.0
    assert [int(v) for v in q[0, :len(rows)]] == [int(e) for _, e in rows]
    # symmetry: x -> -x gives q -> -q and the same d
    x = TI.activations(g, 2, 1024)
    q1, d1, b1 = orc.quantize_q8k(x)
    q2, d2, b2 = orc.quantize_q8k(-x)
    assert np.array_equal(q2, -q1) and np.array_equal(d1, d2) and np.array_equal(b2, -b1)


def check_identity_quantization(orc):
    """Integer x with |x| = 127 in EVERY 256-block quantizes to itself (d = 1), so
    the whole product reduces to an integer matmul checked with numpy int64."""
    g = TI.rng(99, 3)
    for R, K, T in ((4, 256, 1), (8, 512, 3), (12, 1024, 5), (33, 1024, 8)):
        x = g.integers(-127, 128, size=(T, K)).astype(np.float32)
        x[:, ::256] = 127 * np.where(g.integers(0, 2, size=(T, K // 256)) > 0, 1, -1)
        q, d, _ = orc.quantize_q8k(x)
        assert np.all(d == 1.0) and np.array_equal(q.astype(np.float32), x)
        W = TI.pq2_matrix(g, R, K)
        wn, dn = np_decode_pq2(W)
        I = orc.group_dots("pq2_0", W, q)
        ref = np.einsum("tgk,rgk->trg", x.astype(np.int64).reshape(T, K // 128, 128), wn.reshape(R, K // 128, 128))
        assert np.array_equal(I.astype(np.int64), ref)


def check_brute_force_grid(orc):
    """The pages' validation grid shape: batch widths 1-5, 7, 8; rows 4, 8, 12
    (plus 1, 5, 33); inner sizes 256, 512, 1024 -- y vs a float64 brute force."""
    g = TI.rng(99, 4)
    for fmt in ("pq2_0", "ptq1_0"):
        for K in (256, 512, 1024):
            for R in (1, 4, 5, 8, 12, 33):
                W = TI.pq2_matrix(g, R, K) if fmt == "pq2_0" else TI.ptq1_matrix(g, R, K)
                wn, dn = np_decode_pq2(W) if fmt == "pq2_0" else np_decode_ptq1(W)
                for T in (1, 2, 3, 4, 5, 7, 8):
                    x = TI.activations(g, T, K)
                    q, dx, _ = orc.quantize_q8k(x)
                    y, mag = orc.matmul(fmt, W, q, dx, with_mag=True)
                    ref = brute_y(wn, dn, q, dx)
                    assert np.all(rel_ok(y, ref, mag, 1e-12)), (fmt, K, R, T)
                    I = orc.group_dots(fmt, W, q)
                    Iref = np.einsum("tgk,rgk->trg", q.astype(np.int64).reshape(T, K // 128, 128), wn.reshape(R, K // 128, 128))
                    assert np.array_equal(I.astype(np.int64), Iref), (fmt, K, R, T)


def check_invariants(orc):
    P = pages()
    g = TI.rng(99, 5)
    R, K, T = 6, 1024, 3
    G = K // 128
    x = TI.activations(g, T, K)
    q, dx, bs = orc.quantize_q8k(x)
    d = g.uniform(0.01, 0.05, size=(R, G)).astype(np.float16)
    # all-zero weights -> I = 0 and y = +0 exactly
    W0 = pack_pq2_from_w(np.zeros((R, K), int), d)
    y0 = orc.matmul("pq2_0", W0, q, dx)
    assert not orc.group_dots("pq2_0", W0, q).any() and np.all(y0 == 0) and not np.signbit(y0).any()
    # all +1 -> I_g = sum of the 8 partial sums of the group; all -1 -> the negation
    Wp = pack_pq2_from_w(np.ones((R, K), int), d)
    Wm = pack_pq2_from_w(-np.ones((R, K), int), d)
    Ip = orc.group_dots("pq2_0", Wp, q)
    Im = orc.group_dots("pq2_0", Wm, q)
    gs = bs.astype(np.int64).reshape(T, G, 8).sum(axis=2)
    assert np.array_equal(Ip.astype(np.int64), np.broadcast_to(gs[:, None, :], Ip.shape))
    assert np.array_equal(Im, -Ip)
    assert np.array_equal(orc.matmul("pq2_0", Wm, q, dx), -orc.matmul("pq2_0", Wp, q, dx))
    # extremes: q = +-127 everywhere with w = +-1 -> |I| = 128 * 127; in the
    # pages' u = w + 1 form the same block reaches 128 * 2 * 127, and times the
    # slot factor 16 that is the printed int32 bound
    xe = np.full((1, K), 127.0, np.float32)
    qe, dxe, _ = orc.quantize_q8k(xe)
    Ie = orc.group_dots("pq2_0", Wp, qe)
    assert np.all(Ie == 128 * 127)
    dot_u = Ie.astype(np.int64) + qe.astype(np.int64).reshape(1, G, 128).sum(axis=2)[:, None, :]
    assert np.all(dot_u * 16 == P["int32_bound_x16"])
    # w -> -w negates I and y exactly; x -> -x negates y exactly
    W = TI.pq2_matrix(g, R, K)
    wn, _ = np_decode_pq2(W)
    dn = np.ascontiguousarray(W[..., 0:2]).view("<f2")[..., 0]
    Wneg = pack_pq2_from_w(-wn, dn)
    assert np.array_equal(orc.group_dots("pq2_0", Wneg, q), -orc.group_dots("pq2_0", W, q))
    y = orc.matmul("pq2_0", W, q, dx)
    assert np.array_equal(orc.matmul("pq2_0", Wneg, q, dx), -y)
    qn, dxn, _ = orc.quantize_q8k(-x)
    assert np.array_equal(orc.matmul("pq2_0", W, qn, dxn), -y)
    # permuting rows permutes y
    perm = g.permutation(R)
    assert np.array_equal(orc.matmul("pq2_0", W[perm], q, dx), y[:, perm])
    # row-range evaluation equals the full evaluation
    assert np.array_equal(orc.matmul("pq2_0", W, q, dx, rows=(2, 5)), y[:, 2:5])
    assert np.array_equal(orc.matmul("pq2_0", W, q, dx, threads=3), y)


CHECKS = [check_half, check_pq2_decode, check_ptq1_decode, check_q8k, check_identity_quantization,
          check_brute_force_grid, check_invariants]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_pin(orc, check):
    check(orc)


def test_workload_sizes():
    """The canonical byte counts per 128 weights are the pages' bits per weight."""
    P = pages()
    g = TI.rng(99, 6)
    assert TI.pq2_matrix(g, 2, 256).nbytes * 8 / (2 * 256) == P["pq2_bits_per_weight"]
    assert TI.ptq1_matrix(g, 2, 256).nbytes * 8 / (2 * 256) == P["ptq1_bits_per_weight"]

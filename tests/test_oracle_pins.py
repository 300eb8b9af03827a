"""Pins of the fp64 oracle against facts that do not come from the oracle itself:
hand-derived byte positions of the weight layouts, exact rational arithmetic,
closed forms, brute force on tiny shapes, textbook library routines,
invariants, and the structural numbers the pages print.

Each pin is written so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a swapped gate/up, an unstable sort)
fails at least one of them; ``test_planted_mistakes_are_caught`` checks that on
the CPU by planting such slips into the oracle and re-running the pins.
"""
import itertools
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle.formats as F
import oracle.layer as L
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ============================================================ layouts (hand-derived positions)

def test_q2_layout_hand_derived():
    # 128 x 256 matrix, every code 2 (byte 0b10101010) and every scale 1.0, except:
    #   (n=70, k=200): tile 1*4+3 = 7, byte 7*1024 + 6*16 + 8//4 = 7266, bits 0-1 -> code 3: 0xAB
    #   (n=5,  k=63):  tile 0,          byte 5*16 + 15 = 95,                bits 6-7 -> code 0: 0x2A
    #   scale of (n=70, block 6): ((1*2) + 1)*256 + 6*4 + 2 = 794 -> 0.5
    N, K = 128, 256
    codes = np.full(N * K // 4, 0xAA, dtype=np.uint8)
    codes[7266] = 0xAB
    codes[95] = 0x2A
    scales = np.full(N * K // 32, 0x3C00, dtype=np.uint16)
    scales[794] = 0x3800
    W = F.decode_q2(codes, scales, N, K)
    expect = np.zeros((N, K))
    expect[70, 200] = 0.5
    expect[5, 63] = -2.0
    np.testing.assert_array_equal(W, expect)
    # scale-block mapping: all codes 3 -> W = scale; block (n=127, b=7) is index
    # ((1*2) + 1)*256 + 63*4 + 3 = 1023
    codes[:] = 0xFF
    scales[794] = 0x3C00
    scales[1023] = 0x4000
    W = F.decode_q2(codes, scales, N, K)
    expect = np.ones((N, K))
    expect[127, 224:256] = 2.0
    np.testing.assert_array_equal(W, expect)


def _pack_q2_writer(C):
    """Writer-direction packer of the Q2 layout, written as nested loops over
    tiles, rows and bytes (independent of the oracle's reader)."""
    N, K = C.shape
    out = bytearray(N * K // 4)
    pos = 0
    for ng in range(N // 64):
        for kc in range(K // 64):
            for r in range(64):
                for q in range(16):
                    b = 0
                    for i in range(4):
                        b |= int(C[ng * 64 + r, kc * 64 + 4 * q + i]) << (2 * i)
                    out[pos] = b
                    pos += 1
    return np.frombuffer(bytes(out), dtype=np.uint8)


def _pack_scales_writer(S):
    """S[n, b] (fp16 bits) -> flat array in the scale layout, as nested loops."""
    N, B = S.shape
    out = []
    for ng in range(N // 64):
        for bq in range(B // 4):
            for r in range(64):
                for i in range(4):
                    out.append(S[ng * 64 + r, bq * 4 + i])
    return np.array(out, dtype=np.uint16)


def _fp16_from_bits(b):
    return struct.unpack("<e", struct.pack("<H", int(b)))[0]


def test_q2_layout_writer_reader_agree():
    rng = np.random.default_rng(11)
    N, K = 128, 384
    C = rng.integers(0, 4, size=(N, K))
    S = np.abs(rng.standard_normal((N, K // 32)) * 0.02).astype(np.float16).view(np.uint16)
    W = F.decode_q2(_pack_q2_writer(C), _pack_scales_writer(S), N, K)
    expect = np.array([[_fp16_from_bits(S[n, k // 32]) * (C[n, k] - 2) for k in range(K)] for n in range(N)])
    np.testing.assert_array_equal(W, expect)


def _pack_q3_hi_writer(Hb):
    """Writer for the Q3 high-bit plane: per (tile, row) a 64-bit word whose bit
    32*(w//2) + 8*(w%2) + (j%8) + 16*(j//8) holds weight 16*w + j of the tile row."""
    N, K = Hb.shape
    out = bytearray()
    for ng in range(N // 64):
        for kc in range(K // 64):
            for r in range(64):
                word = 0
                for w in range(4):
                    for j in range(16):
                        if Hb[ng * 64 + r, kc * 64 + 16 * w + j]:
                            word |= 1 << (32 * (w // 2) + 8 * (w % 2) + (j % 8) + 16 * (j // 8))
                out += word.to_bytes(8, "little")
    return np.frombuffer(bytes(out), dtype=np.uint8)


def test_q3_layout_hand_derived():
    # 64 x 128; every lo code 2, every hi bit 0, scales 1.0 -> W = 1*(2-4) = -2
    # except (n=3, k=105): k%64 = 41 = 16*2 + 9 -> bit 32*1 + 0 + 1 + 16 = 49 of the
    # 64-bit word at byte (tile 1)*512 + 3*8 = 536 -> byte 542, bit 1.  c = 2 + 4 = 6 -> W = +2.
    N, K = 64, 128
    lo = np.full(N * K // 4, 0xAA, dtype=np.uint8)
    hi = np.zeros(N * K // 8, dtype=np.uint8)
    hi[542] = 0x02
    scales = np.full(N * K // 32, 0x3C00, dtype=np.uint16)
    W = F.decode_q3(lo, hi, scales, N, K)
    expect = np.full((N, K), -2.0)
    expect[3, 105] = 2.0
    np.testing.assert_array_equal(W, expect)


def test_q3_layout_writer_reader_agree():
    rng = np.random.default_rng(12)
    N, K = 64, 256
    C = rng.integers(0, 8, size=(N, K))
    S = np.abs(rng.standard_normal((N, K // 32)) * 0.02).astype(np.float16).view(np.uint16)
    W = F.decode_q3(_pack_q2_writer(C & 3), _pack_q3_hi_writer(C >> 2), _pack_scales_writer(S), N, K)
    expect = np.array([[_fp16_from_bits(S[n, k // 32]) * (C[n, k] - 4) for k in range(K)] for n in range(N)])
    np.testing.assert_array_equal(W, expect)


def test_bf16_tiled_layout_hand_derived():
    # 64 x 16: element (n=1, k=9) at ((0)*2 + 1)*512 + 1*8 + 1 = 521
    w = np.zeros(64 * 16, dtype=np.uint16)
    w[521] = 0x3F80          # 1.0
    w[0] = 0xC000            # (0, 0) = -2.0
    W = F.decode_bf16_tiled(w, 64, 16)
    expect = np.zeros((64, 16))
    expect[1, 9] = 1.0
    expect[0, 0] = -2.0
    np.testing.assert_array_equal(W, expect)


# Expert slicing of a bank.  Three experts at H = 128, I = 128: per expert W13 is [2I, H] = [256, 128]
# (gate rows 0..127, then up rows 128..255) and W2 is [H, I] = [128, 128].  Per expert that is, in the
# 2-bit code plane, 256*128/4 = 8,192 bytes of W13 and 128*128/4 = 4,096 of W2; in fp16 scales 1,024 and
# 512; in the 3-bit high plane 4,096 and 2,048 bytes; in bf16 32,768 and 16,384 elements.  Expert j starts
# at j times those counts.  Every weight of the bank is 0 except five markers at positions worked out by
# hand from the layout definitions (tile t = (n // 64) * (K // 64) + k // 64 with K = 128, so two tiles per
# 64-row band):
#
#   marker                          W13/W2 (n, k)   tile   code byte in the matrix              bits
#   A  expert 1, gate[5, 7]   = +1  W13 (5, 7)       0     0*1024 +  5*16 +  7//4 =   81        6-7
#   B  expert 1, up[3, 70]    = -1  W13 (131, 70)    5     5*1024 +  3*16 +  6//4 = 5169        4-5
#   C  expert 2, down[100, 33]= +2  W2  (100, 33)    2     2*1024 + 36*16 + 33//4 = 2632        2-3
#   D  expert 2, gate[127,127]= -1  W13 (127, 127)   3     3*1024 + 63*16 + 63//4 = 4095        6-7
#   E  expert 2, up[0, 0]     = +1  W13 (128, 0)     4     4*1024 +  0    +  0    = 4096        0-1
#
# Scales are 1.0 except B's block, 0.5: scale index ((131//64)*(128//128) + (70//32)//4)*256 + 3*4 + 2 = 526,
# and C's block, 2.0: ((100//64)*1 + (33//32)//4)*256 + 36*4 + 1 = 401.
# Q3 high bits (8 bytes per (tile, row); k % 64 = 16w + j -> bit 32(w//2) + 8(w%2) + j%8 + 16(j//8)):
#   B  (131, 70): k%64 = 6 = 16*0 + 6 -> bit 6 of the word at 5*512 + 3*8 = 2584 -> byte 2584, bit 6
#   D  (127, 127): k%64 = 63 = 16*3 + 15 -> bit 32 + 8 + 7 + 16 = 63 of the word at 3*512 + 63*8 = 2040
#                  -> byte 2047, bit 7
# bf16 elements ((n//64)*(K//8) + k//8)*512 + (n%64)*8 + k%8 with K//8 = 16:
#   A (5, 7): 0*512 + 40 + 7 = 47          B (131, 70): (2*16 + 8)*512 + 24 + 6 = 20510
#   C (100, 33): (16 + 4)*512 + 288 + 1 = 10529 (in W2)
#   D (127, 127): (16 + 15)*512 + 504 + 7 = 16383      E (128, 0): (2*16)*512 = 16384

_XM_H, _XM_I = 128, 128
_XM_EXPECT = {   # (expert, matrix, row, col) -> value
    (1, "gate", 5, 7): 1.0, (1, "up", 3, 70): -1.0, (2, "down", 100, 33): 2.0,
    (2, "gate", 127, 127): -1.0, (2, "up", 0, 0): 1.0,
}


def _xm_bank(fmt):
    n13_codes, n2_codes, n13_sc, n2_sc, n13_hi, n2_hi = 8192, 4096, 1024, 512, 4096, 2048
    if fmt == "bf16":
        w13 = np.zeros(3 * 32768, dtype=np.uint16)
        w2 = np.zeros(3 * 16384, dtype=np.uint16)
        w13[1 * 32768 + 47] = 0x3F80             # A +1
        w13[1 * 32768 + 20510] = 0xBF80          # B -1
        w2[2 * 16384 + 10529] = 0x4000           # C +2
        w13[2 * 32768 + 16383] = 0xBF80          # D -1
        w13[2 * 32768 + 16384] = 0x3F80          # E +1
        return {"w13": w13, "w2": w2}
    s13 = np.full(3 * n13_sc, 0x3C00, dtype=np.uint16)
    s2 = np.full(3 * n2_sc, 0x3C00, dtype=np.uint16)
    s13[1 * n13_sc + 526] = 0x3800               # B's block: 0.5
    s2[2 * n2_sc + 401] = 0x4000                 # C's block: 2.0
    if fmt == "q2":                               # code 2 everywhere (weight 0)
        c13 = np.full(3 * n13_codes, 0xAA, dtype=np.uint8)
        c2 = np.full(3 * n2_codes, 0xAA, dtype=np.uint8)
        c13[1 * n13_codes + 81] = 0xEA           # A: bits 6-7 = 3 -> +1
        c13[1 * n13_codes + 5169] = 0x8A         # B: bits 4-5 = 0 -> -2 * 0.5
        c2[2 * n2_codes + 2632] = 0xAE           # C: bits 2-3 = 3 -> +1 * 2.0
        c13[2 * n13_codes + 4095] = 0x6A         # D: bits 6-7 = 1 -> -1
        c13[2 * n13_codes + 4096] = 0xAB         # E: bits 0-1 = 3 -> +1
        return {"w13": c13, "w13_scale": s13, "w2": c2, "w2_scale": s2}
    # q3: lo 0 and hi 1 everywhere (c = 4, weight 0)
    c13 = np.zeros(3 * n13_codes, dtype=np.uint8)
    c2 = np.zeros(3 * n2_codes, dtype=np.uint8)
    h13 = np.full(3 * n13_hi, 0xFF, dtype=np.uint8)
    h2 = np.full(3 * n2_hi, 0xFF, dtype=np.uint8)
    c13[1 * n13_codes + 81] = 0x40               # A: lo 1, hi 1 -> c 5 -> +1
    c13[1 * n13_codes + 5169] = 0x20             # B: lo 2 ...
    h13[1 * n13_hi + 2584] = 0xBF                # ... hi 0 -> c 2 -> -2 * 0.5
    c2[2 * n2_codes + 2632] = 0x04               # C: lo 1, hi 1 -> +1 * 2.0
    c13[2 * n13_codes + 4095] = 0xC0             # D: lo 3 ...
    h13[2 * n13_hi + 2047] = 0x7F                # ... hi 0 -> c 3 -> -1
    c13[2 * n13_codes + 4096] = 0x01             # E: lo 1, hi 1 -> +1
    return {"w13": c13, "w13_hi": h13, "w13_scale": s13, "w2": c2, "w2_hi": h2, "w2_scale": s2}


@pytest.mark.parametrize("fmt", ["q2", "q3", "bf16"])
def test_expert_matrices_slices_the_right_expert_and_projection(fmt):
    bank = _xm_bank(fmt)
    for j in range(3):
        wg, wu, wd = F.expert_matrices(fmt, bank, _XM_H, _XM_I, j)
        assert wg.shape == (_XM_I, _XM_H) and wu.shape == (_XM_I, _XM_H) and wd.shape == (_XM_H, _XM_I)
        for name, m in (("gate", wg), ("up", wu), ("down", wd)):
            expect = np.zeros(m.shape)
            for (e, mat, r, c), v in _XM_EXPECT.items():
                if e == j and mat == name:
                    expect[r, c] = v
            np.testing.assert_array_equal(m, expect, err_msg=f"{fmt} expert {j} {name}")


def test_dequant_exact_for_every_fp16_scale_and_code():
    # 63,488 finite fp16 patterns = the blocks of a 64 x 31,744 matrix; each block's
    # 32 weights cycle through the four codes.  Expected values in exact rationals.
    finite = [b for b in range(1 << 16) if (b & 0x7C00) != 0x7C00]
    assert len(finite) == 63488
    N, K = 64, 31744
    S = np.array(finite, dtype=np.uint16).reshape(N, K // 32)
    C = np.tile(np.arange(4), (N, K // 4))
    codes = np.zeros(N * K // 4, dtype=np.uint8)
    # fast writer: byte of (n, k) per the layout, via index arithmetic on whole arrays
    n = np.arange(N)[:, None]
    k = np.arange(K)[None, :]
    byte = ((n // 64) * (K // 64) + k // 64) * 1024 + (n % 64) * 16 + (k % 64) // 4
    np.bitwise_or.at(codes, byte.ravel(), (C << (2 * (k % 4))).astype(np.uint8).ravel())
    scales = _pack_scales_writer(S)
    W = F.decode_q2(codes, scales, N, K)
    # every (scale, code) pair, checked exactly
    for ni in range(N):
        for b in range(K // 32):
            s = Fraction(_fp16_from_bits(S[ni, b]))
            for c in range(4):
                assert Fraction(float(W[ni, 32 * b + c])) == s * (c - 2)
    # and re-quantisation returns the codes wherever the scale is non-zero
    Sf = np.repeat(np.vectorize(_fp16_from_bits)(S), 32, axis=1)
    nz = Sf != 0
    np.testing.assert_array_equal(np.rint(W[nz] / Sf[nz]) + 2, C[nz])


# ============================================================ conversions

def test_bf16_and_fp16_bits():
    assert F.bf16_to_f64(np.uint16(0x3F80)) == 1.0
    assert F.bf16_to_f64(np.uint16(0xC000)) == -2.0
    assert F.bf16_to_f64(np.uint16(0x0001)) == 2.0 ** -133
    assert F.bf16_to_f64(np.uint16(0x7F7F)) == (2 - 2.0 ** -7) * 2.0 ** 127
    assert F.fp16_to_f64(np.uint16(0x3C00)) == 1.0
    assert F.fp16_to_f64(np.uint16(0x0001)) == 2.0 ** -24
    assert F.fp16_to_f64(np.uint16(0x7BFF)) == 65504.0


def test_f64_to_bf16_round_to_nearest_even():
    cases = {
        1.0: 0x3F80,
        1.0 + 2.0 ** -8: 0x3F80,                    # tie -> even (down)
        1.0 + 3 * 2.0 ** -8: 0x3F82,                # tie -> even (up)
        1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F81,       # just above the tie
        -(1.0 + 2.0 ** -7): 0xBF81,
        2.0 ** -130: 0x0008,                        # bf16 subnormal
        3.4e38: 0x7F80,                             # overflows to +inf
        0.0: 0x0000,
    }
    for v, bits in cases.items():
        assert int(F.f64_to_bf16_bits(np.array([v]))[0]) == bits, v
    rng = np.random.default_rng(3)
    a = rng.standard_normal(5000) * 10.0 ** rng.integers(-40, 38, 5000)
    fast = F.f64_to_bf16_bits(a)
    slow = np.array([F._round_one_to_bf16(float(v)) for v in a], dtype=np.uint16)
    np.testing.assert_array_equal(fast, slow)


# ============================================================ routing

def _bf16(a):
    return synth.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def test_router_logits_against_exact_sums():
    rng = np.random.default_rng(5)
    T, E, H = 3, 7, 40                       # E != H so a transposed operand cannot pass
    xb = _bf16(rng.standard_normal((T, H)))
    wb = _bf16(rng.standard_normal((E, H)) * 0.1)
    bias = rng.standard_normal(E).astype(np.float32)
    got = L.router_logits(xb, wb, bias)
    xv = [[struct.unpack("<f", struct.pack("<I", int(b) << 16))[0] for b in row] for row in xb]
    wv = [[struct.unpack("<f", struct.pack("<I", int(b) << 16))[0] for b in row] for row in wb]
    for t in range(T):
        for e in range(E):
            ref = math.fsum([xv[t][h] * wv[e][h] for h in range(H)] + [float(bias[e])])
            assert abs(got[t, e] - ref) <= 1e-13 * (1 + abs(ref))


def _brute_topk(logits_row, k):
    best, best_set = None, None
    for sub in itertools.combinations(range(len(logits_row)), k):   # lexicographic order
        s = math.fsum(logits_row[list(sub)])
        if best is None or s > best:
            best, best_set = s, sub
    return set(best_set)


def test_topk_matches_brute_force_subsets():
    rng = np.random.default_rng(6)
    for trial in range(200):
        E, k = 8, 3
        l = np.round(rng.standard_normal((1, E)) * 2, 1)        # coarse values -> frequent ties
        got = L.select_topk(l, k)[0]
        assert set(got.tolist()) == _brute_topk(l[0], k)
        # the order is by logit descending, ties by index ascending
        keys = [(-l[0, e], e) for e in got]
        assert keys == sorted(keys)


def test_topk_forced_tie_goes_to_lower_index():
    rng = np.random.default_rng(7)
    H = 64
    w = rng.standard_normal((6, H)) * 0.05
    w[5] = w[2] = np.abs(w[2]) + 0.3                  # rows 2 and 5 identical and large
    x = np.abs(rng.standard_normal((2, H))) + 0.1     # positive x -> rows 2/5 have the top logit
    ids, gates, margin, logits = L.route(_bf16(x), _bf16(w), 1)
    assert (ids[:, 0] == 2).all()
    assert (gates == 1.0).all()
    assert (margin == 0.0).all()


def test_gates():
    rng = np.random.default_rng(8)
    l = rng.standard_normal((50, 16)) * 3
    for k in (1, 4, 16):
        ids = L.select_topk(l, k)
        g = L.renormalised_gates(l, ids)
        assert np.all(np.abs(g.sum(axis=1) - 1.0) <= 1e-15)
        # renormalised softmax == softmax of the selected logits (textbook routine)
        sel = np.take_along_axis(l, ids.astype(np.int64), axis=1)
        np.testing.assert_allclose(g, scipy.special.softmax(sel, axis=1), rtol=1e-14, atol=0)
        if k == 1:
            assert (g == 1.0).all()
        if k == 16:   # all experts: the full softmax, reordered
            full = scipy.special.softmax(l, axis=1)
            np.testing.assert_allclose(g, np.take_along_axis(full, ids.astype(np.int64), axis=1), rtol=1e-14)
    np.testing.assert_allclose(L.softmax(l), scipy.special.softmax(l, axis=1), rtol=1e-14)


def test_margin_hand_case():
    l = np.array([[5.0, 4.0, 3.0, 3.5]])
    assert L.topk_margin(l, 2)[0] == 0.5          # sorted 5, 4 | 3.5, 3
    assert L.topk_margin(l, 1)[0] == 1.0
    assert L.topk_margin(l, 4)[0] == np.inf


# ============================================================ permutation

def test_permute_is_stable_counting_sort():
    rng = np.random.default_rng(9)
    for T, k, E in ((1, 10, 512), (4, 10, 512), (37, 3, 5), (64, 4, 16)):
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        for with_shared in (False, True):
            off, srt, inv = L.permute(ids, E, with_shared)
            group = list(ids.reshape(-1)) + ([E] * T if with_shared else [])
            ref = sorted(range(len(group)), key=lambda r: (group[r], r))     # stable library sort
            np.testing.assert_array_equal(srt, ref)
            counts = np.bincount(group, minlength=E + 1)
            np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(counts)]))
            np.testing.assert_array_equal(inv[srt], np.arange(len(group)))      # inverse map
            assert len(off) == E + 2


# ============================================================ FFN

def test_silu_closed_forms():
    ln3 = math.log(3.0)
    assert L.silu(np.array(0.0)) == 0.0
    assert abs(L.silu(np.array(ln3)) - 0.75 * ln3) <= 4e-16          # sigmoid(ln 3) = 3/4
    assert abs(L.silu(np.array(-ln3)) + 0.25 * ln3) <= 4e-16         # sigmoid(-ln 3) = 1/4
    a = np.random.default_rng(1).standard_normal(1000) * 5
    np.testing.assert_allclose(L.silu(a), a * scipy.special.expit(a), rtol=1e-15, atol=1e-300)
    # saturated tails: SiLU(a) -> 0 as a -> -inf and SiLU(a) = a for large a, with no
    # warning (exp(-a) overflowing to inf is the expected route to the limit)
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("error")
        tails = L.silu(np.array([-1e4, -800.0, 800.0, 1e4]))
    assert tails[0] == 0.0 and tails[1] == 0.0
    assert tails[2] == 800.0 and tails[3] == 1e4


def test_expert_ffn_closed_form():
    # x = v * e_k0; gate column alpha, up column beta, every down weight gamma:
    # a_j = v*alpha = ln 3, b_j = v*beta = 2, h_j = 0.75 ln 3 * 2, y_n = I * gamma * 1.5 ln 3.
    H, I, k0, v = 48, 20, 7, 0.5
    alpha, beta, gamma = 2 * math.log(3.0), 4.0, 0.125
    x = np.zeros((1, H)); x[0, k0] = v
    wg = np.zeros((I, H)); wg[:, k0] = alpha
    wu = np.zeros((I, H)); wu[:, k0] = beta
    wd = np.full((H, I), gamma)
    y = L.expert_ffn(x, wg, wu, wd)
    np.testing.assert_allclose(y, np.full((1, H), I * gamma * 1.5 * math.log(3.0)), rtol=1e-15)
    # swapping the roles of gate and up changes the result: SiLU(2) * ln 3 != SiLU(ln 3) * 2
    assert abs(L.expert_ffn(x, wu, wg, wd)[0, 0] - y[0, 0]) > 0.1


def test_single_expert_layer_equals_dense_swiglu():
    # E = 1, k = 1, no shared expert: the layer is one dense SwiGLU FFN with gate 1.
    rng = np.random.default_rng(10)
    H, I, T = 128, 128, 5
    tens = synth.expert_tensors(99, 0, 0, "q2", H, I)
    wg, wu, wd = F.expert_matrices("q2", tens, H, I)
    xb = _bf16(rng.standard_normal((T, H)))
    wr = _bf16(rng.standard_normal((1, H)))
    out, ids, gates, _ = L.layer_forward(xb, wr, 1, lambda e: (wg, wu, wd))
    x = F.bf16_to_f64(xb)
    ref = np.array([[math.fsum(
        (lambda h: [h[j] * wd[n, j] for j in range(I)])(
            [ (x[t] @ wg[j]) * scipy.special.expit(x[t] @ wg[j]) * (x[t] @ wu[j]) for j in range(I)]))
        for n in range(H)] for t in range(T)])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert (ids == 0).all() and (gates == 1.0).all()


# ============================================================ whole layer

def _tiny_layer(seed=21, E=6, H=128, I=128, fmt="q2"):
    tens = synth.bank(seed, 0, fmt, range(E + 1), H, I)       # expert E is the shared one
    fn = L.bank_expert_fn(fmt, tens, H, I)
    wr = synth.router_weight(seed, 0, E, H, std=0.1)
    return tens, fn, wr


def test_layer_equals_dense_masked_brute_force():
    E, k, H, I, T = 6, 2, 128, 128, 7
    _, fn, wr = _tiny_layer(E=E, H=H, I=I)
    xb = synth.activations(21, 0, T, H)
    bias = np.linspace(-0.5, 0.5, E).astype(np.float32)
    out, ids, gates, _ = L.layer_forward(xb, wr, k, fn, lambda: fn(E), bias=bias)
    x = F.bf16_to_f64(xb)
    wv = F.bf16_to_f64(wr)
    for t in range(T):
        logits = np.array([math.fsum(list(x[t] * wv[e]) + [float(bias[e])]) for e in range(E)])
        sel = sorted(_brute_topk(logits, k))
        g = scipy.special.softmax(logits[sel])
        terms = []
        for e in range(E):                                  # dense over all experts, masked
            ye = L.expert_ffn(x[t:t + 1], *fn(e))[0]
            m = g[sel.index(e)] if e in sel else 0.0
            terms.append(m * ye)
        ref = np.sum(terms, axis=0) + L.expert_ffn(x[t:t + 1], *fn(E))[0]
        np.testing.assert_allclose(out[t], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_layer_invariants():
    E, k, H, I, T = 6, 2, 128, 128, 9
    tens, fn, wr = _tiny_layer(E=E, H=H, I=I)
    xb = synth.activations(22, 0, T, H)
    out, ids, gates, _ = L.layer_forward(xb, wr, k, fn, lambda: fn(E))
    # token permutation permutes the outputs
    perm = np.random.default_rng(2).permutation(T)
    out_p, ids_p, _, _ = L.layer_forward(xb[perm], wr, k, fn, lambda: fn(E))
    np.testing.assert_allclose(out_p, out[perm], rtol=0, atol=1e-14 * np.abs(out).max())
    np.testing.assert_array_equal(ids_p, ids[perm])
    # all codes 2 -> every weight 0 -> output exactly 0
    zero = {kk: (np.full_like(v, 0xAA) if kk in ("w13", "w2") else v) for kk, v in tens.items()}
    zfn = L.bank_expert_fn("q2", zero, H, I)
    out_z, _, _, _ = L.layer_forward(xb, wr, k, zfn, lambda: zfn(E))
    assert (out_z == 0.0).all()
    # doubling every down-projection scale (fp16 exponent + 1) doubles the output exactly
    dbl = dict(tens)
    s = tens["w2_scale"].astype(np.uint32)
    assert ((s & 0x7C00) < 0x7800).all()            # no scale near the fp16 top: doubling is exact
    normal = (s & 0x7C00) != 0
    # normal: exponent + 1; subnormal: significand * 2 (which carries into the exponent exactly)
    dbl["w2_scale"] = np.where(normal, s + 0x0400, (s & 0x8000) | ((s & 0x3FF) << 1)).astype(np.uint16)
    dfn = L.bank_expert_fn("q2", dbl, H, I)
    out_d, _, _, _ = L.layer_forward(xb, wr, k, dfn, lambda: dfn(E))
    np.testing.assert_array_equal(out_d, 2.0 * out)


def test_combine_matches_layer_through_permutation():
    E, k, H, I, T = 6, 2, 128, 128, 5
    _, fn, wr = _tiny_layer(E=E, H=H, I=I)
    xb = synth.activations(23, 0, T, H)
    resid = synth.activations(24, 0, T, H)
    out, ids, gates, _ = L.layer_forward(xb, wr, k, fn, lambda: fn(E), residual_bits=resid)
    off, srt, inv = L.permute(ids, E, True)
    x = F.bf16_to_f64(xb)
    y_sorted = np.zeros((len(srt), H))
    for p, r in enumerate(srt):
        t = r // k if r < T * k else r - T * k
        e = ids.reshape(-1)[r] if r < T * k else E
        y_sorted[p] = L.expert_ffn(x[t:t + 1], *fn(int(e)))[0]
    np.testing.assert_allclose(L.combine(y_sorted, inv, gates, True, resid), out, rtol=1e-13, atol=1e-13)


def test_cached_layer_hits_plus_misses_is_full_layer():
    E, k, H, I, T = 6, 3, 128, 128, 8
    _, fn, wr = _tiny_layer(E=E, H=H, I=I)
    xb = synth.activations(25, 0, T, H)
    slot_row = np.array([3, -1, 0, -1, 1, -1])         # experts 0, 2, 4 resident in slots 3, 0, 1
    expert_of_slot = {3: 0, 0: 2, 1: 4}
    out_h, ids, gates, misses, _ = L.cached_layer_forward(
        xb, wr, k, slot_row, lambda s: fn(expert_of_slot[s]), lambda: fn(E))
    ref_misses = sorted(t * k + i for t in range(T) for i in range(k) if slot_row[ids[t, i]] < 0)
    np.testing.assert_array_equal(misses, ref_misses)
    full, ids_f, gates_f, _ = L.layer_forward(xb, wr, k, fn, lambda: fn(E))
    x = F.bf16_to_f64(xb)
    miss_sum = np.zeros_like(full)
    for r in ref_misses:
        t, i = divmod(r, k)
        miss_sum[t] += gates[t, i] * L.expert_ffn(x[t:t + 1], *fn(int(ids[t, i])))[0]
    np.testing.assert_allclose(out_h + miss_sum, full, rtol=1e-13, atol=1e-13 * np.abs(full).max())


def test_residual_bf16_hand_cases():
    one = np.array([[0x3F80]], dtype=np.uint16)
    assert int(L.residual_bf16(one, np.array([[2.0 ** -8]]))[0, 0]) == 0x3F80          # tie -> even
    assert int(L.residual_bf16(one, np.array([[2.0 ** -8 + 2.0 ** -20]]))[0, 0]) == 0x3F81
    assert int(L.residual_bf16(one, np.array([[-3.0]]))[0, 0]) == 0xC000                 # 1 - 3 = -2


def test_rms_norm_closed_forms():
    # a constant row c normalises to sign(c) * 1/sqrt(1 + eps/c^2): exactly 1.0 in bf16 for |c| >= 1
    x = np.full((2, 64), 0x4040, dtype=np.uint16)          # 3.0
    x[1] = 0xC040                                           # -3.0
    xn = L.rms_norm_bf16(x)
    assert (xn[0] == 0x3F80).all() and (xn[1] == 0xBF80).all()
    # scaling a row by a power of two leaves its normalisation unchanged (eps aside: rows of O(1))
    rng = np.random.default_rng(4)
    xb = _bf16(rng.standard_normal((5, 256)))
    x2 = _bf16(F.bf16_to_f64(xb) * 4.0)
    np.testing.assert_array_equal(L.rms_norm_bf16(xb, eps=0.0), L.rms_norm_bf16(x2, eps=0.0))
    # unit RMS up to bf16 rounding
    v = F.bf16_to_f64(L.rms_norm_bf16(xb))
    assert np.all(np.abs(np.sqrt((v * v).mean(axis=1)) - 1.0) < 4e-3)
    # one stack step: residual of the normalised layer input
    step, xn2 = L.stack_step(xb, lambda z: np.ones((5, 256)))
    np.testing.assert_array_equal(step, L.residual_bf16(xb, np.ones((5, 256))))


def test_rel_max_err():
    assert L.rel_max_err([1.0, 1.0], [1.0, -1.0]) == 2.0
    assert L.rel_max_err([3.0, 4.0], [3.0, 4.0]) == 0.0


# ============================================================ the pages' structural numbers

def test_model_shape_constants_from_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "model_shape.json")))
    c = synth.CONFIGS
    for w in ("decode", "prefill", "stack", "cache"):
        s = c[w].shape
        assert s.n_experts == g["experts_per_layer"]["value"]
        assert s.top_k == g["routed_per_token"]["value"]
        assert int(s.shared) == g["shared_per_token"]["value"]
        assert s.hidden == g["hidden"]["value"]
    assert c["stack"].layers == g["layers"]["value"] == c["cache"].layers
    assert g["layers"]["value"] * g["experts_per_layer"]["value"] == g["experts_total"]["value"]
    assert g["layers"]["value"] * g["routed_per_token"]["value"] == g["expert_blocks_per_token"]["value"]
    assert c["prefill"].tokens[0] == g["prefill_chunk_max_tokens"]["value"]
    assert c["decode"].tokens[1] == 1 + g["mtp_draft_max_tokens"]["value"]
    # bytes of one 2-bit expert from the format definition: 3*H*I weights at 2 bits
    # plus one fp16 scale per 32 weights; about 700 of them per extra GiB of VRAM.
    H, I = c["decode"].shape.hidden, c["decode"].shape.inter
    q2_bytes = 3 * H * I * 2 // 8 + 3 * H * I // 32 * 2
    assert q2_bytes == 1_536_000 == sum(synth.expert_nbytes("q2", H, I).values())
    per_gib = 2 ** 30 / q2_bytes
    assert abs(per_gib - g["experts_per_extra_gb"]["value"]) / 700 < 0.02


# ============================================================ planted mistakes

def _swap_gate_up(orig):
    def f(x, wg, wu, wd):
        return orig(x, wu, wg, wd)
    return f


def _mutations():
    import oracle.layer as Lm
    import oracle.formats as Fm
    orig_codes = Fm.q2_codes
    orig_topk = Lm.select_topk
    orig_ffn = Lm.expert_ffn
    orig_perm = Lm.permute
    orig_gates = Lm.renormalised_gates
    orig_silu = Lm.silu

    def codes_msb_first(codes, N, K):
        c = orig_codes(codes, N, K)
        return ((c & 1) << 1) | (c >> 1)

    def topk_high_index(logits, k):
        E = logits.shape[1]
        return (E - 1 - orig_topk(logits[:, ::-1], k)).astype(np.int32)

    def gates_not_renormalised(logits, ids):
        return np.take_along_axis(Lm.softmax(logits), ids.astype(np.int64), axis=1)

    def permute_reverse_within_group(ids, E, with_shared):
        off, srt, inv = orig_perm(ids, E, with_shared)
        srt = srt.copy()
        for g in range(E + 1):
            srt[off[g]:off[g + 1]] = srt[off[g]:off[g + 1]][::-1]
        inv = np.empty_like(srt); inv[srt] = np.arange(len(srt))
        return off, srt, inv

    def silu_sign_slip(a):
        return a / (1.0 + np.exp(a))

    def ffn_dropped_up(x, wg, wu, wd):
        return Lm.silu(x @ wg.T) @ wd.T

    orig_matrices = Fm.expert_matrices

    def matrices_gate_up_swapped(fmt, tensors, H, I, j=0):
        wg, wu, wd = orig_matrices(fmt, tensors, H, I, j)
        return wu, wg, wd

    def matrices_always_expert_0(fmt, tensors, H, I, j=0):
        return orig_matrices(fmt, tensors, H, I, 0)

    def matrices_scale_stride_off(fmt, tensors, H, I, j=0):
        # expert j's fp16 scales read from the previous expert's block (a per-expert offset slip)
        if fmt == "bf16" or j == 0:
            return orig_matrices(fmt, tensors, H, I, j)
        t = dict(tensors)
        n13, n2 = 2 * I * H // 32, H * I // 32
        t["w13_scale"] = np.concatenate([tensors["w13_scale"][n13:], tensors["w13_scale"][:n13]])
        t["w2_scale"] = np.concatenate([tensors["w2_scale"][n2:], tensors["w2_scale"][:n2]])
        return orig_matrices(fmt, t, H, I, j)

    return [
        (Fm, "q2_codes", codes_msb_first, [test_q2_layout_hand_derived, test_q2_layout_writer_reader_agree]),
        (Lm, "select_topk", topk_high_index, [test_topk_forced_tie_goes_to_lower_index]),
        (Lm, "renormalised_gates", gates_not_renormalised, [test_gates]),
        (Lm, "permute", permute_reverse_within_group, [test_permute_is_stable_counting_sort]),
        (Lm, "silu", silu_sign_slip, [test_silu_closed_forms, test_expert_ffn_closed_form]),
        (Lm, "expert_ffn", _swap_gate_up(orig_ffn), [test_expert_ffn_closed_form]),
        (Lm, "expert_ffn", ffn_dropped_up, [test_single_expert_layer_equals_dense_swiglu]),
        (Fm, "expert_matrices", matrices_gate_up_swapped, [_xm_pin_all_formats]),
        (Fm, "expert_matrices", matrices_always_expert_0, [_xm_pin_all_formats]),
        (Fm, "expert_matrices", matrices_scale_stride_off, [_xm_pin_all_formats]),
    ]


def _xm_pin_all_formats():
    for fmt in ("q2", "q3", "bf16"):
        test_expert_matrices_slices_the_right_expert_and_projection(fmt)


@pytest.mark.parametrize("case", range(10))
def test_planted_mistakes_are_caught(case, monkeypatch):
    mod, name, bad, pins = _mutations()[case]
    monkeypatch.setattr(mod, name, bad)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()

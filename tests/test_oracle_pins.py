"""Pins of the CPU oracle against facts outside itself (no GPU).

Each test checks the oracle against a closed form, a textbook value, an invariant,
a value printed on the pages (tests/golden/), a library routine, or brute force,
so that a dropped term, a wrong sign or index, or a transposed operand fails.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import integrate, special, stats

from oracle import cache as C
from oracle import codebook as cb
from oracle import decode as D
from oracle import encode as E
from oracle import layout as L
from oracle import rotation as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class Lay:
    def __init__(self, d, hq, hkv, k_kind, k_bits, v_kind, v_bits):
        self.head_dim, self.n_q_heads, self.n_kv_heads = d, hq, hkv
        self.k_kind, self.k_bits, self.v_kind, self.v_bits = k_kind, k_bits, v_kind, v_bits


def _rand_state(lay, seed):
    rng = np.random.default_rng(seed)
    d = lay.head_dim
    sk = np.where(rng.integers(0, 2, d) == 1, -1, 1).astype(np.int8)
    sv = np.where(rng.integers(0, 2, d) == 1, -1, 1).astype(np.int8)
    S = rng.standard_normal((d, d)).astype(np.float32)
    return C.make_state(lay, sk, sv, S)


# --------------------------------------------------------------------------- rotation
def test_hadamard_textbook_entries():
    assert np.array_equal(R.sylvester_hadamard(2), [[1, 1], [1, -1]])
    assert np.array_equal(R.sylvester_hadamard(4), [[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])


@pytest.mark.parametrize("d", [1, 2, 8, 64, 128, 256, 512])
def test_hadamard_orthogonality(d):
    H = R.sylvester_hadamard(d)
    assert np.array_equal(H @ H.T, d * np.eye(d))
    assert np.array_equal(H, H.T)


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_rotation_preserves_norm(d):
    rng = np.random.default_rng(d)
    s = np.where(rng.integers(0, 2, d) == 1, -1, 1)
    P = R.rotation_matrix(s)
    assert np.max(np.abs(P.T @ P - np.eye(d))) < 1e-12
    x = rng.standard_normal((16, d))
    assert np.max(np.abs(np.linalg.norm(x @ P.T, axis=1) - np.linalg.norm(x, axis=1))) < 1e-12
    # the sign flip comes before the transform: column j of Pi is s_j H[:, j] / sqrt(d)
    H = R.sylvester_hadamard(d)
    j = int(rng.integers(d))
    assert np.allclose(P[:, j], s[j] * H[:, j] / math.sqrt(d), atol=0, rtol=0)


def test_splitmix64_published_vector():
    g = R.SplitMix64(1234567)
    assert [g.next() for _ in range(5)] == [6457827717110365317, 3203168211198807973, 9817491932198370423,
                                            4593380528125082431, 16408922859458223821]


def test_box_muller_state_is_standard_normal():
    words, S = R.reference_rotation_state(256, 42)
    x = S.astype(np.float64).ravel()
    assert abs(x.mean()) < 4.5 / math.sqrt(x.size)
    assert abs(x.var() - 1.0) < 4.5 * math.sqrt(2.0 / x.size)
    assert stats.kstest(x, "norm").pvalue > 1e-4
    s = R.mask_to_signs(words, 256)
    assert abs(int(np.sum(s))) < 4.5 * 16


# --------------------------------------------------------------------------- codebook
@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_coordinate_density_moments(d):
    # a coordinate of a uniform unit vector: total mass 1, mean 0, E[X^2] = 1/d
    m0 = integrate.quad(lambda x: cb.coord_pdf(x, d), -1, 1, points=[0], limit=200)[0]
    m2 = integrate.quad(lambda x: x * x * cb.coord_pdf(x, d), -1, 1, points=[0], limit=200)[0]
    assert abs(m0 - 1) < 1e-10 and abs(m2 - 1.0 / d) < 1e-12
    assert abs(cb.coord_cdf(0.0, d) - 0.5) < 1e-15


def test_coordinate_density_matches_sphere_samples():
    d = 64
    rng = np.random.default_rng(0)
    g = rng.standard_normal((20000, d))
    x = (g / np.linalg.norm(g, axis=1, keepdims=True))[:, 0]
    assert stats.kstest(x, lambda t: cb.coord_cdf(t, d)).pvalue > 1e-4


@pytest.mark.parametrize("d,expect", [(64, 0.1001259), (128, 0.0706616), (256, 0.0499165)])
def test_one_bit_closed_form(d, expect):
    # 1-bit Lloyd-Max: c = E|X| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)); per-vector MSE 1 - d c^2
    c, t = cb.lloyd_max(d, 1)
    closed = math.exp(special.gammaln(d / 2) - special.gammaln((d + 1) / 2)) / math.sqrt(math.pi)
    assert abs(c[1] - closed) < 1e-13 and abs(c[0] + closed) < 1e-13 and t[0] == 0.0
    assert abs(closed - expect) < 5e-8
    assert abs(d * cb.distortion(c, d) - (1 - d * closed * closed)) < 1e-12


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lloyd_max_conditions_by_independent_quadrature(d, bits):
    c, t = cb.lloyd_max(d, bits)
    assert np.all(np.diff(c) > 0)
    assert np.max(np.abs(c + c[::-1])) < 1e-15
    assert np.array_equal(t, 0.5 * (c[:-1] + c[1:]))
    edges = np.concatenate(([-1.0], t, [1.0]))
    for i in range(len(c)):
        m0 = integrate.quad(lambda x: cb.coord_pdf(x, d), edges[i], edges[i + 1], limit=200, epsabs=1e-15)[0]
        m1 = integrate.quad(lambda x: x * cb.coord_pdf(x, d), edges[i], edges[i + 1], limit=200, epsabs=1e-15)[0]
        assert abs(m1 / m0 - c[i]) < 1e-10 * max(1.0, abs(c[i]) * math.sqrt(d))


def test_lloyd_max_is_a_local_minimum():
    d, bits = 128, 3
    c, _ = cb.lloyd_max(d, bits)

    def mse(cc):
        t = 0.5 * (cc[:-1] + cc[1:])
        e = np.concatenate(([-1.0], t, [1.0]))
        return sum(integrate.quad(lambda x: (x - cc[i]) ** 2 * cb.coord_pdf(x, d), e[i], e[i + 1], limit=200)[0]
                   for i in range(len(cc)))

    base = mse(c)
    assert abs(base - cb.distortion(c, d)) < 1e-12
    for i in range(len(c)):
        for eps in (1e-3, -1e-3):
            cc = c.copy()
            cc[i] += eps / math.sqrt(d)
            assert mse(cc) > base


# Gaussian Lloyd-Max quantiser, J. Max (1960), positive output levels and MSE:
MAX1960 = {2: ([0.4528, 1.510], 0.1175), 3: ([0.2451, 0.7560, 1.344, 2.152], 0.03454),
           4: ([0.1284, 0.3881, 0.6568, 0.9423, 1.256, 1.618, 2.069, 2.733], 0.009497)}


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_large_d_limit_is_gaussian_lloyd_max(bits):
    d = 512
    c, _ = cb.lloyd_max(d, bits)
    levels, mse = MAX1960[bits]
    got = c[len(c) // 2:] * math.sqrt(d)
    assert np.max(np.abs(got - levels) / levels) < 0.01
    assert abs(d * cb.distortion(c, d) - mse) / mse < 0.01


@pytest.mark.parametrize("d", [64, 128])
def test_distortion_decreases_with_bits_and_matches_monte_carlo(d):
    rng = np.random.default_rng(d)
    g = rng.standard_normal((4000, d))
    u = g / np.linalg.norm(g, axis=1, keepdims=True)
    prev = np.inf
    for bits in (1, 2, 3, 4):
        c, t = cb.lloyd_max(d, bits)
        D0 = cb.distortion(c, d)
        assert D0 < prev
        prev = D0
        idx = np.searchsorted(t, u, side="left")   # independent of the oracle's counting rule
        err = np.sum((u - c[idx]) ** 2, axis=1)     # per-vector squared error
        se = err.std() / math.sqrt(len(err))
        assert abs(err.mean() - d * D0) < 4.0 * se


# --------------------------------------------------------------------------- packing
@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_pack_round_trip(bits, d):
    rng = np.random.default_rng(bits * 1000 + d)
    x = rng.integers(0, 1 << bits, size=(5, d))
    w = L.pack_codes(x, bits)
    assert w.shape == (5, L.words_for(d, bits)) and w.dtype == np.uint32
    assert np.array_equal(L.unpack_codes(w, bits, d), x)
    top = np.full((1, d), (1 << bits) - 1)
    assert np.array_equal(L.unpack_codes(L.pack_codes(top, bits), bits, d), top)
    s = rng.integers(0, 2, size=(3, d)).astype(bool)
    assert np.array_equal(L.unpack_signs(L.pack_signs(s), d), s)


def test_pack_bit_positions_by_hand():
    # 3-bit: ten codes per word, code j at bits 3j; bits 30..31 stay zero
    codes = np.array([[1, 2, 3, 4, 5, 6, 7, 0, 1, 2, 7]])
    w = L.pack_codes(np.pad(codes, ((0, 0), (0, 53))), 3)
    assert int(w[0, 0]) == 0b00_010_001_000_111_110_101_100_011_010_001
    assert int(w[0, 1]) == 7
    # 2-bit: four per byte, LSB first
    w2 = L.pack_codes(np.array([[3, 0, 1, 2] + [0] * 60]), 2)
    assert int(w2[0, 0]) == 0b10_01_00_11
    # 8-bit: byte j of the little-endian row
    w8 = L.pack_codes(np.array([[0x11, 0x22, 0x33, 0x44] + [0] * 60]), 8)
    assert int(w8[0, 0]) == 0x44332211
    # signs: bit j%32 of word j/32
    sg = np.zeros((1, 64), dtype=bool)
    sg[0, [0, 31, 33]] = True
    assert list(L.pack_signs(sg)[0]) == [0x80000001, 0x2]


def test_compression_ratios_against_printed_values():
    g = json.load(open(os.path.join(GOLDEN, "compression_ratios.json")))
    # the default vllm-metal pair (q8_0 K / q3_0 V) on head_dim 128 is our affine-8 K +
    # rotated 3-bit LM V layout; its printed ratio must come out of the byte accounting
    row = g["ratios_vs_fp16"]["rows"][0]
    assert (row["k_quant"], row["v_quant"]) == ("q8_0", "q3_0")
    ratio = L.compression_ratio(128, "affine8", 8, "lm_rot", 3)
    assert round(ratio, 2) == row["ratio"]
    assert sum(L.bytes_per_token_head(128, "affine8", 8, "lm_rot", 3).values()) == 200
    # 3-bit keys (+ QJL) and 2-bit values sit in the benchmark page's 4.5x-5x band
    band = g["memory_band"]
    for d in (64, 128):
        r = L.compression_ratio(d, "lm_qjl", 3, "group_sym", 2)
        assert band["lo"] - 0.3 <= r <= band["hi"]
    assert L.compression_ratio(128, "lm_qjl", 3, "group_sym", 2) == 512 / 112
    assert sum(L.bytes_per_token_head(64, "lm_qjl", 3, "group_sym", 2).values()) == 60


def test_narrow_affine_key_ratios_against_printed_values():
    """The guide's other printed rows: q5_0 / q4_0 / uint2 keys with q3_0 values come out of
    the layout's byte accounting to the printed precision (3.37x, 3.76x, 4.92x).  The
    int2 / q2_0 row (printed 5.82x) is 512 / 88 bytes; this layout stores 2-bit value codes
    sixteen to a word (84 bytes, 6.10x) -- the printed figure equals 2-bit codes fifteen to a
    word, the 30-bit payload of the ten-to-a-word 3-bit packing (recorded as a reading)."""
    g = json.load(open(os.path.join(GOLDEN, "compression_ratios.json")))
    rows = {(r["k_quant"], r["v_quant"]): r["ratio"] for r in g["ratios_vs_fp16"]["rows"]}
    kbits = {"q8_0": 8, "q5_0": 5, "q4_0": 4, "uint2": 2, "int2": 2}
    vbits = {"q3_0": 3, "q2_0": 2}
    for (kq, vq), printed in rows.items():
        ours = L.compression_ratio(128, "affine8", kbits[kq], "lm_rot", vbits[vq])
        if (kq, vq) == ("int2", "q2_0"):
            assert round(ours, 2) == 6.10
            assert round(512 / (48 + 4 * -(-128 // 15) + 4), 2) == printed
        else:
            assert round(ours, 2) == printed, (kq, vq, ours, printed)
    assert sum(L.bytes_per_token_head(128, "affine8", 5, "lm_rot", 3).values()) == 152


# --------------------------------------------------------------------------- QJL estimator
def test_qjl_sign_identity_and_unbiased_score():
    """E_S[sign(<s,r>) <s,q>] = sqrt(2/pi) <q,r>/|r| makes the full score unbiased."""
    d = 64
    lay = Lay(d, 1, 1, "lm_qjl", 3, "group_sym", 2)
    rng = np.random.default_rng(7)
    k = rng.standard_normal(d)
    q = 0.8 * k + 0.6 * rng.standard_normal(d)      # correlated with k, so the shrinkage is visible
    truth = float(q @ k) / math.sqrt(d)
    full, lm_only = [], []
    c32, t32 = cb.codebook_f32(d, 3)
    M = 4096
    for m in range(M):
        s = np.where(rng.integers(0, 2, d) == 1, -1, 1).astype(np.int8)
        S = rng.standard_normal((d, d)).astype(np.float32)
        st = {"signs_k": s, "S": S, "cb_k": (c32, t32)}
        e = E.encode_k_lm_qjl(k[None], s, S, c32, t32)
        kd = {"idx": e["idx"], "sigma": np.where(e["qjl"], 1.0, -1.0),
              "n": np.linalg.norm(k)[None], "gamma": np.linalg.norm(e["y"] - c32[e["idx"]], axis=1)}
        full.append(D._scores_compressed(lay, q, kd, st)[0])
        kd0 = dict(kd, gamma=np.zeros(1))
        lm_only.append(D._scores_compressed(lay, q, kd0, st)[0])
    full, lm_only = np.array(full), np.array(lm_only)
    se = full.std() / math.sqrt(M)
    assert abs(full.mean() - truth) < 4.5 * se
    # the codebook-only estimate is shrunk toward zero (biased); QJL removes that
    se0 = lm_only.std() / math.sqrt(M)
    assert truth - lm_only.mean() > 4.5 * max(se0, 1e-12)
    # the shrink factor is E[<y, c[idx]>] = 1 - d * distortion for a Lloyd-Max codebook
    shrink = 1.0 - d * cb.distortion(cb.lloyd_max(d, 3)[0], d)
    assert abs(lm_only.mean() - shrink * truth) < 4.5 * se0 + 1e-3 * truth


@pytest.mark.parametrize("s_dtype", ["float64", "float16"])
@pytest.mark.parametrize("bits", [2, 3])
def test_qjl_unbiased_through_the_stored_planes(bits, s_dtype):
    """The whole LM+QJL chain as it is stored -- encode, pack into the k_codes / k_signs /
    k_aux planes, read back the fp16 n and gamma and the sign bits, score -- is an unbiased
    estimate of <q, k>/sqrt(d) over independent (Pi, S) draws (vLLM guide section 2, steps
    2-3: the residual's sign sketch makes the expected inner-product estimate equal to the
    true one).  A norm, residual norm or sign stored wrongly (gamma^2, the residual's norm
    before the codebook subtraction, an inverted bit) biases the mean by several standard
    errors.  With S rounded to fp16 the estimate stays unbiased: only S's distribution
    enters the expectation, and every rounded row is still a symmetric random direction."""
    d = 64
    lay = Lay(d, 1, 1, "lm_qjl", bits, "group_sym", 2)
    rng = np.random.default_rng(100 + bits)
    k = rng.standard_normal(d)
    q = 0.8 * k + 0.6 * rng.standard_normal(d)
    truth = float(q @ k) / math.sqrt(d)
    c32, t32 = cb.codebook_f32(d, bits)
    M = 4096
    got, lm_only = np.empty(M), np.empty(M)
    for m in range(M):
        s = np.where(rng.integers(0, 2, d) == 1, -1, 1).astype(np.int8)
        S = rng.standard_normal((d, d)).astype(s_dtype)
        st = {"signs_k": s, "S": S, "cb_k": (c32, t32)}
        planes = C.encode_k(lay, k[None], st)
        kd = C.read_k(lay, {n: planes[n] for n in ("k_codes", "k_signs", "k_aux")}, st)
        got[m] = D._scores_compressed(lay, q, kd, st)[0]
        lm_only[m] = D._scores_compressed(lay, q, dict(kd, gamma=np.zeros(1)), st)[0]
    se = got.std() / math.sqrt(M)
    assert abs(got.mean() - truth) < 4.5 * se, (got.mean(), truth, se)
    # the correction is not vacuous: without it the same stored codes are biased
    assert truth - lm_only.mean() > 8 * se


def test_mse_only_keys_score_is_the_shrunk_inner_product():
    """MSE-only keys (no QJL residual): over independent rotations the score of the whole
    oracle chain (encode, pack, read back, score) averages (1 - d D) <q, k>/sqrt(d), D the
    per-coordinate distortion of the Lloyd-Max codebook: E[<y, c[idx]>] = 1 - d D for a
    unit vector, and the rotation makes the error isotropic."""
    d = 64
    lay = Lay(d, 1, 1, "lm_mse", 3, "group_sym", 2)
    rng = np.random.default_rng(11)
    k = rng.standard_normal(d)
    q = 0.8 * k + 0.6 * rng.standard_normal(d)
    truth = float(q @ k) / math.sqrt(d)
    c32, t32 = cb.codebook_f32(d, 3)
    M = 4096
    got = []
    for m in range(M):
        s = np.where(rng.integers(0, 2, d) == 1, -1, 1).astype(np.int8)
        st = {"signs_k": s, "cb_k": (c32, t32)}
        planes = C.encode_k(lay, k[None], st)
        kd = C.read_k(lay, {"k_codes": planes["k_codes"], "k_aux": planes["k_aux"]}, st)
        got.append(D._scores_compressed(lay, q, kd, st)[0])
    got = np.array(got)
    se = got.std() / math.sqrt(M)
    shrink = 1.0 - d * cb.distortion(cb.lloyd_max(d, 3)[0], d)
    assert truth - got.mean() > 4.5 * se                       # biased toward zero
    assert abs(got.mean() - shrink * truth) < 4.5 * se + 1e-3 * truth
    # and the decoded key is n Pi^T c[idx]: rotating it back gives n c[idx] exactly
    khat = D.reconstruct_k(lay, kd, st)[0]
    y = R.rotation_matrix(s) @ khat
    assert np.max(np.abs(y - kd["n"][0] * c32[kd["idx"][0]])) < 1e-12


# --------------------------------------------------------------------------- encoders: special cases
def test_group_sym_grid_and_ties_by_hand():
    # 2-bit, amax 0.375 -> Delta = 0.25 exactly; levels Delta*(idx-1.5) reconstruct exactly
    v = np.zeros(32)
    v[:4] = [-0.375, -0.125, 0.125, 0.375]
    v[4:8] = [0.25, -0.25, 0.0, 0.0625]        # ties: 0.25/0.25+1.5 = 2.5 -> 2, -1+1.5=0.5 -> 0, 1.5 -> 2
    e = E.encode_v_group_sym(v[None], 2)
    assert float(e["scale16"][0, 0]) == 0.25
    assert list(e["idx"][0, :8]) == [0, 1, 2, 3, 2, 0, 2, 2]
    # exact ties are decided by round-half-to-even and compared, never excluded
    assert not e["near_idx"][0, :8].any()
    # an inexact value 2^-24 above a tie is within 1e-6 of the boundary: excluded
    v2 = v.copy()
    v2[8] = 0.25 + 2.0 ** -24
    e2 = E.encode_v_group_sym(v2[None], 2)
    assert e2["near_idx"][0, 8] and e2["idx"][0, 8] == 3 and not e2["near_idx"][0, 4]
    vhat = 0.25 * (e["idx"][0, :4] - 1.5)
    assert np.array_equal(vhat, v[:4])
    z = E.encode_v_group_sym(np.zeros((1, 32)), 4)
    assert float(z["scale16"][0, 0]) == 0.0 and np.all(z["idx"] == 8)


def test_affine8_grid_by_hand():
    k = np.arange(32) * 8.0 / 16.0            # 0 .. 15.5 step 0.5 -> a = 15.5/255 (fp16), m = 0
    e = E.encode_k_affine(k[None])
    a = float(e["a16"][0, 0])
    assert a == float(np.float16(15.5 / 255))
    assert e["q"][0, 0] == 0 and e["q"][0, -1] == 255
    k2 = np.full(32, 3.0)
    e2 = E.encode_k_affine(k2[None])
    assert float(e2["a16"][0, 0]) == 0 and np.all(e2["q"] == 0)
    # values on the grid m + a*q reconstruct exactly
    k3 = np.float16(-1.0) + np.float16(2.0 ** -4) * np.arange(32).astype(np.float64)
    k3[-1] = -1.0 + 255 * 2.0 ** -4
    e3 = E.encode_k_affine(k3[None])
    assert float(e3["a16"][0, 0]) == 2.0 ** -4
    assert np.array_equal(-1.0 + 2.0 ** -4 * e3["q"][0], k3)


@pytest.mark.parametrize("bits", [2, 4, 5])
def test_affine_keys_narrow_widths_by_hand(bits):
    """q5_0 / q4_0 / 2-bit affine keys (vllm-metal guide, compression-ratio table): the block
    min goes to code 0 and the max to 2^b - 1, values on the grid m + a q reconstruct exactly,
    exact half-way points go to the even code, a flat block has a = 0 and codes 0, and the
    5-bit row packs into its two planes at the documented bit positions."""
    top = (1 << bits) - 1
    a, m = 2.0 ** -4, -0.5
    q = np.arange(32) % (top + 1)
    k = m + a * q.astype(np.float64)
    k[0], k[1] = m, m + a * top
    e = E.encode_k_affine(k[None], bits)
    assert float(e["a16"][0, 0]) == a and float(e["m16"][0, 0]) == m
    assert e["q"][0, 0] == 0 and e["q"][0, 1] == top
    assert np.array_equal(m + a * e["q"][0], k) and not e["near_idx"].any()
    w = k.copy()
    w[2:2 + min(top, 30)] = m + a * (np.arange(min(top, 30)) + 0.5)
    e2 = E.encode_k_affine(w[None], bits)
    lo = np.arange(min(top, 30))
    assert np.array_equal(e2["q"][0, 2:2 + len(lo)], np.where(lo % 2 == 0, lo, lo + 1))
    e3 = E.encode_k_affine(np.full((1, 32), 0.7), bits)
    assert float(e3["a16"][0, 0]) == 0 and np.all(e3["q"] == 0)
    if bits == 5:
        codes = np.zeros((1, 64), dtype=np.int64)
        codes[0, 0], codes[0, 9], codes[0, 40], codes[0, 63] = 31, 17, 16, 5
        w5 = L.pack_codes(codes, 5)
        assert w5.shape == (1, 10)                      # 8 nibble words + 2 fifth-bit words
        assert int(w5[0, 0]) == 0xF and int(w5[0, 1]) == 0x10 and int(w5[0, 5]) == 0x0
        assert int(w5[0, 7]) == 0x50000000
        assert int(w5[0, 8]) == (1 << 0) | (1 << 9) and int(w5[0, 9]) == 1 << 8
        assert np.array_equal(L.unpack_codes(w5, 5, 64), codes)


@pytest.mark.parametrize("bits", [2, 4])
def test_group_minmax_values_grid_and_ties_by_hand(bits):
    """Min/max values (benchmark page): min -> code 0, max -> code L-1, values on the grid
    m + a k reconstruct exactly, a value exactly half-way goes to the even code, a flat
    group has a = 0 and codes 0."""
    top = (1 << bits) - 1
    a = 2.0 ** -3
    m = -0.75
    k = np.arange(32) % (top + 1)
    v = m + a * k.astype(np.float64)
    v[0], v[1] = m, m + a * top                  # the group's min and max
    e = E.encode_v_group_asym(v[None], bits)
    assert float(e["a16"][0, 0]) == a and float(e["m16"][0, 0]) == m
    assert e["idx"][0, 0] == 0 and e["idx"][0, 1] == top
    assert np.array_equal(m + a * e["idx"][0], v)
    assert not e["near_idx"].any()
    # exact half-way points: ties to the even code
    w = v.copy()
    w[2:2 + top] = m + a * (np.arange(top) + 0.5)
    e2 = E.encode_v_group_asym(w[None], bits)
    half = e2["idx"][0, 2:2 + top]
    lo = np.arange(top)
    assert np.array_equal(half, np.where(lo % 2 == 0, lo, lo + 1))
    assert not e2["near_idx"].any()
    e3 = E.encode_v_group_asym(np.full((1, 32), 0.3), bits)
    assert float(e3["a16"][0, 0]) == 0 and np.all(e3["idx"] == 0)
    # reconstruction error of N(0,1) groups stays within half a step plus the fp16 rounding of m
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 64)).astype(np.float16).astype(np.float64)
    e4 = E.encode_v_group_asym(x, bits)
    ah = np.repeat(e4["a16"].astype(np.float64), 32, -1)
    mh = np.repeat(e4["m16"].astype(np.float64), 32, -1)
    lo32 = np.repeat(x.reshape(50, 2, 32).min(-1), 32, -1)
    assert np.all(np.abs(mh + ah * e4["idx"] - x) <= ah / 2 + np.abs(mh - lo32) + ah * 2.0 ** -10 * top + 1e-12)


def test_benchmark_memory_table_reproduced_by_the_layout():
    """The benchmark page's 4096-token cache, 512 MB fp16 -> 113 MB, with its last 128 tokens
    in fp16: keys read as 2 Lloyd-Max bits + the 1-bit QJL sketch ("3-bit keys", R1 reading)
    and values as 2-bit group-32 min/max give 100 bytes per token and kv-head at d = 128,
    6.25 bits per K/V element pair, and the printed total to the megabyte."""
    g = json.load(open(os.path.join(GOLDEN, "compression_ratios.json")))["memory_table"]
    per = sum(L.bytes_per_token_head(128, "lm_qjl", 2, "group_asym", 2).values())
    assert per == 100
    fp16_per_token = g["fp16_mb"] * 2 ** 20 / g["tokens"]            # bytes per token, all layers
    heads_x_layers = fp16_per_token / (4 * 128)                         # (kv-head, layer) pairs
    buf = g["fp16_buffer_tokens"]
    total = buf * fp16_per_token + (g["tokens"] - buf) * heads_x_layers * per
    assert round(total / 2 ** 20) == g["compressed_mb"]
    assert L.compression_ratio(128, "lm_qjl", 2, "group_asym", 2) == 5.12


def test_key_on_centroids_has_zero_residual():
    d = 128
    rng = np.random.default_rng(3)
    c32, t32 = cb.codebook_f32(d, 3)
    s = np.where(rng.integers(0, 2, d) == 1, -1, 1)
    idx = rng.integers(0, 8, d)
    y = c32.astype(np.float64)[idx]
    k = (R.rotation_matrix(s).T @ y) * 2.5       # Pi^T c[idx], scaled
    e = E.encode_k_lm_qjl(k[None], s, rng.standard_normal((d, d)).astype(np.float32), c32, t32)
    # normalising divides by |k| = 2.5 |c[idx]|, so y is c[idx]/|c[idx]|, not c[idx]; undo it
    assert np.allclose(e["y"][0] * np.linalg.norm(y), y, atol=1e-15)
    k_unit = R.rotation_matrix(s).T @ (y / np.linalg.norm(y))
    y2 = R.rotation_matrix(s) @ k_unit
    assert np.allclose(y2, y / np.linalg.norm(y), atol=1e-15)


def test_zero_residual_when_unit_vector_lands_on_centroids():
    d = 64
    c32, t32 = cb.codebook_f32(d, 2)
    rng = np.random.default_rng(11)
    s = np.ones(d, dtype=np.int8)
    # a unit vector whose rotated coordinates are all +-c: |y|^2 = d c^2 must equal 1,
    # so use a synthetic one-entry codebook scaled to that norm
    cval = 1.0 / math.sqrt(d)
    cc = np.array([-cval, cval], dtype=np.float32)
    tt = np.array([0.0], dtype=np.float32)
    y = np.where(rng.integers(0, 2, d) == 1, cval, -cval)
    k = R.rotation_matrix(s).T @ y
    e = E.encode_k_lm_qjl(k[None], s, rng.standard_normal((d, d)).astype(np.float32), cc, tt)
    assert float(e["g16"][0]) < 1e-7


# --------------------------------------------------------------------------- decode
KINDS = [("lm_qjl", 3, "group_sym", 2), ("lm_qjl", 4, "group_sym", 4), ("lm_qjl", 2, "group_sym", 2),
         ("affine8", 8, "lm_rot", 3), ("affine8", 8, "lm_rot", 2),
         ("affine8", 5, "lm_rot", 3), ("affine8", 4, "lm_rot", 3), ("affine8", 2, "lm_rot", 2),
         ("lm_mse", 3, "lm_rot", 3), ("lm_mse", 4, "group_sym", 4), ("lm_mse", 2, "lm_rot", 2),
         ("f16", 16, "lm_rot", 3), ("f16", 16, "group_sym", 2),
         ("lm_qjl", 2, "group_asym", 2), ("lm_qjl", 3, "group_asym", 4)]


def _keys(kind, k):
    """16-bit keys are stored as given: feed values of that type."""
    return k.astype(np.float16).astype(np.float64) if kind[0] == "f16" else k


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("d", [64, 128])
def test_fast_decode_equals_bruteforce(kind, d):
    lay = Lay(d, 4, 2, *kind)
    st = _rand_state(lay, d)
    rng = np.random.default_rng(5)
    B, T, Rn = 2, 40, 6
    k = _keys(kind, rng.standard_normal((B, 2, T, d)))
    v = rng.standard_normal((B, 2, T, d))
    pk, pv = C.encode_k(lay, k, st), C.encode_v(lay, v, st)
    planes = {n: a for n, a in {**pk, **pv}.items() if n in ("k_codes", "k_signs", "k_aux", "v_codes", "v_aux")}
    q = rng.standard_normal((B, 4, d)) * 2
    rk = rng.standard_normal((B, 2, Rn, d))
    rv = rng.standard_normal((B, 2, Rn, d))
    fast = D.decode_attention(lay, q, planes, T, st, rk, rv)
    slow = D.decode_attention_bruteforce(lay, q, planes, T, st, rk, rv)
    assert np.max(np.abs(fast - slow)) < 1e-12
    # the compressed attention stays close to exact attention on the original values
    exact = D.exact_attention(lay, q, np.concatenate([k, rk], 2), np.concatenate([v, rv], 2))
    cos = np.sum(fast * exact, -1) / np.linalg.norm(fast, axis=-1) / np.linalg.norm(exact, axis=-1)
    assert np.mean(cos) > 0.75 and np.min(cos) > 0.5


@pytest.mark.parametrize("kind", [("lm_qjl", 3, "group_sym", 2), ("lm_qjl", 4, "group_sym", 4)])
@pytest.mark.parametrize("nq", [2, 4])
def test_multi_query_decode_is_causal_masked_attention(kind, nq):
    """Several queries per step: one masked attention matrix over the reconstructed cache
    (every query sees all compressed tokens; recent token r is visible to query j when
    r <= R - NQ + j) equals the oracle, which cuts the recent buffer per query."""
    d, T, Rn = 64, 37, 7
    lay = Lay(d, 4, 2, *kind)
    st = _rand_state(lay, 11)
    rng = np.random.default_rng(12)
    B = 2
    k = rng.standard_normal((B, 2, T, d))
    v = rng.standard_normal((B, 2, T, d))
    pk, pv = C.encode_k(lay, k, st), C.encode_v(lay, v, st)
    planes = {n: a for n, a in {**pk, **pv}.items() if n in ("k_codes", "k_signs", "k_aux", "v_codes", "v_aux")}
    q = rng.standard_normal((B, nq, 4, d)) * 2
    rk = rng.standard_normal((B, 2, Rn, d))
    rv = rng.standard_normal((B, 2, Rn, d))
    got = D.decode_attention_multi(lay, q, planes, T, st, rk, rv)
    allowed = np.ones((nq, T + Rn), dtype=bool)
    for j in range(nq):
        allowed[j, T + (Rn - nq + j) + 1:] = False
    for b in range(B):
        for g in range(2):
            sl = {n: planes[n][b, g, :T] for n in planes}
            K = np.concatenate([D.reconstruct_k(lay, C.read_k(lay, sl, st), st), rk[b, g]])
            V = np.concatenate([D.reconstruct_v(lay, C.read_v(lay, sl, st), st), rv[b, g]])
            for h in range(2 * g, 2 * g + 2):
                S = q[b, :, h] @ K.T / math.sqrt(d)                 # [nq, T + R]
                S = np.where(allowed, S, -np.inf)
                P = np.exp(S - S.max(axis=1, keepdims=True))
                P /= P.sum(axis=1, keepdims=True)
                assert np.max(np.abs(P @ V - got[b, :, h])) < 1e-12
    # causality: tokens after a query's own position do not move it; the last query is the
    # single-query decode over the whole buffer
    rk2, rv2 = rk.copy(), rv.copy()
    rk2[:, :, Rn - 1] += 5.0
    rv2[:, :, Rn - 1] -= 3.0
    got2 = D.decode_attention_multi(lay, q, planes, T, st, rk2, rv2)
    assert np.array_equal(got2[:, :nq - 1], got[:, :nq - 1])
    assert not np.allclose(got2[:, nq - 1], got[:, nq - 1])
    one = D.decode_attention(lay, q[:, nq - 1], planes, T, st, rk, rv)
    assert np.max(np.abs(one - got[:, nq - 1])) == 0.0


def test_no_compressed_tokens_is_exact_sdpa():
    torch = pytest.importorskip("torch")
    lay = Lay(64, 4, 2, "lm_qjl", 3, "group_sym", 2)
    st = _rand_state(lay, 1)
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 4, 64))
    rk = rng.standard_normal((1, 2, 17, 64))
    rv = rng.standard_normal((1, 2, 17, 64))
    out = D.decode_attention(lay, q, {}, 0, st, rk, rv)
    tq = torch.from_numpy(q)[:, :, None, :]
    tk = torch.from_numpy(np.repeat(rk, 2, axis=1))
    tv = torch.from_numpy(np.repeat(rv, 2, axis=1))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[:, :, 0, :].numpy()
    assert np.max(np.abs(out - ref)) < 1e-13


@pytest.mark.parametrize("kind", KINDS)
def test_one_token_and_identical_keys(kind):
    d = 64
    lay = Lay(d, 2, 1, *kind)
    st = _rand_state(lay, 2)
    rng = np.random.default_rng(4)
    k1 = _keys(kind, rng.standard_normal((1, 1, 1, d)))
    v = rng.standard_normal((1, 1, 5, d))
    q = rng.standard_normal((1, 2, d))
    pk = C.encode_k(lay, np.repeat(k1, 5, axis=2), st)
    pv = C.encode_v(lay, v, st)
    planes = {n: a for n, a in {**pk, **pv}.items() if n in ("k_codes", "k_signs", "k_aux", "v_codes", "v_aux")}
    vhat = D.reconstruct_v(lay, C.read_v(lay, {n: planes[n][0, 0] for n in ("v_codes", "v_aux")}, st), st)
    out5 = D.decode_attention(lay, q, planes, 5, st)
    assert np.max(np.abs(out5[0] - vhat.mean(axis=0))) < 1e-13       # equal keys: plain mean
    out1 = D.decode_attention(lay, q, planes, 1, st)
    assert np.max(np.abs(out1[0] - vhat[0])) < 1e-14                   # one token: that value


def test_value_reconstruction_quality_band():
    """Loose band only: the pages quote cos 0.940 (2-bit V) and 0.997 (4-bit V) at head_dim 256,
    without saying what the cosine is taken over."""
    rng = np.random.default_rng(0)
    v = rng.standard_normal((2000, 256))
    for bits, lo, hi in ((2, 0.88, 0.96), (4, 0.99, 1.0)):
        e = E.encode_v_group_sym(v, bits)
        Lv = 1 << bits
        vh = np.repeat(e["scale16"].astype(np.float64), 32, -1) * (e["idx"] - (Lv - 1) / 2)
        cos = np.mean(np.sum(v * vh, 1) / np.linalg.norm(v, axis=1) / np.linalg.norm(vh, axis=1))
        assert lo < cos <= hi

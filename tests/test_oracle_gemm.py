"""Pins for the oracle's grouped GEMM (CPU only).

The pages print no worked example, so the GEMM is pinned by:
  * special cases that reduce to a library routine (all scales 1.0 -> numpy fp64 matmul
    of the decoded codes, rounded by numpy's float16 conversion);
  * closed forms (one-hot rows select a B element exactly; constant blocks give
    k*a*b*sa*sb; a scale sweep over every finite E4M3FN code);
  * invariants (sign flip, scale exponent +1, K-block permutation, group independence);
  * exact rational brute force on tiny shapes, with values decoded by the OCP table and
    torch's float8_e4m3fn (not by the oracle).
Each is chosen so that a plausible slip in the oracle (wrong nibble order, wrong scale
index, transposed operand, dropped or wrong-signed term) fails at least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import load_golden
from synthetic import make_inputs

E2M1 = load_golden("ocp_fp4_e2m1_values.txt")
E2M1_ARR = np.array([E2M1[c] for c in range(16)], dtype=np.float64)
E4M3_ARR = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()

ONE = 0x38  # E4M3FN 1.0


def pack(codes):
    """[rows, k] codes (0..15) -> [rows, k/2] bytes, low nibble = even k."""
    codes = np.asarray(codes, dtype=np.uint8)
    return np.ascontiguousarray(codes[:, 0::2] | (codes[:, 1::2] << 4))


def unpack(packed):
    lo = packed & 0x0F
    hi = packed >> 4
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def dequant_lib(packed, sf):
    """Decoded operand from the OCP table (E2M1) and torch (E4M3FN): [rows, k] float64."""
    codes = unpack(packed)
    vals = E2M1_ARR[codes]
    scales = np.repeat(E4M3_ARR[sf], 16, axis=1)
    return vals * scales


def run(m, n, k, A, B, SFA, SFB, **kw):
    return oracle.grouped(m, n, k, A, B, SFA, SFB, want_exact=True, **kw)


def f16_bits_numpy(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def same_f16(a_bits, b_bits):
    """Bitwise equal fp16 arrays, except that +0 and -0 count as equal (signed zero is
    not part of the result: the sign of an exact zero sum depends on summation order)."""
    a = np.where((a_bits & 0x7FFF) == 0, 0, a_bits)
    b = np.where((b_bits & 0x7FFF) == 0, 0, b_bits)
    return np.array_equal(a, b)


def test_unit_scales_reduce_to_numpy_matmul():
    rng = np.random.default_rng(11)
    m, n, k = [7, 33], 24, 256
    A = [pack(rng.integers(0, 16, (mi, k))) for mi in m]
    B = [pack(rng.integers(0, 16, (n, k))) for _ in m]
    SFA = [np.full((mi, k // 16), ONE, np.uint8) for mi in m]
    SFB = [np.full((n, k // 16), ONE, np.uint8) for _ in m]
    res = run(m, n, k, A, B, SFA, SFB)
    for i in range(len(m)):
        want = E2M1_ARR[unpack(A[i])] @ E2M1_ARR[unpack(B[i])].T
        assert np.array_equal(res.exact[i], want)
        assert same_f16(res.C[i], f16_bits_numpy(want))


def test_nibble_order_low_nibble_is_even_k():
    # A row 0 = byte 0x21 then zeros: element k=0 is code 1 (0.5), k=1 is code 2 (1.0)
    k, n = 32, 2
    A = np.zeros((1, k // 2), np.uint8)
    A[0, 0] = 0x21
    # B row 0 selects k=0 with value 1.0, B row 1 selects k=1 with value 1.0
    Bc = np.zeros((n, k), np.uint8)
    Bc[0, 0] = 0x2
    Bc[1, 1] = 0x2
    ones = lambda r: np.full((r, k // 16), ONE, np.uint8)
    res = run([1], n, k, [A], [pack(Bc)], [ones(1)], [ones(n)])
    assert list(res.exact[0][0]) == [0.5, 1.0]


def test_one_hot_rows_select_b_elements_exactly():
    rng = np.random.default_rng(3)
    m, n, k = 40, 48, 512
    j = rng.permutation(k)[:m]            # row r picks K index j[r]
    Ac = np.zeros((m, k), np.uint8)
    Ac[np.arange(m), j] = 0x2             # E2M1 1.0
    SFA = np.full((m, k // 16), ONE, np.uint8)
    Bc = rng.integers(0, 16, (n, k)).astype(np.uint8)
    SFB = rng.integers(0x01, 0x7F, (n, k // 16)).astype(np.uint8)   # all finite positive codes
    res = run([m], n, k, [pack(Ac)], [pack(Bc)], [SFA], [SFB])
    Bd = dequant_lib(pack(Bc), SFB)
    want = Bd[:, j].T                      # [m, n]
    assert np.array_equal(res.exact[0], want)
    assert same_f16(res.C[0], f16_bits_numpy(want))


def test_constant_blocks_closed_form():
    # a = b = 1.0, sa = sb = 2^-3, k = 512 -> C = 512 * 2^-6 = 8.0 everywhere
    m, n, k = 5, 16, 512
    A = np.full((m, k // 2), 0x22, np.uint8)
    B = np.full((n, k // 2), 0x22, np.uint8)
    SFA = np.full((m, k // 16), 0x20, np.uint8)
    SFB = np.full((n, k // 16), 0x20, np.uint8)
    res = run([m], n, k, [A], [B], [SFA], [SFB])
    assert np.all(res.exact[0] == 8.0)
    assert np.all(res.C[0] == 0x4800)     # fp16 8.0
    # a = 6, b = -1.5, sa = 448, sb = 2^-9, k = 256: 256 * 6 * -1.5 * 448 * 2^-9 = -2016
    A = np.full((1, 128), 0x77, np.uint8)
    B = np.full((1, 128), 0xBB, np.uint8)
    res = run([1], 1, 256, [A], [B], [np.full((1, 16), 0x7E, np.uint8)], [np.full((1, 16), 0x01, np.uint8)])
    assert res.exact[0][0, 0] == -2016.0


def test_scale_sweep_every_finite_e4m3fn_code():
    codes = [c for c in range(256) if c not in (0x7F, 0xFF)]
    m, n, k = len(codes), 16, 256
    # row r: one-hot 1.0 at K = 16*(r % 16) + (r // 16) % 16, with that block's SFA = codes[r]
    Ac = np.zeros((m, k), np.uint8)
    SFA = np.full((m, k // 16), ONE, np.uint8)
    pos = [(16 * (r % 16) + (r // 16) % 16) for r in range(m)]
    for r, c in enumerate(codes):
        Ac[r, pos[r]] = 0x2
        SFA[r, pos[r] // 16] = c
    rng = np.random.default_rng(5)
    Bc = rng.integers(0, 16, (n, k)).astype(np.uint8)
    SFB = np.full((n, k // 16), ONE, np.uint8)
    res = run([m], n, k, [pack(Ac)], [pack(Bc)], [SFA], [SFB])
    for r, c in enumerate(codes):
        want = E4M3_ARR[c] * E2M1_ARR[Bc[:, pos[r]]]
        assert np.array_equal(res.exact[0][r], want), hex(c)


def test_sign_flip_negates_exactly():
    inp = make_inputs([9, 17], 32, 512, seed=21)
    base = oracle.grouped_inputs(inp, want_exact=True)
    flipped = [a ^ 0x88 for a in inp.A]     # bit 3 of every nibble is the sign
    res = oracle.grouped(inp.m, inp.n, inp.k, flipped, inp.B, inp.SFA, inp.SFB, want_exact=True)
    for i in range(inp.g):
        assert np.array_equal(res.exact[i], -base.exact[i])
        nz = base.exact[i] != 0
        assert np.array_equal((res.C[i] ^ 0x8000)[nz], base.C[i][nz])


def test_scale_exponent_plus_one_doubles_exactly():
    inp = make_inputs([6, 11], 40, 256, seed=22)
    base = oracle.grouped_inputs(inp, want_exact=True)
    SFA2 = [s + 8 for s in inp.SFA]          # codes 0x10..0x28: exponent field +1
    res = oracle.grouped(inp.m, inp.n, inp.k, inp.A, inp.B, SFA2, inp.SFB, want_exact=True)
    SFB2 = [s + 8 for s in inp.SFB]
    res2 = oracle.grouped(inp.m, inp.n, inp.k, inp.A, inp.B, inp.SFA, SFB2, want_exact=True)
    for i in range(inp.g):
        assert np.array_equal(res.exact[i], 2.0 * base.exact[i])
        assert np.array_equal(res2.exact[i], 2.0 * base.exact[i])


def test_k_block_permutation_invariance_and_transpose_sensitivity():
    inp = make_inputs([13], 24, 512, seed=23)
    base = oracle.grouped_inputs(inp, want_exact=True)
    nb = inp.k // 16
    perm = np.random.default_rng(1).permutation(nb)
    def permute(q, sf):
        qb = q.reshape(q.shape[0], nb, 8)[:, perm, :].reshape(q.shape)
        return np.ascontiguousarray(qb), np.ascontiguousarray(sf[:, perm])
    A2, SA2 = permute(inp.A[0], inp.SFA[0])
    B2, SB2 = permute(inp.B[0], inp.SFB[0])
    res = oracle.grouped([13], 24, 512, [A2], [B2], [SA2], [SB2], want_exact=True)
    assert np.array_equal(res.exact[0], base.exact[0])
    # permuting only B's blocks must change the result (the K pairing matters)
    res_b = oracle.grouped([13], 24, 512, [inp.A[0]], [B2], [inp.SFA[0]], [SB2], want_exact=True)
    assert not np.array_equal(res_b.exact[0], base.exact[0])


def test_groups_are_independent():
    inp = make_inputs([5, 7, 3], 20, 256, seed=24)
    base = oracle.grouped_inputs(inp, want_exact=True)
    inp.B[1] = np.ascontiguousarray(inp.B[1][::-1])
    inp.SFA[2] = inp.SFA[2] + 1
    res = oracle.grouped_inputs(inp, want_exact=True)
    assert np.array_equal(res.exact[0], base.exact[0])
    assert not np.array_equal(res.exact[1], base.exact[1])
    assert not np.array_equal(res.exact[2], base.exact[2])


@pytest.mark.parametrize("m,n,k", [([1, 2], 16, 256), ([3], 17, 512), ([5, 1, 4], 18, 256)])
def test_exact_rational_brute_force_tiny(m, n, k):
    inp = make_inputs(m, n, k, seed=sum(m) * 100 + n)
    res = oracle.grouped_inputs(inp, want_exact=True)
    for i, mi in enumerate(m):
        Ad = dequant_lib(inp.A[i], inp.SFA[i])
        Bd = dequant_lib(inp.B[i], inp.SFB[i])
        for r in range(mi):
            for c in range(n):
                s = sum((Fraction(Ad[r, kk]) * Fraction(Bd[c, kk]) for kk in range(k)), Fraction(0))
                assert Fraction(res.exact[i][r, c]) == s
                assert same_f16(res.C[i][r:r+1, c], f16_bits_numpy([float(s)]))


def test_synthetic_workload_sums_are_exact_and_abs_sum_consistent():
    # A medium case with the workload distribution: fp64 sums equal numpy's fp64 matmul of
    # the library-decoded operands (sums are exact, so any order agrees), and |C| <= abssum.
    inp = make_inputs([33, 64], 96, 1536, seed=1111)
    res = oracle.grouped_inputs(inp, want_exact=True)
    for i in range(inp.g):
        want = dequant_lib(inp.A[i], inp.SFA[i]) @ dequant_lib(inp.B[i], inp.SFB[i]).T
        assert np.array_equal(res.exact[i], want)
        assert same_f16(res.C[i], f16_bits_numpy(want))
        assert np.all(np.abs(res.exact[i]) <= res.abssum[i])
        absw = np.abs(dequant_lib(inp.A[i], inp.SFA[i])) @ np.abs(dequant_lib(inp.B[i], inp.SFB[i])).T
        assert np.array_equal(res.abssum[i], absw)


def test_empty_group_and_argument_errors():
    inp = make_inputs([0, 4], 16, 256, seed=2)
    res = oracle.grouped_inputs(inp, want_exact=True)
    assert res.C[0].shape == (0, 16)
    with pytest.raises(ValueError):
        oracle.grouped([4], 16, 256, [inp.A[1][:, :10]], inp.B[1:], inp.SFA[1:], inp.SFB[1:])

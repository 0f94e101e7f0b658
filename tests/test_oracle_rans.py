"""Pins for oracle.rans ([D-Quant] §3.1 Eq. (2), §4.2 Eq. (3), Appendix A
Algorithm 2): round trip, container length, the bit-insertion closed form of
a uniform table, a hand-worked example and the code-length bound."""

import numpy as np
import pytest

import oracle as O


def _uniform_table(b):
    M = 1 << b
    f = np.full(M, 256 // M, np.int64)
    return f, np.arange(M, dtype=np.int64) * (256 // M)


def _bit_insertion_encode(m, b, C):
    """Closed form of Eq. (2) for f_m = 2^(8-b): Enc(x, m) keeps the low 8-b
    bits of x, writes m above them and moves the rest of x up by b bits."""
    lowbits = 8 - b
    x = 1 << 23
    pushed = []
    for sym in reversed(list(m)):
        while x >= (1 << (31 - b)):          # 2^23 * 2^(8-b)
            pushed.append(x & 0xFF)
            x >>= 8
        x = ((x >> lowbits) << 8) | (int(sym) << lowbits) | (x & ((1 << lowbits) - 1))
    out = list(x.to_bytes(4, "little")) + pushed[::-1]
    return np.array(out + [0] * (C - len(out)), np.uint8)


def test_hand_worked_uniform_example():
    # M = 2, f = [128, 128]: every encode step inserts one bit at bit 7.
    # Symbols m_0..m_15 below are encoded from m_15 down to m_0 (a_1..a_16).
    # Seven steps lift x from 2^23 to 2^30 + (a_1..a_7 at bits 13..7), so the
    # first push is the byte a_7 << 7 = 0x80; the low six bits then hold
    # a_1..a_6 = 101001b = 41 while a_8..a_15 are inserted; the second push is
    # a_15 << 7 | 41 = 0x29; the final state is 2^23 + a_16 << 7 + a_8..a_14
    # (1010011b = 83) = 0x8000D3.  Container: state LE, then the last pushed
    # byte first, then zero padding.
    m = [1, 0, 1, 1, 0, 0, 1, 0, 1, 1, 1, 0, 0, 1, 0, 1]
    f, c = _uniform_table(1)
    cont, k = O.rans_encode(np.array([m]), f, c, 8)
    assert cont[0].tolist() == [0xD3, 0x00, 0x80, 0x00, 0x29, 0x80, 0x00, 0x00]
    assert k[0] == 2
    sym, x_end, ptr = O.rans_decode(cont, f, c, 16)
    assert sym[0].tolist() == m and x_end[0] == O.L_RANS and ptr[0] == 6


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_uniform_tables_match_bit_insertion(b):
    rng = np.random.default_rng(b)
    f, c = _uniform_table(b)
    n = 200
    C = 4 + (n * b + 7) // 8 + 2
    m = rng.integers(0, 1 << b, (20, n))
    cont, _ = O.rans_encode(m, f, c, C)
    for s in range(20):
        assert np.array_equal(cont[s], _bit_insertion_encode(m[s], b, C))


@pytest.mark.parametrize("M,n", [(8, 1024), (6, 1024), (8, 128), (6, 128), (16, 256)])
def test_round_trip_and_framing(M, n):
    f, c = O.build_table(M, n, 1.4)
    rng = np.random.default_rng(M + n)
    # draw symbols from the table's own law, plus a few all-expensive streams
    m = rng.choice(M, size=(40, n), p=f / 256.0)
    m[0] = 0
    m[1] = M - 1
    C = int(np.ceil((O.rate_table(f)[m].sum(axis=1).max() / 65536 + 40) / 8)) + 8
    cont, k = O.rans_encode(m, f, c, C)
    assert cont.shape == (40, C) and cont.dtype == np.uint8
    sym, x_end, ptr = O.rans_decode(cont, f, c, n)
    assert np.array_equal(sym, m)
    assert np.all(x_end == O.L_RANS)
    assert np.array_equal(ptr, 4 + k)
    for s in range(40):
        assert np.all(cont[s, 4 + k[s]:] == 0)


def test_code_length_bound():
    """8k <= sum_i -log2(f_mi / 256) + (n + k) 2^-15 log2(e): each encode step
    scales the state by 256 / f within a relative 2^-15 and the state ends at
    least as large as it started."""
    for M, n in [(8, 1024), (6, 1024), (8, 128)]:
        f, c = O.build_table(M, n, 1.4)
        rng = np.random.default_rng(7)
        m = rng.choice(M, size=(300, n), p=f / 256.0)
        rtrue = (8 - np.log2(f.astype(np.float64)))[m].sum(axis=1)
        cont, k = O.rans_encode(m, f, c, int(rtrue.max() / 8) + 16)
        slack = (n + k) * 2.0 ** -15 * np.log2(np.e)
        assert np.all(8 * k <= rtrue + slack)
        assert np.all(8 * k >= rtrue - 8 - slack)


def test_budget_implies_fit():
    """A fixed-point rate within B_fx = (8C - 32) 2^16 always fits C bytes."""
    f, c = O.build_table(6, 1024, 1.4)
    r = O.rate_table(f)
    rng = np.random.default_rng(8)
    m = rng.choice(6, size=(400, 1024), p=f / 256.0)
    R = r[m].sum(axis=1)
    C = int(np.ceil(R.max() / 65536 / 8)) + 4       # tightest C for the worst row
    keep = R <= O.budget_fx(C)
    assert keep.sum() > 0
    cont, k = O.rans_encode(m[keep], f, c, C)
    assert np.all(4 + k <= C)


@pytest.mark.parametrize("M,C", [(8, 331), (6, 231), (3, 200)])
def test_decode_then_reencode_reproduces_the_container(M, C):
    """The decoder inverts the encoder: encoding the decoded symbols again gives
    the same C bytes, for random symbol streams drawn from the table itself."""
    rng = np.random.default_rng(M + C)
    f, c = O.build_table(M, 1024, 1.4)
    q = np.asarray(f, np.float64) / 256.0
    m = rng.choice(M, size=(32, 1024), p=q)
    r = O.rate_table(f)
    fits = r[m].sum(axis=1) <= O.budget_fx(C)
    m = m[fits]
    cont, _ = O.rans_encode(m, f, c, C)
    sym, x_end, ptr = O.rans_decode(cont, f, c, 1024)
    assert np.array_equal(sym, m)
    assert np.all(x_end == O.L_RANS)
    again, _ = O.rans_encode(sym, f, c, C)
    assert np.array_equal(again, cont)

"""rANS coder and the fixed-size container.

Follows [D-Quant] §3.1 Eq. (2) (the encoder maps state x and symbol m to
floor(x / f_m) 2^p + (x mod f_m) + c_m with precision p = 8; symbols are
encoded backwards so that decoding yields them in stream order), §4.2 Eq. (3)
(a stream occupies exactly C bytes, sigma bits of which hold the final state)
and Appendix A, Algorithm 2 (which states that the decoder starts from the
little-endian state at the head of the container and consumes bytes forwards).

Readings (the page leaves them open):
  * 32-bit state, L = 2^23, sigma = 32, so the state lives in [2^23, 2^31).
  * Encoder: start at x = L; for i = n-1 down to 0, while x >= 2^23 f_m push
    the low byte of x and shift x right by 8, then apply Eq. (2).
  * Container: bytes 0..3 hold the final state little-endian, then the pushed
    bytes in reverse push order (the last pushed byte is read first), then
    zero bytes up to C.

The decoder here is written as the inverse of that encoder: each symbol is
recovered by undoing Eq. (2), and each byte the encoder pushed to keep its
state below 2^23 f_m is pulled back when the state drops below L.
"""

import numpy as np

from .model import L_RANS, PROB_BITS

_U64 = np.uint64


def rans_encode(m, f, c, container_bytes):
    """Encode symbol rows m [N, n] into containers [N, C] (uint8).

    Returns (containers, payload_len) where payload_len counts pushed bytes.
    Raises if a stream does not fit (cannot happen when its fixed-point rate
    is within the budget; see the length bound in the tests)."""
    m = np.asarray(m, np.int64)
    N, n = m.shape
    C = int(container_bytes)
    fm = np.asarray(f, np.int64)[m].astype(_U64)
    cm = np.asarray(c, np.int64)[m].astype(_U64)
    x = np.full(N, L_RANS, _U64)
    pushed = np.zeros((N, max(C - 4, 1)), np.uint8)
    k = np.zeros(N, np.int64)
    rows = np.arange(N)
    for i in range(n - 1, -1, -1):
        fi = fm[:, i]
        x_max = _U64(L_RANS >> PROB_BITS) * _U64(1 << 8) * fi
        while True:
            ren = x >= x_max
            if not ren.any():
                break
            r = rows[ren]
            if (k[r] >= C - 4).any():
                raise ValueError("stream does not fit its container")
            pushed[r, k[r]] = (x[r] & _U64(255)).astype(np.uint8)
            k[r] += 1
            x[r] >>= _U64(8)
        x = (x // fi) * _U64(1 << PROB_BITS) + (x % fi) + cm[:, i]
    cont = np.zeros((N, C), np.uint8)
    for b in range(4):
        cont[:, b] = ((x >> _U64(8 * b)) & _U64(255)).astype(np.uint8)
    for s in range(N):
        kk = int(k[s])
        cont[s, 4:4 + kk] = pushed[s, :kk][::-1]
    return cont, k


def _undo_eq2(xp, f, c):
    """Inverse of Eq. (2) for one state per row.

    The encoder's output x' = floor(x / f_m) 2^p + (x mod f_m) + c_m has its
    low p bits, the slot x' mod 2^p = (x mod f_m) + c_m, inside
    [c_m, c_m + f_m), and those intervals tile [0, 2^p) in symbol order; so m
    is the last symbol whose cumulative frequency c_m does not exceed the slot,
    and x = f_m floor(x' / 2^p) + (slot - c_m)."""
    slot = xp & ((1 << PROB_BITS) - 1)
    m = np.searchsorted(c, slot, side="right") - 1
    return m, f[m] * (xp >> PROB_BITS) + (slot - c[m])


def rans_decode(cont, f, c, n):
    """Recover the n symbols of each container row by running the encoder
    backwards: read the final state, undo Eq. (2) once per symbol in stream
    order, and after each step pull back, one at a time, the bytes the encoder
    pushed before that step (it pushed while its state was at least 2^23 f_m,
    which leaves the undone state below L = 2^23 exactly when a byte is due).

    Returns (m [N, n] int64, end_state [N], bytes_read [N]); a well-formed
    stream ends at the encoder's start state L.  Raises if a stream would read
    past its container."""
    cont = np.asarray(cont, np.uint8)
    N, C = cont.shape
    f = np.asarray(f, np.int64)
    c = np.asarray(c, np.int64)
    x = np.zeros(N, np.int64)
    for b in range(4):
        x |= cont[:, b].astype(np.int64) << (8 * b)
    ptr = np.full(N, 4, np.int64)
    out = np.zeros((N, n), np.int64)
    rows = np.arange(N)
    for i in range(n):
        out[:, i], x = _undo_eq2(x, f, c)
        while True:
            due = x < L_RANS
            if not due.any():
                break
            r = rows[due]
            if (ptr[r] >= C).any():
                raise ValueError("decoder ran past the container")
            x[r] = (x[r] << 8) | cont[r, ptr[r]].astype(np.int64)
            ptr[r] += 1
    return out, x, ptr

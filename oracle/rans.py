"""rANS coder and the fixed-size container.

Follows [D-Quant] §3.1 Eq. (2) (Enc / Dec of the integer state with precision
p = 8; symbols are encoded backwards so that decoding runs forwards), §4.2
Eq. (3) (a stream occupies exactly C bytes; sigma is the final-state
overhead) and Appendix A, Algorithm 2 (the state is read little-endian from
the first sigma/8 bytes; each step looks up T[z] for z = x mod 2^p, updates
x = f floor(x / 2^p) + z - c, then shifts in one byte at a time while x < L).

Readings (the page leaves them open):
  * 32-bit state, L = 2^23, sigma = 32, so the state lives in [2^23, 2^31).
  * Encoder: start at x = L; for i = n-1 down to 0, while x >= 2^23 f_m push
    the low byte of x and shift x right by 8, then apply Eq. (2).
  * Container: bytes 0..3 hold the final state little-endian, then the pushed
    bytes in reverse push order (the last pushed byte is read first), then
    zero bytes up to C.
"""

import numpy as np

from .model import L_RANS, PROB_BITS, decode_table

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


def rans_decode(cont, f, c, n):
    """Decode n symbols from each container row (Algorithm 2).

    Returns (m [N, n] int64, end_state [N], bytes_read [N]).  Raises if a
    stream would read past its container."""
    cont = np.asarray(cont, np.uint8)
    N, C = cont.shape
    sym, fz, bias = decode_table(f, c)
    x = np.zeros(N, np.int64)
    for b in range(4):
        x |= cont[:, b].astype(np.int64) << (8 * b)
    ptr = np.full(N, 4, np.int64)
    out = np.zeros((N, n), np.int64)
    rows = np.arange(N)
    for i in range(n):
        z = x & 255
        out[:, i] = sym[z]
        x = fz[z] * (x >> PROB_BITS) + bias[z]
        while True:
            ren = x < L_RANS
            if not ren.any():
                break
            r = rows[ren]
            if (ptr[r] >= C).any():
                raise ValueError("decoder ran past the container")
            x[r] = (x[r] << 8) | cont[r, ptr[r]].astype(np.int64)
            ptr[r] += 1
    return out, x, ptr

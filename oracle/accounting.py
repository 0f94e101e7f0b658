"""Bits-per-value accounting and the budget -> container-size helper.

Follows [D-Quant] §3.1 (storage is reported in bits per value including the
quantised symbols and the metadata; INT2 with an FP16 scale and zero point per
128 values costs 2.25), §5.1 "Implementation details" (331/231-byte K/V
containers with 8/6 levels are 2.26 bits per value; groups of 1024 values),
§5.4 (2.68 bits to keys, 1.84 to values) and Appendix B (FP16 metadata and an
INT8 windowed channel mean for keys).

Reading: per token-layer the cache holds one K and one V container, an fp16
(scale, offset) pair for each, and, for each window of W tokens, an INT8 key
mean of n values plus its fp16 scale, so
    bpe = 8 (C_K + C_V + 2*(2+2) + (n + 2)/W) / (2 n).
With 331/231, n = 1024, W = 128 this is 2.2579 (the page's 2.26); keys alone
8 (331 + 4 + 1026/128) / 1024 = 2.680, values alone 8 (231 + 4) / 1024 = 1.836.

Budget helper: total = floor(bpe 2n/8 - (8 + (n+2)/W)) bytes of container per
token-layer, split in the page's K:V proportion 331:562 (rounded to nearest,
ties to even) so that 2.26 gives back 331/231.
"""

import math


def bits_per_elem(c_k, c_v, n, window, metadata=True):
    if metadata:
        return 8.0 * (c_k + c_v + 2 * (2 + 2) + (n + 2) / window) / (2.0 * n)
    return 8.0 * (c_k + c_v) / (2.0 * n)


def containers_for_budget(bpe, n, window):
    total = math.floor(bpe * 2.0 * n / 8.0 - (8.0 + (n + 2) / window))
    c_k = round(total * 331 / 562)          # Python round: ties to even
    return c_k, total - c_k

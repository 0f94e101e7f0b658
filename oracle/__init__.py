"""CPU oracle for D-Quant-style entropy-coded KV-cache quantisation.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding) may import, call, link or execute anything in this package.
Its only callers are ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.

It is a plain, slow restatement of what the method computes, written from the
page "D-Quant: Driftable Entropy Coding for KV Cache Quantization" (cited
below as [D-Quant], with its section, equation, algorithm or appendix).  Where
the page leaves an arithmetic detail open, the oracle fixes one reading; every
such reading is listed in the repository's design notes and restated in the
docstring of the function that takes it.

Arithmetic rules (they make the encoder's output a single, reproducible value):
  * every float operation is one IEEE-754 binary32 or binary64 operation,
    rounded to nearest-even; numpy elementwise ufuncs on float32/float64
    arrays are exactly that, and the code never lets numpy pick a reduction
    order for a floating sum (sums are explicit loops);
  * no fused multiply-add anywhere;
  * min / max / integer sums are order-free and use numpy freely.

Modules:
  model      probability model, integer rANS table, rate and lambda tables
  transform  per-head Hadamard rotation, windowed key channel mean (INT8)
  quant      FitMinMax, Drift, least-squares Refit, the Algorithm-1 encoder
  rans       rANS coder and the fixed-size container format
  attention  dequantise-then-attend reference in float64 (plain and factored)
  accounting bits-per-value accounting and the budget -> container helper
  pipeline   whole-cache encode/decode used by the tests and the baseline
  fixedwidth the fixed-width comparator of Appendix B (nearest rounding,
             power-of-two symbol widths)

Parity unpinned: none of the functions here lacks a pin; the pins live in
tests/test_oracle_*.py (marked not-gpu).
"""

from .model import (L_RANS, PROB_BITS, SIGMA_BITS, budget_fx, order_stat_probs, sharpen,
                    integer_table, build_table, rate_table, lambda_table,
                    decode_table, level_midpoints, level_values_fp16)
from .transform import fwht_f32, hadamard_f64, rotate_heads, key_window_mean
from .quant import (fit_minmax, drift, refit, refit_f64, lane_sum_f64,
                    nearest_levels, encode_streams_alg1)
from .rans import rans_encode, rans_decode
from .attention import (dequantize_f64, attention_plain_f64,
                        attention_factored_f64, attention_with_residual_f64)
from .accounting import bits_per_elem, containers_for_budget
from .pipeline import OracleParams, encode_cache, decode_cache_symbols
from .fixedwidth import (fw_bits, fw_container_bytes, fw_pack, fw_unpack, encode_streams_fw,
                         encode_cache_fw)

__all__ = [
    "L_RANS", "PROB_BITS", "SIGMA_BITS", "budget_fx", "order_stat_probs", "sharpen",
    "level_midpoints", "level_values_fp16",
    "refit_f64", "lane_sum_f64", "nearest_levels",
    "integer_table", "build_table", "rate_table", "lambda_table",
    "decode_table", "fwht_f32", "hadamard_f64", "rotate_heads",
    "key_window_mean", "fit_minmax", "drift", "refit", "encode_streams_alg1",
    "rans_encode", "rans_decode", "dequantize_f64", "attention_plain_f64",
    "attention_factored_f64", "attention_with_residual_f64", "bits_per_elem", "containers_for_budget",
    "OracleParams", "encode_cache", "decode_cache_symbols",
    "fw_bits", "fw_container_bytes", "fw_pack", "fw_unpack", "encode_streams_fw", "encode_cache_fw",
]

"""Reference int8 KV-cache quantization and decode over the quantized cache (oracle side,
test infrastructure).

Source: the decode benchmark of "rename context to context_autoregressive" (MaxText PR 1453,
Description) runs with an int8-quantized KV cache (``quantize_kvcache=True`` together with
``quantization=int8``). The pages name the setting but not its arithmetic, so the plainest
reading is taken:

* symmetric absmax quantization, one scale per cached row, i.e. per (sequence, kv head, cache
  position) over the head dimension: ``amax = max_d |x_d|``, ``scale = amax / 127``,
  ``code_d = round(x_d / scale)`` (round half to even), clipped to [-127, 127]; a row of
  zeros gets scale 0 and codes 0. The rounding decisions are taken in float32: ``amax`` is
  exact, the quotient ``amax / 127`` and each ``x_d / scale`` are correctly rounded float32
  divisions.
* the cache stores the codes and the scales; attention reads the dequantized values
  ``code * scale`` (exact in float64) and is otherwise the decode attention of ``decode_ref``.
"""

import numpy as np

from .attention import _f64, decode_ref


def kv_quantize_ref(x):
    """Quantize every row (last axis) of ``x`` (numpy or CPU torch, any float dtype whose values
    are exact in float32). Returns (codes int8 of x's shape, scales float32 of x.shape[:-1])."""
    x32 = _f64(x).astype(np.float32)  # bf16 and fp32 values are exact in float32
    rows = x32.reshape(-1, x32.shape[-1])
    codes = np.zeros(rows.shape, dtype=np.int8)
    scales = np.zeros(rows.shape[0], dtype=np.float32)
    for i in range(rows.shape[0]):
        amax = np.float32(np.max(np.abs(rows[i]))) if rows.shape[1] else np.float32(0)
        if amax == 0:
            continue
        s = np.float32(amax / np.float32(127))
        c = np.rint(rows[i] / s)  # float32 quotient, then round half to even
        codes[i] = np.clip(c, -127, 127).astype(np.int8)
        scales[i] = s
    return codes.reshape(x32.shape), scales.reshape(x32.shape[:-1])


def dequantize_ref(codes, scales):
    """code * scale per row, in float64 (exact)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def decode_int8_ref(q, k_codes, k_scales, v_codes, v_scales, lengths, scale):
    """Decode attention over an int8 cache: the dequantized cache fed to ``decode_ref``.

    q: [B, Hq, D]; k_codes, v_codes: [B, Hkv, Lmax, D] int8; k_scales, v_scales: [B, Hkv, Lmax]
    float32. Returns (O [B, Hq, D], LSE [B, Hq]) float64.
    """
    k = dequantize_ref(k_codes, k_scales)
    v = dequantize_ref(v_codes, v_scales)
    return decode_ref(q, k, v, lengths, scale)

"""Oracle: per-token asymmetric min/max quantizer (test infrastructure only).

Source: DiffKV review page, "Core claim" and the free-parameter ledger -- important tokens
are stored as K8V4 (8-bit keys, 4-bit values), moderately important ones as K4V2.  The page
does not print the quantizer; the reading taken is the plain
per-token, per-head asymmetric min/max scheme over the 128 channels of one key or value row:

    mn, mx  = min and max of the row's fp16 values (exact in float32)
    s32     = fl32( fl32(mx - mn) / (2^b - 1) )        two float32 round-to-nearest-even ops
    s16     = fp16(s32) rounded to nearest even; if that is 0 while mx > mn, 2^-24 instead
    z16     = mn + 0  (an fp16 value already; adding +0 stores a -0 minimum as +0)
    inv     = fl32(1 / s16) when s16 > 0, else 0
    code_i  = min( rint_even( fl32( fl32(x_i - z16) * inv ) ), 2^b - 1 )
    x_hat_i = fl32( code_i * s16 + z16 )                one rounding (a fused multiply-add)

x_i - z16 >= 0 always, so no lower clamp is needed.  Scale and zero are stored as fp16.
A token demoted from K8V4 to K4V2 after its fp16 row is gone is re-quantized from the fp16
rounding of its K8V4 reconstruction (``requantize_from``).
"""
import numpy as np

K_BITS = {2: 8, 1: 4}     # tier -> key bits   (HIGH = 2 -> K8, LOW = 1 -> K4)
V_BITS = {2: 4, 1: 2}     # tier -> value bits (HIGH -> V4, LOW -> V2)


def quantize_rows(x, bits):
    """x: fp16 [n][d] -> (codes uint8 [n][d], scale fp16 [n], zero fp16 [n])."""
    x = np.asarray(x, dtype=np.float16)
    lq = np.float32(2 ** bits - 1)
    xf = x.astype(np.float32)
    mn = xf.min(axis=1)
    mx = xf.max(axis=1)
    rng = (mx - mn).astype(np.float32)                 # float32 subtraction
    s32 = (rng / lq).astype(np.float32)                # float32 division
    s16 = s32.astype(np.float16)                       # round to nearest even
    tiny = np.float16(2.0 ** -24)
    s16 = np.where((s16 == 0) & (mx > mn), tiny, s16).astype(np.float16)
    z16 = (mn + np.float32(0)).astype(np.float16)      # exact; -0 becomes +0
    sf = s16.astype(np.float32)
    pos = sf > 0
    inv = np.zeros_like(sf)
    inv[pos] = np.float32(1.0) / sf[pos]               # float32 division
    diff = (xf - z16.astype(np.float32)[:, None]).astype(np.float32)
    y = (diff * inv[:, None]).astype(np.float32)
    codes = np.minimum(np.rint(y), lq).astype(np.uint8)   # rint: half to even
    return codes, s16, z16


def dequantize_rows(codes, scale, zero):
    """codes uint8 [n][d], scale/zero fp16 [n] -> float32 [n][d] = fl32(code*scale + zero).

    code*scale + zero is exact in float64 (an 8-bit integer times an fp16 value plus an fp16
    value fits in 53 bits), so one rounding to float32 is exactly a fused multiply-add.
    """
    c = np.asarray(codes, dtype=np.float64)
    s = np.asarray(scale, dtype=np.float16).astype(np.float64)[:, None]
    z = np.asarray(zero, dtype=np.float16).astype(np.float64)[:, None]
    return (c * s + z).astype(np.float32)


def requantize_from(codes, scale, zero, bits):
    """Demotion: fp16(x_hat) of the stored row, then quantize at the lower bit width."""
    xh = dequantize_rows(codes, scale, zero).astype(np.float16)
    return quantize_rows(xh, bits)

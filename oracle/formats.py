"""Weight-format decode (oracle; test infrastructure only).

The pages name the expert formats MXFP4, NVFP4, FP8 and BF16 (FreeToken README
feature list "Broad MoE & ecosystem support"; supported-models guide, sections
"how quantizations land" and "CPU layer split") but print no bit layouts.  The
decoders below follow the public definitions of those encodings:

  E2M1  (4 bit)  sign | 2-bit exponent (bias 1) | 1-bit mantissa, no Inf/NaN
  E8M0  (8 bit)  pure power of two 2^(b-127); 0xFF is NaN
  E4M3  (8 bit)  sign | 4-bit exponent (bias 7) | 3-bit mantissa; subnormals
                 when the exponent field is 0; S.1111.111 is NaN; no Inf
  BF16           upper 16 bits of an IEEE binary32

and the record layout of one expert (sections at 256-byte aligned offsets;
W13 = gate rows then up rows; two E2M1 codes per byte, element 2i in the low
nibble).  Every value is produced exactly in float64.

Parity: pinned (all 16 / 256 / 256 codes against the published value tables,
torch's float8_e4m3fn / float8_e8m0fnu casts, and invariants; see tests).
"""
from __future__ import annotations

import numpy as np

FMT_BF16, FMT_MXFP4, FMT_NVFP4, FMT_FP8_B128 = "bf16", "mxfp4", "nvfp4", "fp8_b128"


def e2m1_value(code) -> np.ndarray:
    """E2M1 code (0..15) -> value.  Exponent field 0 is the subnormal row
    (mantissa * 2^-1 * 2^(1-bias) = m * 0.5); otherwise (1 + m/2) * 2^(e-1)."""
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag).astype(np.float64)


def e8m0_value(b) -> np.ndarray:
    """E8M0 scale byte -> 2^(b-127); 0xFF encodes NaN."""
    b = np.asarray(b, dtype=np.int64)
    v = np.exp2(b.astype(np.float64) - 127.0)
    return np.where(b == 255, np.nan, v)


def e4m3_value(b) -> np.ndarray:
    """OCP E4M3 ("FN") byte -> value.  Bias 7; exponent field 0 is subnormal
    (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN (no infinities)."""
    b = np.asarray(b, dtype=np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag).astype(np.float64)


def bf16_value(u16) -> np.ndarray:
    """bf16 bit pattern (uint16) -> value (exact)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def unpack_e2m1(packed: np.ndarray, K: int) -> np.ndarray:
    """[N, K/2] bytes -> [N, K] codes; element 2i = low nibble, 2i+1 = high."""
    p = np.asarray(packed, dtype=np.uint8)
    N = p.shape[0]
    out = np.empty((N, K), dtype=np.uint8)
    out[:, 0::2] = p & 0x0F
    out[:, 1::2] = p >> 4
    return out


def dequant_mxfp4(packed: np.ndarray, scales: np.ndarray, N: int, K: int) -> np.ndarray:
    """MXFP4: w[n,k] = E2M1(code[n,k]) * E8M0(scale[n, k//32])."""
    codes = unpack_e2m1(packed.reshape(N, K // 2), K)
    sc = e8m0_value(scales.reshape(N, K // 32))
    return e2m1_value(codes) * np.repeat(sc, 32, axis=1)


def dequant_nvfp4(packed: np.ndarray, scales: np.ndarray, tensor_scale: float,
                  N: int, K: int) -> np.ndarray:
    """NVFP4: w[n,k] = E2M1(code[n,k]) * E4M3(scale[n, k//16]) * tensor_scale."""
    codes = unpack_e2m1(packed.reshape(N, K // 2), K)
    sc = e4m3_value(scales.reshape(N, K // 16))
    return e2m1_value(codes) * np.repeat(sc, 16, axis=1) * float(tensor_scale)


def dequant_fp8_b128(q: np.ndarray, scales: np.ndarray, N: int, K: int) -> np.ndarray:
    """FP8 block: w[n,k] = E4M3(q[n,k]) * scale[n//128, k//128] (fp32 scales)."""
    v = e4m3_value(q.reshape(N, K))
    sc = np.asarray(scales, dtype=np.float32).reshape(N // 128, K // 128).astype(np.float64)
    return v * np.repeat(np.repeat(sc, 128, axis=0), 128, axis=1)


def dequant_bf16(raw: np.ndarray, N: int, K: int) -> np.ndarray:
    return bf16_value(np.asarray(raw).view(np.uint16).reshape(N, K))


# ----------------------------------------------------------------------------
# expert record layout (the oracle's own reading of the storage spec)
# ----------------------------------------------------------------------------
def _sections(fmt: str, H: int, I: int):
    if fmt == FMT_BF16:
        return [("w13", 4 * I * H), ("w2", 2 * H * I)]
    if fmt == FMT_MXFP4:
        return [("w13", I * H), ("w13s", I * H // 16), ("w2", H * I // 2), ("w2s", H * I // 32)]
    if fmt == FMT_NVFP4:
        return [("w13", I * H), ("w13s", I * H // 8), ("w2", H * I // 2), ("w2s", H * I // 16),
                ("ts", 12)]
    if fmt == FMT_FP8_B128:
        return [("w13", 2 * I * H), ("w13s", 2 * I * H // (128 * 128) * 4),
                ("w2", H * I), ("w2s", H * I // (128 * 128) * 4)]
    raise ValueError(fmt)


def record_sections(fmt: str, H: int, I: int) -> dict:
    out, pos = {}, 0
    for name, n in _sections(fmt, H, I):
        pos = -(-pos // 256) * 256
        out[name] = (pos, n)
        pos += n
    return out


def decode_record(record: np.ndarray, fmt: str, H: int, I: int):
    """One expert record (bytes) -> (W_gate [I,H], W_up [I,H], W_down [H,I]) float64."""
    rec = np.asarray(record, dtype=np.uint8).reshape(-1)
    sec = record_sections(fmt, H, I)

    def raw(name):
        off, n = sec[name]
        return rec[off:off + n]

    if fmt == FMT_BF16:
        w13 = dequant_bf16(raw("w13"), 2 * I, H)
        wd = dequant_bf16(raw("w2"), H, I)
    elif fmt == FMT_MXFP4:
        w13 = dequant_mxfp4(raw("w13"), raw("w13s"), 2 * I, H)
        wd = dequant_mxfp4(raw("w2"), raw("w2s"), H, I)
    elif fmt == FMT_NVFP4:
        ts = raw("ts").view(np.float32).astype(np.float64)
        codes = raw("w13").reshape(2 * I, H // 2)
        sc = raw("w13s").reshape(2 * I, H // 16)
        wg = dequant_nvfp4(codes[:I], sc[:I], ts[0], I, H)
        wu = dequant_nvfp4(codes[I:], sc[I:], ts[1], I, H)
        w13 = np.concatenate([wg, wu], axis=0)
        wd = dequant_nvfp4(raw("w2"), raw("w2s"), ts[2], H, I)
    elif fmt == FMT_FP8_B128:
        w13 = dequant_fp8_b128(raw("w13"), raw("w13s").view(np.float32), 2 * I, H)
        wd = dequant_fp8_b128(raw("w2"), raw("w2s").view(np.float32), H, I)
    else:
        raise ValueError(fmt)
    return w13[:I], w13[I:], wd

"""Seeded synthetic inputs for the MoE layer forward.

This module only *produces input bytes*: router logits, bf16 activations and
expert weight records in the four storage formats.  It holds none of the
layer's arithmetic (no routing, no permutation, no FFN, no combine, no weight
decode).  Both the CPU oracle and the GPU path consume what it writes.

Workloads follow the MoE serving setting of the FreeToken pages (page 2,
section "MoE strategies" and "expert bank & LRU slot cache"; page 5, the
measured-performance table and production configuration), with the shapes of
the five synthetic layers listed in `WORKLOADS`.

Record layout (one expert = one record; identical rule used by every consumer,
each of which implements it on its own):

  every section starts at a 256-byte aligned offset inside the record, in the
  order below; the record stride is the payload rounded up to 256 bytes.

  bf16      w13  [2I][H]  bf16          w2  [H][I]  bf16
  mxfp4     w13  [2I][H/2] E2M1 pairs   w13s [2I][H/32] E8M0
            w2   [H][I/2]  E2M1 pairs   w2s  [H][I/32]  E8M0
  nvfp4     w13  [2I][H/2]              w13s [2I][H/16] E4M3
            w2   [H][I/2]               w2s  [H][I/16]  E4M3
            ts   fp32[3] = per-tensor scale of (gate, up, down)
  fp8_b128  w13  [2I][H]  E4M3          w13s fp32 [2I/128][H/128]
            w2   [H][I]   E4M3          w2s  fp32 [H/128][I/128]

  W13 rows 0..I-1 are the gate projection, rows I..2I-1 the up projection.
  Two E2M1 codes share a byte: element 2i in the low nibble, 2i+1 in the high.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

FORMATS = ("bf16", "mxfp4", "nvfp4", "fp8_b128")
FMT_ID = {"bf16": 0, "mxfp4": 1, "nvfp4": 2, "fp8_b128": 3}
ALIGN = 256
WEIGHT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    E: int
    I: int
    k: int
    fmt: str
    seed: int
    zipf: float | None = None      # Zipf exponent of the expert bias, None = no bias
    domains: int = 0               # >0: rotating domain-biased routing (cache workload)
    batches: int = 1               # batches in one pass of the cache workload
    pool_slots: int = 0            # >0: HBM expert pool of this many slots
    shared_I: int = 0              # >0: one always-on bf16 shared expert of this width

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five synthetic layers.  Sizes and distributions are the ones stated for
# each workload; names describe the workload, not where it was listed.
WORKLOADS = {
    "tiny_bf16": Workload("tiny_bf16", T=64, H=256, E=8, I=128, k=2, fmt="bf16", seed=1),
    "decode_mxfp4": Workload("decode_mxfp4", T=8, H=2048, E=256, I=512, k=8, fmt="mxfp4", seed=2),
    "prefill_nvfp4": Workload("prefill_nvfp4", T=4096, H=2048, E=256, I=512, k=8, fmt="nvfp4",
                              seed=3, zipf=1.1),
    "fp8_lru_pool": Workload("fp8_lru_pool", T=2048, H=4096, E=512, I=1024, k=8, fmt="fp8_b128",
                             seed=4, zipf=1.2, domains=6, batches=12, pool_slots=160),
    "large_prefill_mxfp4": Workload("large_prefill_mxfp4", T=16384, H=7168, E=256, I=2048, k=8,
                                    fmt="mxfp4", seed=5, zipf=1.0, shared_I=2048),
}


# ----------------------------------------------------------------------------
# seed mixing (splitmix64) so that every stream is addressable on its own
# ----------------------------------------------------------------------------
_M64 = (1 << 64) - 1


def _splitmix64(z: int) -> int:
    z = (z + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def sub_seed(*parts: int) -> int:
    h = 0x1234_5678
    for p in parts:
        h = _splitmix64(h ^ (int(p) & _M64))
    return h & ((1 << 63) - 1)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


# stream tags
_LOGITS, _X, _W, _RANK, _SHARED = 1, 2, 3, 4, 5


# ----------------------------------------------------------------------------
# record layout
# ----------------------------------------------------------------------------
def _round_up(v: int, a: int = ALIGN) -> int:
    return (v + a - 1) // a * a


def section_sizes(fmt: str, H: int, I: int) -> list[tuple[str, int]]:
    """(name, bytes) of each section of one expert record, in record order."""
    if fmt == "bf16":
        return [("w13", 2 * I * H * 2), ("w2", H * I * 2)]
    if fmt == "mxfp4":
        return [("w13", 2 * I * H // 2), ("w13s", 2 * I * H // 32),
                ("w2", H * I // 2), ("w2s", H * I // 32)]
    if fmt == "nvfp4":
        return [("w13", 2 * I * H // 2), ("w13s", 2 * I * H // 16),
                ("w2", H * I // 2), ("w2s", H * I // 16), ("ts", 12)]
    if fmt == "fp8_b128":
        return [("w13", 2 * I * H), ("w13s", (2 * I // 128) * (H // 128) * 4),
                ("w2", H * I), ("w2s", (H // 128) * (I // 128) * 4)]
    raise ValueError(fmt)


def record_layout(fmt: str, H: int, I: int) -> dict:
    offs, pos, payload = {}, 0, 0
    for name, nbytes in section_sizes(fmt, H, I):
        pos = _round_up(pos)
        offs[name] = (pos, nbytes)
        pos += nbytes
        payload += nbytes
    return {"sections": offs, "payload": payload, "stride": _round_up(pos)}


def check_shape(fmt: str, H: int, I: int) -> None:
    blk = {"bf16": 8, "mxfp4": 32, "nvfp4": 16, "fp8_b128": 128}[fmt]
    if H % max(blk, 32) or I % max(blk, 32):
        raise ValueError(f"H={H}, I={I} must be multiples of {max(blk, 32)} for {fmt}")


# ----------------------------------------------------------------------------
# quantizers: float weights -> stored bytes (input production only)
# ----------------------------------------------------------------------------
# E2M1 magnitudes are 0, .5, 1, 1.5, 2, 3, 4, 6 for codes 0..7; the midpoints
# between neighbours decide the nearest code, and a value exactly on a midpoint
# goes to the neighbour with the even code (round half to even).
_E2M1_MID = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _e2m1_encode(v: torch.Tensor) -> torch.Tensor:
    a = v.abs().clamp(max=6.0)
    code = torch.zeros_like(a, dtype=torch.int32)
    for i, t in enumerate(_E2M1_MID):
        above = a > t
        tie_up = (a == t) & ((i + 1) % 2 == 0)
        code += (above | tie_up).to(torch.int32)
    sign = torch.signbit(v)
    return (code | (sign.to(torch.int32) << 3)).to(torch.uint8)


def _pack_nibbles(codes: torch.Tensor) -> torch.Tensor:
    lo = codes[..., 0::2]
    hi = codes[..., 1::2]
    return (lo | (hi << 4)).to(torch.uint8)


def _e4m3_bytes(v: torch.Tensor) -> torch.Tensor:
    v = v.float().clamp(-448.0, 448.0)
    return v.to(torch.float8_e4m3fn).view(torch.uint8)


def _e4m3_as_float(b: torch.Tensor) -> torch.Tensor:
    return b.view(torch.float8_e4m3fn).float()


def quantize_mxfp4(w: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """w [N,K] float -> (packed codes [N,K/2] u8, E8M0 scales [N,K/32] u8).

    OCP MX conversion: shared exponent = floor(log2(block amax)) - 2 (the
    largest E2M1 exponent), elements rounded to nearest-even and saturated."""
    N, K = w.shape
    blk = w.float().reshape(N, K // 32, 32)
    amax = blk.abs().amax(dim=-1)
    e = torch.floor(torch.log2(amax.clamp(min=2.0 ** -126))) - 2.0
    e = e.clamp(-126.0, 127.0)
    scale_byte = (e + 127.0).to(torch.uint8)
    q = blk / torch.exp2(e).unsqueeze(-1)
    codes = _e2m1_encode(q).reshape(N, K)
    return _pack_nibbles(codes), scale_byte


def quantize_nvfp4(w: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor, float]:
    """w [N,K] -> (packed codes [N,K/2], E4M3 block scales [N,K/16], fp32 tensor scale)."""
    N, K = w.shape
    wf = w.float()
    ts = float(wf.abs().amax()) / (6.0 * 448.0)
    if ts == 0.0:
        ts = 1.0
    ts = float(np.float32(ts))
    blk = wf.reshape(N, K // 16, 16)
    amax = blk.abs().amax(dim=-1)
    sb = _e4m3_bytes(amax / (6.0 * ts))
    sbf = _e4m3_as_float(sb)
    denom = (sbf * ts).unsqueeze(-1)
    q = torch.where(denom > 0, blk / torch.where(denom > 0, denom, torch.ones_like(denom)),
                    torch.zeros_like(blk))
    codes = _e2m1_encode(q).reshape(N, K)
    return _pack_nibbles(codes), sb, ts


def quantize_fp8_b128(w: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """w [N,K] -> (E4M3 codes [N,K] u8, fp32 scales [N/128][K/128])."""
    N, K = w.shape
    blk = w.float().reshape(N // 128, 128, K // 128, 128)
    amax = blk.abs().amax(dim=(1, 3))
    s = (amax / 448.0).to(torch.float32)
    s = torch.where(s > 0, s, torch.ones_like(s))
    q = _e4m3_bytes(blk / s[:, None, :, None]).reshape(N, K)
    return q, s.contiguous()


def _bf16_bytes(w: torch.Tensor) -> torch.Tensor:
    return w.to(torch.bfloat16).contiguous().view(torch.uint8).reshape(w.shape[0], -1)


# ----------------------------------------------------------------------------
# expert records
# ----------------------------------------------------------------------------
def expert_float_weights(seed: int, layer: int, e: int, H: int, I: int, device="cpu",
                         std: float = WEIGHT_STD, tag: int = _W):
    g = _gen(sub_seed(seed, tag, layer, e), device)
    w13 = torch.randn((2 * I, H), generator=g, device=device, dtype=torch.float32) * std
    w2 = torch.randn((H, I), generator=g, device=device, dtype=torch.float32) * std
    return w13, w2


def encode_record(fmt: str, w13: torch.Tensor, w2: torch.Tensor) -> torch.Tensor:
    """Float weights of one expert -> one record (uint8 [stride])."""
    I2, H = w13.shape
    I = I2 // 2
    lay = record_layout(fmt, H, I)
    rec = torch.zeros(lay["stride"], dtype=torch.uint8, device=w13.device)

    def put(name, t: torch.Tensor):
        off, nbytes = lay["sections"][name]
        flat = t.contiguous().view(torch.uint8).reshape(-1)
        assert flat.numel() == nbytes, (name, flat.numel(), nbytes)
        rec[off:off + nbytes] = flat

    if fmt == "bf16":
        put("w13", _bf16_bytes(w13))
        put("w2", _bf16_bytes(w2))
    elif fmt == "mxfp4":
        c, s = quantize_mxfp4(w13)
        put("w13", c); put("w13s", s)
        c, s = quantize_mxfp4(w2)
        put("w2", c); put("w2s", s)
    elif fmt == "nvfp4":
        cg, sg, tg = quantize_nvfp4(w13[:I])
        cu, su, tu = quantize_nvfp4(w13[I:])
        put("w13", torch.cat([cg, cu], 0)); put("w13s", torch.cat([sg, su], 0))
        c, s, td = quantize_nvfp4(w2)
        put("w2", c); put("w2s", s)
        put("ts", torch.tensor([tg, tu, td], dtype=torch.float32, device=w13.device))
    elif fmt == "fp8_b128":
        q, s = quantize_fp8_b128(w13)
        put("w13", q); put("w13s", s)
        q, s = quantize_fp8_b128(w2)
        put("w2", q); put("w2s", s)
    else:
        raise ValueError(fmt)
    return rec


def make_expert_records(fmt: str, E: int, H: int, I: int, seed: int, layer: int = 0,
                        device="cpu", experts=None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Records of experts 0..E-1 (or the listed subset) as uint8 [n, stride]."""
    check_shape(fmt, H, I)
    lay = record_layout(fmt, H, I)
    ids = list(range(E)) if experts is None else list(experts)
    if out is None:
        out = torch.empty((len(ids), lay["stride"]), dtype=torch.uint8, device=device)
    for row, e in enumerate(ids):
        w13, w2 = expert_float_weights(seed, layer, e, H, I, device=device)
        out[row] = encode_record(fmt, w13, w2)
    return out


def make_shared_record(seed: int, H: int, I_s: int, device="cpu") -> torch.Tensor:
    w13, w2 = expert_float_weights(seed, 0, 0, H, I_s, device=device, tag=_SHARED)
    return encode_record("bf16", w13, w2).reshape(1, -1)


# ----------------------------------------------------------------------------
# router logits and activations
# ----------------------------------------------------------------------------
def expert_bias(E: int, s: float | None, seed: int, domain: int = 0) -> np.ndarray:
    """Zipf(s) expert bias: b_e = -s * ln(rank_e), ranks a seeded permutation of 1..E,
    so that softmax(b) is the Zipf(s) probability mass over experts."""
    if not s:
        return np.zeros(E, dtype=np.float32)
    rng = np.random.default_rng(sub_seed(seed, _RANK, domain))
    rank = rng.permutation(E) + 1
    return (-s * np.log(rank.astype(np.float64))).astype(np.float32)


def make_logits(wl: Workload, batch: int = 0, T: int | None = None, layer: int = 0) -> np.ndarray:
    """Router logits of one batch: N(0,1) noise + the batch's domain bias.  Layers other
    than 0 (a stack of layers) draw their own noise and their own expert ranking for
    the same domain."""
    T = wl.T if T is None else T
    extra = (layer,) if layer else ()
    rng = np.random.default_rng(sub_seed(wl.seed, _LOGITS, batch, *extra))
    noise = rng.standard_normal((T, wl.E), dtype=np.float32)
    domain = (batch % wl.domains) if wl.domains else 0
    bseed = sub_seed(wl.seed, layer) if layer else wl.seed
    return (noise + expert_bias(wl.E, wl.zipf, bseed, domain)[None, :]).astype(np.float32)


def make_x(wl: Workload, batch: int = 0, T: int | None = None) -> np.ndarray:
    """bf16 activations ~N(0,1), returned as their uint16 bit patterns [T,H]."""
    T = wl.T if T is None else T
    rng = np.random.default_rng(sub_seed(wl.seed, _X, batch))
    v = rng.standard_normal((T, wl.H), dtype=np.float32)
    return torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def algorithmic_expert_bytes(fmt: str, H: int, I: int) -> int:
    return record_layout(fmt, H, I)["payload"]


def describe(wl: Workload) -> dict:
    d = dataclasses.asdict(wl)
    d["record_stride"] = record_layout(wl.fmt, wl.H, wl.I)["stride"]
    d["expert_payload_bytes"] = algorithmic_expert_bytes(wl.fmt, wl.H, wl.I)
    return d


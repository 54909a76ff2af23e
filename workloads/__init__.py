"""Seeded synthetic inputs for the MoE layer, shared by the tests, the smoke check
and the benchmark.

This module holds none of the layer's arithmetic: no router product, no top-k,
no expert product.  It only draws random numbers and stores them in the formats
the layer consumes (fp32, bf16 bit patterns, symmetric int4 with fp16 group-32
scales, symmetric int8 with fp16 per-row scales).  Turning a Gaussian draw into
stored int4/int8 codes is part of producing an input, not of the layer.

Shapes follow the Flash-Next MoE layer on the pages about serving
Qwen3.8-Flash-Next (TandemLLM docs chapter 17, Table 17.1: 512 experts a layer,
10 routed plus 1 shared per token, a 2,560-wide residual stream).  The expert
width 1024 is an assumption; the pages do not state it.

Recipe (every draw seeded; PCG64 streams keyed by (seed, role[, expert])):
  hidden x          ~ N(0, 1)
  router Wr [E, d]  ~ N(0, std = 1/sqrt(d))
  gate/up [F, d]    ~ N(0, std = 1/sqrt(d));  down [d, F] ~ N(0, std = 1/sqrt(F))
  shared expert     same recipe, width Fs
  bf16 storage      round-to-nearest-even of the fp32 draw
  int4 g32          s = fp16(max|w_group|/7), q = clip(rint(w/s), -7, 7); s=0 -> q=0
  int8 per row      s = fp16(max|w_row|/127), q = clip(rint(w/s), -127, 127)
  b-bit g32         s = fp16(max|w_group|/(2^(b-1)-1)), q = clip(rint(w/s), +-(2^(b-1)-1)),
                    b = 2, 3, 5, 6, 7, 8 (one int8 per code)
  mxfp4             E = ceil(log2(max|w_group| / 6)) (E8M0 byte E + 127; 0 for a
                    zero group), code = the e2m1 magnitude nearest |w| / 2^E
                    (a midpoint goes to the smaller one) with w's sign
  Zipf bias         bias_e = -c * 1.1 * ln(r_e), r a seeded permutation of 1..E,
                    c = ZIPF_C (chosen so the hottest expert gets about 10x the
                    mean load on the seeded T=16384 input).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

F32, BF16, I4G32, I8ROW = "f32", "bf16", "i4g32", "i8row"
# b-bit group-32 formats: symmetric codes, one int8 each, fp16 scale per 32 along K
IG32 = {2: "i2g32", 3: "i3g32", 5: "i5g32", 6: "i6g32", 7: "i7g32", 8: "i8g32"}
IG32_BITS = {v: b for b, v in IG32.items()}
# OCP MX FP4 (e2m1 codes + E8M0 scale per 32 along K), W4A4 routed experts
MXFP4 = "mxfp4"
ZIPF_S = 1.1
ZIPF_C = 0.22


@dataclass(frozen=True)
class LayerConfig:
    name: str
    index: int
    T: int
    d: int
    E: int
    k: int
    F: int
    n_shared: int
    Fs: int
    act: str          # hidden / output dtype: f32 | bf16
    router: str       # router weight dtype: f32 | bf16
    expert: str       # routed expert weights: f32 | bf16 | i4g32 | i{2..8}g32 | mxfp4
    shared: str       # shared expert weights: f32 | bf16 | i8row
    zipf: bool = False
    extra_T: tuple = field(default_factory=tuple)

    @property
    def seed(self) -> int:
        return 0x5EED0000 + self.index

    def with_T(self, T: int) -> "LayerConfig":
        return replace(self, T=T)


CONFIGS = {
    "tiny_fp32": LayerConfig("tiny_fp32", 0, T=64, d=256, E=16, k=2, F=128, n_shared=0, Fs=0,
                             act=F32, router=F32, expert=F32, shared=F32),
    "bf16_T512": LayerConfig("bf16_T512", 1, T=512, d=2560, E=512, k=10, F=1024, n_shared=1,
                             Fs=1024, act=BF16, router=BF16, expert=BF16, shared=BF16),
    "int4_T4096": LayerConfig("int4_T4096", 2, T=4096, d=2560, E=512, k=10, F=1024, n_shared=1,
                              Fs=1024, act=BF16, router=BF16, expert=I4G32, shared=I8ROW),
    "int4_decode": LayerConfig("int4_decode", 3, T=16, d=2560, E=512, k=10, F=1024, n_shared=1,
                               Fs=1024, act=BF16, router=BF16, expert=I4G32, shared=I8ROW,
                               extra_T=(32,)),
    "zipf_T16384": LayerConfig("zipf_T16384", 4, T=16384, d=2560, E=512, k=10, F=1024,
                               n_shared=1, Fs=1024, act=BF16, router=BF16, expert=I4G32,
                               shared=I8ROW, zipf=True),
}


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_i4g32(w: np.ndarray):
    """[rows, K] float -> (packed uint8 [rows, K/2], fp16 bits [rows, K/32])."""
    rows, K = w.shape
    assert K % 32 == 0
    g = w.reshape(rows, K // 32, 32).astype(np.float32)
    s16 = (np.abs(g).max(axis=2) / np.float32(7.0)).astype(np.float16)
    s = s16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(g / np.where(s > 0, s, 1)), 0)
    q = np.clip(q, -7, 7).astype(np.int8).reshape(rows, K)
    return pack_int4(q), s16.view(np.uint16)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """int codes in [-8, 7], [rows, K] -> bytes with element 2j in the low nibble."""
    u = (np.asarray(q).astype(np.int16) & 15).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def quantize_ig32(w: np.ndarray, b: int):
    """[rows, K] float -> (int8 codes [rows, K] in [-(2^(b-1)-1), 2^(b-1)-1],
    fp16 bits [rows, K/32]); s = fp16(max|w_group| / (2^(b-1)-1))."""
    rows, K = w.shape
    assert K % 32 == 0
    qmax = (1 << (b - 1)) - 1
    g = w.reshape(rows, K // 32, 32).astype(np.float32)
    s16 = (np.abs(g).max(axis=2) / np.float32(qmax)).astype(np.float16)
    s = s16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(g / np.where(s > 0, s, 1)), 0)
    q = np.clip(q, -qmax, qmax).astype(np.int8).reshape(rows, K)
    return q, s16.view(np.uint16)


# e2m1 magnitudes by code (bits 2..0) and the midpoints between neighbours
_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def quantize_mxfp4(w: np.ndarray):
    """[rows, K] float -> (packed e2m1 uint8 [rows, K/2], E8M0 uint8 [rows, K/32])."""
    rows, K = w.shape
    assert K % 32 == 0
    g = w.reshape(rows, K // 32, 32).astype(np.float64)
    amax = np.abs(g).max(axis=2)
    m, ex = np.frexp(amax / 6.0)                   # amax/6 = m 2^ex, m in [0.5, 1)
    E = np.where(amax > 0, ex - (m == 0.5), -127)  # ceil(log2(amax / 6))
    E = np.clip(E, -127, 127)
    a = np.abs(g) / np.ldexp(1.0, E)[..., None]
    code = np.searchsorted(_E2M1_MID, a, side="left").astype(np.uint8)
    code |= np.where((g < 0) & (code > 0), 8, 0).astype(np.uint8)
    code = code.reshape(rows, K)
    return (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8), (E + 127).astype(np.uint8)


def quantize_i8row(w: np.ndarray):
    """[rows, K] float -> (int8 [rows, K], fp16 bits [rows])."""
    w = w.astype(np.float32)
    s16 = (np.abs(w).max(axis=1) / np.float32(127.0)).astype(np.float16)
    s = s16.astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(w / np.where(s > 0, s, 1)), 0)
    return np.clip(q, -127, 127).astype(np.int8), s16.view(np.uint16)


def store(w: np.ndarray, fmt: str):
    """Store an fp32 matrix [rows, K] in ``fmt``; returns (q, scales or None)."""
    if fmt == F32:
        return np.ascontiguousarray(w, np.float32), None
    if fmt == BF16:
        return to_bf16_bits(w), None
    if fmt == I4G32:
        return quantize_i4g32(w)
    if fmt == I8ROW:
        return quantize_i8row(w)
    if fmt in IG32_BITS:
        return quantize_ig32(w, IG32_BITS[fmt])
    if fmt == MXFP4:
        return quantize_mxfp4(w)
    raise ValueError(fmt)


def _normal(rng, shape, std):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def expert_weights(cfg: LayerConfig, e: int):
    """Stored (gate, up, down) of routed expert e; each is (q, scales)."""
    rng = _rng(cfg.seed, 2, e)
    wg = _normal(rng, (cfg.F, cfg.d), 1.0 / np.sqrt(cfg.d))
    wu = _normal(rng, (cfg.F, cfg.d), 1.0 / np.sqrt(cfg.d))
    wd = _normal(rng, (cfg.d, cfg.F), 1.0 / np.sqrt(cfg.F))
    return store(wg, cfg.expert), store(wu, cfg.expert), store(wd, cfg.expert)


def shared_weights(cfg: LayerConfig):
    rng = _rng(cfg.seed, 3)
    sg = _normal(rng, (cfg.Fs, cfg.d), 1.0 / np.sqrt(cfg.d))
    su = _normal(rng, (cfg.Fs, cfg.d), 1.0 / np.sqrt(cfg.d))
    sd = _normal(rng, (cfg.d, cfg.Fs), 1.0 / np.sqrt(cfg.Fs))
    return store(sg, cfg.shared), store(su, cfg.shared), store(sd, cfg.shared)


def hidden(cfg: LayerConfig, T: int | None = None):
    T = cfg.T if T is None else T
    x = _rng(cfg.seed, 0, T).standard_normal((T, cfg.d), dtype=np.float32)
    return store(x, cfg.act)[0]


def router_weights(cfg: LayerConfig):
    wr = _normal(_rng(cfg.seed, 1), (cfg.E, cfg.d), 1.0 / np.sqrt(cfg.d))
    return store(wr, cfg.router)[0]


def zipf_bias(cfg: LayerConfig, c: float = ZIPF_C):
    if not cfg.zipf:
        return None
    r = _rng(cfg.seed, 4).permutation(cfg.E) + 1
    return (-c * ZIPF_S * np.log(r.astype(np.float64))).astype(np.float32)


def stack_experts(cfg: LayerConfig, experts=None, threads: int | None = None) -> dict:
    """All routed experts stacked: wg/wu [E, F, ...], wd [E, d, ...] (+ _s scales)."""
    E = cfg.E
    experts = range(E) if experts is None else experts
    threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda e: expert_weights(cfg, e), experts))
    out = {}
    for i, name in enumerate(("wg", "wu", "wd")):
        out[name] = np.stack([p[i][0] for p in parts])
        if parts[0][i][1] is not None:
            out[name + "_s"] = np.stack([p[i][1] for p in parts])
    return out


def generate(cfg: LayerConfig, T: int | None = None, threads: int | None = None) -> dict:
    """Every stored input of one layer call, as numpy arrays (canonical layouts)."""
    inp = {"x": hidden(cfg, T), "wr": router_weights(cfg), "bias": zipf_bias(cfg)}
    inp.update(stack_experts(cfg, threads=threads))
    if cfg.n_shared:
        (sg, sgs), (su, sus), (sd, sds) = shared_weights(cfg)
        inp.update(sg=sg, sg_s=sgs, su=su, su_s=sus, sd=sd, sd_s=sds)
    return inp

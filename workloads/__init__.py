"""Seeded synthetic inputs for the pair-biased attention workloads.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the method's arithmetic, so both the fp64 oracle (under
``oracle/``) and the HIP path can be fed from it without sharing any code.

Workloads (all values standard normal, as the task's configurations state):

* ``tiny_fp32``       rows B=32, tokens N=32, heads H=4, d=32, fp32,
                       key mask 0 on 3 of the 32 keys (about 10 %, drawn).
* ``tri_attn_n384``   triangle attention: B=384 rows, N=384, H=4, d=32, bf16,
                       last 5 % of keys masked (keys 365..383).
* ``pairformer_apb``  Pairformer AttentionPairBias: B=1, N=768, H=16, d=24, bf16.
* ``dit_apb_x48``     diffusion-transformer AttentionPairBias: B=48 noise copies,
                       N=384, H=16, d=48, bf16, one bias shared by the copies.
* ``msa_pwa``         MSA pair-weighted averaging: S=1024 MSA rows, N=768,
                       H=8, d=32, bf16, no QK term.
* ``msa_row_attn``    MSA row attention with pair bias, the operation the
                       pair-weighted average replaces: B=1024 MSA rows,
                       N=768, H=8, d=32, bf16, one bias shared by the rows,
                       last 5 % of keys masked (keys 730..767).

* ``bias_proj_tri_n384``   pair-bias projection Linear(LayerNorm(z)) for the
                       triangle attention above: z [384, 384, c=128] bf16,
                       H=4 heads.
* ``bias_proj_pairformer`` the same projection for the Pairformer pair bias:
                       z [768, 768, c=128] bf16, H=16 heads.
* ``local_atom_attn``  windowed (sequence-local) atom attention with pair
                       bias: B=48 diffusion copies, N=3072 atoms (384 tokens at
                       8 atoms each), H=4, d=32, bf16, blocks of 32 queries
                       each attending 128 keys, local bias [4, 96, 32, 128],
                       last 5 % of atoms masked (154 of 3072).
  Windowed-attention draw order: Q, K, V, G, bias, dO, then the mask.
  Projection inputs: z = standard normal plus a standard-normal shift per
  pair position (so that the LayerNorm has a mean to remove), rounded to
  bf16; gamma = 1 + 0.25 N(0,1), beta = 0.25 N(0,1) and w = N(0,1)/sqrt(c)
  in float32; dbias standard normal in bf16.  Draw order: z, shift, gamma,
  beta, w, dbias.

Where the workloads come from: the AlphaFold3 open-source implementation page
(molayo1419.me, "Show HN: AlphaFold3 open-source implementation"), sections
"Model Efficiency" (triangle attention reused from OpenFold; the 48 diffusion
copies handled as an extra batch dimension) and "MSA Pair Averaging Efficiency"
(the pair-weighted average that replaces MSA row attention, and with it
the row attention itself, whose pair-biased form the page names as the
DS4Sci MSARowAttentionWithPairBias kernel).

Draw order per workload (generator ``numpy.random.default_rng(seed)``):
attention: Q, K, V, G, bias, dO, then the masked key indices (tiny case only);
pair-weighted average: b, V, G, dO.
"""
from __future__ import annotations

import dataclasses
import numpy as np

__all__ = [
    "AttnConfig", "PwaConfig", "ProjConfig", "LocalConfig", "CONFIGS", "ATTN_CONFIGS", "PWA_CONFIGS", "PROJ_CONFIGS", "LOCAL_CONFIGS",
    "bf16_round_bits", "bf16_bits_to_f32", "attention_inputs", "pwa_inputs",
    "scaled_attention_config", "scaled_pwa_config", "bias_proj_inputs", "local_inputs",
]


@dataclasses.dataclass(frozen=True)
class AttnConfig:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "f32" or "bf16"
    mask: str             # "none", "random:<count>", "tail:<count>"
    seed: int

    @property
    def kind(self) -> str:
        return "attention"


@dataclasses.dataclass(frozen=True)
class PwaConfig:
    name: str
    S: int
    N: int
    H: int
    d: int
    dtype: str
    mask: str
    seed: int

    @property
    def kind(self) -> str:
        return "pwa"


@dataclasses.dataclass(frozen=True)
class ProjConfig:
    name: str
    N: int
    H: int
    c: int
    seed: int

    @property
    def kind(self) -> str:
        return "bias_proj"


@dataclasses.dataclass(frozen=True)
class LocalConfig:
    name: str
    B: int
    H: int
    N: int
    d: int
    mask: str
    seed: int
    dtype: str = "bf16"

    @property
    def kind(self) -> str:
        return "local_attention"


CONFIGS = {
    "tiny_fp32": AttnConfig("tiny_fp32", B=32, H=4, N=32, d=32, dtype="f32",
                            mask="random:3", seed=1001),
    "tri_attn_n384": AttnConfig("tri_attn_n384", B=384, H=4, N=384, d=32, dtype="bf16",
                                mask="tail:19", seed=1002),
    "pairformer_apb": AttnConfig("pairformer_apb", B=1, H=16, N=768, d=24, dtype="bf16",
                                 mask="none", seed=1003),
    "dit_apb_x48": AttnConfig("dit_apb_x48", B=48, H=16, N=384, d=48, dtype="bf16",
                              mask="none", seed=1004),
    "msa_pwa": PwaConfig("msa_pwa", S=1024, N=768, H=8, d=32, dtype="bf16",
                         mask="none", seed=1005),
    "msa_row_attn": AttnConfig("msa_row_attn", B=1024, H=8, N=768, d=32, dtype="bf16",
                               mask="tail:38", seed=1006),
    "bias_proj_tri_n384": ProjConfig("bias_proj_tri_n384", N=384, H=4, c=128, seed=1007),
    "bias_proj_pairformer": ProjConfig("bias_proj_pairformer", N=768, H=16, c=128, seed=1008),
    "local_atom_attn": LocalConfig("local_atom_attn", B=48, H=4, N=3072, d=32, mask="tail:154", seed=1009),
}
ATTN_CONFIGS = [c for c in CONFIGS.values() if c.kind == "attention"]
PWA_CONFIGS = [c for c in CONFIGS.values() if c.kind == "pwa"]
PROJ_CONFIGS = [c for c in CONFIGS.values() if c.kind == "bias_proj"]
LOCAL_CONFIGS = [c for c in CONFIGS.values() if c.kind == "local_attention"]


def scaled_attention_config(cfg: AttnConfig, **overrides) -> AttnConfig:
    """Same workload recipe with some sizes replaced (for reduced parity cases)."""
    return dataclasses.replace(cfg, **overrides)


def scaled_pwa_config(cfg: PwaConfig, **overrides) -> PwaConfig:
    return dataclasses.replace(cfg, **overrides)


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); return raw uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _store(x: np.ndarray, dtype: str, want64: bool = True):
    """Return (storage array, float64 copy of the exact stored values or None)."""
    if dtype == "f32":
        s = np.ascontiguousarray(x, dtype=np.float32)
        return s, (s.astype(np.float64) if want64 else None)
    if dtype == "bf16":
        bits = bf16_round_bits(x)
        return bits, (bf16_bits_to_f32(bits).astype(np.float64) if want64 else None)
    raise ValueError(f"unknown dtype {dtype}")


def _key_mask(spec: str, N: int, rng) -> np.ndarray | None:
    if spec == "none":
        return None
    kind, _, count = spec.partition(":")
    count = int(count)
    keep = np.ones(N, dtype=np.uint8)
    if kind == "random":
        idx = rng.choice(N, size=min(count, N), replace=False)
        keep[idx] = 0
    elif kind == "tail":
        if count > 0:
            keep[N - min(count, N):] = 0
    else:
        raise ValueError(f"unknown mask spec {spec}")
    return keep


def attention_inputs(cfg: AttnConfig, seed: int | None = None, with_grad: bool = True,
                     with_f64: bool = True):
    """Draw one attention workload.

    Returns a dict with storage arrays (``q``, ``k``, ``v``, ``g``, ``bias``,
    ``dout``: uint16 bf16 bits or float32) and their exact float64 values
    (``q64`` ...), plus ``key_mask`` (uint8 [N], 1 = keep, or None).
    Layouts: q, k, v, g, dout [B, H, N, d]; bias [H, N, N].
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, H, N, d = cfg.B, cfg.H, cfg.N, cfg.d
    out = {"cfg": cfg}
    names = ["q", "k", "v", "g", "bias"] + (["dout"] if with_grad else [])
    for name in names:
        shape = (H, N, N) if name == "bias" else (B, H, N, d)
        x = rng.standard_normal(shape, dtype=np.float32)
        out[name], out[name + "64"] = _store(x, cfg.dtype, with_f64)
        del x
    out["key_mask"] = _key_mask(cfg.mask, N, rng)
    return out


def pwa_inputs(cfg: PwaConfig, seed: int | None = None, with_grad: bool = True,
               with_f64: bool = True):
    """Draw one pair-weighted-average workload.

    Layouts: b [H, N, N]; v, g, dout [S, N, H, d] (MSA row, token, head, channel).
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    S, N, H, d = cfg.S, cfg.N, cfg.H, cfg.d
    out = {"cfg": cfg}
    names = ["b", "v", "g"] + (["dout"] if with_grad else [])
    for name in names:
        shape = (H, N, N) if name == "b" else (S, N, H, d)
        x = rng.standard_normal(shape, dtype=np.float32)
        out[name], out[name + "64"] = _store(x, cfg.dtype, with_f64)
        del x
    out["key_mask"] = _key_mask(cfg.mask, N, rng)
    return out


def bias_proj_inputs(cfg: ProjConfig, seed: int | None = None, with_f64: bool = True):
    """Draw one pair-bias projection workload.

    Returns ``z`` (uint16 bf16 bits, [N, N, c]), ``gamma``, ``beta`` ([c]) and
    ``w`` ([H, c]) as float32, ``dbias`` (bf16 bits, [H, N, N]), and float64
    copies of the exact stored values (``z64`` ...).
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    N, H, c = cfg.N, cfg.H, cfg.c
    out = {"cfg": cfg}
    z = rng.standard_normal((N, N, c), dtype=np.float32)
    z += rng.standard_normal((N, N, 1), dtype=np.float32)
    out["z"], out["z64"] = _store(z, "bf16", with_f64)
    del z
    out["gamma"], out["gamma64"] = _store(1.0 + 0.25 * rng.standard_normal(c), "f32")
    out["beta"], out["beta64"] = _store(0.25 * rng.standard_normal(c), "f32")
    out["w"], out["w64"] = _store(rng.standard_normal((H, c)) / np.sqrt(c), "f32")
    out["dbias"], out["dbias64"] = _store(rng.standard_normal((H, N, N), dtype=np.float32), "bf16", with_f64)
    return out


def local_inputs(cfg: LocalConfig, seed: int | None = None, with_grad: bool = True, with_f64: bool = True):
    """Draw one windowed-attention workload.

    Layouts: q, k, v, g, dout [B, H, N, d]; bias [H, ceil(N/32), 32, 128]
    (head, query block, query in block, window slot); key_mask [N] or None.
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, H, N, d = cfg.B, cfg.H, cfg.N, cfg.d
    out = {"cfg": cfg}
    names = ["q", "k", "v", "g", "bias"] + (["dout"] if with_grad else [])
    for name in names:
        shape = (H, -(-N // 32), 32, 128) if name == "bias" else (B, H, N, d)
        x = rng.standard_normal(shape, dtype=np.float32)
        out[name], out[name + "64"] = _store(x, cfg.dtype, with_f64)
        del x
    out["key_mask"] = _key_mask(cfg.mask, N, rng)
    return out

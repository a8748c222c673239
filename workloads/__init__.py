"""Seeded synthetic inputs for the draft-tree build and target-side verify path.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark.  It only *draws inputs*: random logits, the processed probability
rows a caller hands to the verify step, prefix lengths, slot/page maps, bf16
Q/K/V, uniforms and the TLI vocabulary pairing.  It performs none of the
method's own arithmetic (no top-k, no tree build, no attention, no accept walk,
no compaction, no remap, no GEMM) and imports neither the oracle nor the HIP
binding.

Recipes (every config draws from one ``numpy.random.SeedSequence`` spawned into
named child streams in a fixed order, each drawn with ``Generator(PCG64)``):

* probabilities are ``softmax(logits / T)`` evaluated in float64 from the fp32
  logits and rounded once to fp32 -- the method consumes processed
  distributions supplied by the caller (zero-to-sglang ch.10, section 5.1);
* uniforms are ``k * 2**-24`` with an integer ``k`` in ``[0, 2**24)`` so that
  every uniform carries at most 24 significant bits;
* bf16 tensors are fp32 normals rounded to bf16 (round-to-nearest-even) and are
  stored as their raw ``uint16`` bit patterns;
* page size 1 pools use a shuffled slot permutation; page size > 1 pools use a
  shuffled permutation of physical pages (non-contiguous page chains).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Config",
    "CONFIGS",
    "get_config",
    "generate",
    "softmax_rows",
    "to_bf16_bits",
    "bf16_bits_to_f32",
    "uniforms24",
    "num_draft_rows",
    "pool_size",
]

# Order in which the named child streams are spawned; never reorder (it would
# change every input of every config).
_STREAMS = (
    "draft_logits",
    "target_logits",
    "root",
    "prefix_len",
    "slots",
    "q",
    "k",
    "v",
    "u_accept",
    "u_draw",
    "tli_pairing",
    "tli_hidden",
    "tli_weight",
    "tli_draft_logits",
    "extra",
)


@dataclasses.dataclass(frozen=True)
class Config:
    """Shape and distribution of one synthetic workload."""

    name: str
    seed: int
    B: int                      # batch (requests)
    k: int                      # topk per draft step
    S: int                      # num_steps (draft steps)
    N: int                      # num_draft_tokens, root included
    V: int                      # vocab of the rows the verify reads (target vocab)
    mode: str                   # "greedy" | "stochastic"
    logit_std: float            # std of the fp32 logits
    temperature: float = 1.0
    # tree-verify attention (None: the config has no attention stage)
    Hq: Optional[int] = None
    Hkv: Optional[int] = None
    D: Optional[int] = None
    page: int = 1
    L_min: Optional[int] = None
    L_max: Optional[int] = None
    layers: int = 1
    # TLI (heterogeneous vocabularies)
    V_draft: Optional[int] = None
    K_inter: Optional[int] = None
    H_draft: Optional[int] = None
    w_std: float = 0.02

    @property
    def R(self) -> int:
        return num_draft_rows(self.k, self.S)

    @property
    def M(self) -> int:
        return pool_size(self.k, self.S)

    @property
    def has_attention(self) -> bool:
        return self.Hq is not None

    @property
    def is_tli(self) -> bool:
        return self.V_draft is not None

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def num_draft_rows(k: int, S: int) -> int:
    """Draft distribution rows per request: the root's, then one per frontier
    slot of every draft step but the last."""
    return 1 + (S - 1) * k


def pool_size(k: int, S: int) -> int:
    """Candidates produced by the draft steps: k at the first step, k*k after."""
    return k + (S - 1) * k * k


CONFIGS: Dict[str, Config] = {
    # Tiny EAGLE tree verify (one seed, greedy, page size 1).
    "c1": Config(name="c1", seed=1001, B=2, k=2, S=3, N=6, V=1000, mode="greedy",
                 logit_std=2.0, Hq=4, Hkv=4, D=64, page=1, L_min=256, L_max=256),
    # Linear (topk=1) stochastic verify, no attention shape given.
    "c2": Config(name="c2", seed=1002, B=16, k=1, S=4, N=5, V=128256, mode="stochastic",
                 logit_std=3.0, temperature=1.0),
    # EAGLE-2 tree verify with the Llama-3-8B attention shape (the metric's workload).
    "c3": Config(name="c3", seed=1003, B=32, k=8, S=5, N=64, V=128256, mode="greedy",
                 logit_std=3.0, Hq=32, Hkv=8, D=128, page=1, L_min=512, L_max=4096),
    # Paged tree verify, page size 16, stochastic at T=0.7.
    "c4": Config(name="c4", seed=1004, B=64, k=4, S=4, N=32, V=128256, mode="stochastic",
                 logit_std=3.0, temperature=0.7, Hq=32, Hkv=8, D=128, page=16,
                 L_min=1024, L_max=8192),
    # TLI heterogeneous-vocabulary draft step plus linear stochastic verify.
    "c5": Config(name="c5", seed=1005, B=64, k=1, S=4, N=5, V=128256, mode="stochastic",
                 logit_std=3.0, temperature=1.0, V_draft=151936, K_inter=60000,
                 H_draft=896, w_std=0.02),
}


def get_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    return cfg.replace(**overrides) if overrides else cfg


# ----------------------------------------------------------------------------
# elementary draws
# ----------------------------------------------------------------------------

def _streams(seed: int) -> Dict[str, np.random.Generator]:
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.Generator(np.random.PCG64(ss)) for name, ss in zip(_STREAMS, children)}


def softmax_rows(logits: np.ndarray, temperature: float = 1.0, chunk_rows: int = 32) -> np.ndarray:
    """Processed distribution handed to the verify step: softmax(logits / T)
    along the last axis, evaluated in float64 and rounded once to fp32."""
    x = np.asarray(logits, dtype=np.float32)
    flat = x.reshape(-1, x.shape[-1])
    out = np.empty(flat.shape, dtype=np.float32)
    buf = np.empty((min(chunk_rows, max(1, flat.shape[0])), flat.shape[1]), dtype=np.float64)
    inv_t = 1.0 / float(temperature)
    for s in range(0, flat.shape[0], chunk_rows):
        n = min(chunk_rows, flat.shape[0] - s)
        z = buf[:n]
        z[...] = flat[s:s + n]
        if inv_t != 1.0:
            z *= inv_t
        z -= z.max(axis=1, keepdims=True)
        np.exp(z, out=z)
        z /= z.sum(axis=1, keepdims=True)
        out[s:s + n] = z
    return out.reshape(x.shape)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def uniforms24(rng: np.random.Generator, shape) -> np.ndarray:
    """fp32 uniforms k * 2**-24, k integer in [0, 2**24)."""
    k = rng.integers(0, 1 << 24, size=shape, dtype=np.int64)
    return (k.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def _normal_f32(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _normal_bf16(rng: np.random.Generator, shape, std: float = 1.0, chunk: int = 1 << 24) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        out[s:s + m] = to_bf16_bits(_normal_f32(rng, (m,), std))
    return out.reshape(shape)


# ----------------------------------------------------------------------------
# per-config generation
# ----------------------------------------------------------------------------

def _paged_layout(cfg: Config, rng: np.random.Generator, prefix_len: np.ndarray,
                  slack_pages: int = 8):
    """Physical placement of every request's logical positions 0 .. L_b+N-1.

    Returns ``(page_table [B, max_pages] int32 (-1 = unused), num_pages)``.
    With page size 1 a "page" is one slot and the table is the slot map.
    """
    P = cfg.page
    need = (prefix_len.astype(np.int64) + cfg.N + P - 1) // P           # pages per request
    max_pages = int(need.max())
    total = int(need.sum()) + slack_pages
    perm = rng.permutation(total).astype(np.int32)
    table = np.full((cfg.B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(cfg.B):
        n = int(need[b])
        table[b, :n] = perm[off:off + n]
        off += n
    return table, total


def generate(cfg: Config, *, with_attention: bool = True, with_rows: bool = True,
             with_logits: bool = False) -> Dict[str, np.ndarray]:
    """Draw every input of ``cfg``.  Large configs take seconds.

    Keys (present when the config has the stage):
      draft_probs [B,R,V] f32 -- processed draft distributions (A1 input, q rows)
      draft_logits [B,R,V] f32 -- the logits they are softmax(. / T) of (with_logits)
      target_logits [B,N,V] f32 -- stochastic: the logits p is softmax(. / T) of (with_logits)
      target      [B,N,V] f32 -- greedy: raw logits; stochastic: processed p
      root_token [B] i32, prefix_len [B] i32
      u_accept, u_draw [B,N] f32 (stochastic)
      q [B,N,Hq,D], k_pool/v_pool [slots,Hkv,D] (bf16 bits, uint16), page_table [B,max_pages] i32
      tli_*: inter_ids [K], tgt_ids [K], fallback, hidden [S,B,H] bf16, weight [K,H] bf16,
             q_pruned [B,R,K] f32
    """
    rs = _streams(cfg.seed)
    out: Dict[str, np.ndarray] = {}
    B, N, V, R = cfg.B, cfg.N, cfg.V, cfg.R

    out["root_token"] = rs["root"].integers(0, V, size=B, dtype=np.int64).astype(np.int32)
    if cfg.L_min is not None:
        pl = rs["prefix_len"].integers(cfg.L_min, cfg.L_max + 1, size=B, dtype=np.int64)
    else:
        pl = np.zeros(B, dtype=np.int64)
    out["prefix_len"] = pl.astype(np.int32)

    if with_rows:
        if cfg.is_tli:
            # The draft proposes over the K intersection ids; its processed
            # rows are scattered into target-vocab rows by the remap stage.
            dl = _normal_f32(rs["tli_draft_logits"], (B, R, cfg.K_inter), cfg.logit_std)
            out["q_pruned"] = softmax_rows(dl, cfg.temperature)
            del dl
        else:
            dl = _normal_f32(rs["draft_logits"], (B, R, V), cfg.logit_std)
            out["draft_probs"] = softmax_rows(dl, cfg.temperature)
            if with_logits:
                out["draft_logits"] = dl
            del dl
        tl = _normal_f32(rs["target_logits"], (B, N, V), cfg.logit_std)
        if cfg.mode == "greedy":
            out["target"] = tl
        else:
            out["target"] = softmax_rows(tl, cfg.temperature)
            if with_logits:
                out["target_logits"] = tl
            del tl
        if cfg.mode == "stochastic":
            out["u_accept"] = uniforms24(rs["u_accept"], (B, N))
            out["u_draw"] = uniforms24(rs["u_draw"], (B, N))

    if cfg.has_attention and with_attention:
        table, num_pages = _paged_layout(cfg, rs["slots"], pl)
        out["page_table"] = table
        slots = num_pages * cfg.page
        out["q"] = _normal_bf16(rs["q"], (B, N, cfg.Hq, cfg.D))
        out["k_pool"] = _normal_bf16(rs["k"], (slots, cfg.Hkv, cfg.D))
        out["v_pool"] = _normal_bf16(rs["v"], (slots, cfg.Hkv, cfg.D))

    if cfg.is_tli:
        pr = rs["tli_pairing"]
        inter = np.sort(pr.choice(cfg.V_draft, size=cfg.K_inter, replace=False)).astype(np.int32)
        tgt = pr.choice(cfg.V, size=cfg.K_inter, replace=False).astype(np.int32)
        # fallback: a draft id outside the intersection
        mask = np.ones(cfg.V_draft, dtype=bool)
        mask[inter] = False
        outside = np.flatnonzero(mask)
        out["inter_ids"] = inter
        out["tgt_ids"] = tgt
        out["fallback"] = np.int32(outside[pr.integers(0, outside.size)])
        out["hidden"] = _normal_bf16(rs["tli_hidden"], (cfg.S, B, cfg.H_draft))
        out["weight"] = _normal_bf16(rs["tli_weight"], (cfg.K_inter, cfg.H_draft), cfg.w_std)
    return out


def sample_tokens(rng: np.random.Generator, V: int, n: int) -> np.ndarray:
    """Uniform token ids (used for id-remap inputs)."""
    return rng.integers(0, V, size=n, dtype=np.int64).astype(np.int32)


def extra_rng(cfg: Config, salt: int = 0) -> np.random.Generator:
    """A further seeded stream of ``cfg`` for test-only draws."""
    ss = np.random.SeedSequence([cfg.seed, 0xE7A, salt])
    return np.random.Generator(np.random.PCG64(ss))

"""Seeded synthetic workloads standing in for the NanoGPT-256 caches and the
larger GQA caches the PGKQ path is measured on.

Recipe (identical for every consumer):

* ``SeedSequence(20261010 + config_id)`` spawns eight children, in this order:
  channel scales, outlier channel indices, keys, queries, values, RHT signs,
  QJL projection, value QJL projection (the first seven are the same as when
  seven were spawned).  The key and value children each spawn one grandchild per
  (sequence, kv-head) stream, so any stream can be regenerated on its own.
  Every child drives a ``numpy.random.Generator(PCG64(child))``.
* channel scale[h, c] = exp(0.5 * N(0, 1)); ``n_outliers`` channels per kv-head,
  drawn without replacement, are multiplied by ``outlier_mult``.
* K[b, h, t, c] = scale[h, c] * N(0, 1), cast to the key dtype (fp32 or fp16).
* q ~ N(0, 1), cast to the query dtype (fp32, or bf16 by round-to-nearest-even).
* V ~ N(0, 1), cast to fp16.
* RHT signs: Rademacher +-1 per (kv-head, channel), int8.
* QJL projection S[h, j, c] ~ N(0, 1), cast to fp32, one m x d matrix per kv-head;
  the value projection (for coded values) likewise, d x d.

Only draws and dtype casts live here: nothing of the method's arithmetic.
"""

from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

BASE_SEED = 20261010
_CHILDREN = ("scales", "outliers", "keys", "queries", "values", "signs", "proj", "proj_v")


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    config_id: int
    n_seq: int
    n_q: int
    n_kv: int
    n_tokens: int
    head_dim: int
    b_main: int
    b_angle: int
    qjl_m: int
    k_dtype: str  # "f32" | "f16"
    q_dtype: str  # "f32" | "bf16"
    n_outliers: int
    outlier_mult: float
    reorder: bool = False
    n_splits: int = 0
    description: str = ""
    layers: int = 1  # model layers flattened into the kv-heads (cache tokens count each layer)

    @property
    def group(self) -> int:
        return self.n_q // self.n_kv

    @property
    def n_streams(self) -> int:
        return self.n_seq * self.n_kv

    @property
    def proj_rows(self) -> int:
        # the projection is drawn even when QJL is off so that every other
        # input of a configuration stays the same across its variants
        return self.qjl_m if self.qjl_m > 0 else self.head_dim

    def with_(self, **kw) -> "WorkloadConfig":
        return replace(self, **kw)


CONFIGS = {
    # NanoGPT-256 cache, one decode step: 6 layers x 4 heads flattened into 24
    # kv-heads (= query heads), head_dim 64, 128 cached tokens.
    "nano_t128": WorkloadConfig("nano_t128", 1, 1, 24, 24, 128, 64, 3, 2, 64, "f32", "f32", 2, 8.0,
                         description="NanoGPT-256 cache, 6Lx4H, d64, T128, B1, b3/2, QJL m64", layers=6),
    # Full NanoGPT-256 context, batch 64.
    "nano_b64_t512": WorkloadConfig("nano_b64_t512", 2, 64, 24, 24, 512, 64, 3, 2, 64, "f32", "f32", 2, 8.0,
                          description="NanoGPT-256 full context, B64, d64, T512, b3/2, QJL m64", layers=6),
    "nano_b64_t512_b4": WorkloadConfig("nano_b64_t512_b4", 2, 64, 24, 24, 512, 64, 4, 3, 0, "f32", "f32", 2, 8.0,
                          description="NanoGPT-256 full context, B64, d64, T512, b4/3, no QJL", layers=6),
    # GQA decode at scale.
    "gqa_b16_t32k": WorkloadConfig("gqa_b16_t32k", 3, 16, 32, 8, 32768, 128, 3, 2, 128, "f16", "bf16", 4, 10.0,
                         n_splits=8,
                         description="GQA 32q/8kv, d128, T32768, B16, b3/2, QJL m128, split-K"),
    # Bulk encode: the 4 194 304 keys of the 32k-token GQA cache, with the channel reorder step.
    "gqa_b16_t32k_encode": WorkloadConfig("gqa_b16_t32k_encode", 3, 16, 32, 8, 32768, 128, 3, 2, 128, "f16", "bf16", 4, 10.0,
                         reorder=True,
                         description="bulk encode of 4194304 fp16 keys, d128, reorder on, b3/2, QJL m128"),
    # Long context, one stream.
    "gqa_b1_t131k": WorkloadConfig("gqa_b1_t131k", 5, 1, 32, 8, 131072, 128, 4, 3, 128, "f16", "bf16", 4, 10.0,
                         n_splits=256,
                         description="GQA 32q/8kv, d128, T131072, B1, b4/3, QJL m128, 256 splits"),
}


def _children(cfg: WorkloadConfig):
    ss = np.random.SeedSequence(BASE_SEED + cfg.config_id)
    return dict(zip(_CHILDREN, ss.spawn(len(_CHILDREN))))


def _rng(seed_seq) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_seq))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).copy()
    nan = np.isnan(x)
    out[nan] = x[nan]
    return out


def channel_scales(cfg: WorkloadConfig) -> np.ndarray:
    ch = _children(cfg)
    z = _rng(ch["scales"]).standard_normal((cfg.n_kv, cfg.head_dim))
    scale = np.exp(0.5 * z)
    orng = _rng(ch["outliers"])
    for h in range(cfg.n_kv):
        idx = orng.choice(cfg.head_dim, size=cfg.n_outliers, replace=False)
        scale[h, idx] *= cfg.outlier_mult
    return scale


def _stream_child(cfg: WorkloadConfig, which: str, b: int, h: int):
    kids = _children(cfg)[which].spawn(cfg.n_streams)
    return kids[b * cfg.n_kv + h]


def stream_keys(cfg: WorkloadConfig, b: int, h: int, scales: np.ndarray | None = None) -> np.ndarray:
    """Keys of one (sequence, kv-head) stream, [n_tokens, head_dim] in the key dtype."""
    if scales is None:
        scales = channel_scales(cfg)
    z = _rng(_stream_child(cfg, "keys", b, h)).standard_normal((cfg.n_tokens, cfg.head_dim))
    k = z * scales[h][None, :]
    return k.astype(np.float16 if cfg.k_dtype == "f16" else np.float32)


def stream_values(cfg: WorkloadConfig, b: int, h: int) -> np.ndarray:
    """Values of one stream, [n_tokens, head_dim] fp16."""
    z = _rng(_stream_child(cfg, "values", b, h)).standard_normal(
        (cfg.n_tokens, cfg.head_dim), dtype=np.float32)
    return z.astype(np.float16)


def queries(cfg: WorkloadConfig) -> np.ndarray:
    """[n_seq, n_q, head_dim] float32 holding values of the query dtype."""
    q = _rng(_children(cfg)["queries"]).standard_normal(
        (cfg.n_seq, cfg.n_q, cfg.head_dim), dtype=np.float32)
    return bf16_round(q) if cfg.q_dtype == "bf16" else q


def rht_signs(cfg: WorkloadConfig) -> np.ndarray:
    r = _rng(_children(cfg)["signs"]).integers(0, 2, size=(cfg.n_kv, cfg.head_dim))
    return (2 * r - 1).astype(np.int8)


def projection(cfg: WorkloadConfig) -> np.ndarray:
    s = _rng(_children(cfg)["proj"]).standard_normal(
        (cfg.n_kv, cfg.proj_rows, cfg.head_dim), dtype=np.float32)
    return s


def value_projection(cfg: WorkloadConfig) -> np.ndarray:
    """A second Gaussian projection [n_kv, head_dim, head_dim] fp32, for the value
    sketch when the values are coded as well."""
    return _rng(_children(cfg)["proj_v"]).standard_normal(
        (cfg.n_kv, cfg.head_dim, cfg.head_dim), dtype=np.float32)


def make_inputs(cfg: WorkloadConfig, streams=None, with_values: bool = True) -> dict:
    """All inputs of a configuration.

    ``streams``: None for every (sequence, kv-head) stream, else an iterable of
    (b, h) pairs; keys/values are then returned as dicts keyed by (b, h).
    """
    scales = channel_scales(cfg)
    out = {
        "cfg": cfg,
        "scales": scales,
        "q": queries(cfg),
        "signs": rht_signs(cfg),
        "S": projection(cfg),
    }
    if streams is None:
        kd = np.float16 if cfg.k_dtype == "f16" else np.float32
        K = np.empty((cfg.n_seq, cfg.n_kv, cfg.n_tokens, cfg.head_dim), dtype=kd)
        V = np.empty((cfg.n_seq, cfg.n_kv, cfg.n_tokens, cfg.head_dim), dtype=np.float16) \
            if with_values else None
        for b in range(cfg.n_seq):
            for h in range(cfg.n_kv):
                K[b, h] = stream_keys(cfg, b, h, scales)
                if with_values:
                    V[b, h] = stream_values(cfg, b, h)
        out["K"] = K
        out["V"] = V
    else:
        out["K"] = {(b, h): stream_keys(cfg, b, h, scales) for (b, h) in streams}
        out["V"] = {(b, h): stream_values(cfg, b, h) for (b, h) in streams} if with_values else None
    return out

"""Seeded synthetic inputs for the flow-matching action-expert denoise loop.

This module only *draws* inputs: model weights, per-layer prefix K/V, start
noise and time schedules, with the shapes of the workloads described on the
pages (a 36-layer action expert, chunk 50x75 or 50x55, prefix KV of 256 or 512
tokens per layer).  It holds none of the method's arithmetic.  Both the CPU
oracle (through the tests) and the HIP library (through the tests, the smoke
check and the benchmark) consume what it returns, so the two sides never
generate their own inputs.

Encodings returned:
  * bf16 tensors as ``uint16`` arrays holding the bfloat16 bit patterns
    (round-to-nearest-even from the float32 draw, done by torch's CPU cast);
  * fp8 tensors as ``uint8`` arrays holding OCP E4M3FN codes plus one float32
    scale per output row (``s_n = max_k |W[n,k]| / 448``, ``s_n = 1`` for an
    all-zero row, codes by torch's round-to-nearest-even cast of ``W / s_n``
    clamped to +-448);
  * MXFP4 tensors (the gate and up linears of the ``fp8_mxfp4gu`` tier) as
    ``uint8`` arrays of OCP E2M1 codes, two per byte (element 2j in the low
    nibble), ``[N, K/2]``, plus one E8M0 block scale per 32 inputs
    ``uint8 [N, K/32]`` (value 2^(e - 127)): per block, X = 2^(floor(log2
    max|W|) - 2) (X = 1 for an all-zero block) and codes = nearest E2M1 value
    of W / X, ties to even, clamped to +-6 (the OCP MX conversion);
  * biases, noise and schedules as float32.

Random streams: every tensor has its own ``numpy.random.default_rng`` stream
keyed by ``[seed, model_tag, tensor_id, layer]``; request ``b`` of a batch
draws its noise and prefix K/V from streams keyed by ``b`` alone, so request
``b`` of a batched workload equals the batch-1 workload of request ``b``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np
import torch

__all__ = [
    "ExpertConfig", "CONFIGS", "config", "make_weights", "make_prefix",
    "make_noise", "make_schedule", "apply_variant", "BLOCK_LINEARS",
    "BackboneConfig", "BACKBONES", "backbone", "make_backbone_weights", "make_embeddings",
]

# Per-layer linears of the expert block that the fp8 tier quantizes.
BLOCK_LINEARS = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


@dataclasses.dataclass(frozen=True)
class ExpertConfig:
    """Shapes and conventions of one workload (all sizes in elements)."""
    name: str
    model_tag: int          # weights/requests are keyed by this: same tag => same model
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    prefix_len: int
    horizon: int
    action_dim: int
    n_steps: int
    batch: int
    weight_dtype: str = "bf16"      # "bf16", "fp8_e4m3", or "fp8_mxfp4gu" (E4M3, gate/up MXFP4)
    time_emb_dim: int = 256
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6
    time_scale: float = 1000.0
    weight_std: float = 0.02

    @property
    def m_rows(self) -> int:
        return self.batch * self.horizon

    def replace(self, **kw) -> "ExpertConfig":
        return dataclasses.replace(self, **kw)


# The five workloads: tiny oracle-scale expert, LingBot-shaped expert, the
# V2-shaped longer loop, the fp8 tier and batched replica serving.
CONFIGS: Dict[int, ExpertConfig] = {
    1: ExpertConfig("tiny_2L_h256", 1, 2, 256, 4, 2, 64, 704, 32, 16, 7, 10, 1),
    2: ExpertConfig("lingbot_36L_h1024_b1", 2, 36, 1024, 16, 2, 128, 4096, 256, 50, 75, 10, 1),
    3: ExpertConfig("v2_36L_h1536_b1", 3, 36, 1536, 16, 2, 128, 6144, 512, 50, 55, 50, 1),
    4: ExpertConfig("lingbot_36L_h1024_fp8_b1", 2, 36, 1024, 16, 2, 128, 4096, 256, 50, 75, 25, 1,
                    weight_dtype="fp8_e4m3"),
    5: ExpertConfig("lingbot_36L_h1024_b64", 2, 36, 1024, 16, 2, 128, 4096, 256, 50, 75, 10, 64),
}


def config(i: int) -> ExpertConfig:
    return CONFIGS[i]


_TENSOR_IDS = {
    "in_w": 1, "in_b": 2, "out_w": 3, "out_b": 4, "t1_w": 5, "t1_b": 6, "t2_w": 7, "t2_b": 8,
    "mod_w": 9, "mod_b": 10, "wq": 11, "wk": 12, "wv": 13, "wo": 14, "wg": 15, "wu": 16,
    "wd": 17, "modf_w": 18, "modf_b": 19,
}


def _draw(cfg: ExpertConfig, seed: int, name: str, layer: int, shape) -> np.ndarray:
    rng = np.random.default_rng([seed, cfg.model_tag, _TENSOR_IDS[name], layer])
    x = rng.standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(cfg.weight_std)
    return x


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (torch's round-to-nearest-even cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def to_e4m3_rowwise(x: np.ndarray):
    """float32 [N, K] -> (E4M3FN codes uint8 [N, K], float32 scales [N])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1).astype(np.float64)
    s = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
    t = torch.from_numpy(x) / torch.from_numpy(s)[:, None]
    t = t.clamp_(-448.0, 448.0)
    q = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return q, s


_E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def to_mxfp4_blocks(x: np.ndarray):
    """float32 [N, K] (K % 32 == 0) -> (packed E2M1 codes uint8 [N, K/2],
    E8M0 scales uint8 [N, K/32]); see the module docstring."""
    x = np.asarray(x, dtype=np.float64)
    N, K = x.shape
    blk = x.reshape(N, K // 32, 32)
    amax = np.max(np.abs(blk), axis=2)
    e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0).astype(np.int64)
    v = np.abs(blk) / np.exp2(e)[:, :, None]
    v = np.minimum(v, 6.0)
    d = np.abs(v[..., None] - _E2M1_VALUES)                   # distance to each of the 8 magnitudes
    best = d.min(axis=-1, keepdims=True)
    cand = (d == best)
    # ties: the even code (codes 0..7 in increasing magnitude order)
    even = cand & (np.arange(8) % 2 == 0)
    idx = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    code = (idx | np.where(blk < 0, 8, 0)).astype(np.uint8).reshape(N, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def make_weights(cfg: ExpertConfig, seed: int = 0, weight_dtype: Optional[str] = None) -> dict:
    """All weights of one expert, as raw encodings (see the module docstring).

    Layout is torch ``nn.Linear`` ``[out, in]``, row-major.  Per-layer tensors
    are lists of length ``n_layers``.  ``weight_dtype`` overrides the config's
    block-linear dtype (the fp8 workload's bf16 reference uses the same draws).
    """
    wd = weight_dtype or cfg.weight_dtype
    H, A, L = cfg.hidden, cfg.action_dim, cfg.n_layers
    qd, kvd, I = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim, cfg.intermediate
    E = cfg.time_emb_dim
    W: Dict[str, object] = {"weight_dtype": wd}
    W["in_w"] = to_bf16_bits(_draw(cfg, seed, "in_w", 0, (H, A)))
    W["in_b"] = _draw(cfg, seed, "in_b", 0, (H,))
    W["out_w"] = to_bf16_bits(_draw(cfg, seed, "out_w", 0, (A, H)))
    W["out_b"] = _draw(cfg, seed, "out_b", 0, (A,))
    W["t1_w"] = to_bf16_bits(_draw(cfg, seed, "t1_w", 0, (H, E)))
    W["t1_b"] = _draw(cfg, seed, "t1_b", 0, (H,))
    W["t2_w"] = to_bf16_bits(_draw(cfg, seed, "t2_w", 0, (H, H)))
    W["t2_b"] = _draw(cfg, seed, "t2_b", 0, (H,))
    W["modf_w"] = to_bf16_bits(_draw(cfg, seed, "modf_w", 0, (2 * H, H)))
    W["modf_b"] = _draw(cfg, seed, "modf_b", 0, (2 * H,))
    shapes = {"wq": (qd, H), "wk": (kvd, H), "wv": (kvd, H), "wo": (H, qd),
              "wg": (I, H), "wu": (I, H), "wd": (H, I)}
    W["mod_w"], W["mod_b"] = [], []
    for name in BLOCK_LINEARS:
        W[name] = []
        if wd in ("fp8_e4m3", "fp8_mxfp4gu"):
            W["s" + name[1]] = []
    for l in range(L):
        W["mod_w"].append(to_bf16_bits(_draw(cfg, seed, "mod_w", l, (6 * H, H))))
        W["mod_b"].append(_draw(cfg, seed, "mod_b", l, (6 * H,)))
        for name in BLOCK_LINEARS:
            x = _draw(cfg, seed, name, l, shapes[name])
            if wd == "bf16":
                W[name].append(to_bf16_bits(x))
            elif wd == "fp8_e4m3" or (wd == "fp8_mxfp4gu" and name not in ("wg", "wu")):
                q, s = to_e4m3_rowwise(x)
                W[name].append(q)
                W["s" + name[1]].append(s)
            elif wd == "fp8_mxfp4gu":
                q, s = to_mxfp4_blocks(x)
                W[name].append(q)
                W["s" + name[1]].append(s)
            else:
                raise ValueError(f"unknown weight dtype {wd!r}")
    return W


def apply_variant(W: dict, variant: str, cfg: ExpertConfig, velocity_bias=None) -> dict:
    """Structured weight sets for closed-form checks (returns a modified copy).

    * ``zero_blocks``: every block linear zeroed (codes 0, fp8 scales 1).
    * ``gate_closed``: all modulation weights and biases zeroed, final ones too.
    * ``gate_open``: 1.0 added to the bias of both gate chunks (chunks 2 and 5 of
      the six per-layer modulation chunks), so block outputs dominate.
    * ``const_velocity``: out-projection weight zeroed, bias set to
      ``velocity_bias`` (float32 [action_dim]).
    """
    V = {k: (list(v) if isinstance(v, list) else v) for k, v in W.items()}
    H = cfg.hidden
    if variant == "zero_blocks":
        for name in BLOCK_LINEARS:
            V[name] = [np.zeros_like(a) for a in V[name]]
            if ("s" + name[1]) in V:
                V["s" + name[1]] = [np.ones_like(s) for s in V["s" + name[1]]]
    elif variant == "gate_closed":
        V["mod_w"] = [np.zeros_like(a) for a in V["mod_w"]]
        V["mod_b"] = [np.zeros_like(a) for a in V["mod_b"]]
        V["modf_w"] = np.zeros_like(V["modf_w"])
        V["modf_b"] = np.zeros_like(V["modf_b"])
    elif variant == "gate_open":
        nb = []
        for b in V["mod_b"]:
            b = b.copy()
            b[2 * H:3 * H] += np.float32(1.0)
            b[5 * H:6 * H] += np.float32(1.0)
            nb.append(b)
        V["mod_b"] = nb
    elif variant == "const_velocity":
        V["out_w"] = np.zeros_like(V["out_w"])
        V["out_b"] = np.asarray(velocity_bias, dtype=np.float32).copy()
    else:
        raise ValueError(f"unknown variant {variant!r}")
    return V


def make_prefix(cfg: ExpertConfig, seed: int = 0, requests: Optional[List[int]] = None):
    """Per-layer prefix K and V, bf16 bits ``[B, L, P, n_kv, d_h]``, N(0, 1).

    ``requests`` selects which request streams fill the batch (default
    ``range(cfg.batch)``).
    """
    reqs = list(range(cfg.batch)) if requests is None else list(requests)
    shp = (cfg.n_layers, cfg.prefix_len, cfg.n_kv_heads, cfg.head_dim)
    K = np.empty((len(reqs),) + shp, dtype=np.uint16)
    V = np.empty((len(reqs),) + shp, dtype=np.uint16)
    for i, b in enumerate(reqs):
        rk = np.random.default_rng([seed, cfg.model_tag, 2000 + b])
        rv = np.random.default_rng([seed, cfg.model_tag, 3000 + b])
        K[i] = to_bf16_bits(rk.standard_normal(size=shp, dtype=np.float32))
        V[i] = to_bf16_bits(rv.standard_normal(size=shp, dtype=np.float32))
    return K, V


def make_noise(cfg: ExpertConfig, seed: int = 0, requests: Optional[List[int]] = None):
    """Start state x_0 ~ N(0, 1), float32 ``[B, T, A]``."""
    reqs = list(range(cfg.batch)) if requests is None else list(requests)
    x = np.empty((len(reqs), cfg.horizon, cfg.action_dim), dtype=np.float32)
    for i, b in enumerate(reqs):
        r = np.random.default_rng([seed, cfg.model_tag, 1000 + b])
        x[i] = r.standard_normal(size=(cfg.horizon, cfg.action_dim), dtype=np.float32)
    return x


def make_schedule(n_steps: int, batch: int, kind: str = "uniform", seed: int = 0) -> np.ndarray:
    """Times t_{b,0..N}, float32 ``[B, N+1]``.

    ``uniform``: t_k = k / N, each entry computed as float32(k) / float32(N).
    ``warped``: request b uses t_k = (k / N) ** p_b with p_b drawn in [0.5, 2]
    (a per-request schedule, as when batched requests sit at different times).
    """
    k = np.arange(n_steps + 1, dtype=np.float32)
    u = k / np.float32(n_steps)
    if kind == "uniform":
        return np.tile(u, (batch, 1)).astype(np.float32)
    if kind == "warped":
        r = np.random.default_rng([seed, 4242, n_steps, batch])
        p = r.uniform(0.5, 2.0, size=batch)
        out = np.empty((batch, n_steps + 1), dtype=np.float32)
        for b in range(batch):
            out[b] = (u.astype(np.float64) ** p[b]).astype(np.float32)
        out[:, 0] = 0.0
        out[:, -1] = 1.0
        return out
    raise ValueError(f"unknown schedule kind {kind!r}")


# ----------------------------------------------------------------------------
# The prefix backbone (the step before the loop): a decoder whose per-layer
# K/V become the expert's prefix cache, so its n_layers, n_kv_heads and
# head_dim equal the expert's.
# ----------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class BackboneConfig:
    name: str
    model_tag: int
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    prefix_len: int
    batch: int
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6
    weight_std: float = 0.02
    weight_dtype: str = "bf16"   # or "fp8_e4m3": per-row E4M3 linears as for the expert

    def replace(self, **kw) -> "BackboneConfig":
        return dataclasses.replace(self, **kw)


# tiny (for the tiny expert) and the LingBot-shaped 36-layer prefix backbone
# (Qwen2.5-VL-3B text widths: hidden 2048, 16 query / 2 KV heads of 128,
# SwiGLU 11008; prefix 256 = 3 views x 64 merged patches + 64 text tokens)
BACKBONES: Dict[int, BackboneConfig] = {
    1: BackboneConfig("backbone_tiny_2L_h256", 11, 2, 256, 4, 2, 64, 704, 32, 1),
    2: BackboneConfig("backbone_lingbot_36L_h2048", 12, 36, 2048, 16, 2, 128, 11008, 256, 1),
}


def backbone(i: int) -> BackboneConfig:
    return BACKBONES[i]


_BB_IDS = {"n1": 1, "n2": 2, "wq": 3, "wk": 4, "wv": 5, "wo": 6, "wg": 7, "wu": 8, "wd": 9}


def make_backbone_weights(cfg: BackboneConfig, seed: int = 0, weight_dtype: Optional[str] = None) -> dict:
    """Per-layer lists: ``n1``, ``n2`` RMSNorm weights float32 [H] (1 + N(0, 0.1^2));
    ``wq`` [n_q*d_h, H], ``wk``, ``wv`` [n_kv*d_h, H], ``wo`` [H, n_q*d_h],
    ``wg``, ``wu`` [I, H], ``wd`` [H, I], N(0, std^2), as bf16 bits, or for
    ``fp8_e4m3`` as per-row E4M3FN codes with fp32 row scales ``sq`` .. ``sd``
    (the rule of the expert's E4M3 tier) from the same draws."""
    wd = weight_dtype or cfg.weight_dtype
    H, I = cfg.hidden, cfg.intermediate
    qd, kvd = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    shapes = {"wq": (qd, H), "wk": (kvd, H), "wv": (kvd, H), "wo": (H, qd), "wg": (I, H), "wu": (I, H),
              "wd": (H, I)}
    W: Dict[str, list] = {k: [] for k in _BB_IDS}
    if wd == "fp8_e4m3":
        for name in shapes:
            W["s" + name[1]] = []
    elif wd != "bf16":
        raise ValueError(f"unknown backbone weight dtype {wd!r}")
    for l in range(cfg.n_layers):
        for name in ("n1", "n2"):
            r = np.random.default_rng([seed, cfg.model_tag, _BB_IDS[name], l])
            W[name].append((1.0 + 0.1 * r.standard_normal(H)).astype(np.float32))
        for name, shp in shapes.items():
            r = np.random.default_rng([seed, cfg.model_tag, _BB_IDS[name], l])
            x = r.standard_normal(size=shp, dtype=np.float32) * np.float32(cfg.weight_std)
            if wd == "bf16":
                W[name].append(to_bf16_bits(x))
            else:
                q, sc = to_e4m3_rowwise(x)
                W[name].append(q)
                W["s" + name[1]].append(sc)
    return W


def make_embeddings(cfg: BackboneConfig, seed: int = 0, requests: Optional[List[int]] = None) -> np.ndarray:
    """Prefix token embeddings (vision patches + text), bf16 bits ``[B, P, H]``,
    N(0, 1); request b from its own stream."""
    reqs = list(range(cfg.batch)) if requests is None else list(requests)
    out = np.empty((len(reqs), cfg.prefix_len, cfg.hidden), dtype=np.uint16)
    for i, b in enumerate(reqs):
        r = np.random.default_rng([seed, cfg.model_tag, 5000 + b])
        out[i] = to_bf16_bits(r.standard_normal(size=(cfg.prefix_len, cfg.hidden), dtype=np.float32))
    return out

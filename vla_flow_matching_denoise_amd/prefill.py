"""``Prefill``: owns one prefix K/V construction context (argument marshalling only).

Backbone weights arrive as raw encodings (bf16 bit patterns as uint16, or
E4M3 codes as uint8 with fp32 row scales; fp32 RMSNorm weights), are placed in device memory by torch, handed to
``vla_prefill_create`` (which repacks and copies them) and released.
``__call__`` passes device pointers of torch tensors to ``vla_prefill`` on
torch's current stream; every step runs in the HIP library.
"""
from __future__ import annotations

import ctypes
from typing import Optional

from . import binding as B
from .expert import to_device

LINEARS = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def backbone_dims(n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, prefix_len, batch,
                  rope_theta=1.0e6, rms_eps=1.0e-6, weight_dtype="bf16") -> B.VlaBackboneDims:
    wd = {"bf16": B.VLA_BF16, "fp8_e4m3": B.VLA_FP8_E4M3}[weight_dtype] if isinstance(weight_dtype, str) \
        else int(weight_dtype)
    return B.VlaBackboneDims(n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, prefix_len, batch,
                             rope_theta, rms_eps, wd)


def backbone_dims_from_config(cfg, batch: Optional[int] = None, prefix_len: Optional[int] = None):
    return backbone_dims(cfg.n_layers, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate,
                         cfg.prefix_len if prefix_len is None else prefix_len,
                         cfg.batch if batch is None else batch, cfg.rope_theta, cfg.rms_eps, cfg.weight_dtype)


class Prefill:
    def __init__(self, raw: dict, dims: B.VlaBackboneDims, device: str = "cuda"):
        import torch
        self.dims = dims
        self.device = device
        keep = []

        def arr(name):
            ts = [to_device(a, device) for a in raw[name]]
            keep.extend(ts)
            ptrs = (ctypes.c_void_p * dims.n_layers)(*[t.data_ptr() for t in ts])
            keep.append(ptrs)
            return ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p))

        w = B.VlaBackboneWeights()
        w.norm1 = arr("n1")
        w.norm2 = arr("n2")
        for name in LINEARS:
            setattr(w, name, arr(name))
            sname = "s" + name[1]
            if sname in raw:                   # E4M3 row scales
                setattr(w, sname, arr(sname))
        torch.cuda.synchronize()
        self.ctx = B.vla_prefill_create(w, dims)
        del keep

    def set_option(self, option: int, value: int) -> None:
        B.vla_prefill_set_option(self.ctx, option, value)

    def __call__(self, embeddings, prefix_k=None, prefix_v=None):
        """embeddings: int16 (bf16 bits) device tensor [B, P, H]. Returns
        (prefix_k, prefix_v) int16 tensors [B, L, P, n_kv, d_h]."""
        import torch
        d = self.dims
        shape = (d.batch, d.n_layers, d.prefix_len, d.n_kv_heads, d.head_dim)
        if tuple(embeddings.shape) != (d.batch, d.prefix_len, d.hidden):
            raise ValueError(f"embeddings shape {tuple(embeddings.shape)} != {(d.batch, d.prefix_len, d.hidden)}")
        if prefix_k is None:
            prefix_k = torch.empty(shape, dtype=torch.int16, device=embeddings.device)
        if prefix_v is None:
            prefix_v = torch.empty(shape, dtype=torch.int16, device=embeddings.device)
        B.vla_prefill_set_stream(self.ctx, torch.cuda.current_stream().cuda_stream)
        B.vla_prefill(self.ctx, embeddings.data_ptr(), prefix_k.data_ptr(), prefix_v.data_ptr())
        return prefix_k, prefix_v

    def device_bytes(self) -> int:
        return B.vla_prefill_device_bytes(self.ctx)

    def close(self) -> None:
        if getattr(self, "ctx", None):
            B.vla_prefill_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

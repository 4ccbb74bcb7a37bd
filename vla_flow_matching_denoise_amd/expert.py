"""``Expert``: owns one library context; uploads weights with PyTorch.

Argument marshalling only: weights arrive as raw encodings (bf16 bit patterns
as uint16, E4M3FN codes as uint8, fp32 biases/scales), are placed in device
memory by torch, handed to ``vla_expert_create`` (which repacks and copies
them), and released.  ``denoise`` passes device pointers of torch tensors to
``vla_denoise`` on torch's current stream.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np

from . import binding as B

BLOCK = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def make_dims(n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, action_dim, horizon,
              prefix_len, batch, time_emb_dim=256, rope_theta=1.0e6, rms_eps=1.0e-6, time_scale=1000.0,
              weight_dtype="bf16") -> B.VlaDims:
    wd = {"bf16": B.VLA_BF16, "fp8_e4m3": B.VLA_FP8_E4M3,
          "fp8_mxfp4gu": B.VLA_FP8_E4M3_MXFP4_GU}[weight_dtype] if isinstance(weight_dtype, str) \
        else int(weight_dtype)
    return B.VlaDims(n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate, action_dim, horizon,
                     prefix_len, batch, time_emb_dim, rope_theta, rms_eps, time_scale, wd)


def dims_from_config(cfg, batch: Optional[int] = None) -> B.VlaDims:
    return make_dims(cfg.n_layers, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate,
                     cfg.action_dim, cfg.horizon, cfg.prefix_len, cfg.batch if batch is None else batch,
                     cfg.time_emb_dim, cfg.rope_theta, cfg.rms_eps, cfg.time_scale, cfg.weight_dtype)


def to_device(a, device="cuda"):
    """numpy array (uint16 = bf16 bits, kept as int16) or torch tensor -> contiguous device tensor."""
    import torch
    if isinstance(a, torch.Tensor):
        return a.to(device).contiguous()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    return torch.from_numpy(a).to(device)


class Expert:
    def __init__(self, raw: dict, dims: B.VlaDims, device: str = "cuda"):
        import torch
        self.dims = dims
        self.device = device
        keep = []

        def dev(a):
            t = to_device(a, device)
            keep.append(t)
            return t.data_ptr()

        def arr(name):
            ptrs = (ctypes.c_void_p * dims.n_layers)(*[dev(a) for a in raw[name]])
            keep.append(ptrs)
            return ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p))

        w = B.VlaWeights()
        for name in ("in_w", "in_b", "out_w", "out_b", "t1_w", "t1_b", "t2_w", "t2_b", "modf_w", "modf_b"):
            setattr(w, name, dev(raw[name]))
        w.mod_w = arr("mod_w")
        w.mod_b = arr("mod_b")
        for name in BLOCK:
            setattr(w, name, arr(name))
            sname = "s" + name[1]
            if sname in raw:
                setattr(w, sname, arr(sname))
        torch.cuda.synchronize()
        self.ctx = B.vla_expert_create(w, dims)
        del keep

    def set_option(self, option: int, value: int) -> None:
        B.vla_set_option(self.ctx, option, value)

    def get_option(self, option: int) -> int:
        return B.vla_get_option(self.ctx, option)

    @property
    def persistent_active(self) -> bool:
        """True when calls run as the single persistent kernel (one launch of
        one workgroup per CU, all resident together)."""
        return B.vla_get_option(self.ctx, B.VLA_OPT_PERSISTENT_ACTIVE) == 1

    def denoise(self, prefix_k, prefix_v, noise, t_schedule, n_steps: int, out=None, prefix_valid=None):
        """All arguments torch device tensors (prefix as int16/bf16 bits); returns ``out``.
        ``prefix_valid``: optional int32 device tensor [B] of valid prefix tokens per request."""
        import torch
        if out is None:
            out = torch.empty_like(noise)
        B.vla_set_stream(self.ctx, torch.cuda.current_stream().cuda_stream)
        if prefix_valid is None:
            B.vla_denoise(self.ctx, prefix_k.data_ptr(), prefix_v.data_ptr(), noise.data_ptr(),
                          t_schedule.data_ptr(), n_steps, out.data_ptr())
        else:
            if prefix_valid.dtype != torch.int32 or not prefix_valid.is_cuda:
                raise ValueError("prefix_valid must be an int32 CUDA tensor")
            B.vla_denoise_varlen(self.ctx, prefix_k.data_ptr(), prefix_v.data_ptr(), prefix_valid.data_ptr(),
                                 noise.data_ptr(), t_schedule.data_ptr(), n_steps, out.data_ptr())
        return out

    def device_bytes(self) -> int:
        return B.vla_device_bytes(self.ctx)

    def close(self) -> None:
        if getattr(self, "ctx", None):
            B.vla_expert_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

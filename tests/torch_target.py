"""An independent formulation of the synthetic target's forward from torch library routines.

Used only to pin the target oracle. It keeps no cache: every call runs the whole token
history in one causal pass, with an explicit boolean [queries, keys] mask per layer (keys
p <= q, and q - p < W on sliding layers) through torch.nn.functional.scaled_dot_product_attention
(GQA via enable_gqa). RoPE is a complex rotation of the (i, i + hd/2) pairs; RMSNorm, SiLU and
the projections are F.rms_norm, F.silu and F.linear. float64 on the CPU; bf16 shapes round the
cached K/V and the captured streams to bf16 through torch's own conversion.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


class TorchTarget:
    def __init__(self, shape, weights):
        self.sh = shape
        self.w = {k: torch.as_tensor(np.asarray(v, dtype=np.float64)) for k, v in weights.items()}
        self.bf16 = shape.act_dtype == "bf16"

    def _c(self, x):
        return x.to(torch.float32).to(torch.bfloat16).to(torch.float64) if self.bf16 else x

    def _rms(self, x, g):
        return F.rms_norm(x, (x.shape[-1],), weight=self.w[g], eps=self.sh.rms_eps)

    def _rope(self, x, pos):
        hd = x.shape[-1]
        half = hd // 2
        freqs = torch.pow(torch.tensor(self.sh.rope_theta, dtype=torch.float64),
                          -2.0 * torch.arange(half, dtype=torch.float64) / hd)
        ang = pos.to(torch.float64)[:, None] * freqs[None, :]
        rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]  # [n, 1, half]
        z = torch.complex(x[..., :half], x[..., half:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    def forward(self, tokens):
        """All rows of `tokens` (positions 0..n-1): (argmax, top-2 margins, captured streams)."""
        sh = self.sh
        n = len(tokens)
        pos = torch.arange(n)
        x = F.embedding(torch.as_tensor(np.asarray(tokens)), self.w["embed"])
        caps = {}
        q_idx, k_idx = pos[:, None], pos[None, :]
        for l in range(sh.layers):
            p = f"layers.{l}."
            mask = k_idx <= q_idx
            if sh.layer_kind(l) == "sliding":
                mask = mask & (q_idx - k_idx < sh.window)
            h = self._rms(x, p + "in_norm")
            q = F.linear(h, self.w[p + "q"]).reshape(n, sh.q_heads, sh.head_dim)
            k = F.linear(h, self.w[p + "k"]).reshape(n, sh.kv_heads, sh.head_dim)
            v = F.linear(h, self.w[p + "v"]).reshape(n, sh.kv_heads, sh.head_dim)
            q = self._rope(self._rms(q, p + "q_norm"), pos)
            k = self._c(self._rope(self._rms(k, p + "k_norm"), pos))
            v = self._c(v)
            o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], k.transpose(0, 1)[None],
                                               v.transpose(0, 1)[None], attn_mask=mask[None, None],
                                               enable_gqa=True)[0].transpose(0, 1).reshape(n, -1)
            x = x + F.linear(o, self.w[p + "o"])
            h2 = self._rms(x, p + "post_norm")
            x = x + F.linear(F.silu(F.linear(h2, self.w[p + "gate"])) * F.linear(h2, self.w[p + "up"]),
                             self.w[p + "down"])
            if l in sh.capture_layers:
                caps[l] = x.clone()
        capture = self._c(torch.cat([caps[l] for l in sh.capture_layers], dim=1))
        logits = F.linear(self._rms(x, "final_norm"), self.w["lm_head"])
        top = torch.topk(logits, 2, dim=1).values
        return (torch.argmax(logits, dim=1).numpy(), (top[:, 0] - top[:, 1]).numpy(), capture.numpy())

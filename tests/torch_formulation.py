"""An independent formulation of the drafter forward, built from torch library routines.

Used only to pin the oracle. It keeps no ring at all: it holds the whole committed
history of residual rows, recomputes every context K/V from it, and attends with an
explicit boolean [queries, keys] mask over absolute positions, through
torch.nn.functional.scaled_dot_product_attention (GQA via enable_gqa). RoPE is written
as a complex rotation of the (i, i + hd/2) pairs, or for the adjacent pairing of a DSpark
shape of the (2i, 2i + 1) pairs through torch.view_as_complex. Everything runs in float64
on the CPU; bf16 shapes round the inputs and the cached K/V (context and block) to bf16
through torch's own conversion. The DSpark form attends with no mask at all and runs its
Markov chain through F.embedding / F.linear / torch.argmax.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def _t(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float64))


class TorchDrafter:
    def __init__(self, shape, weights):
        self.sh = shape
        self.w = {k: _t(v) for k, v in weights.items() if not hasattr(v, "packed")}
        self.bf16 = shape.act_dtype == "bf16"

    def _c(self, x):
        if not self.bf16:
            return x
        return x.to(torch.float32).to(torch.bfloat16).to(torch.float64)

    def _rms(self, x, name):
        return F.rms_norm(x, (x.shape[-1],), weight=self.w[name], eps=self.sh.rms_eps)

    def _rope(self, x, pos):
        # x: [..., seq, heads, hd]; rotate pair i (elements (i, i+hd/2), or (2i, 2i+1) for the
        # adjacent pairing) by pos * theta^(-2i/hd)
        hd = x.shape[-1]
        half = hd // 2
        freqs = torch.pow(torch.tensor(self.sh.rope_theta, dtype=torch.float64),
                          -torch.arange(0, hd, 2, dtype=torch.float64) / hd)
        ang = torch.outer(torch.as_tensor(pos, dtype=torch.float64), freqs)  # [seq, half]
        rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]
        if getattr(self.sh, "rope_style", "neox") == "traditional":
            z = torch.view_as_complex(x.reshape(*x.shape[:-1], half, 2).contiguous()) * rot
            return torch.view_as_real(z).reshape(x.shape)
        z = torch.complex(x[..., :half], x[..., half:]) * rot
        return torch.cat([z.real, z.imag], dim=-1)

    def context_kv(self, history):
        """K/V of every committed row, positions 0..n-1, per layer."""
        sh = self.sh
        r = self._c(_t(history))
        c = self._rms(F.linear(r, self.w["fc"]), "enc_norm")
        pos = np.arange(r.shape[0])
        out = []
        for l in range(sh.layers):
            p = f"layers.{l}."
            k = F.linear(c, self.w[p + "k"]).unflatten(-1, (sh.kv_heads, sh.head_dim))
            v = F.linear(c, self.w[p + "v"]).unflatten(-1, (sh.kv_heads, sh.head_dim))
            k = self._rope(self._rms(k, p + "k_norm"), pos)
            out.append((self._c(k), self._c(v)))
        return out

    def forward(self, history, anchor, block):
        """Hidden rows [B+1, H] and logits [B, V] of the block drafted after `history`."""
        sh = self.sh
        e = len(history)
        qpos = np.arange(e, e + block + 1)
        kpos = np.arange(0, e + block + 1)
        mask = torch.as_tensor(np.abs(qpos[:, None] - kpos[None, :]) <= sh.window)
        x = self._layers(history, [anchor] + [sh.mask_id] * block, qpos, mask)
        z = self._rms(x[1:], "final_norm")
        return x.numpy(), F.linear(z, self.w["lm_head"]).numpy()

    def forward_dspark(self, history, anchor, gamma):
        """DSpark block after `history`: hidden rows [gamma, H], backbone logits [gamma, V]
        of every row, and the Markov chain's tokens [gamma] (no attention mask)."""
        sh = self.sh
        e = len(history)
        x = self._layers(history, [anchor] + [sh.mask_id] * (gamma - 1), np.arange(e, e + gamma), None)
        logits = F.linear(self._rms(x, "final_norm"), self.w["lm_head"])
        toks = []
        prev = torch.tensor([anchor])
        for i in range(gamma):
            u = F.embedding(prev, self.w["markov_w1"])  # [1, rank]
            score = logits[i] + F.linear(u, self.w["markov_w2"])[0]
            prev = torch.argmax(score, dim=0, keepdim=True)
            toks.append(int(prev[0]))
        return x.numpy(), logits.numpy(), np.array(toks)

    def _layers(self, history, ids, qpos, mask):
        sh = self.sh
        ctx = self.context_kv(history)
        x = F.embedding(torch.tensor(ids), self.w["embed"])
        for l in range(sh.layers):
            p = f"layers.{l}."
            h = self._rms(x, p + "in_norm")
            q = F.linear(h, self.w[p + "q"]).unflatten(-1, (sh.q_heads, sh.head_dim))
            k = F.linear(h, self.w[p + "k"]).unflatten(-1, (sh.kv_heads, sh.head_dim))
            v = F.linear(h, self.w[p + "v"]).unflatten(-1, (sh.kv_heads, sh.head_dim))
            q = self._rope(self._rms(q, p + "q_norm"), qpos)
            k = self._c(self._rope(self._rms(k, p + "k_norm"), qpos))
            v = self._c(v)
            kall = torch.cat([ctx[l][0], k], dim=0).transpose(0, 1)[None]  # [1, nkv, Nk, hd]
            vall = torch.cat([ctx[l][1], v], dim=0).transpose(0, 1)[None]
            o = F.scaled_dot_product_attention(q.transpose(0, 1)[None], kall, vall,
                                               attn_mask=mask, enable_gqa=True)
            o = o[0].transpose(0, 1).flatten(-2)
            x = x + F.linear(o, self.w[p + "o"])
            h2 = self._rms(x, p + "post_norm")
            a = F.silu(F.linear(h2, self.w[p + "gate"])) * F.linear(h2, self.w[p + "up"])
            x = x + F.linear(a, self.w[p + "down"])
        return x

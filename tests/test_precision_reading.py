"""Why activations stay real numbers between the GEMMs of a bf16 drafter (the precision
reading of the whole build): a sensitivity experiment on the drafter forward, CPU only.

The forward is the torch formulation (float64, bf16 inputs and cached K/V). Its F.linear is
wrapped so that every GEMM's activation operand passes through a rounding rule first, and
each reading is run twice with two rules that a correct implementation could equally use:

- every GEMM operand rounded to bf16: straight from float64, against through float32 first
  (the two differ only where the float32 step moves a value across a bf16 tie);
- operands kept real: unrounded, against the bf16 hi/lo pair hi + lo with hi = bf16(x) and
  lo = bf16(x - hi) that the MFMA kernels multiply (about 16 significant bits).

Rounding every operand lets a single differently rounded operand flip further roundings
downstream, so the two runs drift apart until the logits differ by more than the 1e-2 top-2
margin under which argmax indices are compared exactly. With real operands the two runs stay
an order of magnitude closer, well inside it.
"""
import numpy as np
import pytest
import torch

import tests.torch_formulation as TF
from block_drafting_dflash_amd import synth
from oracle.dflash_oracle import round_bf16

MARGIN = 1e-2  # top-2 logit margin above which argmax indices must agree exactly

MID = synth.Shape(hidden=512, layers=5, q_heads=8, kv_heads=2, head_dim=64, intermediate=1536, vocab=8192,
                  target_streams=5, target_width=512, window=256, weight_dtype="bf16", act_dtype="bf16")


def bf16_direct(x):
    return torch.as_tensor(round_bf16(x.numpy()))


def bf16_via_f32(x):
    return x.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def hi_lo_pair(x):
    hi = torch.as_tensor(round_bf16(x.numpy()))
    return hi + torch.as_tensor(round_bf16((x - hi).numpy()))


def forward_with(monkeypatch, sh, w, history, rule):
    linear = torch.nn.functional.linear
    if rule is not None:
        monkeypatch.setattr(TF.F, "linear", lambda x, wt, b=None: linear(rule(x), wt))
    try:
        return TF.TorchDrafter(sh, w).forward(history, 5, 4)
    finally:
        monkeypatch.setattr(TF.F, "linear", linear)


def drift(a, b):
    (xa, la), (xb, lb) = a, b
    rel = np.linalg.norm(xa - xb, axis=1) / np.linalg.norm(xb, axis=1)
    return float(rel.max()), float(np.abs(la - lb).max())


@pytest.mark.parametrize("name", ["mid", "muse"])
def test_real_operands_keep_two_correct_forwards_inside_the_argmax_margin(monkeypatch, name):
    sh = {"mid": MID, "muse": synth.MUSE_BF16}[name]
    w = synth.make_weights(sh)
    history = synth.resid_rows(sh, 200, 0)
    run = lambda rule: forward_with(monkeypatch, sh, w, history, rule)  # noqa: E731
    hid_all, logit_all = drift(run(bf16_direct), run(bf16_via_f32))
    hid_real, logit_real = drift(run(None), run(hi_lo_pair))
    print(f"{name}: every operand rounded: hidden {hid_all:.3g}, logits {logit_all:.3g}; "
          f"real operands: hidden {hid_real:.3g}, logits {logit_real:.3g}")
    # rounding every operand: the two runs end up a sizeable part of the margin apart in the
    # logits at the mid shape, beyond it at the Muse shape
    assert logit_all > (MARGIN if name == "muse" else MARGIN / 2)
    # real operands: an order of magnitude closer, far inside the margin
    assert logit_real < MARGIN / 5
    assert hid_all > 5 * hid_real and logit_all > 5 * logit_real

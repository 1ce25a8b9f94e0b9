"""dflash_lm_head_argmax_noalloc (argmax keys in the library's fixed per-GPU array) against
dflash_lm_head_argmax (keys in the context's workspace), through the C-ABI: the indices are
bit-identical, over two calls in a row whose second takes fewer rows, on bf16, 4-bit and f32
shapes; argument errors are refused before anything is enqueued."""
import pytest
import torch

from block_drafting_dflash_amd import binding, synth

pytestmark = pytest.mark.gpu

SHAPES = {
    "bf16": synth.Shape(hidden=512, layers=1, q_heads=8, kv_heads=2, head_dim=64, intermediate=768, vocab=20480,
                        target_streams=2, target_width=256, window=20, weight_dtype="bf16", act_dtype="bf16"),
    "f32": synth.Shape(hidden=256, layers=1, q_heads=4, kv_heads=2, head_dim=64, intermediate=384, vocab=4096,
                       target_streams=3, target_width=128, window=9, weight_dtype="f32", act_dtype="f32"),
}
SHAPES["q4"] = SHAPES["bf16"].with_(weight_dtype="q4")


@pytest.mark.parametrize("kind", ["bf16", "q4", "f32"])
def test_noalloc_argmax_matches_the_workspace_argmax(kind):
    sh = SHAPES[kind]
    g = binding.Drafter(sh, binding.to_device(sh, synth.make_weights(sh)), max_block=4)
    L = binding.lib()
    stream = torch.cuda.current_stream().cuda_stream
    for call, n in enumerate((40, 5)):  # two launches of rows (32 + 8), then one of 5
        rows = torch.from_numpy(synth.verify_hidden(sh, n, 50 + call)).to(g.act_dtype).cuda()
        want = torch.full((n,), -1, dtype=torch.int32, device="cuda")
        got = torch.full((n,), -2, dtype=torch.int32, device="cuda")
        assert L.dflash_lm_head_argmax(g.ctx, rows.data_ptr(), n, want.data_ptr(), stream) == 0
        assert L.dflash_lm_head_argmax_noalloc(g.ctx, rows.data_ptr(), n, got.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        assert torch.equal(got.cpu(), want.cpu()), (kind, call)
        assert int(want.min()) >= 0 and int(want.max()) < sh.vocab


def test_noalloc_argmax_argument_errors():
    sh = SHAPES["f32"]
    g = binding.Drafter(sh, binding.to_device(sh, synth.make_weights(sh)), max_block=4)
    L = binding.lib()
    stream = torch.cuda.current_stream().cuda_stream
    rows = torch.from_numpy(synth.verify_hidden(sh, 3, 0)).cuda()
    out = torch.empty(3, dtype=torch.int32, device="cuda")
    assert L.dflash_lm_head_argmax_noalloc(None, rows.data_ptr(), 3, out.data_ptr(), stream) == 1
    assert L.dflash_lm_head_argmax_noalloc(g.ctx, None, 3, out.data_ptr(), stream) == 1
    assert L.dflash_lm_head_argmax_noalloc(g.ctx, rows.data_ptr(), 0, out.data_ptr(), stream) == 3
    assert L.dflash_lm_head_argmax_noalloc(g.ctx, rows.data_ptr(), 3, None, stream) == 1

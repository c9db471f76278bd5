"""The allocation-free forward entry point (tp_block_shard_forward_noalloc): through the C ABI,
its partials equal those of tp_block_shard_forward with a caller workspace, bit for bit, for both
halves of every rank, on two calls in a row, the second with a smaller batch."""
import numpy as np
import pytest

from tensor_transformer_block_amd.inputs import BlockShape, make_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts, never run there
    pytest.skip("no GPU", allow_module_level=True)

MED = BlockShape(name="noalloc-med", index=240, d_model=512, n_heads=8, n_kv_heads=2,
                 head_dim=128, ffn_dim=1376, tp=2, w_dtype="bf16", act_dtype="bf16",
                 ffn_act="silu", mode="decode", kv_lens=(37, 100, 5), n_tokens=3)
# The larger batch first (64 tokens: the split-K GEMMs' partial tiles fill more of the scratch),
# then a smaller one, then a Q8_0 decode of one token.
CASES = [MED.with_(name="noalloc-batched-64", index=241, tp=4, n_heads=8, n_kv_heads=4,
                   ffn_dim=1408, kv_lens=tuple(range(40, 40 + 64 * 3, 3)), n_tokens=64),
         MED,
         BlockShape(name="noalloc-q8", index=242, d_model=640, n_heads=8, n_kv_heads=2,
                    head_dim=256, ffn_dim=1280, tp=2, w_dtype="q8_0", act_dtype="bf16",
                    ffn_act="gelu_tanh", mode="decode", kv_lens=(300,), n_tokens=1)]


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def test_no_alloc_matches_workspace_entry_point():
    from tensor_transformer_block_amd import binding as B
    from tensor_transformer_block_amd.block import DeviceBlock
    for s in CASES:
        blk = DeviceBlock(make_inputs(s, seed=5))
        d, T, N = blk.desc, blk.T, blk.N
        got = torch.empty_like(blk.partials[0])
        print(f"noalloc {s.name}: T={T} N={N} workspace {blk.ws_bytes} B", flush=True)
        B.tp_partial_reduce(d, T, None, 0, blk.x, None, blk.gamma1, blk.xn)
        for r in range(N):
            # The ATTN half rewrites the same new K and V into the cache on both calls.
            blk.attn_half(r)
            got.fill_(float("nan"))
            B.tp_block_shard_forward_noalloc(d, r, B.TP_HALF_ATTN, blk.shards[0][r], blk.batch,
                                             blk.xn, blk.kv[0][r], got)
            torch.cuda.synchronize()
            assert torch.equal(_bits(got), _bits(blk.partials[r])), f"{s.name} ATTN rank {r}"
        B.tp_partial_reduce(d, T, blk.partials, N, blk.x, blk.h1, blk.gamma2, blk.xn2)
        for r in range(N):
            blk.ffn_half(r)
            got.fill_(float("nan"))
            B.tp_block_shard_forward_noalloc(d, r, B.TP_HALF_FFN, blk.shards[0][r], blk.batch,
                                             blk.xn2, None, got)
            torch.cuda.synchronize()
            assert torch.equal(_bits(got), _bits(blk.partials[r])), f"{s.name} FFN rank {r}"
        assert bool(torch.isfinite(blk.partials.float()).all())
        del blk


def test_no_alloc_refuses_a_batch_beyond_its_scratch():
    from tensor_transformer_block_amd import binding as B
    s = MED.with_(name="noalloc-prefill", mode="prefill", kv_lens=(8192,), n_tokens=8192,
                  ffn_dim=16384)
    d = B.make_desc(s)
    b = B.make_batch("prefill", 8192, 1, 512, 8192, 16, 16, 16, 16)
    need = B.tp_workspace_size(d, b)
    assert need > 16 << 20
    with pytest.raises(B.TPError) as ei:
        B.tp_block_shard_forward_noalloc(d, 0, B.TP_HALF_FFN, 256, b, 256, None, 256)
    assert ei.value.status == B.TP_ERR_BUFFER_TOO_SMALL
    assert "static scratch" in ei.value.detail

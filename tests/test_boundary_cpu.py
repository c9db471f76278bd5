"""The C-ABI library on the host (no GPU needed): it loads, exports every declared symbol, and
validates every argument before any HIP call, returning the documented status."""
import os
import re

import pytest

from tensor_transformer_block_amd import binding as B
from tensor_transformer_block_amd.inputs import CONFIGS, weight_shapes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "tp_block.h")).read()
    return sorted(set(re.findall(r"^(?:tp_status|const char\*|size_t|uint64_t)\s+(tp_\w+)\(",
                                 text, flags=re.M)))


def test_exports_every_declared_symbol():
    L = B.lib()
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(B.EXPORTED)


def _err(fn, *a, **k):
    with pytest.raises(B.TPError) as ei:
        fn(*a, **k)
    return ei.value.status, ei.value.detail


def desc_of(name, **over):
    d = B.make_desc(CONFIGS[name])
    for k, v in over.items():
        setattr(d, k, v)
    return d


# Per-rank weight bytes of the five workloads (all ranks = N times these).
EXPECTED_PAYLOAD = {
    "tiny-llama-fp32": 1_581_056, "llama3-8b-decode": 218_103_808,
    "llama3-8b-batched": 109_051_904, "llama-70b-prefill": 213_909_504,
    "gemma-q8-decode": 48_742_400,
}


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_shard_layout_is_one_nth(name):
    s = CONFIGS[name]
    d = B.make_desc(s)
    full = 0
    for k, (o, i) in weight_shapes(s).items():
        full += o * i * {"f32": 4, "bf16": 2, "q8_0": 34 / 32}[s.w_dtype]
    for r in range(s.tp):
        lay = B.tp_shard_weights_size(d, r)
        assert lay.payload_bytes * s.tp == full
        assert lay.payload_bytes == EXPECTED_PAYLOAD[name]
        regs = [lay.qkv, lay.o, lay.gate_up, lay.down]
        if s.w_dtype == "q8_0":
            regs += [lay.qkv_scale, lay.o_scale, lay.gate_up_scale, lay.down_scale]
        assert sum(r_.bytes for r_ in regs) == lay.payload_bytes
        for r_ in regs:
            assert r_.offset % 256 == 0
            assert r_.offset + r_.bytes <= lay.alloc_bytes
        offs = sorted((r_.offset, r_.offset + r_.bytes) for r_ in regs)
        assert all(a[1] <= b[0] for a, b in zip(offs, offs[1:]))


def test_validation_divisibility_and_rank():
    st, msg = _err(B.tp_shard_weights_size, desc_of("tiny-llama-fp32", tp_degree=3), 0)
    assert st == B.TP_ERR_NOT_DIVISIBLE and "divide" in msg
    st, _ = _err(B.tp_shard_weights_size, desc_of("llama3-8b-decode", n_kv_heads=6), 0)
    assert st == B.TP_ERR_NOT_DIVISIBLE
    st, _ = _err(B.tp_shard_weights_size, desc_of("llama3-8b-decode", ffn_dim=14337), 0)
    assert st == B.TP_ERR_NOT_DIVISIBLE
    for bad in (-1, 2, 100):
        st, _ = _err(B.tp_shard_weights_size, desc_of("llama3-8b-decode"), bad)
        assert st == B.TP_ERR_RANK


def test_validation_quant_alignment():
    # Q8_0 row-parallel splits must fall on 32-weight block boundaries.
    st, msg = _err(B.tp_shard_weights_size, desc_of("gemma-q8-decode", ffn_dim=10240 + 32), 0)
    assert st == B.TP_ERR_QUANT_ALIGN, msg
    st, _ = _err(B.tp_shard_weights_size, desc_of("gemma-q8-decode", d_model=2560 + 16), 0)
    assert st == B.TP_ERR_QUANT_ALIGN
    st, _ = _err(B.tp_shard_weights_size,
                 desc_of("gemma-q8-decode", n_heads=2, n_kv_heads=2, head_dim=48), 0)
    assert st == B.TP_ERR_QUANT_ALIGN
    # the same shapes are legal unquantised
    B.tp_shard_weights_size(desc_of("gemma-q8-decode", w_dtype=B.TP_DTYPE_BF16,
                                    ffn_dim=10240 + 32), 0)


def test_validation_unsupported_and_invalid():
    st, _ = _err(B.tp_shard_weights_size, desc_of("llama3-8b-decode", act_dtype=B.TP_DTYPE_F32), 0)
    assert st == B.TP_ERR_UNSUPPORTED
    st, _ = _err(B.tp_shard_weights_size, desc_of("llama3-8b-decode", head_dim=96), 0)
    assert st == B.TP_ERR_UNSUPPORTED
    st, _ = _err(B.tp_shard_weights_size, desc_of("llama3-8b-decode", n_heads=48, n_kv_heads=8), 0)
    assert st == B.TP_ERR_UNSUPPORTED
    st, _ = _err(B.tp_shard_weights_size, desc_of("llama3-8b-decode", w_dtype=7), 0)
    assert st == B.TP_ERR_INVALID_ARG
    st, _ = _err(B.tp_shard_weights_size, desc_of("llama3-8b-decode", d_model=0), 0)
    assert st == B.TP_ERR_INVALID_ARG
    st, _ = _err(B.tp_shard_weights_size, desc_of("llama3-8b-decode", rms_eps=float("nan")), 0)
    assert st == B.TP_ERR_INVALID_ARG
    st, _ = _err(B.tp_shard_weights_size, desc_of("llama3-8b-decode", page_size=12), 0)
    assert st == B.TP_ERR_UNSUPPORTED


def _batch(s, **over):
    kw = dict(mode=s.mode, n_tokens=s.n_tokens, n_seqs=s.n_seqs,
              max_pages=-(-max(s.kv_lens) // s.page_size), max_seq_len=max(s.kv_lens))
    kw.update(over)
    return B.make_batch(**kw)


def test_forward_validates_before_any_launch():
    s = CONFIGS["llama3-8b-decode"]
    d = B.make_desc(s)
    b = _batch(s)
    ws = B.tp_workspace_size(d, b)
    assert ws > 0
    fwd = B.tp_block_shard_forward
    st, _ = _err(fwd, d, 5, B.TP_HALF_ATTN, 16, b, 16, None, 16, 16, ws, stream=0)
    assert st == B.TP_ERR_RANK
    st, _ = _err(fwd, d, 0, 9, 16, b, 16, None, 16, 16, ws, stream=0)
    assert st == B.TP_ERR_INVALID_ARG
    # ATTN needs positions / block table / rope table
    st, msg = _err(fwd, d, 0, B.TP_HALF_ATTN, 16, b, 16, None, 16, 16, ws, stream=0)
    assert st == B.TP_ERR_INVALID_ARG and "positions" in msg
    b2 = _batch(s, positions=16, block_table=16, rope_table=16)
    st, msg = _err(fwd, d, 0, B.TP_HALF_ATTN, 16, b2, 16, None, 16, 16, ws, stream=0)
    assert st == B.TP_ERR_INVALID_ARG and "KV" in msg
    kv = B.tp_kv_cache(k_pages=16, v_pages=16, n_pages=256)
    st, _ = _err(fwd, d, 0, B.TP_HALF_ATTN, 16, b2, 16, kv, 16, 16, ws - 1, stream=0)
    assert st == B.TP_ERR_BUFFER_TOO_SMALL
    st, msg = _err(fwd, d, 0, B.TP_HALF_FFN, 16, b2, 8, None, 16, 16, ws, stream=0)
    assert st == B.TP_ERR_INVALID_ARG and "aligned" in msg
    st, _ = _err(fwd, d, 0, B.TP_HALF_FFN, None, b2, 16, None, 16, 16, ws, stream=0)
    assert st == B.TP_ERR_INVALID_ARG
    # decode batches: one token per sequence; prefill: one sequence
    st, _ = _err(B.tp_workspace_size, d, _batch(s, n_seqs=2))
    assert st == B.TP_ERR_INVALID_ARG
    st, _ = _err(B.tp_workspace_size, d, _batch(s, mode="prefill", n_tokens=8, n_seqs=2))
    assert st == B.TP_ERR_INVALID_ARG
    st, _ = _err(B.tp_workspace_size, d, _batch(s, max_seq_len=4097))
    assert st == B.TP_ERR_INVALID_ARG
    # an empty batch is a valid no-op, even with no buffers
    B.tp_block_shard_forward(d, 0, B.TP_HALF_FFN, None, _batch(s, n_tokens=0, n_seqs=0), None,
                             None, None, None, 0, stream=0)


def test_reduce_validates():
    d = B.make_desc(CONFIGS["llama3-8b-decode"])
    st, _ = _err(B.tp_partial_reduce, d, -1, None, 0, 16, None, 16, 16, stream=0)
    assert st == B.TP_ERR_INVALID_ARG
    st, _ = _err(B.tp_partial_reduce, d, 1, None, 2, 16, 16, None, None, stream=0)
    assert st == B.TP_ERR_INVALID_ARG
    st, _ = _err(B.tp_partial_reduce, d, 1, 16, 2, 16, 16, 16, None, stream=0)
    assert st == B.TP_ERR_INVALID_ARG
    st, _ = _err(B.tp_partial_reduce, d, 1, 16, 2, 8, 16, None, None, stream=0)
    assert st == B.TP_ERR_INVALID_ARG
    B.tp_partial_reduce(d, 0, None, 0, None, None, None, None, stream=0)


def test_workspace_grows_with_tokens():
    s = CONFIGS["llama3-8b-batched"]
    d = B.make_desc(s)
    w1 = B.tp_workspace_size(d, _batch(s, n_tokens=1, n_seqs=1))
    w64 = B.tp_workspace_size(d, _batch(s))
    assert 0 < w1 < w64
    q, a, f = B.tp_workspace_offsets(d, _batch(s))
    assert len({q, a, f}) == 3 and max(q, a, f) < w64


def test_status_strings():
    assert B.tp_status_str(B.TP_OK) == "TP_OK"
    assert B.tp_status_str(B.TP_ERR_QUANT_ALIGN) == "TP_ERR_QUANT_ALIGN"
    assert B.tp_status_str(99) == "TP_ERR_UNKNOWN"


# ----------------------------------------------------------------------------- head and MoE calls

def test_head_layout_and_validation():
    d = B.make_desc(CONFIGS["gemma-q8-decode"])
    lay = B.tp_head_size(d, 1000)
    assert lay.table.bytes == 1000 * 2560                     # one code byte per weight
    assert lay.table_scale.bytes == 1000 * (2560 // 32) * 2   # one fp16 scale per block
    assert lay.payload_bytes == 1000 * 2560 * 34 // 32
    assert lay.table_scale.offset % 256 == 0 and lay.alloc_bytes >= lay.payload_bytes
    lay = B.tp_head_size(B.make_desc(CONFIGS["llama3-8b-decode"]), 128256)
    assert lay.table.bytes == 128256 * 4096 * 2 and lay.table_scale.bytes == 0
    st, _ = _err(B.tp_head_size, d, 0)
    assert st == B.TP_ERR_INVALID_ARG
    st, _ = _err(B.tp_head_pack, d, 1000, 16, 16, B.tp_head_size(d, 1000).alloc_bytes - 1,
                 stream=0)
    assert st == B.TP_ERR_BUFFER_TOO_SMALL
    st, _ = _err(B.tp_embed_lookup, d, 1000, 16, None, 3, 16, stream=0)
    assert st == B.TP_ERR_INVALID_ARG
    st, msg = _err(B.tp_embed_lookup, d, 1000, 16, 16, 3, 8, stream=0)
    assert st == B.TP_ERR_INVALID_ARG and "aligned" in msg
    st, _ = _err(B.tp_lm_head, d, 1000, 16, 16, -1, 16, stream=0)
    assert st == B.TP_ERR_INVALID_ARG
    st, _ = _err(B.tp_lm_head, d, 1000, None, 16, 2, 16, stream=0)
    assert st == B.TP_ERR_INVALID_ARG
    # empty token batches are no-ops, even with no buffers
    B.tp_embed_lookup(d, 1000, None, None, 0, None, stream=0)
    B.tp_lm_head(d, 1000, None, None, 0, None, stream=0)


def test_moe_layout_is_one_nth_and_validates():
    from tensor_transformer_block_amd.inputs import MoEShape
    for name, moe in (("llama3-8b-decode", MoEShape(64, 8, 768)),
                      ("gemma-q8-decode", MoEShape(16, 2, 1024))):
        s = CONFIGS[name]
        d, m = B.make_desc(s), B.make_moe_desc(moe)
        per = {"f32": 4, "bf16": 2, "q8_0": 34 / 32}[s.w_dtype]
        full = 3 * moe.n_experts * moe.expert_ffn * s.d_model * per
        for r in range(s.tp):
            lay = B.tp_moe_shard_size(d, m, r)
            assert lay.payload_bytes * s.tp == full
            regs = [lay.gate, lay.up, lay.down, lay.gate_scale, lay.up_scale, lay.down_scale]
            assert sum(x.bytes for x in regs) == lay.payload_bytes
            assert all(x.offset % 256 == 0 and x.offset + x.bytes <= lay.alloc_bytes for x in regs)
    s = CONFIGS["llama3-8b-decode"]
    d = B.make_desc(s)

    def moe(**kw):
        base = dict(n_experts=64, top_k=8, expert_ffn=768)
        base.update(kw)
        return B.tp_moe_desc(**base)
    assert _err(B.tp_moe_shard_size, d, moe(top_k=17), 0)[0] == B.TP_ERR_INVALID_ARG
    assert _err(B.tp_moe_shard_size, d, moe(top_k=9, n_experts=8), 0)[0] == B.TP_ERR_INVALID_ARG
    assert _err(B.tp_moe_shard_size, d, moe(n_experts=1025), 0)[0] == B.TP_ERR_INVALID_ARG
    assert _err(B.tp_moe_shard_size, d, moe(expert_ffn=769), 0)[0] == B.TP_ERR_NOT_DIVISIBLE
    assert _err(B.tp_moe_shard_size, d, moe(expert_ffn=772), 0)[0] == B.TP_ERR_UNSUPPORTED
    assert _err(B.tp_moe_shard_size, d, moe(), 2)[0] == B.TP_ERR_RANK
    dq = B.make_desc(CONFIGS["gemma-q8-decode"])
    assert _err(B.tp_moe_shard_size, dq, moe(expert_ffn=1040), 0)[0] == B.TP_ERR_QUANT_ALIGN
    ws = B.tp_moe_workspace_size(d, moe(), 4)
    assert ws >= 4 * 8 * 384 * 2
    fwd = B.tp_moe_shard_forward
    st, _ = _err(fwd, d, moe(), 0, 16, 16, 4, 16, 16, 16, 16, ws - 1, stream=0)
    assert st == B.TP_ERR_BUFFER_TOO_SMALL
    st, _ = _err(fwd, d, moe(), 0, 16, 16, 4, None, 16, 16, 16, ws, stream=0)
    assert st == B.TP_ERR_INVALID_ARG
    st, _ = _err(B.tp_moe_route, d, moe(), 16, 16, 2, 16, None, 16, stream=0)
    assert st == B.TP_ERR_INVALID_ARG
    B.tp_moe_shard_forward(d, moe(), 0, None, None, 0, None, None, None, None, 0, stream=0)
    B.tp_moe_route(d, moe(), None, None, 0, None, None, None, stream=0)


def test_shard_project_validation():
    """The projection test helper refuses a bad region and a short workspace before any launch,
    and sizes its workspace for the split-K Q8_0 GEMM of a 64-token batch."""
    d = desc_of("gemma-q8-decode")
    st, _ = _err(B.tp_shard_project_workspace_size, d, 7, 1)
    assert st == B.TP_ERR_INVALID_ARG
    assert B.tp_shard_project_workspace_size(d, 1, 1) == 256
    need = B.tp_shard_project_workspace_size(d, 1, 64)
    assert need > 256
    st, _ = _err(B.tp_shard_project, d, 1, 256, 512, 64, 1024, 2048, need - 256)
    assert st == B.TP_ERR_BUFFER_TOO_SMALL
    st, _ = _err(B.tp_shard_project, d, 4, 256, 512, 1, 1024)
    assert st == B.TP_ERR_INVALID_ARG


def test_traffic_record_hash_ignores_comments_only(tmp_path):
    """The gate/up traffic records carry a hash of their kernels' code: an edit of comments or
    whitespace keeps it, a change of code (or of a string literal holding comment markers) does
    not, and every committed record still matches the current sources."""
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import bench
    src = 'int f(int a) { // add one\n  return a + 1; /* done */ }\nconst char* s = "x // y";\n'
    variants = {
        "comments": 'int f(int a) {  // add two\n\n  return a + 1;   /* done,\n twice */ }\n'
                    'const char* s = "x // y";\n',
        "code": 'int f(int a) { // add one\n  return a + 2; /* done */ }\nconst char* s = "x // y";\n',
        "string": 'int f(int a) { // add one\n  return a + 1; /* done */ }\nconst char* s = "x / y";\n',
    }
    base = tmp_path / "a.hip"
    base.write_text(src)
    d0 = bench.code_digest(["a.hip"], str(tmp_path))
    got = {}
    for k, v in variants.items():
        (tmp_path / f"{k}.hip").write_text(v)
        got[k] = bench.code_digest([f"{k}.hip"], str(tmp_path))
    assert got["comments"] == d0
    assert got["code"] != d0 and got["string"] != d0
    assert bench.code_text(src) == 'int f(int a) { return a + 1; } const char* s = "x // y";'
    for w in ("llama3-8b-decode", "gemma-q8-decode", "llama3-8b-batched", "llama-70b-prefill"):
        assert bench.measured_traffic(w) is not None, w

"""ctypes binding of libtpblock (include/tp_block.h): argument marshalling only.

Functions keep the C names. Tensor arguments may be torch tensors (their device pointer is passed),
plain integers (raw addresses) or None (NULL). `stream` defaults to torch's current HIP stream when
a GPU is present, else NULL. Every non-zero status raises ``TPError`` with the library's detail.
The library must have been built (``tensor_transformer_block_amd.build_lib``); nothing here falls
back to another implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpblock.so")

TP_OK, TP_ERR_INVALID_ARG, TP_ERR_RANK, TP_ERR_NOT_DIVISIBLE = 0, 1, 2, 3
TP_ERR_QUANT_ALIGN, TP_ERR_BUFFER_TOO_SMALL, TP_ERR_UNSUPPORTED, TP_ERR_HIP = 4, 5, 6, 7
TP_DTYPE_F32, TP_DTYPE_BF16, TP_DTYPE_Q8_0 = 0, 1, 2
TP_ACT_SILU, TP_ACT_GELU_TANH = 0, 1
TP_HALF_ATTN, TP_HALF_FFN = 0, 1
TP_MODE_DECODE, TP_MODE_PREFILL = 0, 1

DTYPE_CODES = {"f32": TP_DTYPE_F32, "bf16": TP_DTYPE_BF16, "q8_0": TP_DTYPE_Q8_0}
ACT_CODES = {"silu": TP_ACT_SILU, "gelu_tanh": TP_ACT_GELU_TANH}
MODE_CODES = {"decode": TP_MODE_DECODE, "prefill": TP_MODE_PREFILL}

EXPORTED = (
    "tp_shard_weights_size", "tp_shard_weights", "tp_workspace_size", "tp_rope_table_bytes",
    "tp_rope_table_init", "tp_block_shard_forward", "tp_partial_reduce", "tp_status_str",
    "tp_last_error", "tp_shard_unpack", "tp_dequant_q8_0", "tp_workspace_offsets",
    "tp_block_shard_forward_timed", "tp_head_size", "tp_head_pack", "tp_embed_lookup",
    "tp_lm_head", "tp_moe_shard_size", "tp_moe_shard_weights", "tp_moe_route",
    "tp_moe_workspace_size", "tp_moe_shard_forward", "tp_moe_shard_forward_timed",
    "tp_shard_project", "tp_shard_project_workspace_size", "tp_block_shard_forward_noalloc",
    "tp_block_step", "tp_block_step_timed", "tp_moe_block_step", "tp_moe_block_step_timed",
    "tp_step_workspace_size",
    "tp_step_schedule", "tp_block_step_with_schedule",
)

TP_SCHEDULE_STAGED, TP_SCHEDULE_PER_RANK, TP_SCHEDULE_ALL_RANKS = 0, 1, 2


class tp_block_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "d_model", "n_heads", "n_kv_heads", "head_dim", "ffn_dim", "tp_degree", "page_size",
        "max_position")] + [("rms_eps", ctypes.c_float), ("rope_base", ctypes.c_float)] + [
        (n, ctypes.c_int32) for n in ("w_dtype", "act_dtype", "partial_dtype", "ffn_act")]


class tp_region(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_uint64), ("bytes", ctypes.c_uint64)]


class tp_shard_layout(ctypes.Structure):
    _fields_ = [(n, tp_region) for n in (
        "qkv", "o", "gate_up", "down", "qkv_scale", "o_scale", "gate_up_scale", "down_scale")] + [
        ("payload_bytes", ctypes.c_uint64), ("alloc_bytes", ctypes.c_uint64)]


class tp_head_layout(ctypes.Structure):
    _fields_ = [("table", tp_region), ("table_scale", tp_region),
                ("payload_bytes", ctypes.c_uint64), ("alloc_bytes", ctypes.c_uint64)]


class tp_moe_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_experts", "top_k", "expert_ffn")]


class tp_moe_full_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("wg", "wu", "wd")]


class tp_moe_layout(ctypes.Structure):
    _fields_ = [(n, tp_region) for n in (
        "gate", "up", "down", "gate_scale", "up_scale", "down_scale")] + [
        ("payload_bytes", ctypes.c_uint64), ("alloc_bytes", ctypes.c_uint64)]


class tp_full_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")]


class tp_batch(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "mode", "n_tokens", "n_seqs", "max_pages", "max_seq_len")] + [
        (n, ctypes.c_void_p) for n in ("positions", "seq_lens", "block_table", "rope_table")]


class tp_kv_cache(ctypes.Structure):
    _fields_ = [("k_pages", ctypes.c_void_p), ("v_pages", ctypes.c_void_p),
                ("n_pages", ctypes.c_int32)]


class TPError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status
        self.name = name
        self.detail = detail


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtpblock.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m tensor_transformer_block_amd.build_lib`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, U64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
    sig = {
        "tp_shard_weights_size": [P, I32, P],
        "tp_shard_weights": [P, I32, P, P, U64, P],
        "tp_workspace_size": [P, P, P],
        "tp_step_workspace_size": [P, P, P],
        "tp_step_schedule": [P, P, P],
        "tp_rope_table_bytes": [P, P],
        "tp_rope_table_init": [P, P, U64, P],
        "tp_block_shard_forward": [P, I32, I32, P, P, P, P, P, P, U64, P],
        "tp_block_shard_forward_timed": [P, I32, I32, P, P, P, P, P, P, U64, P, P, P],
        "tp_partial_reduce": [P, I32, P, I32, P, P, P, P, P],
        "tp_shard_unpack": [P, I32, P, P, P],
        "tp_dequant_q8_0": [P, P, P, U64, P],
        "tp_workspace_offsets": [P, P, P, P, P],
        "tp_head_size": [P, I32, P],
        "tp_head_pack": [P, I32, P, P, U64, P],
        "tp_embed_lookup": [P, I32, P, P, I32, P, P],
        "tp_lm_head": [P, I32, P, P, I32, P, P],
        "tp_moe_shard_size": [P, P, I32, P],
        "tp_moe_shard_weights": [P, P, I32, P, P, U64, P],
        "tp_moe_route": [P, P, P, P, I32, P, P, P, P],
        "tp_moe_workspace_size": [P, P, I32, P],
        "tp_moe_shard_forward": [P, P, I32, P, P, I32, P, P, P, P, U64, P],
        "tp_moe_shard_forward_timed": [P, P, I32, P, P, I32, P, P, P, P, U64, P, P, P],
        "tp_shard_project": [P, I32, P, P, I32, P, P, U64, P],
        "tp_shard_project_workspace_size": [P, I32, I32, P],
        "tp_block_shard_forward_noalloc": [P, I32, I32, P, P, P, P, P, P],
        "tp_block_step": [P, P, P, P, P, P, P, P, P, P, P, P, P, U64, P],
        "tp_block_step_with_schedule": [P, I32, P, P, P, P, P, P, P, P, P, P, P, P, U64, P],
        "tp_block_step_timed": [P, P, P, P, P, P, P, P, P, P, P, P, P, U64, P, I32, P, P],
        "tp_moe_block_step": [P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, U64, P,
                              U64, P],
        "tp_moe_block_step_timed": [P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, U64,
                                    P, U64, P, P, P],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = I32
    L.tp_status_str.argtypes = [I32]
    L.tp_status_str.restype = ctypes.c_char_p
    L.tp_last_error.argtypes = []
    L.tp_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int) -> None:
    if status != TP_OK:
        L = lib()
        raise TPError(status, L.tp_status_str(status).decode(), L.tp_last_error().decode())


def ptr(x) -> int | None:
    """Device (or host) address of a tensor, an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def make_desc(shape, partial_dtype: str = "f32", max_position: int | None = None) -> tp_block_desc:
    """tp_block_desc of a BlockShape (or any object with the same attribute names)."""
    return tp_block_desc(
        d_model=shape.d_model, n_heads=shape.n_heads, n_kv_heads=shape.n_kv_heads,
        head_dim=shape.head_dim, ffn_dim=shape.ffn_dim, tp_degree=shape.tp,
        page_size=shape.page_size,
        max_position=max_position if max_position is not None else shape.max_pos,
        rms_eps=shape.rms_eps, rope_base=shape.rope_base,
        w_dtype=DTYPE_CODES[shape.w_dtype], act_dtype=DTYPE_CODES[shape.act_dtype],
        partial_dtype=DTYPE_CODES[partial_dtype], ffn_act=ACT_CODES[shape.ffn_act])


def make_batch(mode, n_tokens, n_seqs, max_pages, max_seq_len, positions=None, seq_lens=None,
               block_table=None, rope_table=None) -> tp_batch:
    return tp_batch(mode=MODE_CODES.get(mode, mode), n_tokens=n_tokens, n_seqs=n_seqs,
                    max_pages=max_pages, max_seq_len=max_seq_len, positions=ptr(positions),
                    seq_lens=ptr(seq_lens), block_table=ptr(block_table),
                    rope_table=ptr(rope_table))


def full_weights(w: dict) -> tp_full_weights:
    return tp_full_weights(**{k: ptr(w.get(k)) for k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")})


# ----------------------------------------------------------------------------- the C calls

def tp_shard_weights_size(desc, rank: int) -> tp_shard_layout:
    out = tp_shard_layout()
    _check(lib().tp_shard_weights_size(ctypes.byref(desc), rank, ctypes.byref(out)))
    return out


def tp_shard_weights(desc, rank, src: tp_full_weights, dst, dst_bytes=None, stream=None) -> None:
    if dst_bytes is None:
        dst_bytes = dst.numel() * dst.element_size()
    _check(lib().tp_shard_weights(ctypes.byref(desc), rank, ctypes.byref(src), ptr(dst), dst_bytes,
                                  _stream(stream)))


def tp_shard_unpack(desc, rank, shard, dst: tp_full_weights, stream=None) -> None:
    _check(lib().tp_shard_unpack(ctypes.byref(desc), rank, ptr(shard), ctypes.byref(dst),
                                 _stream(stream)))


def tp_workspace_size(desc, batch: tp_batch) -> int:
    out = ctypes.c_uint64()
    _check(lib().tp_workspace_size(ctypes.byref(desc), ctypes.byref(batch), ctypes.byref(out)))
    return out.value


def tp_step_workspace_size(desc, batch: tp_batch) -> int:
    out = ctypes.c_uint64()
    _check(lib().tp_step_workspace_size(ctypes.byref(desc), ctypes.byref(batch),
                                        ctypes.byref(out)))
    return out.value


def tp_step_schedule(desc, batch: tp_batch) -> int:
    out = ctypes.c_int32()
    _check(lib().tp_step_schedule(ctypes.byref(desc), ctypes.byref(batch), ctypes.byref(out)))
    return out.value


def tp_workspace_offsets(desc, batch: tp_batch):
    q, a, f = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().tp_workspace_offsets(ctypes.byref(desc), ctypes.byref(batch), ctypes.byref(q),
                                      ctypes.byref(a), ctypes.byref(f)))
    return q.value, a.value, f.value


def tp_rope_table_bytes(desc) -> int:
    out = ctypes.c_uint64()
    _check(lib().tp_rope_table_bytes(ctypes.byref(desc), ctypes.byref(out)))
    return out.value


def tp_rope_table_init(desc, table, table_bytes=None, stream=None) -> None:
    if table_bytes is None:
        table_bytes = table.numel() * table.element_size()
    _check(lib().tp_rope_table_init(ctypes.byref(desc), ptr(table), table_bytes, _stream(stream)))


def tp_block_shard_forward(desc, rank, half, shard, batch: tp_batch, xn, kv: tp_kv_cache | None,
                           partial_out, workspace, workspace_bytes=None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().tp_block_shard_forward(
        ctypes.byref(desc), rank, half, ptr(shard), ctypes.byref(batch), ptr(xn),
        ctypes.byref(kv) if kv is not None else None, ptr(partial_out), ptr(workspace),
        workspace_bytes, _stream(stream)))


def tp_block_shard_forward_timed(desc, rank, half, shard, batch: tp_batch, xn,
                                 kv: tp_kv_cache | None, partial_out, workspace, ev_begin, ev_end,
                                 workspace_bytes=None, stream=None) -> None:
    """ev_begin / ev_end: raw hipEvent_t handles (ints from hipEventCreate) or None."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().tp_block_shard_forward_timed(
        ctypes.byref(desc), rank, half, ptr(shard), ctypes.byref(batch), ptr(xn),
        ctypes.byref(kv) if kv is not None else None, ptr(partial_out), ptr(workspace),
        workspace_bytes, _stream(stream), ev_begin, ev_end))


def tp_block_shard_forward_noalloc(desc, rank, half, shard, batch: tp_batch, xn,
                                   kv: tp_kv_cache | None, partial_out, stream=None) -> None:
    _check(lib().tp_block_shard_forward_noalloc(
        ctypes.byref(desc), rank, half, ptr(shard), ctypes.byref(batch), ptr(xn),
        ctypes.byref(kv) if kv is not None else None, ptr(partial_out), _stream(stream)))


def _step_arrays(shards, kv):
    sh = (ctypes.c_void_p * len(shards))(*[ptr(t) for t in shards])
    kvs = (tp_kv_cache * len(kv))(*kv)
    return sh, kvs


def tp_block_step(desc, shards, batch: tp_batch, kv, x, gamma1, gamma2, partials, xn, h1, xn2,
                  out, workspace, workspace_bytes=None, stream=None) -> None:
    """shards: the N ranks' packed shards; kv: their tp_kv_cache structs (host lists)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    sh, kvs = _step_arrays(shards, kv)
    _check(lib().tp_block_step(ctypes.byref(desc), sh, ctypes.byref(batch), kvs, ptr(x),
                               ptr(gamma1), ptr(gamma2), ptr(partials), ptr(xn), ptr(h1),
                               ptr(xn2), ptr(out), ptr(workspace), workspace_bytes,
                               _stream(stream)))


def tp_block_step_with_schedule(desc, schedule, shards, batch: tp_batch, kv, x, gamma1, gamma2,
                                partials, xn, h1, xn2, out, workspace, workspace_bytes=None,
                                stream=None) -> None:
    """tp_block_step with an explicit TP_SCHEDULE_* (-1: the library's choice)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    sh, kvs = _step_arrays(shards, kv)
    _check(lib().tp_block_step_with_schedule(ctypes.byref(desc), schedule, sh, ctypes.byref(batch),
                                             kvs, ptr(x), ptr(gamma1), ptr(gamma2), ptr(partials),
                                             ptr(xn), ptr(h1), ptr(xn2), ptr(out), ptr(workspace),
                                             workspace_bytes, _stream(stream)))


def tp_block_step_timed(desc, shards, batch: tp_batch, kv, x, gamma1, gamma2, partials, xn, h1,
                        xn2, out, workspace, timed_rank, ev_begin, ev_end, workspace_bytes=None,
                        stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    sh, kvs = _step_arrays(shards, kv)
    _check(lib().tp_block_step_timed(ctypes.byref(desc), sh, ctypes.byref(batch), kvs, ptr(x),
                                     ptr(gamma1), ptr(gamma2), ptr(partials), ptr(xn), ptr(h1),
                                     ptr(xn2), ptr(out), ptr(workspace), workspace_bytes,
                                     _stream(stream), timed_rank, ev_begin, ev_end))


def tp_moe_block_step(desc, moe, shards, moe_shards, batch: tp_batch, kv, x, gamma1, gamma2,
                      router, partials, xn, h1, xn2, out, logits, topk_ids, topk_weights,
                      workspace, moe_workspace, workspace_bytes=None, moe_workspace_bytes=None,
                      stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    if moe_workspace_bytes is None:
        moe_workspace_bytes = moe_workspace.numel() * moe_workspace.element_size()
    sh, kvs = _step_arrays(shards, kv)
    msh = (ctypes.c_void_p * len(moe_shards))(*[ptr(t) for t in moe_shards])
    _check(lib().tp_moe_block_step(
        ctypes.byref(desc), ctypes.byref(moe), sh, msh, ctypes.byref(batch), kvs, ptr(x),
        ptr(gamma1), ptr(gamma2), ptr(router), ptr(partials), ptr(xn), ptr(h1), ptr(xn2),
        ptr(out), ptr(logits), ptr(topk_ids), ptr(topk_weights), ptr(workspace), workspace_bytes,
        ptr(moe_workspace), moe_workspace_bytes, _stream(stream)))


def tp_moe_block_step_timed(desc, moe, shards, moe_shards, batch: tp_batch, kv, x, gamma1, gamma2,
                            router, partials, xn, h1, xn2, out, logits, topk_ids, topk_weights,
                            workspace, moe_workspace, ev_begin, ev_end, workspace_bytes=None,
                            moe_workspace_bytes=None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    if moe_workspace_bytes is None:
        moe_workspace_bytes = moe_workspace.numel() * moe_workspace.element_size()
    sh, kvs = _step_arrays(shards, kv)
    msh = (ctypes.c_void_p * len(moe_shards))(*[ptr(t) for t in moe_shards])
    _check(lib().tp_moe_block_step_timed(
        ctypes.byref(desc), ctypes.byref(moe), sh, msh, ctypes.byref(batch), kvs, ptr(x),
        ptr(gamma1), ptr(gamma2), ptr(router), ptr(partials), ptr(xn), ptr(h1), ptr(xn2),
        ptr(out), ptr(logits), ptr(topk_ids), ptr(topk_weights), ptr(workspace), workspace_bytes,
        ptr(moe_workspace), moe_workspace_bytes, _stream(stream), ev_begin, ev_end))


def tp_partial_reduce(desc, n_tokens, partials, n_partials, residual_in, residual_out, gamma,
                      normed_out, stream=None) -> None:
    _check(lib().tp_partial_reduce(ctypes.byref(desc), n_tokens, ptr(partials), n_partials,
                                   ptr(residual_in), ptr(residual_out), ptr(gamma),
                                   ptr(normed_out), _stream(stream)))


def tp_dequant_q8_0(codes, scales, out, n_blocks, stream=None) -> None:
    _check(lib().tp_dequant_q8_0(ptr(codes), ptr(scales), ptr(out), n_blocks, _stream(stream)))


def tp_shard_project_workspace_size(desc, which: int, n_tokens: int) -> int:
    out = ctypes.c_uint64()
    _check(lib().tp_shard_project_workspace_size(ctypes.byref(desc), which, n_tokens,
                                                 ctypes.byref(out)))
    return out.value


def tp_shard_project(desc, which, shard, x, n_tokens, out, workspace=None, workspace_bytes=None,
                     stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().tp_shard_project(ctypes.byref(desc), which, ptr(shard), ptr(x), n_tokens, ptr(out),
                                  ptr(workspace), workspace_bytes, _stream(stream)))


def tp_head_size(desc, vocab: int) -> tp_head_layout:
    out = tp_head_layout()
    _check(lib().tp_head_size(ctypes.byref(desc), vocab, ctypes.byref(out)))
    return out


def tp_head_pack(desc, vocab, src, dst, dst_bytes=None, stream=None) -> None:
    if dst_bytes is None:
        dst_bytes = dst.numel() * dst.element_size()
    _check(lib().tp_head_pack(ctypes.byref(desc), vocab, ptr(src), ptr(dst), dst_bytes,
                              _stream(stream)))


def tp_embed_lookup(desc, vocab, head, token_ids, n_tokens, x_out, stream=None) -> None:
    _check(lib().tp_embed_lookup(ctypes.byref(desc), vocab, ptr(head), ptr(token_ids), n_tokens,
                                 ptr(x_out), _stream(stream)))


def tp_lm_head(desc, vocab, head, xn, n_tokens, logits, stream=None) -> None:
    _check(lib().tp_lm_head(ctypes.byref(desc), vocab, ptr(head), ptr(xn), n_tokens, ptr(logits),
                            _stream(stream)))


def make_moe_desc(moe) -> tp_moe_desc:
    return tp_moe_desc(n_experts=moe.n_experts, top_k=moe.top_k, expert_ffn=moe.expert_ffn)


def tp_moe_shard_size(desc, moe: tp_moe_desc, rank: int) -> tp_moe_layout:
    out = tp_moe_layout()
    _check(lib().tp_moe_shard_size(ctypes.byref(desc), ctypes.byref(moe), rank, ctypes.byref(out)))
    return out


def tp_moe_shard_weights(desc, moe, rank, src: tp_moe_full_weights, dst, dst_bytes=None,
                         stream=None) -> None:
    if dst_bytes is None:
        dst_bytes = dst.numel() * dst.element_size()
    _check(lib().tp_moe_shard_weights(ctypes.byref(desc), ctypes.byref(moe), rank,
                                      ctypes.byref(src), ptr(dst), dst_bytes, _stream(stream)))


def tp_moe_route(desc, moe, router, xn, n_tokens, logits, topk_ids, topk_weights,
                 stream=None) -> None:
    _check(lib().tp_moe_route(ctypes.byref(desc), ctypes.byref(moe), ptr(router), ptr(xn),
                              n_tokens, ptr(logits), ptr(topk_ids), ptr(topk_weights),
                              _stream(stream)))


def tp_moe_workspace_size(desc, moe, n_tokens: int) -> int:
    out = ctypes.c_uint64()
    _check(lib().tp_moe_workspace_size(ctypes.byref(desc), ctypes.byref(moe), n_tokens,
                                       ctypes.byref(out)))
    return out.value


def tp_moe_shard_forward(desc, moe, rank, shard, xn, n_tokens, topk_ids, topk_weights,
                         partial_out, workspace, workspace_bytes=None, stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().tp_moe_shard_forward(ctypes.byref(desc), ctypes.byref(moe), rank, ptr(shard),
                                      ptr(xn), n_tokens, ptr(topk_ids), ptr(topk_weights),
                                      ptr(partial_out), ptr(workspace), workspace_bytes,
                                      _stream(stream)))


def tp_moe_shard_forward_timed(desc, moe, rank, shard, xn, n_tokens, topk_ids, topk_weights,
                               partial_out, workspace, ev_begin, ev_end, workspace_bytes=None,
                               stream=None) -> None:
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(lib().tp_moe_shard_forward_timed(
        ctypes.byref(desc), ctypes.byref(moe), rank, ptr(shard), ptr(xn), n_tokens,
        ptr(topk_ids), ptr(topk_weights), ptr(partial_out), ptr(workspace), workspace_bytes,
        _stream(stream), ev_begin, ev_end))


def tp_status_str(status: int) -> str:
    return lib().tp_status_str(status).decode()


def tp_last_error() -> str:
    return lib().tp_last_error().decode()

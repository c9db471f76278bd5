"""Device buffers and the C-ABI call sequence of one emulated N-rank block step on one GPU.

A block step (mlxcel issue #488, "Problem": every rank runs in sequence on one device and the
partials are summed locally; TensorSharp "How tensor parallelism works": one reduce per half):

    xn  = RMSNorm(x) * gamma1                               tp_partial_reduce (no partials)
    for r in 0..N-1: P[r] = rank r's attention half          tp_block_shard_forward(ATTN, r)
    h1  = x + sum_r P[r];  xn2 = RMSNorm(h1) * gamma2        tp_partial_reduce
    for r in 0..N-1: P[r] = rank r's FFN half                tp_block_shard_forward(FFN, r)
    out = h1 + sum_r P[r]                                     tp_partial_reduce

Everything runs on the current HIP stream; this module only allocates torch tensors and passes
their addresses. ``copies`` > 1 keeps that many independent sets of shards and KV caches so a
timing loop can rotate through more bytes than the last-level cache holds.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B
from .inputs import BlockInputs, paged_prior_cache


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Storage array (fp32 / bf16 bit patterns / Q8_0 bytes) -> torch tensor on `device`."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16))
        return t.to(device).view(torch.bfloat16)
    if dtype == "q8_0":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)
    raise ValueError(dtype)


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Device tensor -> storage array (inverse of ``to_device``)."""
    if dtype == "bf16":
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    if dtype == "f32":
        return t.contiguous().cpu().numpy().astype(np.float32)
    return t.contiguous().cpu().numpy()


def act_torch_dtype(dtype: str):
    return torch.float32 if dtype == "f32" else torch.bfloat16


class DeviceBlock:
    """One block's shards, caches and buffers on the GPU, for all N emulated ranks."""

    def __init__(self, inp: BlockInputs, device="cuda", partial_dtype: str = "f32",
                 copies: int = 1, keep_full: bool = False):
        s = inp.shape
        self.inp, self.shape, self.device = inp, s, device
        self.N, self.T = s.tp, s.n_tokens
        self.desc = B.make_desc(s, partial_dtype)
        self.partial_dtype = partial_dtype
        adt = act_torch_dtype(s.act_dtype)

        full = {k: to_device(v, s.w_dtype, device) for k, v in inp.weights.items()}
        self.full = full if keep_full else None
        fw = B.full_weights(full)
        self.layouts = [B.tp_shard_weights_size(self.desc, r) for r in range(self.N)]
        self.shards = []          # [copy][rank]
        for _ in range(copies):
            row = []
            for r in range(self.N):
                buf = torch.empty(self.layouts[r].alloc_bytes, dtype=torch.uint8, device=device)
                B.tp_shard_weights(self.desc, r, fw, buf)
                row.append(buf)
            self.shards.append(row)
        torch.cuda.synchronize()
        del fw
        if not keep_full:
            del full

        self.gamma1 = to_device(inp.gamma1, s.act_dtype, device)
        self.gamma2 = to_device(inp.gamma2, s.act_dtype, device)
        self.x = to_device(inp.x, s.act_dtype, device)
        self.positions = torch.from_numpy(inp.positions).to(device)
        self.seq_lens = torch.from_numpy(inp.seq_lens).to(device)
        self.block_table = torch.from_numpy(np.ascontiguousarray(inp.block_table)).to(device)
        self.rope = torch.empty(B.tp_rope_table_bytes(self.desc) // 4, dtype=torch.float32,
                                device=device)
        B.tp_rope_table_init(self.desc, self.rope)

        self.max_pages = int(inp.block_table.shape[1])
        self.max_seq_len = int(max(inp.seq_lens))
        self.batch = B.make_batch(s.mode, self.T, s.n_seqs, self.max_pages, self.max_seq_len,
                                  self.positions, self.seq_lens, self.block_table, self.rope)

        # Per copy, per rank: paged K/V pools holding the owned KV heads' prior keys/values.
        self.kv_host = [paged_prior_cache(inp, r) for r in range(self.N)]
        self.k_pages, self.v_pages, self.kv = [], [], []
        for _ in range(copies):
            kr, vr, cr = [], [], []
            for r in range(self.N):
                kp = to_device(self.kv_host[r][0], s.act_dtype, device)
                vp = to_device(self.kv_host[r][1], s.act_dtype, device)
                kr.append(kp)
                vr.append(vp)
                cr.append(B.tp_kv_cache(k_pages=kp.data_ptr(), v_pages=vp.data_ptr(),
                                        n_pages=inp.n_pages))
            self.k_pages.append(kr)
            self.v_pages.append(vr)
            self.kv.append(cr)

        pdt = torch.float32 if partial_dtype == "f32" else torch.bfloat16
        self.partials = torch.empty((self.N, self.T, s.d_model), dtype=pdt, device=device)
        self.xn = torch.empty((self.T, s.d_model), dtype=adt, device=device)
        self.xn2 = torch.empty_like(self.xn)
        self.h1 = torch.empty_like(self.xn)
        self.out = torch.empty_like(self.xn)
        # tp_block_step may keep one copy per rank (the all-ranks schedule); the per-rank calls
        # use the first copy.
        self.ws_bytes = B.tp_step_workspace_size(self.desc, self.batch)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        self.copies = copies

    # --------------------------------------------------------------------------- the step
    def attn_half(self, rank: int, copy: int = 0, partial=None):
        B.tp_block_shard_forward(self.desc, rank, B.TP_HALF_ATTN, self.shards[copy][rank],
                                 self.batch, self.xn, self.kv[copy][rank],
                                 self.partials[rank] if partial is None else partial,
                                 self.workspace, self.ws_bytes)

    def ffn_half(self, rank: int, copy: int = 0, partial=None, events=None):
        """``events``: optional (begin, end) raw hipEvent_t handles that bracket the gate/up
        projection's kernel execution."""
        out = self.partials[rank] if partial is None else partial
        if events is None:
            B.tp_block_shard_forward(self.desc, rank, B.TP_HALF_FFN, self.shards[copy][rank],
                                     self.batch, self.xn2, None, out, self.workspace,
                                     self.ws_bytes)
        else:
            B.tp_block_shard_forward_timed(self.desc, rank, B.TP_HALF_FFN,
                                           self.shards[copy][rank], self.batch, self.xn2, None,
                                           out, self.workspace, events[0], events[1],
                                           self.ws_bytes)

    def step(self, copy: int = 0, ffn_events=None, x=None, xn_ready=False, next_norm=None):
        """One full block step on the current stream; the result lands in ``self.out``.
        ``ffn_events``: optional per-rank (begin, end) event pairs for the gate/up projections.
        ``x``: the block's input [T, d] (act dtype) in place of ``self.x``; ``xn_ready``: its
        RMSNorm is already in ``self.xn`` (the previous block's final reduce wrote it).
        ``next_norm``: (gamma, xn_out) of the next block: the final reduce also writes the next
        block's input RMSNorm, so that block skips its own."""
        d, T, N = self.desc, self.T, self.N
        x = self.x if x is None else x
        if not xn_ready:
            B.tp_partial_reduce(d, T, None, 0, x, None, self.gamma1, self.xn)
        for r in range(N):
            self.attn_half(r, copy)
        B.tp_partial_reduce(d, T, self.partials, N, x, self.h1, self.gamma2, self.xn2)
        for r in range(N):
            self.ffn_half(r, copy, events=None if ffn_events is None else ffn_events[r])
        g, xo = next_norm if next_norm is not None else (None, None)
        B.tp_partial_reduce(d, T, self.partials, N, self.h1, self.out, g, xo)

    def step_fused(self, copy: int = 0, x=None, timed=None, schedule=None):
        """The same block step in one library call (tp_block_step): for decode batches the
        replicated norms and the two reduces run inside the projections next to them, and (all-
        ranks schedule) each projection and the attention is one launch for every rank.
        ``timed``: (rank, begin, end) raw events bracketing that rank's gate/up projection (the
        all-ranks gate/up launch under that schedule). ``schedule``: a TP_SCHEDULE_* to force."""
        x = self.x if x is None else x
        args = (self.desc, self.shards[copy], self.batch, self.kv[copy], x, self.gamma1,
                self.gamma2, self.partials, self.xn, self.h1, self.xn2, self.out, self.workspace)
        if schedule is not None:
            B.tp_block_step_with_schedule(self.desc, schedule, *args[1:], self.ws_bytes)
        elif timed is None:
            B.tp_block_step(*args, self.ws_bytes)
        else:
            B.tp_block_step_timed(*args, timed[0], timed[1], timed[2], self.ws_bytes)

    def schedule(self) -> int:
        """The TP_SCHEDULE_* tp_block_step takes for this block's batch."""
        return B.tp_step_schedule(self.desc, self.batch)

    # --------------------------------------------------------------------------- readback
    def workspace_views(self):
        """Views of the last forward's intermediates: q [T, Hq/N*hd], a_r [T, Hq/N*hd], m_r."""
        s = self.shape
        qo, ao, fo = B.tp_workspace_offsets(self.desc, self.batch)
        adt = act_torch_dtype(s.act_dtype)
        es = 4 if s.act_dtype == "f32" else 2
        qd = s.n_heads // s.tp * s.head_dim
        fr = s.ffn_dim // s.tp

        def view(off, cols):
            return self.workspace[off: off + self.T * cols * es].view(adt).view(self.T, cols)
        return view(qo, qd), view(ao, qd), view(fo, fr)

    def cache_new_entries(self, rank: int, copy: int = 0):
        """The K and V the last ATTN call of ``rank`` wrote, as [T, Hkv/N, hd] storage arrays."""
        s = self.shape
        kp = to_host(self.k_pages[copy][rank], s.act_dtype)
        vp = to_host(self.v_pages[copy][rank], s.act_dtype)
        ks, vs = [], []
        for t in range(self.T):
            b = int(self.inp.token_seq[t])
            p = int(self.inp.positions[t])
            phys = self.inp.block_table[b, p // s.page_size]
            ks.append(kp[phys, :, p % s.page_size])
            vs.append(vp[phys, :, :, p % s.page_size])
        return np.stack(ks), np.stack(vs)


class BlockStack:
    """A stack of distinct blocks of one shape, as the layers of a decoder: block i's ``out`` is
    block i + 1's input (the residual stream), each block with its own shards, norms and
    per-rank KV caches. One ``step`` runs every block in order on the current stream (capturable
    as one HIP graph); the stack's output is ``self.out``."""

    def __init__(self, inputs, device="cuda", partial_dtype: str = "f32"):
        self.blocks = [DeviceBlock(inp, device=device, partial_dtype=partial_dtype)
                       for inp in inputs]
        self.x = self.blocks[0].x

    @property
    def out(self):
        return self.blocks[-1].out

    def step(self, x=None, ffn_events=None, fused=False, timed=None):
        """Every block in order; block i's final reduce also writes block i + 1's input RMSNorm
        (the same rounded residual it would normalise), saving one launch per block boundary.
        ``ffn_events``: optional per-block lists of per-rank gate/up event pairs. ``fused``:
        each block in one tp_block_step call instead (its projections normalise their input
        themselves, so nothing is carried across the boundary); ``timed``: then optional
        per-block (rank, begin, end) event triples."""
        x = self.x if x is None else x
        if fused:
            for i, blk in enumerate(self.blocks):
                blk.step_fused(x=x, timed=None if timed is None else timed[i])
                x = blk.out
            return
        K = len(self.blocks)
        for i, blk in enumerate(self.blocks):
            nxt = self.blocks[i + 1] if i + 1 < K else None
            blk.step(x=x, xn_ready=i > 0,
                     next_norm=(nxt.gamma1, nxt.xn) if nxt is not None else None,
                     ffn_events=None if ffn_events is None else ffn_events[i])
            x = blk.out


class DeviceHead:
    """The replicated head (one packed [vocab, d] table for the token-embedding lookup and the LM
    head, and the final norm's gamma) on the GPU."""

    def __init__(self, head, desc, device="cuda"):
        s = head.shape
        self.vocab, self.desc, self.shape = head.vocab, desc, s
        self.layout = B.tp_head_size(desc, head.vocab)
        src = to_device(head.table, s.w_dtype, device)
        self.table = torch.empty(self.layout.alloc_bytes, dtype=torch.uint8, device=device)
        B.tp_head_pack(desc, head.vocab, src, self.table)
        torch.cuda.synchronize()
        del src
        self.gamma_f = to_device(head.gamma_f, s.act_dtype, device)
        self.token_ids = torch.from_numpy(head.token_ids).to(device)

    def embed(self, x_out, token_ids=None):
        ids = self.token_ids if token_ids is None else token_ids
        B.tp_embed_lookup(self.desc, self.vocab, self.table, ids, int(ids.numel()), x_out)

    def logits(self, xn, out):
        B.tp_lm_head(self.desc, self.vocab, self.table, xn, int(xn.shape[0]), out)


class ModelStep:
    """A synthetic full-token step around a stack of blocks: embedding lookup, the stack, the
    final RMSNorm (the reduce kernel with no partials) and the LM head. Logits in ``self.logits``
    [T, vocab] fp32."""

    def __init__(self, head, inputs, device="cuda", partial_dtype: str = "f32"):
        self.stack = BlockStack(inputs, device=device, partial_dtype=partial_dtype)
        b0 = self.stack.blocks[0]
        self.head = DeviceHead(head, b0.desc, device=device)
        self.x = torch.empty_like(b0.x)
        self.xn_f = torch.empty_like(b0.x)
        self.logits = torch.empty((b0.T, head.vocab), dtype=torch.float32, device=device)

    def step(self, fused=False):
        b0 = self.stack.blocks[0]
        self.head.embed(self.x)
        self.stack.step(x=self.x, fused=fused)
        B.tp_partial_reduce(b0.desc, b0.T, None, 0, self.stack.out, None, self.head.gamma_f,
                            self.xn_f)
        self.head.logits(self.xn_f, self.logits)


class MoEBlock:
    """A block whose FFN half is the expert-sliced MoE: the dense attention half of a
    ``DeviceBlock`` for every rank, the reduce, the replicated router (computed once), every
    rank's MoE partial and the final reduce, all on the current stream."""

    def __init__(self, inp, minp, device="cuda", partial_dtype: str = "f32", copies: int = 1):
        s, m = inp.shape, minp.moe
        self.attn = DeviceBlock(inp, device=device, partial_dtype=partial_dtype, copies=copies)
        b = self.attn
        self.moe = B.make_moe_desc(m)
        self.m = m
        self.router = to_device(minp.router, s.act_dtype, device)
        full = {k: to_device(getattr(minp, k), s.w_dtype, device) for k in ("wg", "wu", "wd")}
        src = B.tp_moe_full_weights(**{k: v.data_ptr() for k, v in full.items()})
        self.layouts = [B.tp_moe_shard_size(b.desc, self.moe, r) for r in range(b.N)]
        self.shards = []
        for _ in range(copies):
            row = []
            for r in range(b.N):
                buf = torch.empty(self.layouts[r].alloc_bytes, dtype=torch.uint8, device=device)
                B.tp_moe_shard_weights(b.desc, self.moe, r, src, buf)
                row.append(buf)
            self.shards.append(row)
        torch.cuda.synchronize()
        del full
        T = b.T
        self.logits = torch.empty((T, m.n_experts), dtype=torch.float32, device=device)
        self.ids = torch.empty((T, m.top_k), dtype=torch.int32, device=device)
        self.weights = torch.empty((T, m.top_k), dtype=torch.float32, device=device)
        self.ws_bytes = B.tp_moe_workspace_size(b.desc, self.moe, T)
        # One rank's share per rank: the block step then runs every rank's expert gate/up as
        # one launch (the per-rank calls use the first share).
        self.step_ws_bytes = self.ws_bytes * b.N
        self.workspace = torch.empty(self.step_ws_bytes, dtype=torch.uint8, device=device)

    @property
    def out(self):
        return self.attn.out

    def route(self):
        b = self.attn
        B.tp_moe_route(b.desc, self.moe, self.router, b.xn2, b.T, self.logits, self.ids,
                       self.weights)

    def moe_half(self, rank: int, copy: int = 0, partial=None, events=None):
        b = self.attn
        out = b.partials[rank] if partial is None else partial
        if events is None:
            B.tp_moe_shard_forward(b.desc, self.moe, rank, self.shards[copy][rank], b.xn2, b.T,
                                   self.ids, self.weights, out, self.workspace, self.ws_bytes)
        else:
            B.tp_moe_shard_forward_timed(b.desc, self.moe, rank, self.shards[copy][rank], b.xn2,
                                         b.T, self.ids, self.weights, out, self.workspace,
                                         events[0], events[1], self.ws_bytes)

    def step_fused(self, copy: int = 0, moe_ws_bytes: int | None = None, timed=None):
        """The same MoE block step in one library call (tp_moe_block_step): for decode batches
        the norms and the reduces run inside the neighbouring projections. moe_ws_bytes: the
        expert workspace handed to the call (default: every rank's share). ``timed``: (begin,
        end) raw events bracketing the expert gate/up launch of every rank
        (tp_moe_block_step_timed)."""
        b = self.attn
        args = (b.desc, self.moe, b.shards[copy], self.shards[copy], b.batch, b.kv[copy], b.x,
                b.gamma1, b.gamma2, self.router, b.partials, b.xn, b.h1, b.xn2, b.out,
                self.logits, self.ids, self.weights, b.workspace, self.workspace)
        ws = self.step_ws_bytes if moe_ws_bytes is None else moe_ws_bytes
        if timed is None:
            B.tp_moe_block_step(*args, b.ws_bytes, ws)
        else:
            B.tp_moe_block_step_timed(*args, timed[0], timed[1], b.ws_bytes, ws)

    def step(self, copy: int = 0, moe_events=None):
        b = self.attn
        d, T, N = b.desc, b.T, b.N
        B.tp_partial_reduce(d, T, None, 0, b.x, None, b.gamma1, b.xn)
        for r in range(N):
            b.attn_half(r, copy)
        B.tp_partial_reduce(d, T, b.partials, N, b.x, b.h1, b.gamma2, b.xn2)
        self.route()
        for r in range(N):
            self.moe_half(r, copy, events=None if moe_events is None else moe_events[r])
        B.tp_partial_reduce(d, T, b.partials, N, b.h1, b.out, None, None)

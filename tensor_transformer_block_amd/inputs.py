"""Seeded synthetic inputs for the tensor-parallel block shard.

This module is the one piece shared by the HIP path's callers (tests, bench) and the CPU oracle's
callers. It draws random numbers and encodes them in the storage formats the block consumes
(fp32, bf16 bit patterns, Q8_0 blocks, a paged KV layout). It holds none of the block's arithmetic:
no normalisation, projection, rotation, attention, activation or reduction, and no dequantisation.

Workloads (the five block shapes a tensor-parallel decode/prefill step is measured on):

* ``tiny-llama-fp32``   d=256,  4 q / 4 kv heads of 64, SwiGLU 688,   N=2, fp32, decode B=1 L=16
* ``llama3-8b-decode``  d=4096, 32 q / 8 kv heads of 128, SwiGLU 14336, N=2, bf16, decode B=1 L=4096
* ``llama3-8b-batched`` same block, N=4, bf16, batched decode B=64, L=2048 each, 16-token pages
* ``llama-70b-prefill`` d=8192, 64 q / 8 kv heads of 128, SwiGLU 28672, N=8, bf16, prefill T=2048
* ``gemma-q8-decode``   d=2560, 8 q / 2 kv heads of 256, GELU-tanh 10240, N=2, Q8_0 weights, bf16
                        activations, decode B=1 L=8192

Recipe (fixed draw order from ``numpy.random.default_rng([seed, index])``, float32 standard
normals): gamma1, gamma2 as 1 + 0.1 N; Wq, Wk, Wv, Wo, Wg, Wu, Wd as 0.02 N, stored [out, in]
row-major; x as N(0, 1); the prior K cache of every sequence, then the prior V cache, as N(0, 1)
of shape [n_kv_heads, prior_len, head_dim]; then a permutation of the physical page ids.
bf16 storage rounds to nearest even. Q8_0 storage quantises blocks of 32 along the input dim:
d32 = max|w| / 127 (fp32), stored scale fp16(d32) (round to nearest even),
q = clamp(round_half_away_from_zero(w / d32), -127, 127) with the quotient taken in fp64; a zero
block stores d = 0, q = 0. Each block is 34 bytes: the fp16 scale (little endian), then 32 int8.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "bf16", "q8_0")
ACTS = ("silu", "gelu_tanh")
Q8_BLOCK = 32
Q8_BLOCK_BYTES = 34


@dataclass(frozen=True)
class BlockShape:
    """Dimensions and step description of one block shard workload."""

    name: str
    index: int                 # second word of the RNG seed
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    tp: int
    w_dtype: str
    act_dtype: str
    ffn_act: str
    mode: str                  # "decode" (one new token per sequence) or "prefill" (one sequence)
    kv_lens: tuple             # keys attended per sequence, new tokens included
    n_tokens: int              # decode: == number of sequences; prefill: new tokens of sequence 0
    page_size: int = 16
    rms_eps: float = 1e-5
    rope_base: float = 10000.0
    max_position: int = 0      # 0: max(kv_lens)

    @property
    def n_seqs(self) -> int:
        return len(self.kv_lens)

    @property
    def max_pos(self) -> int:
        return self.max_position or max(self.kv_lens)

    def with_(self, **kw) -> "BlockShape":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny-llama-fp32": BlockShape(
        name="tiny-llama-fp32", index=0, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64,
        ffn_dim=688, tp=2, w_dtype="f32", act_dtype="f32", ffn_act="silu", mode="decode",
        kv_lens=(16,), n_tokens=1),
    "llama3-8b-decode": BlockShape(
        name="llama3-8b-decode", index=1, d_model=4096, n_heads=32, n_kv_heads=8, head_dim=128,
        ffn_dim=14336, tp=2, w_dtype="bf16", act_dtype="bf16", ffn_act="silu", mode="decode",
        kv_lens=(4096,), n_tokens=1),
    "llama3-8b-batched": BlockShape(
        name="llama3-8b-batched", index=2, d_model=4096, n_heads=32, n_kv_heads=8, head_dim=128,
        ffn_dim=14336, tp=4, w_dtype="bf16", act_dtype="bf16", ffn_act="silu", mode="decode",
        kv_lens=(2048,) * 64, n_tokens=64),
    "llama-70b-prefill": BlockShape(
        name="llama-70b-prefill", index=3, d_model=8192, n_heads=64, n_kv_heads=8, head_dim=128,
        ffn_dim=28672, tp=8, w_dtype="bf16", act_dtype="bf16", ffn_act="silu", mode="prefill",
        kv_lens=(2048,), n_tokens=2048),
    "gemma-q8-decode": BlockShape(
        name="gemma-q8-decode", index=4, d_model=2560, n_heads=8, n_kv_heads=2, head_dim=256,
        ffn_dim=10240, tp=2, w_dtype="q8_0", act_dtype="bf16", ffn_act="gelu_tanh", mode="decode",
        kv_lens=(8192,), n_tokens=1),
}

# Further shapes for the Q8_0 matrix-core projections (more than four tokens): the Gemma-like
# block in batched decode, and the Llama-3-8B-shaped block quantised to Q8_0 at degree 4 in
# prefill (its row-parallel splits fall on 32-weight block boundaries at N = 4).
EXTRA_WORKLOADS = {
    "gemma-q8-batched": BlockShape(
        name="gemma-q8-batched", index=5, d_model=2560, n_heads=8, n_kv_heads=2, head_dim=256,
        ffn_dim=10240, tp=2, w_dtype="q8_0", act_dtype="bf16", ffn_act="gelu_tanh",
        mode="decode", kv_lens=(2048,) * 64, n_tokens=64),
    "llama3-8b-q8-prefill": BlockShape(
        name="llama3-8b-q8-prefill", index=6, d_model=4096, n_heads=32, n_kv_heads=8,
        head_dim=128, ffn_dim=14336, tp=4, w_dtype="q8_0", act_dtype="bf16", ffn_act="silu",
        mode="prefill", kv_lens=(2048,), n_tokens=2048),
}
WORKLOADS = {**CONFIGS, **EXTRA_WORKLOADS}

WEIGHT_NAMES = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def weight_shapes(s: BlockShape) -> dict:
    """[out, in] of every full (unsharded) weight matrix."""
    qd, kd = s.n_heads * s.head_dim, s.n_kv_heads * s.head_dim
    return {
        "wq": (qd, s.d_model), "wk": (kd, s.d_model), "wv": (kd, s.d_model),
        "wo": (s.d_model, qd),
        "wg": (s.ffn_dim, s.d_model), "wu": (s.ffn_dim, s.d_model),
        "wd": (s.d_model, s.ffn_dim),
    }


# ----------------------------------------------------------------------------- storage encoders

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even) and return the 16-bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    flat_in, flat_out = a.reshape(-1), out.reshape(-1)
    step = 1 << 24
    for i in range(0, flat_in.size, step):
        u = flat_in[i:i + step].view(np.uint32)
        r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
        flat_out[i:i + step] = (r >> np.uint32(16)).astype(np.uint16)
    return out


def q8_0_encode(w: np.ndarray) -> np.ndarray:
    """Encode a float32 [rows, cols] matrix as Q8_0 blocks: uint8 [rows, cols/32*34]."""
    rows, cols = w.shape
    assert cols % Q8_BLOCK == 0, "Q8_0 needs the input dim to be a multiple of 32"
    nb = cols // Q8_BLOCK
    out = np.empty((rows, nb, Q8_BLOCK_BYTES), dtype=np.uint8)
    step = max(1, (1 << 22) // cols)
    for r0 in range(0, rows, step):
        blk = np.asarray(w[r0:r0 + step], dtype=np.float32).reshape(-1, nb, Q8_BLOCK)
        amax = np.max(np.abs(blk), axis=2)
        d32 = (amax / np.float32(127.0)).astype(np.float32)
        d16 = d32.astype(np.float16)
        safe = np.where(d32 > 0, d32, np.float32(1.0)).astype(np.float64)
        v = blk.astype(np.float64) / safe[..., None]
        q = np.sign(v) * np.floor(np.abs(v) + 0.5)
        q = np.clip(q, -127, 127)
        q = np.where((d32 > 0)[..., None], q, 0).astype(np.int8)
        out[r0:r0 + step, :, 0:2] = d16.view(np.uint8).reshape(blk.shape[0], nb, 2)
        out[r0:r0 + step, :, 2:] = q.view(np.uint8)
    return out.reshape(rows, nb * Q8_BLOCK_BYTES)


def _encode(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(a32)
    if dtype == "q8_0":
        return q8_0_encode(a32)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------- the inputs

@dataclass
class BlockInputs:
    """One block step's inputs in storage form (what the GPU receives, bit for bit).

    f32 tensors are float32 arrays, bf16 tensors uint16 bit patterns, Q8_0 weights uint8 blocks.
    """

    shape: BlockShape
    gamma1: np.ndarray
    gamma2: np.ndarray
    weights: dict
    x: np.ndarray                     # [T, d]
    k_prior: list                     # per sequence [n_kv_heads, prior_len, head_dim]
    v_prior: list
    positions: np.ndarray             # int32 [T]
    token_seq: np.ndarray             # int32 [T]: sequence of each token
    seq_lens: np.ndarray              # int32 [B]: keys attended incl. new tokens
    block_table: np.ndarray           # int32 [B, max_pages]
    n_pages: int
    extras: dict = field(default_factory=dict)


def make_inputs(s: BlockShape, seed: int = 0, block: int = 0) -> BlockInputs:
    """One block's inputs. ``block`` > 0 draws another block of the same shape (its own weights,
    norms and prior caches) from the stream ``[seed, index, block]``; block 0 is the workload."""
    rng = np.random.default_rng([seed, s.index] if block == 0 else [seed, s.index, block])
    nrm = lambda shape: rng.standard_normal(shape, dtype=np.float32)

    g1 = (np.float32(1.0) + np.float32(0.1) * nrm(s.d_model)).astype(np.float32)
    g2 = (np.float32(1.0) + np.float32(0.1) * nrm(s.d_model)).astype(np.float32)
    weights = {}
    for name, shp in weight_shapes(s).items():
        w32 = nrm(shp)
        w32 *= np.float32(0.02)
        weights[name] = _encode(w32, s.w_dtype)
        del w32
    T = s.n_tokens
    x = nrm((T, s.d_model))

    B = s.n_seqs
    if s.mode == "decode":
        assert T == B, "decode steps carry one new token per sequence"
        new_per_seq = [1] * B
        positions = np.array([L - 1 for L in s.kv_lens], dtype=np.int32)
        token_seq = np.arange(B, dtype=np.int32)
    elif s.mode == "prefill":
        assert B == 1, "prefill steps carry one sequence"
        L = s.kv_lens[0]
        assert T <= L
        new_per_seq = [T]
        positions = np.arange(L - T, L, dtype=np.int32)
        token_seq = np.zeros(T, dtype=np.int32)
    else:
        raise ValueError(s.mode)
    prior = [L - n for L, n in zip(s.kv_lens, new_per_seq)]
    k_prior = [_encode(nrm((s.n_kv_heads, p, s.head_dim)), s.act_dtype) for p in prior]
    v_prior = [_encode(nrm((s.n_kv_heads, p, s.head_dim)), s.act_dtype) for p in prior]

    pages_per_seq = [-(-L // s.page_size) for L in s.kv_lens]
    n_pages = int(sum(pages_per_seq))
    perm = rng.permutation(n_pages).astype(np.int32)
    max_pages = max(pages_per_seq)
    table = np.zeros((B, max_pages), dtype=np.int32)
    off = 0
    for b, n in enumerate(pages_per_seq):
        table[b, :n] = perm[off:off + n]
        off += n

    return BlockInputs(
        shape=s, gamma1=_encode(g1, s.act_dtype), gamma2=_encode(g2, s.act_dtype),
        weights=weights, x=_encode(x, s.act_dtype), k_prior=k_prior, v_prior=v_prior,
        positions=positions, token_seq=token_seq,
        seq_lens=np.array(s.kv_lens, dtype=np.int32), block_table=table, n_pages=n_pages)


def make_stack_inputs(s: BlockShape, n_blocks: int, seed: int = 0) -> list:
    """Inputs of a stack of ``n_blocks`` distinct blocks of one shape, as the layers of a decoder:
    block 0 is ``make_inputs(s, seed)``; only its x enters the stack (each later block takes the
    previous block's output); every block keeps its own weights, norms and KV caches."""
    return [make_inputs(s, seed, block=i) for i in range(n_blocks)]


# Vocabulary sizes of the model families the workloads are shaped after (the replicated head).
VOCAB = {"tiny-llama-fp32": 512, "llama3-8b-decode": 128256, "llama3-8b-batched": 128256,
         "llama-70b-prefill": 128256, "gemma-q8-decode": 262144, "gemma-q8-batched": 262144,
         "llama3-8b-q8-prefill": 128256}


@dataclass
class HeadInputs:
    """The replicated head around a stack: one table [vocab, d] (storage form, w_dtype) used for
    the token-embedding lookup and as the LM head, the final norm's gamma and the token ids."""

    shape: BlockShape
    vocab: int
    table: np.ndarray                 # f32 / bf16 bits [vocab, d]; Q8_0 bytes [vocab, d/32*34]
    gamma_f: np.ndarray               # [d], activation storage dtype
    token_ids: np.ndarray             # int32 [T]


def make_head_inputs(s: BlockShape, vocab: int, seed: int = 0) -> HeadInputs:
    """Draws from ``[seed, index, 1 << 20]``: gamma_f as 1 + 0.1 N, the table as 0.02 N
    [vocab, d] (stored like the block weights), then T token ids uniform in [0, vocab)."""
    rng = np.random.default_rng([seed, s.index, 1 << 20])
    gf = (np.float32(1.0) + np.float32(0.1) * rng.standard_normal(s.d_model, dtype=np.float32))
    table = np.empty((vocab, s.d_model), dtype=np.float32)
    step = max(1, (1 << 24) // s.d_model)
    for r0 in range(0, vocab, step):
        r1 = min(vocab, r0 + step)
        table[r0:r1] = rng.standard_normal((r1 - r0, s.d_model), dtype=np.float32)
        table[r0:r1] *= np.float32(0.02)
    ids = rng.integers(0, vocab, s.n_tokens, dtype=np.int64).astype(np.int32)
    return HeadInputs(shape=s, vocab=vocab, table=_encode(table, s.w_dtype),
                      gamma_f=_encode(gf.astype(np.float32), s.act_dtype), token_ids=ids)


@dataclass(frozen=True)
class MoEShape:
    """A mixture-of-experts FFN in place of the dense one: n_experts SwiGLU (or GELU-gated)
    experts of width expert_ffn, top_k of them per token."""

    n_experts: int
    top_k: int
    expert_ffn: int


@dataclass
class MoEInputs:
    """Storage-form MoE FFN weights: the router [E, d] (activation dtype), the experts' gate and
    up rows stacked expert-major [E * F_e, d] and their down matrices stacked [E * d, F_e]
    (weight dtype; Q8_0 blocks along the input dim)."""

    shape: BlockShape
    moe: MoEShape
    router: np.ndarray
    wg: np.ndarray
    wu: np.ndarray
    wd: np.ndarray


# A mixture-of-experts block for measurement: a dense attention half (32 query / 4 KV heads of
# 128) and 64 SwiGLU experts of width 768, 8 per token, at degree 2, decoding one token against
# a 4096-token cache.
MOE_WORKLOADS = {
    "moe-decode": (BlockShape(name="moe-decode", index=7, d_model=2048, n_heads=32, n_kv_heads=4,
                              head_dim=128, ffn_dim=768, tp=2, w_dtype="bf16", act_dtype="bf16",
                              ffn_act="silu", mode="decode", kv_lens=(4096,), n_tokens=1),
                   MoEShape(n_experts=64, top_k=8, expert_ffn=768)),
}


def make_moe_inputs(s: BlockShape, moe: MoEShape, seed: int = 0, block: int = 0) -> MoEInputs:
    """Draws from ``[seed, index, 2^21, block]``: router, then every expert's gate rows, up rows
    and down matrix, all 0.02 N."""
    rng = np.random.default_rng([seed, s.index, 1 << 21, block])
    E, F, d = moe.n_experts, moe.expert_ffn, s.d_model

    def draw(rows, cols, dtype):
        a = np.empty((rows, cols), dtype=np.float32)
        step = max(1, (1 << 24) // cols)
        for r0 in range(0, rows, step):
            r1 = min(rows, r0 + step)
            a[r0:r1] = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
            a[r0:r1] *= np.float32(0.02)
        return _encode(a, dtype)
    router = draw(E, d, s.act_dtype)
    wg = draw(E * F, d, s.w_dtype)
    wu = draw(E * F, d, s.w_dtype)
    wd = draw(E * d, F, s.w_dtype)
    return MoEInputs(shape=s, moe=moe, router=router, wg=wg, wu=wu, wd=wd)


def paged_prior_cache(inp: BlockInputs, rank: int):
    """Rank ``rank``'s K and V page pools holding its owned KV heads' prior keys/values.

    K: [n_pages][n_kv_heads / tp][page_size][head_dim]; V is stored transposed,
    [n_pages][n_kv_heads / tp][head_dim][page_size]; activation storage dtype. Slots that hold no
    prior key are zero.
    """
    s = inp.shape
    hk = s.n_kv_heads // s.tp
    g0 = rank * hk
    dt = np.float32 if s.act_dtype == "f32" else np.uint16
    kp = np.zeros((inp.n_pages, hk, s.page_size, s.head_dim), dtype=dt)
    vp = np.zeros((inp.n_pages, hk, s.head_dim, s.page_size), dtype=dt)
    for b in range(s.n_seqs):
        kb, vb = inp.k_prior[b][g0:g0 + hk], inp.v_prior[b][g0:g0 + hk]
        plen = kb.shape[1]
        for pg in range(-(-plen // s.page_size)):
            j0, j1 = pg * s.page_size, min(plen, (pg + 1) * s.page_size)
            phys = inp.block_table[b, pg]
            kp[phys, :, 0:j1 - j0] = kb[:, j0:j1]
            vp[phys, :, :, 0:j1 - j0] = np.swapaxes(vb[:, j0:j1], 1, 2)
    return kp, vp

"""CPU oracle for one Megatron-style tensor-parallel transformer block (fp64, NumPy).

TEST INFRASTRUCTURE ONLY. This code is slow on purpose and is never part of the product path:
only the test suite, the package entry point's smoke check and the benchmark's CPU-baseline leg
may import it. It shares no code with the HIP library or its Python binding.

What it computes, and where the pages fix it:

* TensorSharp, "Multi-GPU & Multi-Node", section "How tensor parallelism works": a block is a
  complementary pair of shardings. Column-parallel QKV and gate/up split their output dim (heads,
  FFN columns) and need no communication; attention or the activation runs per rank over the heads
  that rank owns, against that rank's own KV cache; row-parallel o_proj and down split their input
  dim so each rank emits a partial sum, and one all-reduce per block half makes the hidden state
  identical on every rank. Norms stay replicated on every rank.
* mlxcel issue #488, section "Problem": in the one-device runtime every rank runs in sequence and
  the partials are summed locally ("reduce_sum"); this is the reduction ``block_sharded`` models.
* nnsight PR #677, section "Change": a row-parallel layer is cut along its input features and the
  remaining parallel layers along their output features; a fused weight keeps each rank's rows
  together (the layers compute ``x @ weight.T``).

The pages do not define the block's sublayers. Their published definitions are used:
RMSNorm (Zhang & Sennrich 2019), rotary embedding in its rotate-half form (Su et al. 2021),
softmax attention with grouped KV heads, SiLU (Elfwing et al. 2018) gating as in SwiGLU
(Shazeer 2020), and the tanh form of GELU (Hendrycks & Gimpel 2016).

``block_unsharded`` is the ground truth; ``block_sharded`` is the explicit N-rank computation,
rank by rank and head by head, with the partial sums added in rank order.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------- storage decoders


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64: the pattern is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> float64."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequant_q8_0(blocks: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Q8_0 blocks -> float64 [rows, cols].

    TensorSharp "Requirements & constraints" names block-quantised row-parallel splits; the Q8_0
    format stores, per 32 consecutive weights along the input dim, one fp16 scale d followed by 32
    signed bytes q, and the weight value is d * q.
    """
    nb = cols // 32
    raw = np.asarray(blocks, dtype=np.uint8).reshape(rows, nb, 34)
    d = f16_bits_to_f64(raw[:, :, 0:2].copy().view(np.uint16)[..., 0])
    q = raw[:, :, 2:].copy().view(np.int8).astype(np.float64)
    return (d[..., None] * q).reshape(rows, cols)


def to_f64(a: np.ndarray, dtype: str, shape=None) -> np.ndarray:
    """Stored tensor (fp32 values, bf16 patterns or Q8_0 blocks) -> float64."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    if dtype == "q8_0":
        return dequant_q8_0(a, *shape)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------- sublayers


def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last dim: gamma * x / sqrt(mean(x^2) + eps)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return gamma * (x / np.sqrt(ms + eps))


def rope_cos_sin(position: int, head_dim: int, base: float):
    """Rotary angles for one position: theta_i = base^(-2i/hd), i < hd/2."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / head_dim)
    ang = float(position) * theta
    return np.cos(ang), np.sin(ang)


def rope(vec: np.ndarray, position: int, base: float) -> np.ndarray:
    """Rotate-half rotary embedding of one head vector (or a stack of them, last dim = hd).

    The pair (x_i, x_{i+hd/2}) is rotated by the angle position * theta_i.
    """
    hd = vec.shape[-1]
    c, s = rope_cos_sin(position, hd, base)
    a, b = vec[..., : hd // 2], vec[..., hd // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def gelu_tanh(z: np.ndarray) -> np.ndarray:
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


ACTIVATIONS = {"silu": silu, "gelu_tanh": gelu_tanh}


def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Softmax attention of one query vector over n keys: softmax(q.K^T / sqrt(hd)) . V."""
    s = keys @ q / np.sqrt(q.shape[-1])
    w = np.exp(s - np.max(s))
    w = w / np.sum(w)
    return w @ values


# ----------------------------------------------------------------------------- parameters


def params_f64(inp) -> dict:
    """All block parameters of a ``BlockInputs`` widened to float64 (dequantised for Q8_0)."""
    s = inp.shape
    shapes = {
        "wq": (s.n_heads * s.head_dim, s.d_model), "wk": (s.n_kv_heads * s.head_dim, s.d_model),
        "wv": (s.n_kv_heads * s.head_dim, s.d_model), "wo": (s.d_model, s.n_heads * s.head_dim),
        "wg": (s.ffn_dim, s.d_model), "wu": (s.ffn_dim, s.d_model), "wd": (s.d_model, s.ffn_dim),
    }
    p = {k: to_f64(inp.weights[k], s.w_dtype, shapes[k]) for k in shapes}
    p["gamma1"] = to_f64(inp.gamma1, s.act_dtype)
    p["gamma2"] = to_f64(inp.gamma2, s.act_dtype)
    return p


def caches_f64(inp):
    """Per-sequence logical caches [n_kv_heads, kv_len, hd], prior part filled, rest zero."""
    s = inp.shape
    kc, vc = [], []
    for b in range(s.n_seqs):
        L = int(inp.seq_lens[b])
        k = np.zeros((s.n_kv_heads, L, s.head_dim))
        v = np.zeros_like(k)
        kp = to_f64(inp.k_prior[b], s.act_dtype)
        vp = to_f64(inp.v_prior[b], s.act_dtype)
        k[:, : kp.shape[1]] = kp
        v[:, : vp.shape[1]] = vp
        kc.append(k)
        vc.append(v)
    return kc, vc


# ----------------------------------------------------------------------------- the block


def block_unsharded(s, p, x, kcache, vcache, positions, token_seq, rows=None):
    """The whole block on one device, no sharding: the ground truth.

    s: a BlockShape; p: ``params_f64``; x [T, d] float64; kcache/vcache: per-sequence logical
    caches, updated in place with every new token's post-rotary K and V before any attention.
    rows: token rows whose attention/FFN outputs are wanted (default all); K and V are produced
    for every token since later rows attend to them.
    Returns a dict of float64 intermediates (rows restricted to ``rows``).
    """
    T = x.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    hd, Hq, Hkv = s.head_dim, s.n_heads, s.n_kv_heads
    grp = Hq // Hkv
    xn = rms_norm(x, p["gamma1"], s.rms_eps)
    k = (xn @ p["wk"].T).reshape(T, Hkv, hd)
    v = (xn @ p["wv"].T).reshape(T, Hkv, hd)
    for t in range(T):
        sq, pos = int(token_seq[t]), int(positions[t])
        kcache[sq][:, pos] = rope(k[t], pos, s.rope_base)
        vcache[sq][:, pos] = v[t]
    xr = x[rows]
    q = (xn[rows] @ p["wq"].T).reshape(len(rows), Hq, hd)
    attn = np.zeros((len(rows), Hq, hd))
    for i, t in enumerate(rows):
        sq, pos = int(token_seq[t]), int(positions[t])
        q[i] = rope(q[i], pos, s.rope_base)
        for h in range(Hq):
            g = h // grp
            attn[i, h] = attend(q[i, h], kcache[sq][g, : pos + 1], vcache[sq][g, : pos + 1])
    attn = attn.reshape(len(rows), Hq * hd)
    attn_proj = attn @ p["wo"].T
    h1 = xr + attn_proj
    xn2 = rms_norm(h1, p["gamma2"], s.rms_eps)
    gate = xn2 @ p["wg"].T
    up = xn2 @ p["wu"].T
    m = ACTIVATIONS[s.ffn_act](gate) * up
    ffn_proj = m @ p["wd"].T
    out = h1 + ffn_proj
    return dict(xn=xn[rows], q=q, k_new=np.stack([kcache[int(token_seq[t])][:, int(positions[t])]
                                                  for t in rows]),
                v_new=v[rows], attn=attn, attn_proj=attn_proj, h1=h1, xn2=xn2, gate=gate, up=up,
                m=m, ffn_proj=ffn_proj, out=out)


def shard_slices(s, r: int) -> dict:
    """Rank r's owned index ranges: query heads, KV heads and FFN columns (contiguous blocks)."""
    hq, hk, fr = s.n_heads // s.tp, s.n_kv_heads // s.tp, s.ffn_dim // s.tp
    return dict(q_heads=range(r * hq, (r + 1) * hq), kv_heads=range(r * hk, (r + 1) * hk),
                ffn=range(r * fr, (r + 1) * fr))


def shard_weights(s, p, r: int) -> dict:
    """Rank r's weight slices in logical form.

    Column-parallel (output dim): Wq rows of the owned query heads, Wk/Wv rows of the owned KV
    heads, Wg/Wu rows of the owned FFN columns. Row-parallel (input dim): Wo columns of the owned
    query heads, Wd columns of the owned FFN columns.
    """
    sl = shard_slices(s, r)
    hd = s.head_dim
    qrows = slice(sl["q_heads"].start * hd, sl["q_heads"].stop * hd)
    krows = slice(sl["kv_heads"].start * hd, sl["kv_heads"].stop * hd)
    frows = slice(sl["ffn"].start, sl["ffn"].stop)
    return dict(wq=p["wq"][qrows], wk=p["wk"][krows], wv=p["wv"][krows],
                wo=p["wo"][:, qrows], wg=p["wg"][frows], wu=p["wu"][frows], wd=p["wd"][:, frows])


def block_sharded(s, p, x, kcaches_by_rank, vcaches_by_rank, positions, token_seq, rows=None):
    """The explicit N-rank block: every rank's share computed in sequence, partials reduced.

    kcaches_by_rank[r][seq]: rank r's cache holding only its owned KV heads [hkv/N, L, hd];
    updated in place. Returns the replicated tensors (xn, h1, xn2, out) and, per rank, the
    pre-rotary qkv, post-rotary q, the new K and V, the attention output a_r, m_r and both
    partial sums.
    """
    xn, ranks, red, h1 = attention_sharded(s, p, x, kcaches_by_rank, vcaches_by_rank, positions,
                                           token_seq, rows)
    N = s.tp
    act = ACTIVATIONS[s.ffn_act]
    xn2 = rms_norm(h1, p["gamma2"], s.rms_eps)
    for r in range(N):
        w = ranks[r]["w"]
        m_r = act(xn2 @ w["wg"].T) * (xn2 @ w["wu"].T)
        ranks[r]["m"] = m_r
        ranks[r]["p_ffn"] = m_r @ w["wd"].T
    red2 = ranks[0]["p_ffn"].copy()
    for r in range(1, N):
        red2 = red2 + ranks[r]["p_ffn"]
    out = h1 + red2
    for rk in ranks:
        del rk["w"]
    return dict(xn=xn, h1=h1, xn2=xn2, out=out, attn_sum=red, ffn_sum=red2, ranks=ranks)


def attention_sharded(s, p, x, kcaches_by_rank, vcaches_by_rank, positions, token_seq, rows=None):
    """The attention half of the explicit N-rank block: xn, per-rank shares (pre-rotary qkv,
    rotated q, new K and V, a_r, its o_proj partial, and the rank's weight slices as "w"), their
    rank-ordered sum and h1 = x + that sum (rows restricted to ``rows``)."""
    N = s.tp
    T = x.shape[0]
    rows = np.arange(T) if rows is None else np.asarray(rows)
    hd = s.head_dim
    hq, hk = s.n_heads // N, s.n_kv_heads // N
    grp = s.n_heads // s.n_kv_heads
    xn = rms_norm(x, p["gamma1"], s.rms_eps)
    ranks = []
    for r in range(N):
        w = shard_weights(s, p, r)
        sl = shard_slices(s, r)
        w_qkv = np.concatenate([w["wq"], w["wk"], w["wv"]], axis=0)
        qkv_all = xn @ w_qkv.T
        k_r = qkv_all[:, hq * hd:(hq + hk) * hd].reshape(T, hk, hd)
        v_r = qkv_all[:, (hq + hk) * hd:].reshape(T, hk, hd)
        for t in range(T):
            sq, pos = int(token_seq[t]), int(positions[t])
            for j in range(hk):
                kcaches_by_rank[r][sq][j, pos] = rope(k_r[t, j], pos, s.rope_base)
                vcaches_by_rank[r][sq][j, pos] = v_r[t, j]
        q_r = qkv_all[rows, : hq * hd].reshape(len(rows), hq, hd).copy()
        a_r = np.zeros((len(rows), hq, hd))
        for i, t in enumerate(rows):
            sq, pos = int(token_seq[t]), int(positions[t])
            for j in range(hq):
                q_r[i, j] = rope(q_r[i, j], pos, s.rope_base)
                g_global = sl["q_heads"][j] // grp
                g_local = g_global - sl["kv_heads"].start
                kc = kcaches_by_rank[r][sq][g_local, : pos + 1]
                vc = vcaches_by_rank[r][sq][g_local, : pos + 1]
                a_r[i, j] = attend(q_r[i, j], kc, vc)
        a_r = a_r.reshape(len(rows), hq * hd)
        ranks.append(dict(qkv=qkv_all[rows], q=q_r,
                          k_new=np.stack([kcaches_by_rank[r][int(token_seq[t])][:, int(positions[t])]
                                          for t in rows]),
                          v_new=v_r[rows], a=a_r, p_attn=a_r @ w["wo"].T, w=w))
    red = ranks[0]["p_attn"].copy()
    for r in range(1, N):
        red = red + ranks[r]["p_attn"]
    h1 = x[rows] + red
    return xn[rows], ranks, red, h1


def rank_caches(s, kcache, vcache):
    """Split per-sequence logical caches [Hkv, L, hd] into per-rank owned-head copies."""
    hk = s.n_kv_heads // s.tp
    kr = [[k[r * hk:(r + 1) * hk].copy() for k in kcache] for r in range(s.tp)]
    vr = [[v[r * hk:(r + 1) * hk].copy() for v in vcache] for r in range(s.tp)]
    return kr, vr


def run_block(inp, sharded=True, rows=None):
    """Convenience: widen a BlockInputs and run the sharded (default) or unsharded block."""
    s = inp.shape
    p = params_f64(inp)
    x = to_f64(inp.x, s.act_dtype)
    kc, vc = caches_f64(inp)
    if not sharded:
        res = block_unsharded(s, p, x, kc, vc, inp.positions, inp.token_seq, rows)
        res["kcache"], res["vcache"] = kc, vc
        return res
    kr, vr = rank_caches(s, kc, vc)
    res = block_sharded(s, p, x, kr, vr, inp.positions, inp.token_seq, rows)
    res["kcache_by_rank"], res["vcache_by_rank"] = kr, vr
    return res


def run_stack(inputs, sharded=True, x=None):
    """A stack of blocks, as the layers of a decoder: the residual stream leaves block i as its
    ``out`` and enters block i + 1 as its x (TensorSharp, "Multi-GPU & Multi-Node", section "How
    tensor parallelism works": every rank ends each block half holding the identical hidden state,
    which is what the next layer consumes). ``inputs``: BlockInputs of one shape; the stack input
    is ``x`` (fp64 [T, d]) or else the first one's x. Returns the per-block result dicts (full
    rows, fp64, no rounding between blocks)."""
    if x is None:
        x = to_f64(inputs[0].x, inputs[0].shape.act_dtype)
    results = []
    for inp in inputs:
        s = inp.shape
        p = params_f64(inp)
        kc, vc = caches_f64(inp)
        if sharded:
            kr, vr = rank_caches(s, kc, vc)
            res = block_sharded(s, p, x, kr, vr, inp.positions, inp.token_seq)
        else:
            res = block_unsharded(s, p, x, kc, vc, inp.positions, inp.token_seq)
        res["x"] = x
        results.append(res)
        x = res["out"]
    return results


# ----------------------------------------------------------------------------- the replicated head
# TensorSharp, "Multi-GPU & Multi-Node", section "How tensor parallelism works": the norms, the
# token embeddings and the LM head are held whole on every rank (no sharding, no collective);
# mlxcel issue #488, section "Out of scope", keeps embeddings and LM head replicated too.


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Values exactly representable in fp32 -> nearest bfloat16 (ties to even), as float64: keep
    the top 16 bits of the fp32 pattern after adding 0x7FFF plus the lowest kept bit."""
    u = np.asarray(a, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (r.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def head_table_f64(head) -> np.ndarray:
    """The head's [vocab, d] table widened to fp64 (Q8_0 blocks dequantised exactly)."""
    s = head.shape
    if s.w_dtype == "q8_0":
        return dequant_q8_0(head.table, head.vocab, s.d_model)
    return to_f64(head.table, s.w_dtype)


def embed_lookup(head, table=None) -> np.ndarray:
    """x[t] = row token_ids[t] of the table, as the activation dtype stores it: f32 and bf16 rows
    are taken as stored; a Q8_0 row's dequantised values (exact in fp32) are rounded to bf16."""
    s = head.shape
    table = head_table_f64(head) if table is None else table
    x = table[np.asarray(head.token_ids, dtype=np.int64)]
    if s.w_dtype == "q8_0":
        x = round_to_bf16(x)
    return x


def lm_head(xn: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Logits [T, vocab] = xn [T, d] times the table transposed."""
    return xn @ table.T


def run_model(head, inputs, sharded=True):
    """A synthetic full-token step: embedding lookup, the stack of blocks, the final RMSNorm with
    the head's gamma, and the LM head. Returns dict(x, stack, xn_f, logits)."""
    s = head.shape
    table = head_table_f64(head)
    x = embed_lookup(head, table)
    stack = run_stack(inputs, sharded=sharded, x=x)
    xn_f = rms_norm(stack[-1]["out"], to_f64(head.gamma_f, s.act_dtype), s.rms_eps)
    return dict(x=x, stack=stack, xn_f=xn_f, logits=lm_head(xn_f, table))


# ----------------------------------------------------------------------------- mixture of experts
# TensorSharp, "Multi-GPU & Multi-Node", section "Supported architectures": expert slicing shards
# each expert the way the dense FFN is sharded (gate and up by output column, down by input
# column) and keeps the router whole, so a rank owns 1/N of every expert and the distinct expert
# ids picked for a token refer to the same experts on every rank.


def moe_params_f64(minp) -> dict:
    """Router [E, d] and the experts' gate/up [E, F_e, d] and down [E, d, F_e] in float64."""
    s, m = minp.shape, minp.moe
    E, F, d = m.n_experts, m.expert_ffn, s.d_model
    return dict(router=to_f64(minp.router, s.act_dtype, (E, d)),
                wg=to_f64(minp.wg, s.w_dtype, (E * F, d)).reshape(E, F, d),
                wu=to_f64(minp.wu, s.w_dtype, (E * F, d)).reshape(E, F, d),
                wd=to_f64(minp.wd, s.w_dtype, (E * d, F)).reshape(E, d, F))


def moe_select(logits: np.ndarray, top_k: int):
    """Per token: the top_k experts by router logit, largest first (equal logits: lower expert
    index first), and their weights, the softmax of the selected logits."""
    T, E = logits.shape
    ids = np.zeros((T, top_k), dtype=np.int64)
    w = np.zeros((T, top_k))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))[:top_k]
        ids[t] = order
        sel = logits[t, order]
        ex = np.exp(sel - np.max(sel))
        w[t] = ex / np.sum(ex)
    return ids, w


def moe_route(xn2: np.ndarray, router: np.ndarray, top_k: int):
    """Router logits xn2 . router^T, then ``moe_select``."""
    z = xn2 @ router.T
    ids, w = moe_select(z, top_k)
    return z, ids, w


def moe_ffn_unsharded(act, pm, xn2, ids, w):
    """sum_j w[t, j] * FFN_{ids[t, j]}(xn2[t]) with FFN_e(v) = (act(v Wg_e^T) * (v Wu_e^T)) Wd_e^T."""
    out = np.zeros((xn2.shape[0], pm["wd"].shape[1]))
    for t in range(xn2.shape[0]):
        for j, e in enumerate(ids[t]):
            m = act(xn2[t] @ pm["wg"][e].T) * (xn2[t] @ pm["wu"][e].T)
            out[t] += w[t, j] * (m @ pm["wd"][e].T)
    return out


def moe_ffn_sharded(s, moe, pm, xn2, ids, w):
    """Rank r's partial: its slice F_r of every selected expert's gate/up columns and down rows,
    sum_j w[t, j] * (act(xn2 Wg_e[F_r]^T) * (xn2 Wu_e[F_r]^T)) Wd_e[:, F_r]^T. Returns the
    per-rank partials and activations."""
    N = s.tp
    fr = moe.expert_ffn // N
    act = ACTIVATIONS[s.ffn_act]
    parts, ms = [], []
    for r in range(N):
        cols = slice(r * fr, (r + 1) * fr)
        part = np.zeros((xn2.shape[0], s.d_model))
        mr = np.zeros((xn2.shape[0], len(ids[0]), fr))
        for t in range(xn2.shape[0]):
            for j, e in enumerate(ids[t]):
                m = act(xn2[t] @ pm["wg"][e][cols].T) * (xn2[t] @ pm["wu"][e][cols].T)
                mr[t, j] = m
                part[t] += w[t, j] * (m @ pm["wd"][e][:, cols].T)
        parts.append(part)
        ms.append(mr)
    return parts, ms


def run_moe_block(inp, minp, rows=None):
    """The block with the MoE FFN: the explicit N-rank attention half, the reduce and RMSNorm,
    the replicated router, every rank's MoE partial and the final reduce (rank order)."""
    s, m = inp.shape, minp.moe
    p = params_f64(inp)
    pm = moe_params_f64(minp)
    x = to_f64(inp.x, s.act_dtype)
    kc, vc = caches_f64(inp)
    kr, vr = rank_caches(s, kc, vc)
    xn, ranks, red, h1 = attention_sharded(s, p, x, kr, vr, inp.positions, inp.token_seq, rows)
    xn2 = rms_norm(h1, p["gamma2"], s.rms_eps)
    logits, ids, w = moe_route(xn2, pm["router"], m.top_k)
    parts, ms = moe_ffn_sharded(s, m, pm, xn2, ids, w)
    red2 = parts[0].copy()
    for r in range(1, s.tp):
        red2 = red2 + parts[r]
    for rk in ranks:
        del rk["w"]
    return dict(xn=xn, h1=h1, xn2=xn2, logits=logits, ids=ids, weights=w, partials=parts, m=ms,
                ffn_sum=red2, out=h1 + red2, ranks=ranks)

"""Pins of the CPU oracle against things other than itself (CPU only).

* closed forms and hand-written fixtures (tests/golden/),
* library routines (torch fp64: rms_norm, linear, scaled_dot_product_attention with grouped KV
  heads, silu, gelu-tanh, complex multiplication for the rotary embedding),
* brute force in scalar pure-Python loops on tiny shapes,
* the block-matrix identity the tensor-parallel split rests on (sharded == unsharded),
* shard-map invariants (row-parallel slices concatenate back bit-exactly, fused column rows form
  the same multiset, every rank holds exactly 1/N of the sharded bytes),
* planted mistakes in the oracle, each of which must trip at least one pin.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.block as ob
from tensor_transformer_block_amd.inputs import (
    CONFIGS, BlockShape, f32_to_bf16_bits, make_inputs, q8_0_encode, weight_shapes)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def nrel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


TINY = BlockShape(name="tiny-brute", index=101, d_model=8, n_heads=4, n_kv_heads=2, head_dim=4,
                  ffn_dim=12, tp=2, w_dtype="f32", act_dtype="f32", ffn_act="silu",
                  mode="decode", kv_lens=(3,), n_tokens=1)
SMALL_SHAPES = [
    TINY,
    TINY.with_(name="tiny-n1", index=102, tp=1),
    TINY.with_(name="tiny-gelu-bf16", index=103, w_dtype="bf16", act_dtype="bf16",
               ffn_act="gelu_tanh"),
    TINY.with_(name="tiny-prefill", index=104, mode="prefill", kv_lens=(7,), n_tokens=4),
    TINY.with_(name="tiny-batch", index=105, kv_lens=(3, 1, 5), n_tokens=3, tp=2),
    BlockShape(name="small-q8", index=106, d_model=64, n_heads=4, n_kv_heads=2, head_dim=16,
               ffn_dim=128, tp=2, w_dtype="q8_0", act_dtype="bf16", ffn_act="gelu_tanh",
               mode="decode", kv_lens=(20, 9), n_tokens=2),
    BlockShape(name="small-prefill-n4", index=107, d_model=64, n_heads=8, n_kv_heads=4,
               head_dim=8, ffn_dim=96, tp=4, w_dtype="bf16", act_dtype="bf16", ffn_act="silu",
               mode="prefill", kv_lens=(40,), n_tokens=33),
    CONFIGS["tiny-llama-fp32"],
]


# ----------------------------------------------------------------------------- independent references

def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a))


def torch_decode_storage(a, dtype, shape=None):
    """Storage -> float64 torch tensor through torch's own dtype views (not the oracle's)."""
    if dtype == "f32":
        return _t(np.asarray(a, np.float32)).double()
    if dtype == "bf16":
        return _t(np.asarray(a, np.uint16).view(np.int16)).view(torch.bfloat16).double()
    if dtype == "q8_0":
        rows, cols = shape
        raw = _t(np.asarray(a, np.uint8).reshape(rows, cols // 32, 34))
        d = raw[..., 0:2].contiguous().view(torch.float16).double()          # [rows, nb, 1]
        q = raw[..., 2:].contiguous().view(torch.int8).double()              # [rows, nb, 32]
        return (d * q).reshape(rows, cols)
    raise ValueError(dtype)


def torch_rope(x, pos, base):
    """Rotate-half rotary embedding as a complex product: (a + ib) * exp(i * pos * theta)."""
    hd = x.shape[-1]
    theta = base ** (-torch.arange(0, hd, 2, dtype=torch.float64) / hd)
    z = torch.complex(x[..., : hd // 2], x[..., hd // 2:])
    z = z * torch.polar(torch.ones_like(theta), pos * theta)
    return torch.cat([z.real, z.imag], dim=-1)


def torch_block(inp, x=None):
    """The unsharded block written with torch library routines in float64 (x: an fp64 input in
    place of the stored one)."""
    s = inp.shape
    shp = weight_shapes(s)
    W = {k: torch_decode_storage(inp.weights[k], s.w_dtype, shp[k]) for k in shp}
    g1 = torch_decode_storage(inp.gamma1, s.act_dtype)
    g2 = torch_decode_storage(inp.gamma2, s.act_dtype)
    if x is None:
        x = torch_decode_storage(inp.x, s.act_dtype)
    T, hd, Hq, Hkv = x.shape[0], s.head_dim, s.n_heads, s.n_kv_heads
    xn = F.rms_norm(x, (s.d_model,), g1, eps=s.rms_eps)
    q = F.linear(xn, W["wq"]).view(T, Hq, hd)
    k = F.linear(xn, W["wk"]).view(T, Hkv, hd)
    v = F.linear(xn, W["wv"]).view(T, Hkv, hd)
    pos = torch.from_numpy(inp.positions.astype(np.int64))
    qr = torch.stack([torch_rope(q[t], float(pos[t]), s.rope_base) for t in range(T)])
    kr = torch.stack([torch_rope(k[t], float(pos[t]), s.rope_base) for t in range(T)])
    attn = torch.zeros(T, Hq, hd, dtype=torch.float64)
    for b in range(s.n_seqs):
        L = int(inp.seq_lens[b])
        K = torch.zeros(Hkv, L, hd, dtype=torch.float64)
        V = torch.zeros(Hkv, L, hd, dtype=torch.float64)
        kp = torch_decode_storage(inp.k_prior[b], s.act_dtype)
        vp = torch_decode_storage(inp.v_prior[b], s.act_dtype)
        K[:, : kp.shape[1]] = kp
        V[:, : vp.shape[1]] = vp
        toks = [t for t in range(T) if int(inp.token_seq[t]) == b]
        for t in toks:
            K[:, int(pos[t])] = kr[t]
            V[:, int(pos[t])] = v[t]
        qs = qr[toks].transpose(0, 1).unsqueeze(0)                            # [1, Hq, n, hd]
        mask = torch.arange(L)[None, :] <= pos[toks][:, None]                 # [n, L]
        o = F.scaled_dot_product_attention(qs, K.unsqueeze(0), V.unsqueeze(0), attn_mask=mask,
                                           enable_gqa=True)
        attn[toks] = o[0].transpose(0, 1)
    attn = attn.reshape(T, Hq * hd)
    h1 = x + F.linear(attn, W["wo"])
    xn2 = F.rms_norm(h1, (s.d_model,), g2, eps=s.rms_eps)
    gate, up = F.linear(xn2, W["wg"]), F.linear(xn2, W["wu"])
    act = F.silu(gate) if s.ffn_act == "silu" else F.gelu(gate, approximate="tanh")
    out = h1 + F.linear(act * up, W["wd"])
    return dict(xn=xn, q=qr, k_new=kr, attn=attn, h1=h1, xn2=xn2, m=act * up, out=out)


def brute_block(inp):
    """The unsharded block in scalar pure-Python loops (tiny shapes only)."""
    s = inp.shape
    shp = weight_shapes(s)
    W = {k: torch_decode_storage(inp.weights[k], s.w_dtype, shp[k]).tolist() for k in shp}
    g1 = torch_decode_storage(inp.gamma1, s.act_dtype).tolist()
    g2 = torch_decode_storage(inp.gamma2, s.act_dtype).tolist()
    X = torch_decode_storage(inp.x, s.act_dtype).tolist()
    d, hd, Hq, Hkv, Fd = s.d_model, s.head_dim, s.n_heads, s.n_kv_heads, s.ffn_dim
    half = hd // 2

    def norm(vec, g):
        ms = sum(e * e for e in vec) / len(vec)
        inv = 1.0 / math.sqrt(ms + s.rms_eps)
        return [g[i] * vec[i] * inv for i in range(len(vec))]

    def matvec(Wm, vec):
        return [sum(Wm[o][i] * vec[i] for i in range(len(vec))) for o in range(len(Wm))]

    def rot(vec, p):
        out = [0.0] * hd
        for i in range(half):
            z = complex(vec[i], vec[i + half]) * cmath.exp(1j * p * s.rope_base ** (-2.0 * i / hd))
            out[i], out[i + half] = z.real, z.imag
        return out

    caches = []
    for b in range(s.n_seqs):
        kp = torch_decode_storage(inp.k_prior[b], s.act_dtype).tolist()
        vp = torch_decode_storage(inp.v_prior[b], s.act_dtype).tolist()
        caches.append(({(g, j): kp[g][j] for g in range(Hkv) for j in range(len(kp[g]))},
                       {(g, j): vp[g][j] for g in range(Hkv) for j in range(len(vp[g]))}))
    T = len(X)
    xns = [norm(X[t], g1) for t in range(T)]
    for t in range(T):
        b, p = int(inp.token_seq[t]), int(inp.positions[t])
        kk, vv = matvec(W["wk"], xns[t]), matvec(W["wv"], xns[t])
        for g in range(Hkv):
            caches[b][0][(g, p)] = rot(kk[g * hd:(g + 1) * hd], p)
            caches[b][1][(g, p)] = vv[g * hd:(g + 1) * hd]
    outs = []
    for t in range(T):
        b, p = int(inp.token_seq[t]), int(inp.positions[t])
        qq = matvec(W["wq"], xns[t])
        a = []
        for h in range(Hq):
            g = h * Hkv // Hq
            qh = rot(qq[h * hd:(h + 1) * hd], p)
            sc = [sum(qh[i] * caches[b][0][(g, j)][i] for i in range(hd)) / math.sqrt(hd)
                  for j in range(p + 1)]
            mx = max(sc)
            e = [math.exp(z - mx) for z in sc]
            tot = sum(e)
            a += [sum(e[j] / tot * caches[b][1][(g, j)][i] for j in range(p + 1)) for i in range(hd)]
        h1 = [X[t][i] + v for i, v in enumerate(matvec(W["wo"], a))]
        xn2 = norm(h1, g2)
        gt, up = matvec(W["wg"], xn2), matvec(W["wu"], xn2)
        if s.ffn_act == "silu":
            m = [gt[j] / (1.0 + math.exp(-gt[j])) * up[j] for j in range(Fd)]
        else:
            m = [0.5 * gt[j] * (1 + math.tanh(math.sqrt(2 / math.pi) * (gt[j] + 0.044715 * gt[j] ** 3)))
                 * up[j] for j in range(Fd)]
        outs.append([h1[i] + v for i, v in enumerate(matvec(W["wd"], m))])
    return np.array(outs)


# ----------------------------------------------------------------------------- block-level pins

@pytest.mark.parametrize("s", SMALL_SHAPES, ids=lambda s: s.name)
def test_sharded_equals_unsharded(s):
    """Row-parallel partial sums add up to the unsharded projections (block-matrix identity)."""
    inp = make_inputs(s, seed=3)
    a = oracle.run_block(inp, sharded=True)
    b = oracle.run_block(inp, sharded=False)
    for key in ("xn", "h1", "xn2", "out"):
        assert nrel(a[key], b[key]) <= 1e-12, key
    assert nrel(a["attn_sum"], b["attn_proj"]) <= 1e-12
    assert nrel(a["ffn_sum"], b["ffn_proj"]) <= 1e-12
    hq, hd = s.n_heads // s.tp, s.head_dim
    fr = s.ffn_dim // s.tp
    for r, rk in enumerate(a["ranks"]):
        assert nrel(rk["a"], b["attn"][:, r * hq * hd:(r + 1) * hq * hd]) <= 1e-12
        assert nrel(rk["m"], b["m"][:, r * fr:(r + 1) * fr]) <= 1e-12


@pytest.mark.parametrize("s", SMALL_SHAPES, ids=lambda s: s.name)
def test_oracle_matches_torch_library_block(s):
    inp = make_inputs(s, seed=5)
    ref = torch_block(inp)
    for sharded in (False, True):
        res = oracle.run_block(inp, sharded=sharded)
        for key in ("xn", "h1", "xn2", "out"):
            assert nrel(res[key], ref[key].numpy()) <= 1e-12, (sharded, key)
    res = oracle.run_block(inp, sharded=False)
    assert nrel(res["attn"], ref["attn"].numpy()) <= 1e-12
    assert nrel(res["q"], ref["q"].numpy()) <= 1e-12
    assert nrel(res["m"], ref["m"].numpy()) <= 1e-12


@pytest.mark.parametrize("s", [x for x in SMALL_SHAPES if x.d_model <= 8], ids=lambda s: s.name)
def test_oracle_matches_scalar_brute_force(s):
    inp = make_inputs(s, seed=7)
    ref = brute_block(inp)
    for sharded in (False, True):
        res = oracle.run_block(inp, sharded=sharded)
        assert nrel(res["out"], ref) <= 1e-12, sharded


def test_n1_reduces_sharded_to_unsharded():
    s = TINY.with_(tp=1, index=110)
    inp = make_inputs(s, seed=1)
    a, b = oracle.run_block(inp, True), oracle.run_block(inp, False)
    assert nrel(a["out"], b["out"]) <= 1e-14
    assert nrel(a["ranks"][0]["a"], b["attn"]) <= 1e-14


def test_replicated_state_is_rank_independent():
    """Every rank sees the same xn/xn2; the rank loop order of the reduction is fixed."""
    s = CONFIGS["tiny-llama-fp32"]
    inp = make_inputs(s)
    res = oracle.run_block(inp, True)
    ps = [rk["p_attn"] for rk in res["ranks"]]
    manual = ps[0] + ps[1]
    assert np.array_equal(manual, res["attn_sum"])


# ----------------------------------------------------------------------------- sublayer pins

def test_rms_norm_closed_form_and_library():
    c, eps, d = 3.5, 1e-5, 16
    g = np.linspace(0.5, 1.5, d)
    y = oracle.rms_norm(np.full(d, c), g, eps)
    assert np.allclose(y, g * c / math.sqrt(c * c + eps), rtol=1e-15, atol=0)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, d))
    ref = F.rms_norm(_t(x), (d,), _t(g), eps=eps).numpy()
    assert nrel(oracle.rms_norm(x, g, eps), ref) <= 1e-14
    # scale invariance as eps -> 0
    assert nrel(oracle.rms_norm(7.0 * x, g, 0.0), oracle.rms_norm(x, g, 0.0)) <= 1e-14


def test_rope_golden_hd4():
    doc = json.load(open(os.path.join(GOLDEN, "rope_hd4.json")))
    for c in doc["cases"]:
        y = oracle.rope(np.array(c["x"], dtype=np.float64), c["position"], doc["base"])
        assert np.allclose(y, c["y"], rtol=0, atol=1e-15), c


def test_rope_properties():
    rng = np.random.default_rng(1)
    hd, base = 128, 10000.0
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    assert np.array_equal(oracle.rope(q, 0, base), q)
    y = oracle.rope(q, 4095, base)
    assert np.allclose(q[:64] ** 2 + q[64:] ** 2, y[:64] ** 2 + y[64:] ** 2, rtol=1e-12)
    for p, pp, dl in [(3, 10, 7), (100, 5, 4000), (0, 0, 123)]:
        lhs = oracle.rope(q, p + dl, base) @ oracle.rope(k, pp + dl, base)
        rhs = oracle.rope(q, p, base) @ oracle.rope(k, pp, base)
        assert abs(lhs - rhs) <= 1e-10 * (1 + abs(rhs))
    # hd = 2: a plain rotation by the position (theta_0 = 1)
    y2 = oracle.rope(np.array([0.3, -0.7]), 5, base)
    z = complex(0.3, -0.7) * cmath.exp(5j)
    assert np.allclose(y2, [z.real, z.imag], rtol=0, atol=1e-15)
    ref = torch_rope(_t(q), 77.0, base).numpy()
    assert nrel(oracle.rope(q, 77, base), ref) <= 1e-13


def test_attention_special_cases_and_library():
    rng = np.random.default_rng(2)
    hd = 8
    q, k, v = rng.standard_normal(hd), rng.standard_normal((1, hd)), rng.standard_normal((1, hd))
    assert np.allclose(oracle.attend(q, k, v), v[0], rtol=1e-15)
    kk = np.repeat(rng.standard_normal((1, hd)), 6, axis=0)
    vv = rng.standard_normal((6, hd))
    assert np.allclose(oracle.attend(q, kk, vv), vv.mean(axis=0), rtol=1e-13)
    K, V = rng.standard_normal((9, hd)), rng.standard_normal((9, hd))
    ref = F.scaled_dot_product_attention(_t(q)[None, None, None], _t(K)[None, None],
                                         _t(V)[None, None])[0, 0, 0].numpy()
    assert nrel(oracle.attend(q, K, V), ref) <= 1e-14


def test_activations_library():
    z = np.linspace(-9, 9, 1001)
    assert nrel(oracle.silu(z), F.silu(_t(z)).numpy()) <= 1e-15
    assert nrel(oracle.gelu_tanh(z), F.gelu(_t(z), approximate="tanh").numpy()) <= 1e-15
    assert oracle.silu(np.array(0.0)) == 0.0 and oracle.gelu_tanh(np.array(0.0)) == 0.0


# ----------------------------------------------------------------------------- storage pins

def test_q8_0_golden_blocks():
    doc = json.load(open(os.path.join(GOLDEN, "q8_0_blocks.json")))
    raw, vals = [], []
    for blk in doc["blocks"]:
        bits = int(blk["scale_bits"], 16)
        raw += [bits & 0xFF, bits >> 8] + [q & 0xFF for q in blk["q"]]
        vals += [blk["scale"] * q for q in blk["q"]]
    got = oracle.dequant_q8_0(np.array(raw, dtype=np.uint8), doc["rows"], doc["cols"])
    assert np.array_equal(got.reshape(-1), np.array(vals))


def test_q8_0_encoder_bounds():
    rng = np.random.default_rng(4)
    w = (0.02 * rng.standard_normal((16, 256))).astype(np.float32)
    w[3, 32:64] = 0.0
    blocks = q8_0_encode(w)
    deq = oracle.dequant_q8_0(blocks, 16, 256)
    raw = blocks.reshape(16, 8, 34)
    d16 = raw[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    q = raw[..., 2:].copy().view(np.int8).astype(np.int32)
    wb = w.reshape(16, 8, 32).astype(np.float64)
    amax = np.abs(wb).max(axis=2)
    d32 = amax / 127.0
    err = np.abs(deq.reshape(16, 8, 32) - wb)
    # half a quantisation step plus the fp16 rounding of the scale (at most 127 * |d16 - d32|)
    bound = d32 / 2 + 127 * np.abs(d16 - d32) + 1e-12
    assert np.all(err <= bound[..., None])
    nz = amax > 0
    imax = np.abs(wb).argmax(axis=2)
    qmax = np.take_along_axis(q, imax[..., None], axis=2)[..., 0]
    assert np.all(np.abs(qmax[nz]) == 127)
    assert np.all(d16[~nz] == 0) and np.all(q[~nz] == 0)
    # fp16 scale x int8 code is exact in fp32
    f32 = (d16[..., None].astype(np.float32) * q.astype(np.float32)).astype(np.float64)
    assert np.array_equal(f32, d16[..., None] * q)


def test_bf16_encoder_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1e-3, 3.0e38], dtype=np.float32)
    bits = f32_to_bf16_bits(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    rng = np.random.default_rng(5)
    x = rng.standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)
    assert nrel(oracle.bf16_bits_to_f64(ref), torch.from_numpy(x).to(torch.bfloat16).double().numpy()) == 0


# ----------------------------------------------------------------------------- shard-map pins

@pytest.mark.parametrize("name", ["tiny-llama-fp32", "small-q8", "small-prefill-n4"])
def test_shard_maps_and_bytes(name):
    s = {x.name: x for x in SMALL_SHAPES}[name]
    inp = make_inputs(s)
    p = oracle.params_f64(inp)
    parts = [oracle.shard_weights(s, p, r) for r in range(s.tp)]
    assert np.array_equal(np.concatenate([w["wo"] for w in parts], axis=1), p["wo"])
    assert np.array_equal(np.concatenate([w["wd"] for w in parts], axis=1), p["wd"])
    for key_full, keys in (("qkv", ("wq", "wk", "wv")), ("gu", ("wg", "wu"))):
        full = np.concatenate([p[k] for k in keys], axis=0)
        fused = np.concatenate([np.concatenate([w[k] for k in keys], axis=0) for w in parts])
        a = sorted(map(tuple, full.tolist()))
        b = sorted(map(tuple, fused.tolist()))
        assert a == b, key_full
    counts = [sum(w[k].size for k in w) for w in parts]
    total = sum(p[k].size for k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"))
    assert all(c * s.tp == total for c in counts)


# ----------------------------------------------------------------------------- planted mistakes

def _rope_wrong_sign(vec, position, base):
    hd = vec.shape[-1]
    c, s = ob.rope_cos_sin(position, hd, base)
    a, b = vec[..., : hd // 2], vec[..., hd // 2:]
    return np.concatenate([a * c + b * s, b * c - a * s], axis=-1)


def _rope_interleaved(vec, position, base):
    hd = vec.shape[-1]
    c, s = ob.rope_cos_sin(position, hd, base)
    a, b = vec[..., 0::2], vec[..., 1::2]
    out = np.empty_like(vec)
    out[..., 0::2], out[..., 1::2] = a * c - b * s, b * c + a * s
    return out


def _norm_no_eps(x, gamma, eps):
    return gamma * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True))


def _attend_no_scale(q, keys, values):
    s = keys @ q
    w = np.exp(s - s.max())
    return (w / w.sum()) @ values


def _attend_no_max(q, keys, values):
    s = keys @ q / np.sqrt(q.shape[-1])
    w = np.exp(s)
    return (w / (w.sum() + 1e-3)) @ values


PLANTS = {
    "rope_sign": ("rope", _rope_wrong_sign),
    "rope_interleaved": ("rope", _rope_interleaved),
    "norm_no_eps": ("rms_norm", _norm_no_eps),
    "attn_no_scale": ("attend", _attend_no_scale),
    "attn_bad_normaliser": ("attend", _attend_no_max),
    "silu_for_gelu": ("gelu_tanh", lambda z: z / (1 + np.exp(-z))),
}


@pytest.mark.parametrize("plant", sorted(PLANTS))
def test_planted_mistake_is_caught(plant, monkeypatch):
    fn_name, bad = PLANTS[plant]
    s = {x.name: x for x in SMALL_SHAPES}["small-q8"]
    inp = make_inputs(s, seed=9)
    ref = torch_block(inp)
    monkeypatch.setattr(ob, fn_name, bad)
    if fn_name == "gelu_tanh":
        monkeypatch.setitem(ob.ACTIVATIONS, "gelu_tanh", bad)
    caught = False
    for sharded in (False, True):
        res = oracle.run_block(inp, sharded=sharded)
        caught |= any(nrel(res[k], ref[k].numpy()) > 1e-9 for k in ("xn", "h1", "xn2", "out"))
    assert caught, plant


def test_planted_gqa_mapping_is_caught(monkeypatch):
    """A wrong query-head to KV-head mapping (heads of different groups swapped) must be caught."""
    s = {x.name: x for x in SMALL_SHAPES}["small-prefill-n4"]
    inp = make_inputs(s, seed=2)
    ref = torch_block(inp)
    real = ob.block_unsharded

    def bad_unsharded(s_, p, x, kc, vc, positions, token_seq, rows=None):
        s2 = s_.with_(n_heads=s_.n_heads)
        perm = np.arange(s_.n_heads).reshape(s_.n_kv_heads, -1).T.reshape(-1)
        p2 = dict(p)
        hd = s_.head_dim
        p2["wq"] = p["wq"].reshape(s_.n_heads, hd, -1)[perm].reshape(p["wq"].shape)
        p2["wo"] = p["wo"].reshape(p["wo"].shape[0], s_.n_heads, hd)[:, perm].reshape(p["wo"].shape)
        return real(s2, p2, x, kc, vc, positions, token_seq, rows)

    ok = oracle.run_block(inp, sharded=False)
    assert nrel(ok["out"], ref["out"].numpy()) <= 1e-12
    monkeypatch.setattr(ob, "block_unsharded", bad_unsharded)
    res = ob.run_block(inp, sharded=False)
    assert nrel(res["attn"], ref["attn"].numpy()) > 1e-6


def test_planted_transposed_wo_is_caught():
    s = CONFIGS["tiny-llama-fp32"]          # d == Hq * hd, so a transposed Wo still fits
    inp = make_inputs(s, seed=4)
    ref = torch_block(inp)
    p = oracle.params_f64(inp)
    p["wo"] = p["wo"].T.copy()
    x = oracle.to_f64(inp.x, s.act_dtype)
    kc, vc = oracle.caches_f64(inp)
    res = oracle.block_unsharded(s, p, x, kc, vc, inp.positions, inp.token_seq)
    assert nrel(res["h1"], ref["h1"].numpy()) > 1e-6


# ----------------------------------------------------------------------------- stacks of blocks

STACK_SHAPES = [TINY.with_(name="tiny-stack", index=120),
                TINY.with_(name="tiny-stack-prefill", index=121, mode="prefill", kv_lens=(6,),
                           n_tokens=4, w_dtype="bf16", act_dtype="bf16")]


def _identity_block(inp):
    """The same block with zero o_proj and down weights: both residual branches add exactly 0,
    so the block passes its input through unchanged (a closed form)."""
    import copy
    out = copy.copy(inp)
    out.weights = dict(inp.weights)
    for k in ("wo", "wd"):
        out.weights[k] = np.zeros_like(inp.weights[k])
    return out


@pytest.mark.parametrize("s", STACK_SHAPES, ids=lambda s: s.name)
def test_stack_matches_chained_library_blocks(s):
    """A stack of three blocks against the torch-library block applied three times."""
    from tensor_transformer_block_amd.inputs import make_stack_inputs
    inps = make_stack_inputs(s, 3, seed=4)
    res = oracle.run_stack(inps)
    x = torch_decode_storage(inps[0].x, s.act_dtype)
    for i, inp in enumerate(inps):
        ref = torch_block(inp, x=x)
        assert nrel(res[i]["x"], x.numpy()) <= 1e-12, i
        assert nrel(res[i]["out"], ref["out"].numpy()) <= 1e-12, i
        x = ref["out"]
    # distinct blocks: the draws differ from block to block
    assert not np.array_equal(inps[0].weights["wq"], inps[1].weights["wq"])


@pytest.mark.parametrize("s", STACK_SHAPES, ids=lambda s: s.name)
def test_stack_identity_blocks(s):
    """Identity blocks (zero o_proj and down) pass the residual stream through, so a stack of a
    block and an identity block equals that block alone, in either order; a stack of identity
    blocks returns its input."""
    from tensor_transformer_block_amd.inputs import make_stack_inputs
    b0, b1 = make_stack_inputs(s, 2, seed=6)
    i0, i1 = _identity_block(b0), _identity_block(b1)
    x0 = oracle.to_f64(b0.x, s.act_dtype)
    alone0 = oracle.run_block(b0)["out"]
    assert nrel(oracle.run_stack([b0, i1])[1]["out"], alone0) <= 1e-14
    st = oracle.run_stack([i0, b1])
    assert np.array_equal(st[0]["out"], x0)
    b1x = _with_x(b1, b0.x)
    assert nrel(st[1]["out"], oracle.run_block(b1x)["out"]) <= 1e-14
    assert np.array_equal(oracle.run_stack([i0, i1])[1]["out"], x0)


def _with_x(inp, x):
    import copy
    out = copy.copy(inp)
    out.x = x
    return out


@pytest.mark.parametrize("s", STACK_SHAPES, ids=lambda s: s.name)
def test_stack_sharded_equals_unsharded(s):
    from tensor_transformer_block_amd.inputs import make_stack_inputs
    inps = make_stack_inputs(s, 3, seed=8)
    a, b = oracle.run_stack(inps, sharded=True), oracle.run_stack(inps, sharded=False)
    for i in range(3):
        assert nrel(a[i]["out"], b[i]["out"]) <= 1e-12, i


def test_planted_stack_chaining_is_caught(monkeypatch):
    """A stack that feeds every block the stack input instead of the previous output trips the
    identity-block pin."""
    def wrong_stack(inputs, sharded=True):
        x = ob.to_f64(inputs[0].x, inputs[0].shape.act_dtype)
        res = []
        for inp in inputs:
            s = inp.shape
            kc, vc = ob.caches_f64(inp)
            kr, vr = ob.rank_caches(s, kc, vc)
            r = ob.block_sharded(s, ob.params_f64(inp), x, kr, vr, inp.positions, inp.token_seq)
            r["x"] = x
            res.append(r)
        return res
    monkeypatch.setattr(oracle, "run_stack", wrong_stack)
    with pytest.raises(AssertionError):
        test_stack_identity_blocks(STACK_SHAPES[0])


# ----------------------------------------------------------------------------- the replicated head

HEAD_SHAPES = [TINY.with_(name="tiny-head-f32", index=130, kv_lens=(3, 2), n_tokens=2),
               TINY.with_(name="tiny-head-bf16", index=131, w_dtype="bf16", act_dtype="bf16",
                          mode="prefill", kv_lens=(5,), n_tokens=5),
               BlockShape(name="small-head-q8", index=132, d_model=64, n_heads=4, n_kv_heads=2,
                          head_dim=16, ffn_dim=128, tp=2, w_dtype="q8_0", act_dtype="bf16",
                          ffn_act="gelu_tanh", mode="decode", kv_lens=(9, 4, 1), n_tokens=3)]


def torch_head_table(head):
    s = head.shape
    return torch_decode_storage(head.table, s.w_dtype, (head.vocab, s.d_model))


@pytest.mark.parametrize("s", HEAD_SHAPES, ids=lambda s: s.name)
def test_embedding_lookup_against_library(s):
    """Rows picked by torch's embedding routine from the table as torch decodes it; Q8_0 rows
    rounded to bf16 by torch's own conversion (nearest even)."""
    from tensor_transformer_block_amd.inputs import make_head_inputs
    head = make_head_inputs(s, vocab=37, seed=2)
    ref = F.embedding(torch.from_numpy(head.token_ids.astype(np.int64)), torch_head_table(head))
    if s.w_dtype == "q8_0":
        ref = ref.float().to(torch.bfloat16).double()
    got = oracle.embed_lookup(head)
    assert np.array_equal(got, ref.numpy())


def test_bf16_rounding_closed_forms():
    """Values halfway between two bf16 numbers go to the even one; others to the nearest."""
    one = 1.0
    ulp = 2.0 ** -7                       # bf16 spacing in [1, 2)
    cases = {one + ulp / 2: one, one + 3 * ulp / 2: one + 2 * ulp, one + ulp / 4: one,
             one + 3 * ulp / 4: one + ulp, -(one + ulp / 2): -one, 0.0: 0.0,
             3.0 * 2.0 ** -130: 3.0 * 2.0 ** -130}   # subnormal with 2 significant bits: exact
    for v, want in cases.items():
        assert oracle.round_to_bf16(np.array([v]))[0] == want, v


@pytest.mark.parametrize("s", HEAD_SHAPES, ids=lambda s: s.name)
def test_lm_head_against_library(s):
    from tensor_transformer_block_amd.inputs import make_head_inputs
    head = make_head_inputs(s, vocab=41, seed=3)
    xn = np.random.default_rng(0).standard_normal((4, s.d_model))
    ref = F.linear(torch.from_numpy(xn), torch_head_table(head)).numpy()
    assert nrel(oracle.lm_head(xn, oracle.head_table_f64(head)), ref) <= 1e-13


@pytest.mark.parametrize("s", HEAD_SHAPES, ids=lambda s: s.name)
def test_model_step_against_library_chain(s):
    """Embedding, a stack of two blocks, final RMSNorm and LM head against torch library
    routines chained the same way."""
    from tensor_transformer_block_amd.inputs import make_head_inputs, make_stack_inputs
    head = make_head_inputs(s, vocab=53, seed=5)
    inps = make_stack_inputs(s, 2, seed=5)
    res = oracle.run_model(head, inps)
    W = torch_head_table(head)
    x = F.embedding(torch.from_numpy(head.token_ids.astype(np.int64)), W)
    if s.w_dtype == "q8_0":
        x = x.float().to(torch.bfloat16).double()
    for inp in inps:
        x = torch_block(inp, x=x)["out"]
    xn = F.rms_norm(x, (s.d_model,), torch_decode_storage(head.gamma_f, s.act_dtype),
                    eps=s.rms_eps)
    assert nrel(res["logits"], F.linear(xn, W).numpy()) <= 1e-12


def test_planted_untransposed_head_is_caught(monkeypatch):
    """An LM head that multiplies by the table's first d rows instead of its transpose trips the
    library pin (square table so the shapes still fit)."""
    s = HEAD_SHAPES[0]
    monkeypatch.setattr(oracle, "lm_head", lambda xn, t: xn @ t[: t.shape[1]])
    with pytest.raises(AssertionError):
        from tensor_transformer_block_amd.inputs import make_head_inputs
        head = make_head_inputs(s, vocab=s.d_model, seed=3)
        xn = np.random.default_rng(0).standard_normal((4, s.d_model))
        ref = F.linear(torch.from_numpy(xn), torch_head_table(head)).numpy()
        assert nrel(oracle.lm_head(xn, oracle.head_table_f64(head)), ref) <= 1e-13


# ----------------------------------------------------------------------------- mixture of experts

from tensor_transformer_block_amd.inputs import MoEShape, make_moe_inputs  # noqa: E402

MOE_CASES = [(TINY.with_(name="tiny-moe", index=140, kv_lens=(3, 2), n_tokens=2),
              MoEShape(n_experts=6, top_k=2, expert_ffn=4)),
             (TINY.with_(name="tiny-moe-bf16", index=141, w_dtype="bf16", act_dtype="bf16",
                         ffn_act="gelu_tanh", mode="prefill", kv_lens=(5,), n_tokens=3),
              MoEShape(n_experts=5, top_k=3, expert_ffn=6)),
             (BlockShape(name="small-moe-q8", index=142, d_model=64, n_heads=4, n_kv_heads=2,
                         head_dim=16, ffn_dim=128, tp=2, w_dtype="q8_0", act_dtype="bf16",
                         ffn_act="silu", mode="decode", kv_lens=(7, 3), n_tokens=2),
              MoEShape(n_experts=4, top_k=2, expert_ffn=64))]


def test_moe_select_against_library_and_ties():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((5, 9))
    ids, w = oracle.moe_select(z, 4)
    ref_ids = np.argsort(-z, axis=1, kind="stable")[:, :4]
    assert np.array_equal(ids, ref_ids)
    ref_w = torch.softmax(torch.from_numpy(np.take_along_axis(z, ref_ids, 1)), dim=1).numpy()
    assert nrel(w, ref_w) <= 1e-15
    # equal logits: the lower expert index first; equal weights
    ids, w = oracle.moe_select(np.array([[1.0, 3.0, 3.0, 0.0]]), 2)
    assert ids.tolist() == [[1, 2]] and np.allclose(w, [[0.5, 0.5]], rtol=0, atol=1e-15)
    # every expert selected: the weights are the softmax over all logits, in logit order
    ids, w = oracle.moe_select(z[:1], 9)
    assert nrel(np.sort(w[0]), np.sort(torch.softmax(torch.from_numpy(z[0]), 0).numpy())) <= 1e-15


def _torch_moe_ffn(s, minp, xn2):
    """Routing with torch.topk / torch.softmax and every selected expert's FFN with F.linear."""
    m = minp.moe
    E, F_, d = m.n_experts, m.expert_ffn, s.d_model
    R = torch_decode_storage(minp.router, s.act_dtype)
    Wg = torch_decode_storage(minp.wg, s.w_dtype, (E * F_, d)).view(E, F_, d)
    Wu = torch_decode_storage(minp.wu, s.w_dtype, (E * F_, d)).view(E, F_, d)
    Wd = torch_decode_storage(minp.wd, s.w_dtype, (E * d, F_)).view(E, d, F_)
    x = torch.from_numpy(xn2)
    vals, idx = torch.topk(F.linear(x, R), m.top_k, dim=1)
    w = torch.softmax(vals, dim=1)
    act = F.silu if s.ffn_act == "silu" else (lambda z: F.gelu(z, approximate="tanh"))
    out = torch.zeros(x.shape[0], d, dtype=torch.float64)
    for t in range(x.shape[0]):
        for j in range(m.top_k):
            e = int(idx[t, j])
            out[t] += w[t, j] * F.linear(act(F.linear(x[t], Wg[e])) * F.linear(x[t], Wu[e]), Wd[e])
    return idx.numpy(), out.numpy()


@pytest.mark.parametrize("s,moe", MOE_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_moe_ffn_against_library(s, moe):
    minp = make_moe_inputs(s, moe, seed=1)
    pm = oracle.moe_params_f64(minp)
    xn2 = np.random.default_rng(2).standard_normal((3, s.d_model))
    _, ids, w = oracle.moe_route(xn2, pm["router"], moe.top_k)
    ref_ids, ref = _torch_moe_ffn(s, minp, xn2)
    assert np.array_equal(ids, ref_ids)
    out = oracle.moe_ffn_unsharded(oracle.ACTIVATIONS[s.ffn_act], pm, xn2, ids, w)
    assert nrel(out, ref) <= 1e-12


@pytest.mark.parametrize("s,moe", MOE_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_moe_sharded_equals_unsharded(s, moe):
    """Expert slicing: the rank partials (each rank's slice of every selected expert) add up to
    the unsharded expert mixture."""
    minp = make_moe_inputs(s, moe, seed=3)
    pm = oracle.moe_params_f64(minp)
    xn2 = np.random.default_rng(4).standard_normal((4, s.d_model))
    _, ids, w = oracle.moe_route(xn2, pm["router"], moe.top_k)
    parts, _ = oracle.moe_ffn_sharded(s, moe, pm, xn2, ids, w)
    ref = oracle.moe_ffn_unsharded(oracle.ACTIVATIONS[s.ffn_act], pm, xn2, ids, w)
    assert nrel(sum(parts[1:], parts[0]), ref) <= 1e-12


@pytest.mark.parametrize("s,moe", MOE_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_moe_block_against_unsharded_composition(s, moe):
    """The MoE block (sharded attention, replicated router, sliced experts) against the unsharded
    block's h1 followed by the library MoE FFN."""
    inp = make_inputs(s, seed=5)
    minp = make_moe_inputs(s, moe, seed=5)
    res = oracle.run_moe_block(inp, minp)
    h1 = torch_block(inp)["h1"].numpy()
    xn2 = F.rms_norm(torch.from_numpy(h1), (s.d_model,),
                     torch_decode_storage(inp.gamma2, s.act_dtype), eps=s.rms_eps).numpy()
    ids, ffn = _torch_moe_ffn(s, minp, xn2)
    assert np.array_equal(res["ids"], ids)
    assert nrel(res["out"], h1 + ffn) <= 1e-12


def test_planted_moe_unnormalised_weights_are_caught(monkeypatch):
    """Top-k weights taken from a softmax over all experts (not renormalised) trip the library
    pin."""
    def wrong(logits, top_k):
        ids = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        return ids, np.take_along_axis(p, ids, 1)
    monkeypatch.setattr(ob, "moe_select", wrong)
    with pytest.raises(AssertionError):
        test_moe_ffn_against_library(*MOE_CASES[0])


# (workload, sampled token rows or None for all): the sharded oracle against the unsharded one at
# the workloads' real shapes. The 64-sequence batch and the 2048-token prefill check a few rows
# (every token's K and V are still produced, since the sampled rows attend to them).
P1_REAL = [("llama3-8b-decode", None), ("gemma-q8-decode", None),
           ("llama3-8b-batched", [0, 17, 63]), ("llama-70b-prefill", [0, 1031, 2047])]


@pytest.mark.slow
@pytest.mark.parametrize("name,rows", P1_REAL, ids=lambda v: str(v))
def test_sharded_equals_unsharded_real_shapes(name, rows):
    """Block-matrix identity at the workloads' own shapes (TensorSharp "How tensor parallelism
    works": the reduced partials leave every rank with the hidden state the unsharded block
    computes): every replicated tensor, both partial sums and each rank's owned columns of the
    attention output and of m agree to 1e-12 normwise."""
    from tensor_transformer_block_amd.inputs import WORKLOADS
    s = WORKLOADS[name]
    inp = make_inputs(s, seed=0)
    a = oracle.run_block(inp, sharded=True, rows=rows)
    b = oracle.run_block(inp, sharded=False, rows=rows)
    for key in ("xn", "h1", "xn2", "out"):
        assert nrel(a[key], b[key]) <= 1e-12, key
    assert nrel(a["attn_sum"], b["attn_proj"]) <= 1e-12
    assert nrel(a["ffn_sum"], b["ffn_proj"]) <= 1e-12
    hq, hd, fr = s.n_heads // s.tp, s.head_dim, s.ffn_dim // s.tp
    for r, rk in enumerate(a["ranks"]):
        assert nrel(rk["a"], b["attn"][:, r * hq * hd:(r + 1) * hq * hd]) <= 1e-12
        assert nrel(rk["m"], b["m"][:, r * fr:(r + 1) * fr]) <= 1e-12
        assert nrel(rk["k_new"], b["k_new"][:, r * (s.n_kv_heads // s.tp):
                                            (r + 1) * (s.n_kv_heads // s.tp)]) <= 1e-12

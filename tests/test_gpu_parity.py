"""GPU parity: the HIP path through the C ABI against the CPU oracle, stage by stage.

Tolerances (normwise max|gpu - oracle| / max|oracle| per checked tensor): 1e-4 for the fp32 path,
2e-2 for bf16 activations (bf16 and Q8_0 weights); bit-exact for the shard index maps and the
Q8_0 dequantised values.
"""
import numpy as np
import pytest

from tensor_transformer_block_amd.inputs import CONFIGS, WORKLOADS, BlockShape, make_inputs

from parity_util import TOL, log, nrel, run_and_check, t2np

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts, never run there
    pytest.skip("no GPU", allow_module_level=True)


MED = BlockShape(name="med-bf16-ragged", index=201, d_model=512, n_heads=8, n_kv_heads=2,
                 head_dim=128, ffn_dim=1376, tp=2, w_dtype="bf16", act_dtype="bf16",
                 ffn_act="silu", mode="decode", kv_lens=(37, 100, 5), n_tokens=3)
SHAPES = [
    MED,
    MED.with_(name="med-bf16-single-key", index=202, kv_lens=(1,), n_tokens=1),
    MED.with_(name="med-bf16-batched-gemm", index=203,
              kv_lens=tuple(int(v) for v in np.random.default_rng(7).integers(1, 300, 21)),
              n_tokens=21),
    MED.with_(name="med-bf16-batched-5", index=211, kv_lens=(3, 64, 17, 250, 33), n_tokens=5),
    # 125 key splits of 160 keys: the split merge's per-thread prefetch (16 splits per quarter)
    # and its tail loop.
    MED.with_(name="med-bf16-long-kv", index=234, kv_lens=(20000, 3), n_tokens=2),
    MED.with_(name="med-bf16-batched-64", index=212, tp=4, n_heads=8, n_kv_heads=4,
              ffn_dim=1408, kv_lens=tuple(range(40, 40 + 64 * 3, 3)), n_tokens=64),
    MED.with_(name="med-bf16-prefill", index=204, mode="prefill", kv_lens=(137,), n_tokens=100),
    MED.with_(name="med-bf16-prefill-300", index=213, mode="prefill", kv_lens=(333,),
              n_tokens=300),
    MED.with_(name="med-bf16-prefill-from-empty", index=205, mode="prefill", kv_lens=(70,),
              n_tokens=70, tp=4, n_heads=8, n_kv_heads=4, ffn_dim=1408),
    # Prefill shapes large enough for the 256 x 256 GEMM tiles, with ragged edges: gated
    # gate/up with 600 rows and 8224 columns; o_proj and down with 2000 rows and 6200 columns.
    MED.with_(name="med-bf16-prefill-wide-gated", index=214, mode="prefill", kv_lens=(650,),
              n_tokens=600, ffn_dim=16448),
    BlockShape(name="med-bf16-prefill-wide-rows", index=215, d_model=6200, n_heads=8,
               n_kv_heads=2, head_dim=128, ffn_dim=2176, tp=2, w_dtype="bf16",
               act_dtype="bf16", ffn_act="silu", mode="prefill", kv_lens=(2000,),
               n_tokens=2000),
    # QKV projection paths by token count: 128 <= T < 256 takes the 128-row tiles with the
    # rotary embedding and KV append in the GEMM epilogue; T = 256 exactly takes the split-K
    # projection with no shifted edge tile in M.
    MED.with_(name="med-bf16-prefill-200", index=219, mode="prefill", kv_lens=(241,),
              n_tokens=200),
    MED.with_(name="med-bf16-prefill-256", index=220, mode="prefill", kv_lens=(256,),
              n_tokens=256),
    # Prefill attention over the other GQA group sizes and head dims: one query head per KV
    # head (hd 64 and 128) and eight (hd 64), with a cached prefix and ragged token counts.
    BlockShape(name="med-bf16-prefill-g1-hd64", index=216, d_model=256, n_heads=4, n_kv_heads=4,
               head_dim=64, ffn_dim=512, tp=2, w_dtype="bf16", act_dtype="bf16",
               ffn_act="silu", mode="prefill", kv_lens=(211,), n_tokens=170),
    BlockShape(name="med-bf16-prefill-g1-hd128", index=217, d_model=256, n_heads=4,
               n_kv_heads=4, head_dim=128, ffn_dim=512, tp=2, w_dtype="bf16", act_dtype="bf16",
               ffn_act="silu", mode="prefill", kv_lens=(300,), n_tokens=300),
    BlockShape(name="med-bf16-prefill-g8-hd64", index=218, d_model=256, n_heads=16,
               n_kv_heads=2, head_dim=64, ffn_dim=512, tp=2, w_dtype="bf16", act_dtype="bf16",
               ffn_act="gelu_tanh", mode="prefill", kv_lens=(530,), n_tokens=389),
    # Batched-decode projections on the 16-column band GEMM (at least 192 bands, K a multiple
    # of 128): 37 tokens (a partial third token tile) with o_proj and down 3080 columns wide
    # (a partial last band; the gate/up, whose K of 3080 is not a multiple of 128, takes the
    # split-K GEMM), and 9 tokens with a 3208-column gated gate/up (a partial last band).
    BlockShape(name="med-bf16-band-37", index=226, d_model=3080, n_heads=8, n_kv_heads=2,
               head_dim=128, ffn_dim=6400, tp=2, w_dtype="bf16", act_dtype="bf16",
               ffn_act="gelu_tanh", mode="decode",
               kv_lens=tuple(int(v) for v in np.random.default_rng(10).integers(1, 90, 37)),
               n_tokens=37),
    BlockShape(name="med-bf16-band-9", index=227, d_model=3072, n_heads=8, n_kv_heads=2,
               head_dim=128, ffn_dim=6416, tp=2, w_dtype="bf16", act_dtype="bf16",
               ffn_act="silu", mode="decode", kv_lens=(5, 77, 1, 40, 23, 9, 60, 2, 31),
               n_tokens=9),
    # Batched decode whose every projection takes the split-K QKV or a band GEMM, so the block
    # step runs each stage as one launch for both ranks.
    BlockShape(name="med-bf16-band-all", index=228, d_model=3072, n_heads=8, n_kv_heads=2,
               head_dim=128, ffn_dim=6400, tp=2, w_dtype="bf16", act_dtype="bf16",
               ffn_act="silu", mode="decode",
               kv_lens=tuple(int(v) for v in np.random.default_rng(11).integers(1, 120, 21)),
               n_tokens=21),
    BlockShape(name="med-fp32-g2", index=206, d_model=384, n_heads=4, n_kv_heads=2, head_dim=128,
               ffn_dim=688, tp=2, w_dtype="f32", act_dtype="f32", ffn_act="silu", mode="decode",
               kv_lens=(50, 3), n_tokens=2),
    BlockShape(name="med-fp32-prefill", index=207, d_model=256, n_heads=4, n_kv_heads=4,
               head_dim=64, ffn_dim=688, tp=2, w_dtype="f32", act_dtype="f32", ffn_act="silu",
               mode="prefill", kv_lens=(40,), n_tokens=9),
    BlockShape(name="med-q8-n4", index=208, d_model=512, n_heads=8, n_kv_heads=4, head_dim=64,
               ffn_dim=1536, tp=4, w_dtype="q8_0", act_dtype="bf16", ffn_act="gelu_tanh",
               mode="decode", kv_lens=(33, 200), n_tokens=2),
    BlockShape(name="med-q8-hd256", index=209, d_model=640, n_heads=8, n_kv_heads=2,
               head_dim=256, ffn_dim=1280, tp=2, w_dtype="q8_0", act_dtype="bf16",
               ffn_act="gelu_tanh", mode="decode", kv_lens=(300,), n_tokens=1),
    BlockShape(name="med-bf16-g8", index=210, d_model=256, n_heads=16, n_kv_heads=2,
               head_dim=64, ffn_dim=512, tp=2, w_dtype="bf16", act_dtype="bf16",
               ffn_act="gelu_tanh", mode="decode", kv_lens=(129, 16), n_tokens=2),
    # Q8_0 weights with more than four tokens: the matrix-core projections with per-block scales
    # (split over K for these narrow shapes, whole-K tiles for the 300-token prefill).
    BlockShape(name="med-q8-batched-21", index=222, d_model=512, n_heads=8, n_kv_heads=4,
               head_dim=64, ffn_dim=1536, tp=4, w_dtype="q8_0", act_dtype="bf16",
               ffn_act="gelu_tanh", mode="decode",
               kv_lens=tuple(int(v) for v in np.random.default_rng(9).integers(1, 200, 21)),
               n_tokens=21),
    BlockShape(name="med-q8-batched-64", index=223, d_model=640, n_heads=8, n_kv_heads=2,
               head_dim=128, ffn_dim=1280, tp=2, w_dtype="q8_0", act_dtype="bf16",
               ffn_act="silu", mode="decode", kv_lens=tuple(range(30, 30 + 64 * 2, 2)),
               n_tokens=64),
    BlockShape(name="med-q8-prefill-300", index=224, d_model=512, n_heads=8, n_kv_heads=2,
               head_dim=64, ffn_dim=1536, tp=2, w_dtype="q8_0", act_dtype="bf16",
               ffn_act="gelu_tanh", mode="prefill", kv_lens=(333,), n_tokens=300),
    BlockShape(name="med-q8-hd256-prefill", index=225, d_model=640, n_heads=8, n_kv_heads=2,
               head_dim=256, ffn_dim=1280, tp=2, w_dtype="q8_0", act_dtype="bf16",
               ffn_act="gelu_tanh", mode="prefill", kv_lens=(50,), n_tokens=40),
]


@pytest.mark.parametrize("s", SHAPES, ids=lambda s: s.name)
def test_block_parity_small(s):
    inp = make_inputs(s, seed=11)
    run_and_check(inp, label=s.name)


@pytest.mark.parametrize("name", ["med-bf16-ragged", "med-bf16-prefill-300",
                                  "med-bf16-prefill-wide-rows", "med-bf16-batched-64",
                                  "med-bf16-band-37"])
def test_block_parity_bf16_partials(name):
    """bf16 partial storage on the decode GEMV, the prefill GEMMs (narrow and 256 x 256 tiles)
    and the batched-decode paths (split-K and band GEMMs)."""
    inp = make_inputs({x.name: x for x in SHAPES}[name], seed=12)
    run_and_check(inp, partial_dtype="bf16", label=f"{name}, bf16 partials")


@pytest.mark.parametrize("name", ["tiny-llama-fp32", "llama3-8b-decode", "gemma-q8-decode",
                                  "llama3-8b-batched", "gemma-q8-batched"])
def test_config_parity(name):
    s = WORKLOADS[name]
    log(f"{name}: generating inputs")
    inp = make_inputs(s, seed=0)
    run_and_check(inp, label=name)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llama-70b-prefill", "llama3-8b-q8-prefill"])
def test_config_parity_prefill_sampled(name):
    """2048-token prefill (70B-shaped bf16 at N=8; 8B-shaped Q8_0 at N=4): every row is computed
    on the GPU; sampled rows (first, last, a spread and the tile edges) are computed by the
    oracle one by one."""
    s = WORKLOADS[name]
    log(f"{name}: generating inputs")
    inp = make_inputs(s, seed=0)
    rows = [0, 1, 63, 64, 127, 128, 1000, 1535, 2046, 2047]
    run_and_check(inp, rows=rows, label=f"{name} (sampled rows)")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llama-70b-prefill", "llama3-8b-q8-prefill"])
def test_all_ranks_prefill_matches_staged(name):
    """2048-token prefill (70B-shaped bf16 at N = 8, 8B-shaped Q8_0 at N = 4): the block step with
    one launch per stage for all ranks (QKV, rotary / KV append, attention, o_proj, gate/up,
    down) against the separate per-rank calls: xn bit for bit (the same reduce), and h1, xn2, out,
    the FFN partials and every rank's new K, V to the bf16 tolerance (bf16: the all-ranks QKV
    takes the whole K where the separate calls split it four ways, which changes only the fp32
    summation order before its bf16 rounding); Q8_0 bit for bit (every projection keeps each
    rank's K ranges)."""
    from tensor_transformer_block_amd import binding as B
    from tensor_transformer_block_amd.block import DeviceBlock
    s = WORKLOADS[name]
    log(f"{name}: generating inputs")
    blk = DeviceBlock(make_inputs(s, seed=3))
    assert blk.schedule() == B.TP_SCHEDULE_ALL_RANKS

    def snap():
        torch.cuda.synchronize()
        r = {k: getattr(blk, k).contiguous().view(torch.uint8).cpu()
             for k in ("xn", "h1", "xn2", "out", "partials")}
        for rk in range(blk.N):
            kn, vn = blk.cache_new_entries(rk)
            r[f"kv{rk}"] = (np.ascontiguousarray(kn).view(np.uint8).copy(),
                            np.ascontiguousarray(vn).view(np.uint8).copy())
        return r

    blk.step()
    staged = snap()
    for k in ("xn", "h1", "xn2", "out"):
        getattr(blk, k).fill_(float("nan"))
    blk.step_fused(schedule=B.TP_SCHEDULE_ALL_RANKS)
    got = snap()
    assert torch.equal(got["xn"], staged["xn"])
    errs = {}
    for k in ("h1", "xn2", "out"):
        a = got[k].view(torch.bfloat16).float().numpy()
        b = staged[k].view(torch.bfloat16).float().numpy()
        errs[k] = nrel(a, b)
    pa = got["partials"].view(torch.float32).numpy()
    pb = staged["partials"].view(torch.float32).numpy()
    errs["partials"] = nrel(pa, pb)
    for rk in range(blk.N):
        for nm, a, b in zip(("k", "v"), got[f"kv{rk}"], staged[f"kv{rk}"]):
            fa = (a.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
            fb = (b.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
            errs[f"{nm}_new r{rk}"] = nrel(fa, fb)
    log(f"{name}: all-ranks step vs separate calls: "
        + ", ".join(f"{k} {v:.1e}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= 2e-2, (k, v)
        # Q8_0: the same K ranges, the QKV's fp32 tiles rounded once by the rotary kernel as the
        # separate calls' epilogue rounds them, and the same attention: the same bits.
        if s.w_dtype == "q8_0":
            assert v == 0.0, (k, v)


def test_step_matches_staged_and_graph_replay():
    """The one-call step equals the staged run bit for bit, and a captured HIP graph of the step
    replays to the same bits, with eager work between replays."""
    inp = make_inputs(MED, seed=13)
    blk, _ = run_and_check(inp, label="graph base")
    staged = blk.out.clone()
    blk.step()
    torch.cuda.synchronize()
    assert torch.equal(blk.out, staged)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        blk.step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        blk.step()
    for i in range(3):
        blk.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(blk.out, staged), f"replay {i}"
        _ = (blk.xn.float() * 2).sum().item()  # eager work between replays


# The one-call step: decode shapes take the fused schedule (norms in the QKV and gate/up
# projections, reduces in the last rank's o_proj and down, at most four ranks: one launch per
# projection for all ranks); the batched and prefill shapes take the staged sequence of the same
# calls, batched ones (on the split-K and band GEMMs, or the Q8_0 matrix-core GEMM) as one launch
# per stage for all ranks.
FUSED_STEP = ["med-bf16-ragged", "med-bf16-single-key", "med-q8-n4", "med-q8-hd256",
              "med-fp32-g2", "med-bf16-g8", "med-bf16-long-kv", "med-bf16-batched-64",
              "med-bf16-prefill", "med-bf16-band-all"]


ONE_CALL = ([(n, p) for n in FUSED_STEP for p in ("f32", "bf16")]
            + [(n, "f32") for n in ("tiny-llama-fp32", "llama3-8b-decode", "gemma-q8-decode",
                                    "llama3-8b-batched")]
            + [("llama3-8b-batched", "bf16")]
            # Q8_0 batches: each projection one matrix-core launch for all ranks
            + [(n, p) for n in ("med-q8-batched-21", "med-q8-batched-64", "med-q8-prefill-300")
               for p in ("f32", "bf16")]
            + [("gemma-q8-batched", "f32")])


@pytest.mark.parametrize("name,partial_dtype", ONE_CALL, ids=lambda v: str(v))
def test_one_call_step(name, partial_dtype):
    """tp_block_step: xn, h1, xn2, out and every rank's new K and V against the oracle, and
    against the staged calls on the same inputs (the fused decode schedule feeds the projections
    the unrounded norm, so the two agree to rounding, and exactly where no projection is fused);
    the reduce folded into the last rank's down projection exactly as the reduce kernel adds:
    out == h1 + (((P_0 + P_1) + ...) + P_{N-1}) in fp32 with one rounding. A captured graph of
    the step replays to the same bits."""
    import oracle
    from tensor_transformer_block_amd.block import DeviceBlock, to_host
    s = BY_NAME.get(name) or WORKLOADS.get(name)
    inp = make_inputs(s, seed=23)
    blk = DeviceBlock(inp, partial_dtype=partial_dtype)
    fused = s.mode == "decode" and s.n_tokens <= 4
    tol = {"f32": 1e-4, "bf16": 2e-2}[s.act_dtype]
    tol = max(tol, 2e-2) if partial_dtype == "bf16" else tol
    names = ("xn", "h1", "xn2", "out")

    def snap():
        torch.cuda.synchronize()
        r = {k: t2np(getattr(blk, k)) for k in names}
        for rk in range(blk.N):
            kn, vn = blk.cache_new_entries(rk)
            r[f"k{rk}"] = oracle.to_f64(kn, s.act_dtype)
            r[f"v{rk}"] = oracle.to_f64(vn, s.act_dtype)
        return r

    blk.step()
    staged = snap()
    for k in names:
        getattr(blk, k).fill_(float("nan"))
    blk.step_fused()
    got = snap()
    ref = oracle.run_block(inp, sharded=True)
    errs = {}
    for k in names:
        errs[k] = (nrel(got[k], ref[k]), nrel(got[k], staged[k]))
    for rk in range(blk.N):
        errs[f"k_new r{rk}"] = (nrel(got[f"k{rk}"], ref["ranks"][rk]["k_new"]),
                                nrel(got[f"k{rk}"], staged[f"k{rk}"]))
        errs[f"v_new r{rk}"] = (nrel(got[f"v{rk}"], ref["ranks"][rk]["v_new"]),
                                nrel(got[f"v{rk}"], staged[f"v{rk}"]))
    sched = {0: "staged", 1: "per rank", 2: "all ranks"}[blk.schedule()]
    log(f"one-call step {name} ({partial_dtype} partials, {'fused' if fused else 'staged'}, "
        f"{sched}): "
        + ", ".join(f"{k} {a:.1e}/{b:.1e}" for k, (a, b) in errs.items()))
    for k, (a, b) in errs.items():
        assert a <= tol, (k, a)
        assert b <= tol, (k, b)
        # The staged schedule is the separate calls themselves; the all-ranks batched schedule
        # plans the QKV's K ranges and the attention's key splits for all ranks together, which
        # changes only the order of fp32 additions (to rounding).
        if not fused and sched == "staged":
            assert b == 0.0, (k, b)
    # The all-ranks schedule (one launch per projection for every rank) against the per-rank
    # fused schedule: the same bits everywhere, partials and new cache entries included. (Batched
    # shapes have no per-rank fused schedule; they are compared with the staged calls above.)
    from tensor_transformer_block_amd import binding as B
    if blk.schedule() == B.TP_SCHEDULE_ALL_RANKS and fused:
        def bits(t):
            return t.contiguous().view(torch.uint8).cpu()
        outs = ("xn", "h1", "xn2", "out", "partials")
        all_ranks = {k: bits(getattr(blk, k)) for k in outs}
        def nbits(a):
            return np.ascontiguousarray(a).view(np.uint8).copy()
        kv_all = [tuple(nbits(a) for a in blk.cache_new_entries(rk)) for rk in range(blk.N)]
        for k in outs:
            getattr(blk, k).fill_(float("nan"))
        blk.step_fused(schedule=B.TP_SCHEDULE_PER_RANK)
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(bits(getattr(blk, k)), all_ranks[k]), f"all-ranks vs per-rank {k}"
        for rk in range(blk.N):
            for a, b in zip(kv_all[rk], blk.cache_new_entries(rk)):
                assert np.array_equal(a, nbits(b)), f"all-ranks vs per-rank cache r{rk}"
        log(f"one-call step {name}: all-ranks schedule == per-rank schedule, bit for bit")
    # The folded reduce, bit for bit: out from h1 and the stored FFN partials.
    tdt = torch.float32 if s.act_dtype == "f32" else torch.bfloat16
    acc = blk.partials[0].float().cpu().clone()
    for r in range(1, blk.N):
        acc = acc + blk.partials[r].float().cpu()
    want = (blk.h1.float().cpu() + acc).to(tdt)
    assert torch.equal(want.view(torch.int16 if tdt == torch.bfloat16 else torch.int32),
                       blk.out.cpu().view(torch.int16 if tdt == torch.bfloat16 else torch.int32))
    eager = blk.out.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        blk.step_fused()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        blk.step_fused()
    for i in range(3):
        blk.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(blk.out.view(torch.uint8), eager.view(torch.uint8)), f"replay {i}"
        _ = (blk.xn.float() * 2).sum().item()


STACKS = [(CONFIGS["tiny-llama-fp32"], 3), (MED, 2),
          (MED.with_(name="med-bf16-prefill-stack", index=221, mode="prefill", kv_lens=(150,),
                     n_tokens=130), 2),
          (CONFIGS["llama3-8b-decode"], 2)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("s,k", STACKS, ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_block_stack_parity(s, k):
    """A stack of k distinct blocks (each block's output is the next one's input): every block's
    GPU output against the oracle block run on the GPU's input to that block, and the stack's
    output against the oracle's fp64 chain; a captured graph of the whole stack replays to the
    same bits."""
    import copy
    import oracle
    from tensor_transformer_block_amd.block import BlockStack, to_host
    from tensor_transformer_block_amd.inputs import make_stack_inputs
    tol = {"f32": 1e-4, "bf16": 2e-2}[s.act_dtype]
    log(f"stack {s.name} x{k}: generating inputs")
    inps = make_stack_inputs(s, k, seed=21)
    st = BlockStack(inps)
    st.step()
    torch.cuda.synchronize()
    outs = [to_host(b.out, s.act_dtype) for b in st.blocks]
    x = inps[0].x
    for i, inp in enumerate(inps):
        one = copy.copy(inp)
        one.x = x
        ref = oracle.run_block(one)
        gpu = oracle.to_f64(outs[i], s.act_dtype)
        e = nrel(gpu, ref["out"])
        log(f"  block {i}: out err {e:.3e} (tol {tol:.0e})")
        assert e <= tol, f"block {i}"
        x = outs[i]
    chain = oracle.run_stack(inps)
    e = nrel(oracle.to_f64(outs[-1], s.act_dtype), chain[-1]["out"])
    log(f"  stack out vs fp64 chain: err {e:.3e}")
    assert e <= tol
    eager = st.out.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        st.step()
    for i in range(3):
        for b in st.blocks:
            b.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.out, eager), f"replay {i}"
        _ = (st.x.float() * 2).sum().item()  # eager work between replays


BY_NAME = {x.name: x for x in SHAPES}
HEAD_SHAPES = {"f32": BY_NAME["med-fp32-g2"], "bf16": MED, "q8_0": BY_NAME["med-q8-n4"]}


@pytest.mark.parametrize("wt", ["f32", "bf16", "q8_0"])
def test_embedding_lookup_bit_exact(wt):
    """Rows of the packed table as the activation dtype stores them (Q8_0: dequantised, one
    rounding to bf16), bit for bit; ids outside [0, vocab) clamp to the first / last row."""
    import oracle
    from tensor_transformer_block_amd import binding as B
    from tensor_transformer_block_amd.block import DeviceHead, to_host
    from tensor_transformer_block_amd.inputs import make_head_inputs
    s = HEAD_SHAPES[wt].with_(n_tokens=7, kv_lens=(4,) * 7)
    head = make_head_inputs(s, vocab=1531, seed=3)
    head.token_ids[:4] = [0, 1530, -5, 1531 + 3]
    dh = DeviceHead(head, B.make_desc(s))
    x = torch.empty((7, s.d_model), dtype=torch.float32 if s.act_dtype == "f32" else torch.bfloat16,
                    device="cuda")
    dh.embed(x)
    torch.cuda.synchronize()
    clamped = type(head)(**{**head.__dict__, "token_ids": np.clip(head.token_ids, 0, 1530)})
    ref = oracle.embed_lookup(clamped)
    got = oracle.to_f64(to_host(x, s.act_dtype), s.act_dtype)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("wt,T,vocab", [("f32", 1, 1531), ("f32", 5, 1531), ("bf16", 1, 1531),
                                        ("bf16", 3, 1531), ("bf16", 21, 1531), ("bf16", 100, 1531),
                                        ("bf16", 21, 20011), ("bf16", 64, 20011), ("q8_0", 1, 1531),
                                        ("q8_0", 6, 1531), ("q8_0", 64, 1531),
                                        ("q8_0", 130, 1531)])
def test_lm_head_parity(wt, T, vocab):
    """Logits of the GEMV (few tokens, groups of four beyond that) and of the bf16 matrix-core
    GEMMs (more tokens; up to 64 tokens over a vocabulary wide enough to fill the chip, the
    batched-decode GEMM writing its one tile straight into the logits) against the oracle on the
    same normed input, with ragged vocabulary edges."""
    import oracle
    from tensor_transformer_block_amd import binding as B
    from tensor_transformer_block_amd.block import DeviceHead, to_device
    from tensor_transformer_block_amd.inputs import _encode, make_head_inputs
    s = HEAD_SHAPES[wt].with_(n_tokens=T, kv_lens=(4,) * T)
    head = make_head_inputs(s, vocab=vocab, seed=4)
    dh = DeviceHead(head, B.make_desc(s))
    xn32 = np.random.default_rng(T).standard_normal((T, s.d_model)).astype(np.float32)
    xs = _encode(xn32, s.act_dtype)
    out = torch.full((T, vocab), float("nan"), device="cuda")
    dh.logits(to_device(xs, s.act_dtype, "cuda"), out)
    torch.cuda.synchronize()
    ref = oracle.lm_head(oracle.to_f64(xs, s.act_dtype), oracle.head_table_f64(head))
    e = nrel(t2np(out), ref)
    log(f"lm head {wt} T={T} vocab={vocab}: err {e:.3e}")
    assert e <= {"f32": 1e-4, "bf16": 2e-2, "q8_0": 2e-2}[wt]


MODEL_STEPS = [(CONFIGS["tiny-llama-fp32"], 2, 512), (MED, 2, 3000), (BY_NAME["med-q8-n4"], 2, 2048),
               (CONFIGS["llama3-8b-decode"], 1, 128256)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("s,k,vocab", MODEL_STEPS, ids=lambda v: getattr(v, "name", str(v)))
def test_model_step_parity(s, k, vocab):
    """Embedding, a stack of k blocks, final RMSNorm and LM head: the embedded input bit for bit,
    the logits against the oracle's LM head on the GPU's own normed state (the head kernel) and
    against the oracle's whole fp64 chain; a captured graph of the step replays to the same
    bits."""
    import oracle
    from tensor_transformer_block_amd.block import ModelStep, to_host
    from tensor_transformer_block_amd.inputs import make_head_inputs, make_stack_inputs
    tol = {"f32": 1e-4, "bf16": 2e-2}[s.act_dtype]
    log(f"model step {s.name} x{k} vocab {vocab}: generating inputs")
    head = make_head_inputs(s, vocab=vocab, seed=31)
    inps = make_stack_inputs(s, k, seed=31)
    ms = ModelStep(head, inps)
    ms.step()
    torch.cuda.synchronize()
    ref = oracle.run_model(head, inps)
    x = oracle.to_f64(to_host(ms.x, s.act_dtype), s.act_dtype)
    assert np.array_equal(x, ref["x"])
    table = oracle.head_table_f64(head)
    xn_f = oracle.to_f64(to_host(ms.xn_f, s.act_dtype), s.act_dtype)
    e_head = nrel(t2np(ms.logits), oracle.lm_head(xn_f, table))
    e_all = nrel(t2np(ms.logits), ref["logits"])
    log(f"  logits: head err {e_head:.3e}, whole chain err {e_all:.3e} (tol {tol:.0e})")
    assert e_head <= tol and e_all <= tol
    eager = ms.logits.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ms.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        ms.step()
    for i in range(2):
        ms.logits.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ms.logits, eager), f"replay {i}"
        _ = (ms.x.float() * 2).sum().item()


from tensor_transformer_block_amd.inputs import MOE_WORKLOADS, MoEShape  # noqa: E402

MOE_GPU = [(CONFIGS["tiny-llama-fp32"].with_(name="tiny-moe-gpu", index=230, kv_lens=(16, 5),
                                             n_tokens=2), MoEShape(8, 2, 64)),
           (MED.with_(name="med-moe-bf16", index=231), MoEShape(16, 4, 256)),
           (BY_NAME["med-q8-n4"].with_(name="med-moe-q8", index=232, tp=2, n_kv_heads=2),
            MoEShape(8, 2, 256)),
           (MED.with_(name="med-moe-prefill", index=233, mode="prefill", kv_lens=(60,),
                      n_tokens=40), MoEShape(16, 4, 256)),
           # Four ranks: the one-call step's expert down of every rank in one launch, one wave
           # per rank for each row pair.
           (MED.with_(name="med-moe-n4", index=235, tp=4, n_kv_heads=4, ffn_dim=1408),
            MoEShape(16, 4, 256)),
           (BY_NAME["med-q8-n4"].with_(name="med-moe-q8-n4", index=236), MoEShape(8, 2, 256)),
           (CONFIGS["tiny-llama-fp32"].with_(name="tiny-moe-n4", index=237, tp=4, ffn_dim=704,
                                             kv_lens=(16, 5), n_tokens=2), MoEShape(8, 2, 64)),
           MOE_WORKLOADS["moe-decode"]]


def _moe_tol(s):
    return {"f32": 1e-4, "bf16": 2e-2}[s.act_dtype]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("s,moe", MOE_GPU, ids=lambda v: getattr(v, "name", str(v)))
def test_moe_block_parity(s, moe):
    """The MoE block: router logits against the oracle; the top-k selection bit for bit against
    the oracle's rule applied to the GPU's own fp32 logits (the decision is taken in fp32 on both
    sides) and their weights; every rank's partial against the oracle's expert slices for the
    GPU's selection; the block output against the oracle chain; a graph replay bit-identical."""
    import oracle
    from tensor_transformer_block_amd.block import MoEBlock, to_host
    from tensor_transformer_block_amd.inputs import make_moe_inputs
    tol = _moe_tol(s)
    log(f"moe {s.name}: generating inputs")
    inp = make_inputs(s, seed=41)
    minp = make_moe_inputs(s, moe, seed=41)
    mb = MoEBlock(inp, minp)
    mb.step()
    torch.cuda.synchronize()
    ref = oracle.run_moe_block(inp, minp)
    b = mb.attn
    xn2 = oracle.to_f64(to_host(b.xn2, s.act_dtype), s.act_dtype)
    pm = oracle.moe_params_f64(minp)
    z_gpu = t2np(mb.logits)
    e_z = nrel(z_gpu, xn2 @ pm["router"].T)
    ids_gpu = mb.ids.cpu().numpy().astype(np.int64)
    w_gpu = t2np(mb.weights)
    ids_ref, w_ref = oracle.moe_select(z_gpu, moe.top_k)
    assert np.array_equal(ids_gpu, ids_ref)
    e_w = nrel(w_gpu, w_ref)
    parts_ref, _ = oracle.moe_ffn_sharded(s, moe, pm, xn2, ids_gpu, w_gpu)
    chk = []
    for r in range(s.tp):
        chk.append(nrel(t2np(b.partials[r]), parts_ref[r]))
    e_out = nrel(oracle.to_f64(to_host(b.out, s.act_dtype), s.act_dtype), ref["out"])
    same = np.array_equal(ref["ids"], ids_gpu)
    log(f"  logits {e_z:.3e}, weights {e_w:.3e}, partials {max(chk):.3e}, out {e_out:.3e} "
        f"(tol {tol:.0e}); oracle's own selection {'matches' if same else 'differs'}")
    assert e_z <= tol and e_w <= 1e-5 and max(chk) <= tol
    if same:
        assert e_out <= tol
    eager = b.out.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mb.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        mb.step()
    for i in range(2):
        b.out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(b.out, eager), f"replay {i}"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("s,moe", MOE_GPU, ids=lambda v: getattr(v, "name", str(v)))
def test_moe_one_call_step(s, moe):
    """tp_moe_block_step against the oracle chain: the router logits on the block's own h1, the
    selection by the oracle's rule on the GPU's logits, every rank's partial for that selection,
    and out = h1 + (((P_0 + P_1) + ...) + P_{N-1}) bit for bit from the stored h1 and partials
    (the reduce folded into the last rank's expert-down kernel); a graph replay bit-identical."""
    import oracle
    from tensor_transformer_block_amd.block import MoEBlock, to_host
    from tensor_transformer_block_amd.inputs import make_moe_inputs
    tol = _moe_tol(s)
    inp = make_inputs(s, seed=43)
    minp = make_moe_inputs(s, moe, seed=43)
    mb = MoEBlock(inp, minp)
    mb.step_fused()
    torch.cuda.synchronize()
    b = mb.attn
    ref = oracle.run_moe_block(inp, minp)
    h1 = oracle.to_f64(to_host(b.h1, s.act_dtype), s.act_dtype)
    e_h1 = nrel(h1, ref["h1"])
    xn2 = oracle.rms_norm(h1, oracle.to_f64(inp.gamma2, s.act_dtype), s.rms_eps)
    pm = oracle.moe_params_f64(minp)
    z_gpu = t2np(mb.logits)
    e_z = nrel(z_gpu, xn2 @ pm["router"].T)
    ids_gpu = mb.ids.cpu().numpy().astype(np.int64)
    ids_ref, w_ref = oracle.moe_select(z_gpu, moe.top_k)
    assert np.array_equal(ids_gpu, ids_ref)
    e_w = nrel(t2np(mb.weights), w_ref)
    xn2_s = oracle.to_f64(to_host(b.xn2, s.act_dtype), s.act_dtype)
    parts_ref, _ = oracle.moe_ffn_sharded(s, moe, pm, xn2_s, ids_gpu, t2np(mb.weights))
    e_p = max(nrel(t2np(b.partials[r]), parts_ref[r]) for r in range(s.tp))
    same = np.array_equal(ref["ids"], ids_gpu)
    e_out = nrel(oracle.to_f64(to_host(b.out, s.act_dtype), s.act_dtype), ref["out"])
    log(f"moe one-call {s.name}: h1 {e_h1:.2e}, logits {e_z:.2e}, weights {e_w:.2e}, partials "
        f"{e_p:.2e}, out {e_out:.2e}; oracle's own selection {'matches' if same else 'differs'}")
    assert e_h1 <= tol and e_z <= tol and e_w <= 1e-5 and e_p <= tol
    if same:
        assert e_out <= tol
    tdt = torch.float32 if s.act_dtype == "f32" else torch.bfloat16
    acc = b.partials[0].float().cpu().clone()
    for r in range(1, s.tp):
        acc = acc + b.partials[r].float().cpu()
    want = (b.h1.float().cpu() + acc).to(tdt)
    assert torch.equal(want.view(torch.uint8), b.out.cpu().view(torch.uint8))
    # With one rank's expert workspace the step runs each rank's expert gate/up and down on its
    # own; with every rank's share (above) a decode step runs the gate/up of every rank as one
    # launch and the down of every rank, reduce included, as another: the same bits.
    if s.mode == "decode" and s.tp > 1:
        snap = {k: getattr(b, k).clone() for k in ("out", "partials")}
        b.out.fill_(float("nan"))
        mb.step_fused(moe_ws_bytes=mb.ws_bytes)
        torch.cuda.synchronize()
        for k, v in snap.items():
            assert torch.equal(getattr(b, k).view(torch.uint8), v.view(torch.uint8)), k
        # The measurement variant (events around the all-ranks expert gate/up): the same bits.
        from parity_util import HipEventPair
        ev = HipEventPair()
        b.out.fill_(float("nan"))
        mb.step_fused(timed=(ev.begin, ev.end))
        torch.cuda.synchronize()
        for k, v in snap.items():
            assert torch.equal(getattr(b, k).view(torch.uint8), v.view(torch.uint8)), k
        assert ev.elapsed_us() > 0
        ev.close()
    eager = b.out.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mb.step_fused()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        mb.step_fused()
    for i in range(2):
        b.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(b.out.view(torch.uint8), eager.view(torch.uint8)), f"replay {i}"


@pytest.mark.parametrize("E,k", [(40, 6), (100, 8), (200, 16), (500, 4), (1000, 16)])
def test_moe_topk_ties_and_bounds(E, k):
    """Experts with identical router rows tie exactly; the lower index comes first, also between
    experts that share a lane (64 apart). Every token selects distinct experts. The expert counts
    give each lane 1, 2, 4, 8 and 16 logits."""
    import oracle
    from tensor_transformer_block_amd import binding as B
    from tensor_transformer_block_amd.block import to_device
    from tensor_transformer_block_amd.inputs import _encode
    s = MED.with_(n_tokens=5, kv_lens=(4,) * 5)
    moe = MoEShape(E, k, 256)
    rng = np.random.default_rng(5)
    router = rng.standard_normal((E, s.d_model)).astype(np.float32) * 0.05
    tied = [e for e in (3, 7, 30, 67, 131, 515) if e < E]
    for e in tied[1:]:
        router[e] = router[3]
    router[12] = router[21]
    x = rng.standard_normal((5, s.d_model)).astype(np.float32)
    x[1] = router[3] * 40  # token 1 prefers the tied experts (equal logits)
    rt = to_device(_encode(router, "bf16"), "bf16", "cuda")
    xt = to_device(_encode(x, "bf16"), "bf16", "cuda")
    z = torch.empty((5, E), device="cuda")
    ids = torch.empty((5, k), dtype=torch.int32, device="cuda")
    w = torch.empty((5, k), device="cuda")
    B.tp_moe_route(B.make_desc(s), B.make_moe_desc(moe), rt, xt, 5, z, ids, w)
    torch.cuda.synchronize()
    ids_ref, w_ref = oracle.moe_select(t2np(z), k)
    got = ids.cpu().numpy()
    assert np.array_equal(got, ids_ref)
    n = min(k, len(tied))
    assert list(got[1][:n]) == tied[:n]
    assert all(len(set(row)) == k for row in got)
    assert nrel(t2np(w), w_ref) <= 1e-5


@pytest.mark.parametrize("name", ["tiny-llama-fp32", "llama3-8b-batched", "gemma-q8-decode",
                                  "med-q8-n4"])
def test_shard_maps_bit_exact(name):
    """Unpacking every rank's shard back into zeroed full matrices reproduces the full weights
    byte for byte; each rank's payload is exactly 1/N of the full weight bytes."""
    from tensor_transformer_block_amd import binding as B
    from tensor_transformer_block_amd.block import to_device
    s = CONFIGS.get(name) or {x.name: x for x in SHAPES}[name]
    inp = make_inputs(s, seed=1)
    desc = B.make_desc(s)
    full = {k: to_device(v, s.w_dtype, "cuda") for k, v in inp.weights.items()}
    back = {k: torch.zeros_like(v) for k, v in full.items()}
    total = sum(v.numel() * v.element_size() for v in full.values())
    for r in range(s.tp):
        lay = B.tp_shard_weights_size(desc, r)
        assert lay.payload_bytes * s.tp == total
        buf = torch.empty(lay.alloc_bytes, dtype=torch.uint8, device="cuda")
        B.tp_shard_weights(desc, r, B.full_weights(full), buf)
        B.tp_shard_unpack(desc, r, buf, B.full_weights(back))
    torch.cuda.synchronize()
    for k in full:
        a = full[k].view(torch.uint8) if full[k].dtype != torch.uint8 else full[k]
        b = back[k].view(torch.uint8) if back[k].dtype != torch.uint8 else back[k]
        assert torch.equal(a, b), k


def test_q8_dequant_bit_exact():
    """The library's Q8_0 dequant helper (the device function the embedding lookup and the MoE
    expert kernels use; the projections are checked by the one-hot test below) equals
    fp16(d) * q computed on the host."""
    from tensor_transformer_block_amd import binding as B
    from tensor_transformer_block_amd.inputs import q8_0_encode
    import oracle
    rng = np.random.default_rng(3)
    w = (0.02 * rng.standard_normal((64, 512))).astype(np.float32)
    w[5, :64] = 0
    w[7, 32:64] *= 1e4
    aos = q8_0_encode(w).reshape(64, 16, 34)
    codes = np.ascontiguousarray(aos[..., 2:]).reshape(-1).view(np.int8)
    scales = np.ascontiguousarray(aos[..., :2]).reshape(-1).view(np.uint16)
    c = torch.from_numpy(codes.copy()).cuda()
    sc = torch.from_numpy(scales.copy().view(np.int16)).cuda()
    out = torch.empty(codes.size, dtype=torch.float32, device="cuda")
    B.tp_dequant_q8_0(c, sc, out, scales.size)
    torch.cuda.synchronize()
    ref = oracle.dequant_q8_0(aos.reshape(64, -1), 64, 512).reshape(-1)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)


# (workload, rank, tokens per call): one token and four tokens per call run the dequantising
# GEMV of decode; 64 tokens the matrix-core Q8_0 GEMM split over K (batched decode); 0 means all
# K one-hot rows in one call, the whole-K tiles of prefill.
Q8_PROJ_CASES = [("gemma-q8-decode", 0, 1), ("gemma-q8-decode", 1, 1), ("gemma-q8-decode", 1, 4),
                 ("gemma-q8-decode", 0, 64), ("gemma-q8-decode", 1, 0),
                 ("llama3-8b-q8-prefill", 3, 1), ("llama3-8b-q8-prefill", 2, 64)]
_Q8_CACHE = {}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,rank,T", Q8_PROJ_CASES, ids=lambda v: str(v))
def test_q8_projection_dequant_bit_exact(name, rank, T):
    """The Q8_0 projections as the forward path runs them (tp_shard_project: the same kernel
    choice and main loops, with the fp32 partial epilogue of o_proj and down) on one-hot bf16
    rows: row k of the output is column k of the region as the kernels dequantise it. Every
    region of rank r's shard (QKV, o, gate/up, down) must equal the oracle's d * q of the same
    blocks, bit for bit: the dequantised weights are exact in fp32 and a one-hot product adds
    only zeros to one of them, so any error in forming them shows."""
    import oracle
    from tensor_transformer_block_amd import binding as B
    from tensor_transformer_block_amd.block import to_device
    s = WORKLOADS[name].with_(mode="decode", n_tokens=1, kv_lens=(1,))
    if name not in _Q8_CACHE:
        _Q8_CACHE.clear()
        log(f"q8 projections {name}: generating inputs")
        inp = make_inputs(s, seed=0)
        _Q8_CACHE[name] = (inp, oracle.params_f64(inp))
    inp, p = _Q8_CACHE[name]
    desc = B.make_desc(s)
    full = {k: to_device(v, s.w_dtype, "cuda") for k, v in inp.weights.items()}
    lay = B.tp_shard_weights_size(desc, rank)
    shard = torch.empty(lay.alloc_bytes, dtype=torch.uint8, device="cuda")
    B.tp_shard_weights(desc, rank, B.full_weights(full), shard)
    del full
    w = oracle.shard_weights(s, p, rank)
    regions = {0: np.concatenate([w["wq"], w["wk"], w["wv"]]), 1: w["wo"],
               2: np.concatenate([w["wg"], w["wu"]]), 3: w["wd"]}
    for which, ref in regions.items():
        rows, K = ref.shape
        per = K if T == 0 else T
        eye = torch.eye(K, dtype=torch.bfloat16, device="cuda")
        out = torch.full((K, rows), float("nan"), device="cuda")
        wsb = B.tp_shard_project_workspace_size(desc, which, per)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        for k0 in range(0, K, per):
            B.tp_shard_project(desc, which, shard, eye[k0:k0 + per], per, out[k0:k0 + per], ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy().T.astype(np.float64)
        bad = int(np.count_nonzero(got != ref))
        log(f"q8 {name} rank {rank} region {which} [{rows}x{K}] {per} token(s) per call: "
            f"{bad} of {got.size} values differ")
        assert bad == 0, f"region {which}: {bad} dequantised values differ"


@pytest.mark.parametrize("T", [1, 4])
def test_q8_gemv_activation_range(T):
    """The Q8_0 decode GEMV stages each 16-value chunk of the activations as fp16 times a power of
    two of its own. Rows whose chunks span magnitudes 2^-100 to 2^100, with all-zero chunks among
    them, through the forward path's projection kernels (tp_shard_project, T tokens per call, every
    region of the Gemma-like shard's rank 0): the products must equal the oracle's fp64 products of
    the dequantised weights to 1e-4 of each token's largest output. bf16 values fit fp16's
    significand, so a chunk's dot product with the codes is exact up to fp32 accumulation, and no
    chunk is lost to the range of the others (a shared fp16 scale would flush the small ones)."""
    import oracle
    from tensor_transformer_block_amd import binding as B
    from tensor_transformer_block_amd.block import to_device
    from tensor_transformer_block_amd.inputs import f32_to_bf16_bits
    s = WORKLOADS["gemma-q8-decode"].with_(mode="decode", n_tokens=1, kv_lens=(1,))
    if "gemma-q8-decode" not in _Q8_CACHE:
        _Q8_CACHE.clear()
        inp = make_inputs(s, seed=0)
        _Q8_CACHE["gemma-q8-decode"] = (inp, oracle.params_f64(inp))
    inp, p = _Q8_CACHE["gemma-q8-decode"]
    desc = B.make_desc(s)
    full = {k: to_device(v, s.w_dtype, "cuda") for k, v in inp.weights.items()}
    lay = B.tp_shard_weights_size(desc, 0)
    shard = torch.empty(lay.alloc_bytes, dtype=torch.uint8, device="cuda")
    B.tp_shard_weights(desc, 0, B.full_weights(full), shard)
    del full
    w = oracle.shard_weights(s, p, 0)
    regions = {0: np.concatenate([w["wq"], w["wk"], w["wv"]]), 1: w["wo"],
               2: np.concatenate([w["wg"], w["wu"]]), 3: w["wd"]}
    rng = np.random.default_rng(31)
    for which, ref_w in regions.items():
        rows, K = ref_w.shape
        nch = K // 16
        expo = rng.integers(-100, 101, size=(T, nch)).astype(np.float64)
        expo[:, ::7] = np.nan  # every seventh chunk all zero
        scale = np.where(np.isnan(expo), 0.0, np.exp2(np.nan_to_num(expo)))
        x = rng.standard_normal((T, nch, 16)) * scale[:, :, None]
        xb = f32_to_bf16_bits(x.reshape(T, K).astype(np.float32))
        x64 = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        xt = to_device(xb, "bf16", "cuda")
        out = torch.full((T, rows), float("nan"), device="cuda")
        ws = torch.empty(B.tp_shard_project_workspace_size(desc, which, T), dtype=torch.uint8,
                         device="cuda")
        B.tp_shard_project(desc, which, shard, xt, T, out, ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        ref = x64 @ ref_w.T
        err = np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)
        log(f"q8 activation range region {which} [{rows}x{K}] T={T}: max-abs-rel per token "
            f"{np.array2string(err, precision=2)}")
        assert np.isfinite(got).all(), f"region {which}: non-finite outputs"
        assert err.max() <= 1e-4, f"region {which}: {err.max():.3g}"


# Cache slots holding no key: past each sequence's last position, and a page that no sequence owns
# which the block table's unused entries point at.
STALE_CASES = ["med-bf16-ragged", "med-bf16-batched-64", "med-bf16-prefill", "med-q8-hd256",
               "med-q8-hd256-prefill", "med-fp32-g2", "med-bf16-g8"]


@pytest.mark.parametrize("name", STALE_CASES)
def test_unwritten_cache_slots_never_reach_the_output(name):
    """Page slots no key was written to (past each sequence's last position, and an extra page
    that the block table's unused entries point at) filled with NaN and Inf bit patterns give the
    same step, bit for bit, as zero-filled pools: the attention output, every rank's partials,
    the new K and V, h1 and out (mlxcel issue #488, "Acceptance criteria": no silent wrong
    results)."""
    from tensor_transformer_block_amd import binding as B
    from tensor_transformer_block_amd.block import DeviceBlock
    s = BY_NAME[name]
    inp = make_inputs(s, seed=17)
    extra = inp.n_pages
    inp.n_pages += 1
    ps = s.page_size
    used = [-(-int(L) // ps) for L in inp.seq_lens]
    tab = np.concatenate([inp.block_table, np.full((s.n_seqs, 2), extra, np.int32)], axis=1)
    for b, n in enumerate(used):
        tab[b, n:] = extra
    inp.block_table = np.ascontiguousarray(tab)
    blk = DeviceBlock(inp)
    # Slots holding a prior key (the step writes each new token's slot before attending).
    written = np.zeros((inp.n_pages, ps), dtype=bool)
    for b in range(s.n_seqs):
        prior = int(inp.seq_lens[b]) - (s.n_tokens if s.mode == "prefill" else 1)
        for pos in range(prior):
            written[tab[b, pos // ps], pos % ps] = True
    wm = torch.from_numpy(written).cuda()
    pristine = [(k.clone(), v.clone()) for k, v in zip(blk.k_pages[0], blk.v_pages[0])]

    def run(poison: bool):
        for r in range(blk.N):
            kp, vp = blk.k_pages[0][r], blk.v_pages[0][r]
            kp.copy_(pristine[r][0])
            vp.copy_(pristine[r][1])
            if poison:
                kp.masked_fill_(~wm[:, None, :, None].expand_as(kp), float("nan"))
                vp.masked_fill_(~wm[:, None, None, :].expand_as(vp), float("inf"))
                vp[1::2].masked_fill_(~wm[1::2, None, None, :].expand_as(vp[1::2]), float("nan"))
        d, T, N = blk.desc, blk.T, blk.N
        res = {}
        B.tp_partial_reduce(d, T, None, 0, blk.x, None, blk.gamma1, blk.xn)
        for r in range(N):
            blk.attn_half(r)
            _, av, _ = blk.workspace_views()
            res[f"a r{r}"] = av.clone()
            res[f"P_attn r{r}"] = blk.partials[r].clone()
        B.tp_partial_reduce(d, T, blk.partials, N, blk.x, blk.h1, blk.gamma2, blk.xn2)
        for r in range(N):
            blk.ffn_half(r)
        B.tp_partial_reduce(d, T, blk.partials, N, blk.h1, blk.out, None, None)
        torch.cuda.synchronize()
        res["h1"], res["out"] = blk.h1.clone(), blk.out.clone()
        res = {k: v.float().cpu().numpy() for k, v in res.items()}  # exact widening
        for r in range(N):
            kn, vn = blk.cache_new_entries(r)
            res[f"k_new r{r}"], res[f"v_new r{r}"] = kn, vn
        return res

    clean = run(False)
    dirty = run(True)
    for k in clean:
        assert np.isfinite(clean[k].astype(np.float64)).all(), k
        a, b = np.ascontiguousarray(clean[k]), np.ascontiguousarray(dirty[k])
        assert a.shape == b.shape and a.tobytes() == b.tobytes(), k
    log(f"stale slots {name}: {int((~written).sum())} unwritten slots per head; outputs identical")


@pytest.mark.parametrize("E,k", [(8, 2), (8, 8), (40, 6), (100, 8)])
def test_moe_route_nan_logit(E, k):
    """A NaN router logit ranks as -inf: the selection equals the oracle's rule applied to the
    logits with the NaN replaced by -inf, the NaN expert is picked only when every other one
    is, with weight 0, and no weight is NaN."""
    import oracle
    from tensor_transformer_block_amd import binding as B
    from tensor_transformer_block_amd.block import to_device
    from tensor_transformer_block_amd.inputs import _encode
    s = MED.with_(n_tokens=3, kv_lens=(4,) * 3)
    moe = MoEShape(E, k, 256)
    rng = np.random.default_rng(E + k)
    router = _encode(rng.standard_normal((E, s.d_model)).astype(np.float32) * 0.05, "bf16")
    router[5, 7] = 0x7FC0  # a NaN weight: expert 5's logit is NaN for every token
    x = _encode(rng.standard_normal((3, s.d_model)).astype(np.float32), "bf16")
    rt, xt = to_device(router, "bf16", "cuda"), to_device(x, "bf16", "cuda")
    z = torch.empty((3, E), device="cuda")
    ids = torch.empty((3, k), dtype=torch.int32, device="cuda")
    w = torch.empty((3, k), device="cuda")
    B.tp_moe_route(B.make_desc(s), B.make_moe_desc(moe), rt, xt, 3, z, ids, w)
    torch.cuda.synchronize()
    zh = t2np(z)
    assert np.isnan(zh[:, 5]).all()
    ids_ref, w_ref = oracle.moe_select(np.where(np.isnan(zh), -np.inf, zh), k)
    got = ids.cpu().numpy()
    assert np.array_equal(got, ids_ref)
    wh = t2np(w)
    assert np.isfinite(wh).all() and nrel(wh, w_ref) <= 1e-5
    assert (5 in got[0]) == (k == E)


def test_empty_batch_is_noop():
    from tensor_transformer_block_amd import binding as B
    from tensor_transformer_block_amd.block import DeviceBlock
    inp = make_inputs(MED.with_(kv_lens=(5,), n_tokens=1), seed=2)
    blk = DeviceBlock(inp)
    b0 = B.make_batch("decode", 0, 0, blk.max_pages, blk.max_seq_len, blk.positions,
                      blk.seq_lens, blk.block_table, blk.rope)
    before = blk.partials.clone()
    B.tp_block_shard_forward(blk.desc, 0, B.TP_HALF_ATTN, blk.shards[0][0], b0, blk.xn,
                             blk.kv[0][0], blk.partials[0], blk.workspace, blk.ws_bytes)
    B.tp_partial_reduce(blk.desc, 0, blk.partials, 2, blk.x, blk.h1, blk.gamma2, blk.xn2)
    torch.cuda.synchronize()
    assert torch.equal(before, blk.partials)


@pytest.mark.parametrize("d,n_part,act,part", [
    (512, 1, "bf16", "f32"), (2560, 3, "bf16", "f32"), (4096, 11, "bf16", "bf16"),
    (12288, 11, "bf16", "f32"), (12288, 2, "f32", "f32"), (256, 9, "f32", "f32"),
])
def test_reduce_groups_and_row_widths(d, n_part, act, part):
    """The reduce with and without gamma: rows of one wave, several waves, and two chunks per
    thread (d > 8192), more partials than one load group (tail groups), fp32 and bf16 storage.
    The residual sum is compared bit for bit with the same fp32 order on the host; the norm with
    the fp64 RMSNorm of the stored residual."""
    from tensor_transformer_block_amd import binding as B
    s = MED.with_(d_model=d, n_heads=d // 128, n_kv_heads=d // 128, ffn_dim=2 * d,
                  act_dtype=act, w_dtype="f32" if act == "f32" else "bf16")
    desc = B.make_desc(s, partial_dtype=part)
    T = 3
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}
    g = torch.Generator().manual_seed(d + n_part)
    P = torch.randn(n_part, T, d, generator=g).to(tdt[part])
    x = (torch.randn(T, d, generator=g) * 3).to(tdt[act])
    gamma = (1 + 0.1 * torch.randn(d, generator=g)).to(tdt[act])
    acc = P[0].float().clone()
    for r in range(1, n_part):
        acc = acc + P[r].float()
    ref = (x.float() + acc).to(tdt[act])
    xd, Pd, gd = x.cuda(), P.cuda(), gamma.cuda()
    for with_gamma in (False, True):
        out = torch.full_like(xd, float("nan"))
        nrm = torch.full_like(xd, float("nan"))
        B.tp_partial_reduce(desc, T, Pd, n_part, xd, out, gd if with_gamma else None,
                            nrm if with_gamma else None)
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), ref), f"d={d} n={n_part}: residual differs"
        if with_gamma:
            h = ref.double().numpy()
            want = gamma.double().numpy() * h / np.sqrt((h * h).mean(-1, keepdims=True) + s.rms_eps)
            err = nrel(t2np(nrm), want)
            log(f"reduce d={d} n={n_part} {act}/{part}: norm err {err:.2e}")
            assert err < TOL[act]


def test_reduce_order_and_rounding():
    """h = x + ((P0 + P1) + P2) in fp32 with one rounding: compared with the same order on the
    host in fp32 (one rounding to bf16, nearest even)."""
    from tensor_transformer_block_amd import binding as B
    s = MED.with_(tp=4, n_heads=8, n_kv_heads=4, ffn_dim=1408)
    desc = B.make_desc(s)
    T, d = 5, s.d_model
    g = torch.Generator().manual_seed(0)
    P = (torch.randn(4, T, d, generator=g) * 100).float()
    x = torch.randn(T, d, generator=g).bfloat16()
    acc = P[0].clone()
    for r in range(1, 4):
        acc = acc + P[r]
    ref = (x.float() + acc).bfloat16()
    xd, Pd = x.cuda(), P.cuda()
    out = torch.empty_like(xd)
    B.tp_partial_reduce(desc, T, Pd, 4, xd, out, None, None)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), ref)
    log(f"reduce: max err vs fp64 sum {nrel(t2np(out), (x.double() + P.double().sum(0)).numpy()):.2e}")

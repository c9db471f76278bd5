"""Helpers shared by the GPU parity tests: run the device block stage by stage and compare every
stage with the oracle on the same seeded inputs."""
from __future__ import annotations

import sys
import time

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


class HipEventPair:
    """Two hipEvent_t handles (created through the HIP runtime) for the library's *_timed calls,
    which record them around a launch."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        hs = []
        for _ in range(2):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0, "hipEventCreate failed"
            hs.append(h.value)
        self.begin, self.end = hs

    def elapsed_us(self) -> float:
        ms = self.ct.c_float()
        assert self.hip.hipEventElapsedTime(self.ct.byref(ms), self.begin, self.end) == 0
        return ms.value * 1e3

    def close(self) -> None:
        self.hip.hipEventDestroy(self.begin)
        self.hip.hipEventDestroy(self.end)


def nrel(a, b) -> float:
    """Normwise max-abs-relative error: max|a - b| / max|b|."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = float(np.max(np.abs(b))) if b.size else 0.0
    if b.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)) / max(den, 1e-30))


def t2np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, np.float64)


class StageChecker:
    """Collects (stage, error, tolerance) and asserts at the end with the full table."""

    def __init__(self, label: str, tol: float):
        self.label, self.tol, self.rows = label, tol, []

    def __call__(self, stage: str, gpu, ref, tol: float | None = None):
        e = nrel(gpu, ref)
        self.rows.append((stage, e, self.tol if tol is None else tol))

    def report(self) -> str:
        return "\n".join(f"  {s:<24s} err={e:.3e} tol={t:.1e} {'OK' if e <= t else 'FAIL'}"
                         for s, e, t in self.rows)

    def assert_ok(self):
        log(f"{self.label}\n{self.report()}")
        bad = [r for r in self.rows if not (r[1] <= r[2])]
        assert not bad, f"{self.label}: stages out of tolerance:\n{self.report()}"


def run_and_check(inp, rows=None, partial_dtype: str = "f32", label: str = ""):
    """Run one block step stage by stage on the GPU and check every stage against the oracle.

    rows: token rows checked (all by default); the GPU always computes every row.
    """
    import torch
    import oracle
    from tensor_transformer_block_amd.block import DeviceBlock

    s = inp.shape
    tol = TOL[s.act_dtype]
    if partial_dtype == "bf16":
        tol = max(tol, TOL["bf16"])
    t0 = time.time()
    ref = oracle.run_block(inp, sharded=True, rows=rows)
    log(f"{label}: oracle done in {time.time() - t0:.1f}s")
    sel = np.arange(s.n_tokens) if rows is None else np.asarray(rows)
    blk = DeviceBlock(inp, partial_dtype=partial_dtype)
    chk = StageChecker(f"{label} ({s.name}, N={s.tp}, T={s.n_tokens})", tol)
    d, T, N = blk.desc, blk.T, blk.N
    from tensor_transformer_block_amd import binding as B

    B.tp_partial_reduce(d, T, None, 0, blk.x, None, blk.gamma1, blk.xn)
    torch.cuda.synchronize()
    chk("xn (a1)", t2np(blk.xn)[sel], ref["xn"])
    hq, hd = s.n_heads // N, s.head_dim
    for r in range(N):
        blk.attn_half(r)
        torch.cuda.synchronize()
        rk = ref["ranks"][r]
        qv, av, _ = blk.workspace_views()
        chk(f"q_rot r{r}", t2np(qv)[sel], rk["q"].reshape(len(sel), hq * hd))
        kn, vn = blk.cache_new_entries(r)
        chk(f"k_new r{r}", storage_to_f64(kn, s.act_dtype)[sel], rk["k_new"])
        chk(f"v_new r{r}", storage_to_f64(vn, s.act_dtype)[sel], rk["v_new"])
        chk(f"attn a_r r{r}", t2np(av)[sel], rk["a"])
        chk(f"P_attn r{r}", t2np(blk.partials[r])[sel], rk["p_attn"])
    B.tp_partial_reduce(d, T, blk.partials, N, blk.x, blk.h1, blk.gamma2, blk.xn2)
    torch.cuda.synchronize()
    chk("sum P_attn", t2np(blk.partials.float().sum(0))[sel], ref["attn_sum"])
    chk("h1 (a6)", t2np(blk.h1)[sel], ref["h1"])
    chk("xn2 (a6)", t2np(blk.xn2)[sel], ref["xn2"])
    for r in range(N):
        blk.ffn_half(r)
        torch.cuda.synchronize()
        rk = ref["ranks"][r]
        _, _, mv = blk.workspace_views()
        chk(f"m_r r{r}", t2np(mv)[sel], rk["m"])
        chk(f"P_ffn r{r}", t2np(blk.partials[r])[sel], rk["p_ffn"])
    B.tp_partial_reduce(d, T, blk.partials, N, blk.h1, blk.out, None, None)
    torch.cuda.synchronize()
    chk("sum P_ffn", t2np(blk.partials.float().sum(0))[sel], ref["ffn_sum"])
    chk("out (a9)", t2np(blk.out)[sel], ref["out"])
    chk.assert_ok()
    return blk, ref

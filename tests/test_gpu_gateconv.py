"""GateConv forward and backward on the GPU against the fp64 oracle
("Engram Operators", TileOPs, GateConv section; readings G1-G6).

Comparison rules, derived from the fp32 arithmetic of the kernels:

* alpha: |a - a64| <= a(1-a) (32u smag + 1e-5 |s|) + 8u a, where smag =
  sum |h^ k^| / sqrt(d) bounds the fp32 error of the logit s (a cancelling
  sum of d products) and 8u covers the sigmoid's own evaluation;
* rrms_h, rrms_k: relative 1e-5 (a sum of squares and a reciprocal root);
  rrms_v: relative 1e-5 plus alpha's relative tolerance (rrms_v ~ 1/alpha);
* bf16 tensors (Y, vhat, dH, dk, dv): within one bf16 ulp of the unrounded
  fp64 value, widened by kappa u mag with the oracle's magnitude of every
  term of that element (kappa = 64: the deepest fp32 chain is a row sum of
  up to 28 rounding steps, entered twice); norm-wise against the rounded
  oracle within 2e-3 (half a bf16 ulp is 2^-9 = 1.95e-3 relative);
* fp32 weight gradients: within 2^-14 mag + 1e-6 |ref| (a sequential sum over
  a chunk of up to 512 rows, then over chunk partials, each step at most u
  relative to the magnitude), norm-wise within 1e-5.

The backward is fed the oracle's saved tensors rounded to their storage types
(vhat bf16, alpha and rrms_* fp32), so both sides see the same inputs; one
case feeds both sides the GPU forward's own saved tensors instead.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from numerics import U32, bf16_to_f64, check_bf16, check_rel

pytestmark = pytest.mark.gpu

EPS = 1e-6


def f64(bits):
    return bf16_to_f64(bits)


def dev(a, gpu):
    from gpu_util import to_dev
    return to_dev(a, gpu)


def empty_bf16(shape, gpu):
    import torch
    from gpu_util import poison
    return poison(torch.empty(shape, dtype=torch.bfloat16, device=gpu))


def empty_f32(shape, gpu):
    import torch
    from gpu_util import poison
    return poison(torch.empty(shape, dtype=torch.float32, device=gpu))


def run_fwd(inp, gpu, eps=EPS):
    import torch
    import memory_bound_engram_amd as eg
    M, T, d = inp["H"].shape
    H, k, v = dev(inp["H"], gpu), dev(inp["k"], gpu), dev(inp["v"], gpu)
    wh, wv, cw = dev(inp["wh"], gpu), dev(inp["wv"], gpu), dev(inp["cw"], gpu)
    Y, vhat = empty_bf16((M, T, d), gpu), empty_bf16((M, T, d), gpu)
    al, rh, rk, rv = (empty_f32((M, T), gpu) for _ in range(4))
    eg.engram_gateconv_fwd(H, k, v, wh, wv, cw, Y, vhat, al, rh, rk, rv, eps=eps)
    torch.cuda.synchronize()
    from gpu_util import u16
    return {"Y": u16(Y), "vhat": u16(vhat), "alpha": al.cpu().numpy(), "rh": rh.cpu().numpy(),
            "rk": rk.cpu().numpy(), "rv": rv.cpu().numpy()}


def run_bwd(inp, saved, gpu, repeat=1):
    import torch
    import memory_bound_engram_amd as eg
    from gpu_util import poison, u16
    M, T, d = inp["H"].shape
    args = [dev(inp[x], gpu) for x in ("dY", "H", "k", "v", "wh", "wv", "cw")]
    args += [dev(saved[x], gpu) for x in ("vhat", "alpha", "rh", "rk", "rv")]
    outs = []
    for _ in range(repeat):
        dH, dk, dv = (empty_bf16((M, T, d), gpu) for _ in range(3))
        dwh, dwv, dcw = empty_f32((d,), gpu), empty_f32((d,), gpu), empty_f32((4, d), gpu)
        ws = poison(torch.empty(eg.engram_gateconv_bwd_workspace_bytes(M, T, d), dtype=torch.uint8, device=gpu))
        eg.engram_gateconv_bwd(*args, dH, dk, dv, dwh, dwv, dcw, ws)
        torch.cuda.synchronize()
        outs.append({"dH": u16(dH), "dk": u16(dk), "dv": u16(dv), "dwh": dwh.cpu().numpy(),
                     "dwv": dwv.cpu().numpy(), "dcw": dcw.cpu().numpy()})
    return outs if repeat > 1 else outs[0]


def oracle_fwd(inp, eps=EPS):
    H, k, v = f64(inp["H"]), f64(inp["k"]), f64(inp["v"])
    wh, wv, cw = (inp[x].astype(np.float64) for x in ("wh", "wv", "cw"))
    return oracle.gateconv_fwd_f64(H, k, v, wh, wv, cw, eps=eps, mags=True)


def rounded_saved(ref):
    """The oracle's saved tensors in their storage types."""
    Y, vhat, al, rh, rk, rv = ref[:6]
    return {"vhat": oracle.round_bf16(vhat), "alpha": al.astype(np.float32), "rh": rh.astype(np.float32),
            "rk": rk.astype(np.float32), "rv": rv.astype(np.float32)}


def check_fwd(inp, got, ref):
    Y64, vhat64, al64, rh64, rk64, rv64, magY = ref
    H, k = f64(inp["H"]), f64(inp["k"])
    wh = inp["wh"].astype(np.float64)
    d = H.shape[-1]
    # alpha: conditioning of the logit s = <h^, k^> / sqrt(d)
    hh = H * rh64[..., None] * wh
    kh = k * rk64[..., None] * wh
    s = np.sum(hh * kh, axis=-1) / np.sqrt(d)
    smag = np.sum(np.abs(hh * kh), axis=-1) / np.sqrt(d)
    tol_a = al64 * (1 - al64) * (32 * U32 * smag + 1e-5 * np.abs(s)) + 8 * U32 * al64
    check_rel("alpha", got["alpha"], al64, 0.0, atol=tol_a)
    check_rel("rrms_h", got["rh"], rh64, 1e-5)
    check_rel("rrms_k", got["rk"], rk64, 1e-5)
    rel_a = tol_a / np.maximum(al64, 1e-300)
    check_rel("rrms_v", got["rv"], rv64, 0.0, atol=rv64 * (1e-5 + rel_a))
    v = f64(inp["v"])
    st_vh = check_bf16("vhat", got["vhat"], vhat64, np.abs(vhat64), kappa=8, extra=np.abs(v) * tol_a[..., None])
    st_y = check_bf16("Y", got["Y"], Y64, magY, kappa=64)
    for name, st in (("vhat", st_vh), ("Y", st_y)):
        assert st["sq_diff_rounded"] <= (2e-3) ** 2 * st["sq_rounded"], name
    return st_y


def check_bwd(got, ref):
    dH, dk, dv, dwh, dwv, dcw, mH, mk, mv, mwh, mwv, mcw = ref
    stats = {}
    for name, r, m in (("dH", dH, mH), ("dk", dk, mk), ("dv", dv, mv)):
        st = check_bf16(name, got[name], r, m, kappa=64)
        assert st["sq_diff_rounded"] <= (2e-3) ** 2 * st["sq_rounded"], name
        stats[name] = st
    for name, r, m in (("dwh", dwh, mwh), ("dwv", dwv, mwv), ("dcw", dcw, mcw)):
        g = got[name].astype(np.float64)
        check_rel(name, g, r, 1e-6, atol=2.0 ** -14 * m)
        assert np.linalg.norm(g - r) <= 1e-5 * np.linalg.norm(r), name
    return stats


def oracle_bwd(inp, saved):
    args = [f64(inp[x]) for x in ("dY", "H", "k", "v")]
    args += [inp[x].astype(np.float64) for x in ("wh", "wv", "cw")]
    args += [f64(saved["vhat"])] + [saved[x].astype(np.float64) for x in ("alpha", "rh", "rk", "rv")]
    return oracle.gateconv_bwd_f64(*args, mags=True)


# M, T, d: several chunks with a ragged last one and chunks that cross sequence
# boundaries (at d = 512 also with 16-row chunks); sequences shorter than the
# conv window; a single row; every supported width, 512 to 5120 in steps of
# 512 (each has its own kernels; 4608 runs 9 columns a thread); and more than
# 512 workgroups (563 at d = 512, 625 at d = 2048), where the weight gradients
# are summed in two levels and the last block of 64 partial rows is ragged.
SHAPES = [(2, 37, 5120), (3, 5, 1024), (1, 1, 512), (5, 300, 2048), (7, 3, 3072), (1, 2, 4096), (2, 700, 1536),
          (2, 70, 4608), (3, 33, 2560), (1, 129, 3584), (2, 45, 512), (3, 3000, 512), (1, 20000, 2048),
          # many sequences no longer than the conv window: every chunk crosses hundreds of sequence
          # starts and every row's dc window runs past its sequence's end
          (2000, 1, 5120), (1200, 2, 1024), (600, 4, 2560)]


@pytest.mark.parametrize("M,T,d", SHAPES)
def test_gateconv_fwd_parity(gpu, M, T, d):
    inp = synth.gateconv_inputs(M, T, d, seed=M * 1000 + T, edge=True)
    check_fwd(inp, run_fwd(inp, gpu), oracle_fwd(inp))


@pytest.mark.parametrize("M,T,d", SHAPES)
def test_gateconv_bwd_parity(gpu, M, T, d):
    inp = synth.gateconv_inputs(M, T, d, seed=M * 1000 + T + 7, edge=True)
    saved = rounded_saved(oracle_fwd(inp))
    check_bwd(run_bwd(inp, saved, gpu), oracle_bwd(inp, saved))


@pytest.mark.parametrize("eps", [1e-3, 0.25])
def test_gateconv_other_eps(gpu, eps):
    """The norms' eps is a runtime argument (the page's default is 1e-6):
    other values reach the kernels' rrms_h, rrms_k and rrms_v, checked in
    full against the oracle with the same eps, and the backward runs on
    that forward's saved tensors."""
    inp = synth.gateconv_inputs(2, 45, 1536, seed=31)
    ref = oracle_fwd(inp, eps=eps)
    check_fwd(inp, run_fwd(inp, gpu, eps=eps), ref)
    saved = rounded_saved(ref)
    check_bwd(run_bwd(inp, saved, gpu), oracle_bwd(inp, saved))


def test_gateconv_bwd_from_gpu_saved(gpu):
    """Forward then backward on the GPU, the oracle's backward fed the GPU's
    own saved tensors: the saved layout is what the backward reads."""
    inp = synth.gateconv_inputs(3, 130, 5120, seed=77, edge=True)
    f = run_fwd(inp, gpu)
    saved = {"vhat": f["vhat"], "alpha": f["alpha"], "rh": f["rh"], "rk": f["rk"], "rv": f["rv"]}
    check_bwd(run_bwd(inp, saved, gpu), oracle_bwd(inp, saved))


def test_gateconv_sequences_are_independent(gpu):
    """One call over M sequences writes, per sequence, the same bits as M calls
    over one sequence each (chunks cross sequence starts in the first, not in
    the second); the weight gradients agree to rounding."""
    M, T, d = 3, 45, 1024
    inp = synth.gateconv_inputs(M, T, d, seed=5)
    saved = rounded_saved(oracle_fwd(inp))
    whole_f = run_fwd(inp, gpu)
    whole_b = run_bwd(inp, saved, gpu)
    sums = {x: 0.0 for x in ("dwh", "dwv", "dcw")}
    for m in range(M):
        one = {x: (inp[x][m:m + 1] if inp[x].ndim == 3 else inp[x]) for x in inp}
        sv = {x: saved[x][m:m + 1] for x in saved}
        f = run_fwd(one, gpu)
        b = run_bwd(one, sv, gpu)
        for x in ("Y", "vhat", "alpha", "rh", "rk", "rv"):
            assert np.array_equal(f[x].view(np.uint8), whole_f[x][m:m + 1].view(np.uint8)), x
        for x in ("dH", "dk", "dv"):
            assert np.array_equal(b[x], whole_b[x][m:m + 1]), x
        for x in sums:
            sums[x] = sums[x] + b[x].astype(np.float64)
    for x in sums:
        np.testing.assert_allclose(whole_b[x], sums[x], rtol=1e-5, atol=1e-5 * np.abs(sums[x]).max())


def test_gateconv_bwd_deterministic(gpu):
    inp = synth.gateconv_inputs(2, 600, 5120, seed=11)
    saved = rounded_saved(oracle_fwd(inp))
    a, b = run_bwd(inp, saved, gpu, repeat=2)
    for x in a:
        assert np.array_equal(a[x].view(np.uint8), b[x].view(np.uint8)), x


@pytest.mark.parametrize("d", [5120, 2560, 1536])
def test_gateconv_full_size(gpu, d):
    """M=4 sequences of T=4096 tokens, every output against the oracle: at
    d=5120 the benchmarked workload in the launch configuration the benchmark
    times; at d=2560 and 1536 the backward's 256 x 10 and 768 x 2 column maps
    over 512 workgroups, two resident per CU."""
    M, T = 4, 4096
    inp = synth.gateconv_inputs(M, T, d, seed=2024)
    ref = oracle_fwd(inp)
    st = check_fwd(inp, run_fwd(inp, gpu), ref)
    print(f"gateconv fwd full size d={d}: Y bit-equal to rounded oracle {st['bit_equal_to_rounded_oracle']}/{st['n']}")
    saved = rounded_saved(ref)
    del ref
    check_bwd(run_bwd(inp, saved, gpu), oracle_bwd(inp, saved))


def test_gateconv_graph_capture_replays_match_eager(gpu):
    """Forward + backward (four kernels) captured once in a HIP graph and
    replayed four times, with outputs and workspace poisoned and unrelated
    eager work between replays; every replay equals the eager result."""
    import torch
    import memory_bound_engram_amd as eg
    from gpu_util import poison
    M, T, d = 2, 150, 2048
    inp = synth.gateconv_inputs(M, T, d, seed=21)
    args = {x: dev(inp[x], gpu) for x in inp}
    outs = {x: torch.empty((M, T, d), dtype=torch.bfloat16, device=gpu) for x in ("Y", "vhat", "dH", "dk", "dv")}
    outs.update({x: torch.empty((M, T), dtype=torch.float32, device=gpu) for x in ("alpha", "rh", "rk", "rv")})
    outs.update({"dwh": torch.empty(d, dtype=torch.float32, device=gpu),
                 "dwv": torch.empty(d, dtype=torch.float32, device=gpu),
                 "dcw": torch.empty((4, d), dtype=torch.float32, device=gpu)})
    ws = torch.empty(eg.engram_gateconv_bwd_workspace_bytes(M, T, d), dtype=torch.uint8, device=gpu)
    o = outs

    def step():
        eg.engram_gateconv_fwd(args["H"], args["k"], args["v"], args["wh"], args["wv"], args["cw"], o["Y"],
                               o["vhat"], o["alpha"], o["rh"], o["rk"], o["rv"])
        eg.engram_gateconv_bwd(args["dY"], args["H"], args["k"], args["v"], args["wh"], args["wv"], args["cw"],
                               o["vhat"], o["alpha"], o["rh"], o["rk"], o["rv"], o["dH"], o["dk"], o["dv"], o["dwh"],
                               o["dwv"], o["dcw"], ws)

    step()
    torch.cuda.synchronize()
    ref = {x: t.clone() for x, t in outs.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        for t in list(outs.values()) + [ws]:
            poison(t)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, t in outs.items():
            assert torch.equal(ref[x].view(torch.uint8), t.view(torch.uint8)), f"replay {r}: {x} differs"
        torch.ones(1 << 20, device=gpu).cumsum(0)  # unrelated eager work between replays


def test_gateconv_max_rows(gpu):
    """The largest accepted call, M*T = 4,194,304 rows (M = 1024 sequences of
    T = 4096, d = 512): 512-row chunks, 8192 workgroups, 8192 partial blocks in
    the reduce.  Every sequence holds the same data, so every sequence's
    outputs must equal the first one's bit for bit (all sequences split into
    chunks the same way), the first one's must match the oracle, and each
    weight gradient must be M times the oracle's for one sequence."""
    import torch
    import memory_bound_engram_amd as eg
    from gpu_util import u16
    M, T, d = 1024, 4096, 512
    assert M * T == eg.GATECONV_ROWS_MAX
    one = synth.gateconv_inputs(1, T, d, seed=99)
    big = {x: dev(one[x], gpu).expand(M, T, d).contiguous() for x in ("H", "k", "v", "dY")}
    wh, wv, cw = dev(one["wh"], gpu), dev(one["wv"], gpu), dev(one["cw"], gpu)
    Y, vhat = empty_bf16((M, T, d), gpu), empty_bf16((M, T, d), gpu)
    al, rh, rk, rv = (empty_f32((M, T), gpu) for _ in range(4))
    eg.engram_gateconv_fwd(big["H"], big["k"], big["v"], wh, wv, cw, Y, vhat, al, rh, rk, rv, eps=EPS)
    dH, dk, dv = (empty_bf16((M, T, d), gpu) for _ in range(3))
    dwh, dwv, dcw = empty_f32((d,), gpu), empty_f32((d,), gpu), empty_f32((4, d), gpu)
    ws = torch.empty(eg.engram_gateconv_bwd_workspace_bytes(M, T, d), dtype=torch.uint8, device=gpu)
    eg.engram_gateconv_bwd(big["dY"], big["H"], big["k"], big["v"], wh, wv, cw, vhat, al, rh, rk, rv,
                           dH, dk, dv, dwh, dwv, dcw, ws)
    torch.cuda.synchronize()
    for t in (Y, vhat, al, rh, rk, rv, dH, dk, dv):
        assert torch.equal(t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32),
                           (t[:1].view(torch.int16) if t.dtype == torch.bfloat16 else t[:1].view(torch.int32))
                           .expand_as(t)), "sequences differ"
    got_f = {"Y": u16(Y[:1]), "vhat": u16(vhat[:1]), "alpha": al[:1].cpu().numpy(), "rh": rh[:1].cpu().numpy(),
             "rk": rk[:1].cpu().numpy(), "rv": rv[:1].cpu().numpy()}
    check_fwd(one, got_f, oracle_fwd(one))
    saved = {"vhat": got_f["vhat"], "alpha": got_f["alpha"], "rh": got_f["rh"], "rk": got_f["rk"], "rv": got_f["rv"]}
    ref = oracle_bwd(one, saved)
    got_b = {"dH": u16(dH[:1]), "dk": u16(dk[:1]), "dv": u16(dv[:1]), "dwh": dwh.cpu().numpy() / M,
             "dwv": dwv.cpu().numpy() / M, "dcw": dcw.cpu().numpy() / M}
    check_bwd(got_b, ref)

"""GPU parity of routing, grouping and whole MoE layers (sparse and dense paths)
against the fp64 oracle, through the C ABI."""
import os

import numpy as np
import pytest
import torch

import activation_sparse_expert_amd as moe
import oracle
import synth
from gpu_helpers import (DEV, HostExpert, check_mask, check_route, check_y, run_layer, say,
                         to_dev_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


# ------------------------------------------------------------------ router



@pytest.mark.parametrize("T,d,E,k,renorm,xdt,zipf,xscale", [
    (1, 4096, 8, 2, True, "f16", False, 1 / 64),
    (16, 4096, 8, 2, True, "f16", False, 1 / 64),
    (64, 2048, 64, 6, True, "f16", True, 1.0),
    (256, 6144, 8, 2, True, "bf16", False, 1 / 64),
    (33, 512, 16, 4, False, "f32", False, 1.0),
    (5, 256, 7, 7, True, "f16", False, 1.0),
    (300, 1024, 128, 8, True, "f16", True, 1.0),
    # grouping: more than 8 x 512 pairs (later chunks reload their experts);
    # 1024 experts (the lane masks take the workgroup past 64 KB of LDS), also
    # for a single token, grouped by its own workgroup
    (700, 256, 128, 8, True, "f16", True, 1.0),
    (20, 64, 1024, 4, True, "f16", False, 1.0),
    (1, 64, 1024, 8, True, "bf16", False, 1.0),
])
def test_router(T, d, E, k, renorm, xdt, zipf, xscale):
    xf = synth.tokens_f32(50, T, d, xscale, layer=E)
    Rf = synth.router_f32(50, E, E, d)
    x_bits = xf if xdt == "f32" else synth.to_bits(xf, xdt)
    rdt = "bf16" if xdt == "bf16" else "f16"
    R_bits = synth.to_bits(Rf, rdt)
    bias = synth.zipf_bias(5, E, E, 1.1) if zipf else None
    x = torch.from_numpy(xf).to(DEV) if xdt == "f32" else to_dev_bits(x_bits, xdt)
    R = to_dev_bits(R_bits, rdt)
    b = None if bias is None else torch.from_numpy(bias).to(DEV)
    out = moe.route_topk(x, R, k, renormalize=renorm, bias=b, logits=True)
    torch.cuda.synchronize()
    check_route(x_bits, xdt, R_bits, rdt, E, k, renorm, bias, out, f"router T={T} E={E} k={k}")


@pytest.mark.parametrize("T,d,E,k", [
    (9, 512, 8, 3),         # one workgroup per token computes the logits
    (3, 2048, 64, 6),       # 256 KB of router rows per token: logits kernel over many workgroups
])
def test_router_exact_ties_lowest_index(T, d, E, k):
    Rf = synth.router_f32(51, 0, E, d)
    Rf[5] = Rf[2]
    Rf[7] = Rf[0]
    Rf[6] = Rf[2]
    x_bits = synth.to_f16_bits(synth.tokens_f32(52, T, d, 1.0))
    R_bits = synth.to_f16_bits(Rf)
    out = moe.route_topk(to_dev_bits(x_bits, "f16"), to_dev_bits(R_bits, "f16"), k, logits=True)
    torch.cuda.synchronize()
    lg = out["logits"].cpu().numpy()
    assert np.array_equal(lg[:, 5], lg[:, 2]) and np.array_equal(lg[:, 6], lg[:, 2])
    check_route(x_bits, "f16", R_bits, "f16", E, k, True, None, out, "router ties")
    idx = out["topk_idx"].cpu().numpy()
    for t in range(T):
        row = list(idx[t])
        for a, b in ((2, 5), (2, 6), (5, 6), (0, 7)):
            if a in row and b in row:
                assert row.index(a) < row.index(b)


# ------------------------------------------------------------------ small layers

def build_host_layer(cfg, E, S, d, f, wdt, sparsity, xscale, layer=0):
    experts = [HostExpert(cfg, layer, e, d, f, wdt=wdt) for e in range(E + S)]
    thr = np.array([hx.calibrate(cfg, xscale, sparsity, layer, e) for e, hx in enumerate(experts)],
                   dtype=np.float32)
    return experts, thr


def device_layer(experts, thr, R_bits, rdt, E, S, k, renorm=True, bias=None, dense=False):
    wdt = experts[0].wdt
    d, f = experts[0].d, experts[0].f
    up_q = torch.from_numpy(np.stack([h.up_q for h in experts])).to(DEV)
    up_sz = torch.from_numpy(np.stack([h.up_sz for h in experts]).view(np.int16)).to(DEV)
    gate = to_dev_bits(np.stack([h.gate for h in experts]), wdt)
    down = to_dev_bits(np.stack([h.down for h in experts]), wdt)
    L = moe.Layer(d=d, f=f, E=E, S=S, k=k, renormalize=renorm, router_w=to_dev_bits(R_bits, rdt),
                  up_q=up_q, up_sz=up_sz, gate_t=gate, down=down,
                  thresholds=torch.from_numpy(thr).to(DEV),
                  router_bias=None if bias is None else torch.from_numpy(bias).to(DEV))
    if dense == "gemm":
        # the 256 x 256-tile kernels: up weights in the layer's type, W^down transposed
        L.up_dense = torch.empty((E + S, f, d), dtype=gate.dtype, device=DEV)
        for e in range(E + S):
            moe.materialize_up(up_q[e], up_sz[e], d, gate.dtype, out=L.up_dense[e])
        L.down_dense = moe.transpose_down(down)
    elif dense:
        L.up_dense = torch.empty((E + S, f, d), dtype=torch.bfloat16, device=DEV)
        for e in range(E + S):
            moe.materialize_up_bf16(up_q[e], up_sz[e], d, out=L.up_dense[e])
    return L




def oracle_layer_check(experts, thr, R_bits, rdt, bias, E, S, k, x_bits, y, tr, tokens, dense,
                       what, renorm=True):
    wdt = experts[0].wdt
    sub = x_bits[tokens]
    uq = np.stack([h.up_q for h in experts])
    us = np.stack([h.up_sz for h in experts])
    g = np.stack([h.gate for h in experts])
    dn = np.stack([h.down for h in experts])
    masks_in = None if dense else tr["masks"][tokens]
    y_ref, idx_ref, w_ref, m_ref = oracle.layer_forward(
        sub, wdt, R_bits, rdt, bias, E, k, S, renorm, uq, us, g, dn, wdt, thr, dense=dense,
        topk_in=tr["topk_idx"][tokens], masks_in=masks_in)
    np.testing.assert_allclose(tr["topk_w"][tokens], w_ref, rtol=2e-5, atol=1e-6)
    if not dense:
        # masks against the oracle's own v: recompute per (token, slot)
        for i, t in enumerate(tokens):
            for s in range(k + S):
                e = tr["topk_idx"][t, s] if s < k else E + (s - k)
                v_ref, _, _ = experts[e].oracle_forward(x_bits[t:t + 1], thr[e])
                check_mask(tr["masks"][t, s][None], v_ref, thr[e], f"{what} t={t} slot={s}")
    err = check_y(y[tokens], y_ref, 2e-3, what)
    say(f"{what}: tokens {list(tokens)} max relL2={err:.2e}")


@pytest.mark.parametrize("T,E,S,k,d,f", [(5, 6, 2, 2, 512, 256), (1, 8, 0, 2, 1024, 512),
                                         (12, 4, 1, 4, 2048, 320), (1, 6, 1, 2, 1536, 192),
                                         (7, 4, 0, 2, 3584, 128)])
def test_small_layer_sparse(T, E, S, k, d, f):
    experts, thr = build_host_layer(60, E, S, d, f, "f16", 0.7, 1.0, layer=d)
    R_bits = synth.to_f16_bits(synth.router_f32(60, d, E, d))
    x_bits = synth.to_f16_bits(synth.tokens_f32(61, T, d, 1.0, layer=d))
    L = device_layer(experts, thr, R_bits, "f16", E, S, k)
    y, tr = run_layer(L, to_dev_bits(x_bits, "f16"), moe.PATH_SPARSE)
    check_route(x_bits, "f16", R_bits, "f16", E, k, True, None,
                {"topk_idx": torch.from_numpy(tr["topk_idx"]), "topk_w": torch.from_numpy(tr["topk_w"]),
                 "logits": torch.from_numpy(tr["logits"]),
                 "expert_count": torch.from_numpy(tr["expert_count"]),
                 "expert_offset": torch.from_numpy(np.concatenate([[0], np.cumsum(tr["expert_count"])])),
                 "pair_by_expert": torch.from_numpy(np.argsort(tr["topk_idx"].ravel(), kind="stable"))},
                f"layer router T={T}")
    oracle_layer_check(experts, thr, R_bits, "f16", None, E, S, k, x_bits, y, tr, np.arange(T),
                       False, f"sparse layer T={T} E={E}+{S} k={k} d={d} f={f}")


@pytest.mark.parametrize("T,E,S,k,d,f", [
    (150, 4, 0, 2, 512, 512),    # ~75 tokens per expert: 128-token gate/up passes, one partial
    (9, 6, 1, 2, 1024, 256),     # 64-token passes
    (300, 4, 1, 2, 512, 512),    # ~150 per routed expert, 300 for the shared one: several passes
])
def test_small_layer_dense(T, E, S, k, d, f):
    experts, thr = build_host_layer(62, E, S, d, f, "bf16", 0.7, 1 / 16, layer=d)
    R_bits = synth.to_bf16_bits(synth.router_f32(62, d, E, d))
    x_bits = synth.to_bf16_bits(synth.tokens_f32(63, T, d, 1 / 16, layer=d))
    L = device_layer(experts, thr, R_bits, "bf16", E, S, k, dense=True)
    y, tr = run_layer(L, to_dev_bits(x_bits, "bf16"), moe.PATH_DENSE)
    tokens = np.arange(T) if T <= 16 else np.array([0, 1, 63, 64, 100, T - 1])
    if T > 200:
        tokens = np.concatenate([tokens, [150, 200, 250, 280]])
    oracle_layer_check(experts, thr, R_bits, "bf16", None, E, S, k, x_bits, y, tr, tokens, True,
                       f"dense layer T={T} E={E}+{S} k={k} d={d} f={f}")


@pytest.mark.parametrize("T,E,S,k,d,f,wdt", [
    (150, 4, 0, 2, 512, 512, "bf16"),    # ~75 tokens per expert: one chunk, 3 of 8 row subtiles
    (300, 4, 1, 2, 512, 512, "f16"),     # ~150 per routed expert; the shared one in 2 chunks
    (700, 3, 1, 3, 256, 384, "bf16"),    # 700 per expert: 3 chunks each, every row subtile
    (9, 6, 1, 2, 1024, 256, "f16"),      # a few tokens per expert
    (64, 8, 0, 2, 2048, 1024, "bf16"),   # split of f in the down product
    (120, 8, 1, 2, 512, 256, "f16"),     # 64-row tiles (30 tokens per expert on average):
                                         # the shared expert's 120 tokens in two chunks
    (300, 8, 1, 2, 1024, 512, "bf16"),   # 128-row tiles, three stages (75 per expert on
                                         # average); the shared expert in three chunks
])
def test_small_layer_dense_gemm(T, E, S, k, d, f, wdt):
    """The MFMA GEMM (bf16 and fp16 layers; 256-row tiles, or 64-row tiles
    when the experts average at most 64 tokens) against the oracle's dense
    path: ragged chunks, several chunks per expert, shared experts, and a
    split of f in the down product."""
    experts, thr = build_host_layer(67, E, S, d, f, wdt, 0.7, 1 / 16, layer=d)
    R_bits = synth.to_bits(synth.router_f32(67, d, E, d), wdt)
    x_bits = synth.to_bits(synth.tokens_f32(68, T, d, 1 / 16, layer=d), wdt)
    L = device_layer(experts, thr, R_bits, wdt, E, S, k, dense="gemm")
    y, tr = run_layer(L, to_dev_bits(x_bits, wdt), moe.PATH_DENSE)
    tokens = np.arange(T) if T <= 16 else np.unique(np.array([0, 1, 63, 64, 255, 256, T // 2, T - 1]) % T)
    oracle_layer_check(experts, thr, R_bits, wdt, None, E, S, k, x_bits, y, tr, tokens, True,
                       f"dense GEMM layer {wdt} T={T} E={E}+{S} k={k} d={d} f={f}")
    assert np.isfinite(y).all()


@pytest.mark.parametrize("n,f,d", [(1, 64, 128), (3, 200, 96), (2, 1408, 2048)])
def test_transpose_down_bit_exact(n, f, d):
    a = torch.from_numpy(synth.normal_f32(69, (n, f, d), 0.02)).half().to(DEV)
    t = moe.transpose_down(a)
    torch.cuda.synchronize()
    assert torch.equal(t.cpu(), a.cpu().transpose(1, 2).contiguous())


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16])
def test_materialize_up_matches_oracle(dt):
    d, f = 2048, 48
    w = synth.normal_f32(4243, (f, d), 0.02)
    q_ref, sz_ref = oracle.pack_up_int2(w)
    out = moe.materialize_up(torch.from_numpy(q_ref).to(DEV),
                             torch.from_numpy(sz_ref.view(np.int16)).to(DEV), d, dt)
    torch.cuda.synchronize()
    exact = oracle.dequant_up(q_ref, sz_ref, d)
    if dt == torch.float16:
        ref = exact.astype(np.float16).view(np.uint16)
    else:
        ref = oracle.materialize_up_bf16(q_ref, sz_ref, d)
    assert np.array_equal(out.cpu().view(torch.int16).numpy().view(np.uint16), ref)


@pytest.mark.parametrize("T,E,S,k,d,f,expect", [
    (9, 6, 1, 2, 1024, 256, "sparse"),       # 18 routed pairs < 8 per expert
    (150, 4, 0, 2, 512, 512, "dense"),       # 75 per expert
])
def test_layer_auto_path(T, E, S, k, d, f, expect):
    """MOE_PATH_AUTO takes the dense path from 8 routed tokens per expert on
    average (bf16 layer with dense up weights), else the sparse path: its
    output is bit-identical to the path it names."""
    experts, thr = build_host_layer(64, E, S, d, f, "bf16", 0.7, 1 / 16, layer=d)
    R_bits = synth.to_bf16_bits(synth.router_f32(64, d, E, d))
    x_bits = synth.to_bf16_bits(synth.tokens_f32(65, T, d, 1 / 16, layer=d))
    L = device_layer(experts, thr, R_bits, "bf16", E, S, k, dense=True)
    x = to_dev_bits(x_bits, "bf16")
    y_auto, _ = run_layer(L, x, moe.PATH_AUTO, want_masks=False)
    named = moe.PATH_DENSE if expect == "dense" else moe.PATH_SPARSE
    y_named, _ = run_layer(L, x, named, want_masks=False)
    other = moe.PATH_SPARSE if expect == "dense" else moe.PATH_DENSE
    y_other, _ = run_layer(L, x, other, want_masks=False)
    assert np.array_equal(y_auto, y_named), f"AUTO at T={T} is not the {expect} path"
    assert not np.array_equal(y_auto, y_other)


@pytest.mark.parametrize("wdt,T,expect", [("f16", 1, "sparse"), ("f16", 4, "sparse"),
                                           ("f16", 24, "dense"), ("bf16", 4, "sparse"),
                                           ("bf16", 24, "dense")])
def test_layer_auto_gemm_per_call(wdt, T, expect):
    """MOE_PATH_AUTO on a layer with the GEMM weights decides per call from
    the expected bytes of both paths (16 routed top-2 + 1 shared, d=512,
    f=256, density 0.3: sparse at 1 and 4 tokens, dense at 24).  Its output
    is bit-identical to the path it names and differs from the other, and the
    exported per-expert flags are all-or-none: every expert with tokens on a
    dense call, none on a sparse one (one token included, which is routed
    inside the expert kernel without the grouping step)."""
    E, S, k, d, f = 16, 1, 2, 512, 256
    experts, thr = build_host_layer(74, E, S, d, f, wdt, 0.7, 1.0, layer=d)
    R_bits = synth.to_bits(synth.router_f32(74, d, E, d), wdt)
    x_bits = synth.to_bits(synth.tokens_f32(75, T, d, 1.0, layer=d), wdt)
    L = device_layer(experts, thr, R_bits, wdt, E, S, k, dense="gemm")
    L.density = 0.3
    assert L.auto_dense_min(T) == (1 if expect == "dense" else 0)
    x = to_dev_bits(x_bits, wdt)
    flags = torch.full((E,), 7, dtype=torch.uint8, device=DEV)
    cnt_d = torch.empty(E, dtype=torch.int32, device=DEV)
    y_auto = moe.layer_forward(L, x, path=moe.PATH_AUTO,
                               trace=dict(expert_dense=flags, expert_count=cnt_d))
    torch.cuda.synchronize()
    y_auto = y_auto.cpu().numpy()
    named = moe.PATH_DENSE if expect == "dense" else moe.PATH_SPARSE
    other = moe.PATH_SPARSE if expect == "dense" else moe.PATH_DENSE
    y_named, _ = run_layer(L, x, named, want_masks=False)
    y_other, _ = run_layer(L, x, other, want_masks=False)
    assert np.array_equal(y_auto, y_named), f"AUTO at T={T} is not the {expect} path"
    assert not np.array_equal(y_auto, y_other)
    cnt, fl = cnt_d.cpu().numpy(), flags.cpu().numpy()
    want = (cnt > 0) if expect == "dense" else np.zeros(E, bool)
    assert np.array_equal(fl, want.astype(np.uint8)), (cnt, fl)
    say(f"AUTO per call {wdt} T={T}: {expect}, counts {cnt.tolist()}")


def test_layer_mixed_graph_replay():
    """MOE_PATH_MIXED runs its GEMMs on a library stream forked from the
    caller's stream and joined before the reduce.  Captured in a HIP graph
    (three calls on different tokens sharing one workspace) and replayed three
    times, with eager calls on the same workspace between the replays, every
    replay reproduces the eager outputs bit for bit."""
    E, S, k, d, f, T = 16, 1, 4, 512, 256, 64
    experts, thr = build_host_layer(70, E, S, d, f, "f16", 0.7, 1.0, layer=d)
    R_bits = synth.to_bits(synth.router_f32(70, d, E, d), "f16")
    bias = synth.zipf_bias(71, d, E, 1.1)
    L = device_layer(experts, thr, R_bits, "f16", E, S, k, bias=bias, dense="gemm")
    L.density = 0.3
    assert 1 < L.mixed_dense_min(T) <= T
    xs = [to_dev_bits(synth.to_bits(synth.tokens_f32(76 + i, T, d, 1.0, layer=d), "f16"), "f16")
          for i in range(3)]
    ws = moe.new_workspace(L.workspace_bytes(T))
    ys = torch.zeros((3, T, d), dtype=torch.float32, device=DEV)
    flags = torch.zeros((3, E), dtype=torch.uint8, device=DEV)
    for i in range(3):
        moe.layer_forward(L, xs[i], path=moe.PATH_MIXED, y=ys[i], ws=ws,
                          trace=dict(expert_dense=flags[i]))
    torch.cuda.synchronize()
    y_eager = ys.cpu().numpy().copy()
    fl = flags.cpu().numpy()
    assert fl.any() and not fl.all(), f"not a mixed call: {fl.tolist()}"
    y_dense, _ = run_layer(L, xs[0], moe.PATH_DENSE, want_masks=False)
    assert not np.array_equal(y_eager[0], y_dense)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(3):
            moe.layer_forward(L, xs[i], path=moe.PATH_MIXED, y=ys[i], ws=ws)
    for rep in range(3):
        ys.fill_(7.0)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        stream.synchronize()
        assert np.array_equal(ys.cpu().numpy(), y_eager), f"replay {rep}"
        moe.layer_forward(L, xs[2], path=moe.PATH_MIXED, y=ys[0], ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(ys[0].cpu().numpy(), y_eager[2]), f"eager call after replay {rep}"
    say("MIXED graph replays reproduce the eager outputs bit for bit")


def test_layer_mixed_two_host_threads():
    """Two host threads make MOE_PATH_MIXED calls at the same time, each on
    its own stream and workspace (the binding's foreign calls release the
    interpreter lock).  Both share the device's library stream and fork
    events, which the library serialises; every output equals the one the
    same call gives alone."""
    import threading
    E, S, k, d, f, T = 16, 1, 4, 512, 256, 64
    experts, thr = build_host_layer(70, E, S, d, f, "f16", 0.7, 1.0, layer=d)
    R_bits = synth.to_bits(synth.router_f32(70, d, E, d), "f16")
    bias = synth.zipf_bias(71, d, E, 1.1)
    L = device_layer(experts, thr, R_bits, "f16", E, S, k, bias=bias, dense="gemm")
    L.density = 0.3
    xs = [to_dev_bits(synth.to_bits(synth.tokens_f32(80 + i, T, d, 1.0, layer=d), "f16"), "f16")
          for i in range(2)]
    want = []
    for i in range(2):
        y = moe.layer_forward(L, xs[i], path=moe.PATH_MIXED)
        torch.cuda.synchronize()
        want.append(y.cpu().numpy())
    assert not np.array_equal(want[0], want[1])
    n = 20
    outs = [torch.zeros((n, T, d), dtype=torch.float32, device=DEV) for _ in range(2)]
    wss = [moe.new_workspace(L.workspace_bytes(T)) for _ in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]
    torch.cuda.synchronize()                    # the buffers are filled before the threads start
    errors = []

    def worker(i):
        try:
            torch.cuda.set_device(0)
            with torch.cuda.stream(streams[i]):
                for j in range(n):
                    moe.layer_forward(L, xs[i], path=moe.PATH_MIXED, y=outs[i][j], ws=wss[i])
            streams[i].synchronize()
        except Exception as exc:                 # reported below
            errors.append(repr(exc))

    th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        got = outs[i].cpu().numpy()
        for j in range(n):
            assert np.array_equal(got[j], want[i]), f"thread {i} call {j}"
    say(f"MIXED from two host threads: {2 * n} calls, all bit-identical to the single calls")


def test_layer_mixed_first_call_under_capture():
    """A process whose first MOE_PATH_MIXED call is captured in a graph (the
    library cannot create its stream then) runs that call in order on the
    capturing stream; its replays equal the later forked eager calls.  Run in
    a fresh child process, since this process already holds the stream."""
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    r = subprocess.run([sys.executable, os.path.join(here, "mixed_first_capture.py")],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    say(r.stdout.strip().splitlines()[-1])


@pytest.mark.parametrize("wdt,T,k", [("f16", 64, 4), ("bf16", 64, 4), ("f16", 160, 2)])
def test_layer_mixed_per_expert(wdt, T, k):
    """MOE_PATH_MIXED with dense weights chooses the path per expert in one call:
    under a Zipf-skewed router the hot experts (at least moe_mixed_dense_min
    tokens) and the shared expert take the dense MFMA path, the others the
    sparse kernel.  The exported per-expert flags follow that rule from the
    call's counts, and y matches the oracle run with the same per-expert
    paths (the sparse experts fed the masks of a sparse-path call of the same
    tokens, which the chunking makes identical).  At 160 tokens the hot
    experts hold more than one 64-row dense chunk."""
    E, S, d, f = 16, 1, 512, 256
    experts, thr = build_host_layer(70, E, S, d, f, wdt, 0.7, 1.0, layer=d)
    R_bits = synth.to_bits(synth.router_f32(70, d, E, d), wdt)
    bias = synth.zipf_bias(71, d, E, 1.1)
    x_bits = synth.to_bits(synth.tokens_f32(72, T, d, 1.0, layer=d), wdt)
    L = device_layer(experts, thr, R_bits, wdt, E, S, k, bias=bias, dense="gemm")
    L.density = 0.3
    nstar = L.mixed_dense_min(T)
    assert 1 < nstar <= T, nstar
    x = to_dev_bits(x_bits, wdt)
    flags = torch.zeros(E, dtype=torch.uint8, device=DEV)
    idx_d = torch.empty((T, k), dtype=torch.int32, device=DEV)
    cnt_d = torch.empty(E, dtype=torch.int32, device=DEV)
    w_d = torch.empty((T, k), dtype=torch.float32, device=DEV)
    y = moe.layer_forward(L, x, path=moe.PATH_MIXED,
                          trace=dict(expert_dense=flags, topk_idx=idx_d, expert_count=cnt_d,
                                     topk_w=w_d))
    torch.cuda.synchronize()
    cnt = cnt_d.cpu().numpy()
    fl = flags.cpu().numpy()
    assert np.array_equal(fl, (cnt >= nstar).astype(np.uint8)), (cnt, fl, nstar)
    assert fl.any() and not fl[cnt > 0].all(), f"not a mixed call: counts {cnt.tolist()} n*={nstar}"
    if T > 64:
        assert cnt.max() > 64, "no expert spans several 64-row dense chunks"
    # the sparse experts' masks, from a sparse-path call of the same tokens
    ys, tr = run_layer(L, x, moe.PATH_SPARSE)
    assert np.array_equal(tr["topk_idx"], idx_d.cpu().numpy())
    dense_experts = np.concatenate([fl, np.ones(S, np.uint8) * (T >= nstar)]).astype(np.uint8)
    uq = np.stack([h.up_q for h in experts])
    us = np.stack([h.up_sz for h in experts])
    g = np.stack([h.gate for h in experts])
    dn = np.stack([h.down for h in experts])
    tokens = np.unique(np.array([0, 1, 17, 40, 63, T - 1, T // 2]) % T)
    y_ref, _, w_ref, _ = oracle.layer_forward(
        x_bits[tokens], wdt, R_bits, wdt, bias, E, k, S, True, uq, us, g, dn, wdt, thr,
        topk_in=tr["topk_idx"][tokens], masks_in=tr["masks"][tokens], dense_experts=dense_experts)
    err = check_y(y.cpu().numpy()[tokens], y_ref, 2e-3, f"MIXED per-expert layer {wdt}")
    say(f"MIXED per-expert {wdt}: n*={nstar}, dense experts {np.flatnonzero(fl).tolist()} "
        f"(counts {cnt.tolist()}), shared dense {bool(T >= nstar)}, max relL2 {err:.2e}")


def test_layer_hot_expert_many_chunks():
    """A router bias sends nearly every token to expert 3, which then holds
    about T/tb chunks of the sparse grid with a ragged last one, while the
    other experts hold one or two each and the shared expert's T tokens split
    into chunks as well; sampled tokens from the first, middle and last chunks
    are checked against the oracle."""
    T, E, S, k, d, f = 150, 6, 1, 2, 512, 256
    experts, thr = build_host_layer(66, E, S, d, f, "f16", 0.7, 1.0, layer=d)
    R_bits = synth.to_f16_bits(synth.router_f32(66, d, E, d))
    bias = np.zeros(E, dtype=np.float32)
    bias[3] = 2.0
    x_bits = synth.to_f16_bits(synth.tokens_f32(67, T, d, 1.0, layer=d))
    L = device_layer(experts, thr, R_bits, "f16", E, S, k, bias=bias)
    y, tr = run_layer(L, to_dev_bits(x_bits, "f16"), moe.PATH_SPARSE)
    hist = np.bincount(tr["topk_idx"].ravel(), minlength=E)
    say(f"hot expert: tokens per expert {hist.tolist()}")
    assert hist[3] >= 140
    hot = np.flatnonzero((tr["topk_idx"] == 3).any(axis=1))
    cold = np.flatnonzero(~(tr["topk_idx"] == 3).any(axis=1))
    tokens = np.unique(np.concatenate([hot[:5], hot[len(hot) // 2:len(hot) // 2 + 2], hot[-3:], cold[:2]]))
    oracle_layer_check(experts, thr, R_bits, "f16", bias, E, S, k, x_bits, y, tr, tokens, False,
                       f"hot expert layer T={T} E={E}+{S} k={k}")


def test_layer_repeatable_and_workspace_clean():
    T, E, S, k, d, f = 7, 8, 1, 2, 512, 128
    experts, thr = build_host_layer(64, E, S, d, f, "f16", 0.6, 1.0)
    R_bits = synth.to_f16_bits(synth.router_f32(64, 0, E, d))
    x = to_dev_bits(synth.to_f16_bits(synth.tokens_f32(65, T, d, 1.0)), "f16")
    L = device_layer(experts, thr, R_bits, "f16", E, S, k)
    ws = moe.new_workspace(L.workspace_bytes(T))
    masks = []
    for _ in range(3):
        tr = dict(masks=torch.empty((T, k + S, f), dtype=torch.uint8, device=DEV))
        y = moe.layer_forward(L, x, trace=tr, ws=ws)
        torch.cuda.synchronize()
        masks.append(tr["masks"].cpu().numpy())
    assert all(np.array_equal(masks[0], m) for m in masks[1:])
    # the accumulator and counters are zero again after every call
    lw = moe.workspace_size(moe.OP_LAYER, T, d, f, E, k, S)
    assert ws.numel() >= lw

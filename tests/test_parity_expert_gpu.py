"""GPU parity of the single-expert path (Algorithm 1) and the INT2 packer
against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import activation_sparse_expert_amd as moe
import oracle
import synth
from gpu_helpers import (DEV, Guarded, HostExpert, check_bits_exports, check_mask, check_y,
                         dev_bits, guarded_workspace, say, to_dev_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def run_expert(hx: HostExpert, thr, x_bits, *, T=None, scale=None, ydt=torch.float32,
               y_init=None, accumulate=False):
    """One expert call with y, every export and the workspace canary-guarded;
    the bitmask and nnz exports are checked against the byte mask."""
    ex = hx.to_device(thr)
    x = to_dev_bits(x_bits, hx.wdt)
    T = x.shape[0]
    mask = Guarded((T, hx.f), torch.uint8)
    v = Guarded((T, hx.f), torch.float32)
    bits = Guarded((T, hx.f // 64), torch.int64)
    nnz = Guarded((T,), torch.int32)
    y = Guarded((T, hx.d), y_init.dtype if y_init is not None else ydt, fill=y_init)
    ws = guarded_workspace(moe.workspace_size(moe.OP_EXPERT, T, hx.d, hx.f))
    ts = None if scale is None else torch.tensor(scale, dtype=torch.float32, device=DEV)
    moe.expert_forward_sparse(ex, x, y=y.t, token_scale=ts, accumulate=accumulate,
                              mask_out=mask.t, v_out=v.t, mask_bits=bits.t, nnz=nnz.t, ws=ws.t)
    torch.cuda.synchronize()
    for g, n in ((mask, "mask"), (v, "v"), (bits, "mask_bits"), (nnz, "nnz"), (y, "y"),
                 (ws, "workspace")):
        g.check(f"expert d={hx.d} f={hx.f} T={T} {n}")
    m = mask.t.cpu().numpy()
    check_bits_exports(m, bits.t, nnz.t, f"expert d={hx.d} f={hx.f} T={T}")
    return y.t.float().cpu().numpy(), m, v.t.cpu().numpy()


def check_case(hx, thr, x_bits, what, **kw):
    y, m, v = run_expert(hx, thr, x_bits, **kw)
    v_ref, m_ref, _ = hx.oracle_forward(x_bits, thr)
    ndiff = check_mask(m, v_ref, thr, what)
    scale = kw.get("scale")
    _, _, y_ref = hx.oracle_forward(x_bits, thr, mask_in=m,
                                    scale=None if scale is None else np.asarray(scale, np.float64))
    if kw.get("y_init") is not None and kw.get("accumulate"):
        y_ref = y_ref + kw["y_init"].float().cpu().numpy()
    tol = 2e-3 if kw.get("ydt", torch.float32) == torch.float32 else 1e-2
    err = check_y(y, y_ref, tol, what)
    vscale = np.abs(v_ref).max()
    assert np.abs(v - v_ref).max() <= 1e-5 * vscale + 1e-9, what
    say(f"{what}: nnz/token={m.sum(1).mean():.1f} band-diffs={ndiff} max relL2={err:.2e}")
    return y, m, v


# ------------------------------------------------------------------ packer

@pytest.mark.parametrize("d,f,src", [(256, 64, "f32"), (4096, 96, "f32"), (2048, 40, "f16"),
                                     (6144, 16, "bf16")])
def test_pack_matches_oracle_bit_exact(d, f, src):
    w = synth.normal_f32(777 + d, (f, d), 0.02)
    # edge groups: constant, all zero, signed zeros, exactly representable steps
    w[0, :64] = 0.25
    w[1, :64] = 0.0
    w[1, 64:128] = -0.0
    w[2, :64] = (2.0 ** -7) * (np.arange(64) % 4 - 1.5)
    if src == "f16":
        w = w.astype(np.float16).astype(np.float32)
        wd = torch.from_numpy(w).half().to(DEV)
    elif src == "bf16":
        wd = torch.from_numpy(w).to(torch.bfloat16).to(DEV)
        w = wd.float().cpu().numpy()
    else:
        wd = torch.from_numpy(w).to(DEV)
    q, sz = moe.pack_up_int2(wd)
    torch.cuda.synchronize()
    q_ref, sz_ref = oracle.pack_up_int2(w)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sz.cpu().numpy().view(np.uint16), sz_ref)


def test_materialize_bf16_matches_oracle():
    d, f = 2048, 48
    w = synth.normal_f32(4242, (f, d), 0.02)
    q_ref, sz_ref = oracle.pack_up_int2(w)
    q = torch.from_numpy(q_ref).to(DEV)
    sz = torch.from_numpy(sz_ref.view(np.int16)).to(DEV)
    out = moe.materialize_up_bf16(q, sz, d)
    torch.cuda.synchronize()
    assert np.array_equal(dev_bits(out), oracle.materialize_up_bf16(q_ref, sz_ref, d))


# ------------------------------------------------------------------ tiny expert

@pytest.fixture(scope="module")
def tiny():
    c = synth.CONFIGS[synth.CFG_TINY]
    hx = HostExpert(synth.CFG_TINY, 0, 0, c["d"], c["f"])
    t50 = hx.calibrate(synth.CFG_TINY, c["x_scale"], 0.5)
    x = synth.to_f16_bits(synth.tokens_f32(synth.CFG_TINY, 1, c["d"], c["x_scale"]))
    return hx, t50, x


@pytest.mark.parametrize("which", ["dense", "t50", "inf"])
def test_tiny_expert(tiny, which):
    hx, t50, x = tiny
    thr = {"dense": -1.0, "t50": t50, "inf": np.inf}[which]
    y, m, _ = check_case(hx, thr, x, f"tiny d=256 f=704 {which}")
    if which == "dense":
        assert m.all()
    if which == "inf":
        assert not m.any() and np.all(y == 0.0)


def test_tiny_expert_repeatable(tiny):
    hx, t50, x = tiny
    y1, m1, v1 = run_expert(hx, t50, x)
    y2, m2, v2 = run_expert(hx, t50, x)
    assert np.array_equal(m1, m2) and np.array_equal(v1, v2)
    np.testing.assert_allclose(y1, y2, rtol=1e-6, atol=1e-9)


# ------------------------------------------------------------------ Mixtral-shaped expert

@pytest.fixture(scope="module")
def mixtral():
    c = synth.CONFIGS[synth.CFG_MIXTRAL]
    say("building the d=4096 f=14336 expert on the host")
    hx = HostExpert(synth.CFG_MIXTRAL, 0, 0, c["d"], c["f"])
    thr = {s: hx.calibrate(synth.CFG_MIXTRAL, c["x_scale"], s) for s in (0.5, 0.7, 0.9)}
    thr[0.0] = np.float32(-1.0)
    return hx, thr, c


@pytest.mark.parametrize("sp", [0.0, 0.5, 0.7, 0.9])
def test_mixtral_expert_batch1(mixtral, sp):
    hx, thr, c = mixtral
    x = synth.to_f16_bits(synth.tokens_f32(synth.CFG_MIXTRAL, 1, c["d"], c["x_scale"]))
    _, m, _ = check_case(hx, thr[sp], x, f"d=4096 f=14336 T=1 sparsity {sp}")
    if sp > 0:
        assert abs((1 - m.mean()) - sp) < 0.05


@pytest.mark.parametrize("sp", [0.0, 0.5, 0.7, 0.9])
def test_mixtral_expert_batch4(mixtral, sp):
    """Batch 4 at every sparsity of the workload, 0% (t < 0: every channel of
    every tile active, the heaviest multi-token gather) included."""
    hx, thr, c = mixtral
    x = synth.to_f16_bits(synth.tokens_f32(synth.CFG_MIXTRAL, 4, c["d"], c["x_scale"]))
    _, m, _ = check_case(hx, thr[sp], x, f"d=4096 f=14336 T=4 sparsity {sp}")
    if sp == 0.0:
        assert m.all()


def test_mixtral_expert_infinite_threshold(mixtral):
    hx, thr, c = mixtral
    x = synth.to_f16_bits(synth.tokens_f32(synth.CFG_MIXTRAL, 2, c["d"], c["x_scale"]))
    y, m, _ = run_expert(hx, np.inf, x)
    assert not m.any() and np.all(y == 0.0)


# ------------------------------------------------------------------ shapes and options

@pytest.mark.parametrize("d,f,T,wdt", [
    (64, 128, 1, "f16"), (128, 64, 3, "f16"), (512, 192, 2, "f16"), (1024, 256, 5, "bf16"),
    (2048, 1408, 9, "f16"), (6144, 256, 3, "bf16"), (4096, 320, 17, "f16"), (8192, 128, 2, "bf16"),
    # the widest geometry (4 groups of 64 inputs per lane): d in (8192, 16384]
    (12288, 128, 1, "f16"), (16384, 64, 2, "bf16"), (9216, 192, 3, "f16"),
    # hidden sizes between the geometries' widths: lanes past d/64 groups and
    # threads past d/8 row chunks idle (a multiple of 64 throughout)
    (320, 128, 1, "bf16"), (768, 256, 3, "f16"), (1536, 192, 1, "f16"), (2560, 64, 4, "bf16"),
    (3584, 128, 2, "f16"), (3584, 64, 1, "bf16"), (4160, 64, 1, "f16"), (14336, 64, 1, "bf16"),
])
def test_expert_shapes(d, f, T, wdt):
    hx = HostExpert(90, d, T, d, f, wdt=wdt)
    scale = 1.0 / 16 if d <= 256 else 1.0 / 64
    thr = hx.calibrate(90, scale, 0.7, layer=d)
    x = synth.to_bits(synth.tokens_f32(91, T, d, scale, layer=d), wdt)
    check_case(hx, thr, x, f"d={d} f={f} T={T} {wdt}")


@pytest.mark.parametrize("ydt", [torch.float16, torch.bfloat16])
def test_expert_scale_accumulate_and_output_types(ydt):
    d, f, T = 1024, 512, 3
    hx = HostExpert(92, 0, 0, d, f)
    thr = hx.calibrate(92, 1 / 64, 0.6)
    x = synth.to_f16_bits(synth.tokens_f32(93, T, d, 1 / 64))
    y0 = torch.from_numpy(synth.normal_f32(94, (T, d), 1e-3)).to(ydt).to(DEV)
    check_case(hx, thr, x, f"scaled+accumulate into {ydt}", scale=[0.25, -1.5, 2.0],
               ydt=ydt, y_init=y0, accumulate=True)


def test_workspace_init_and_reuse():
    d, f = 512, 128
    hx = HostExpert(95, 0, 0, d, f)
    ex = hx.to_device(0.0)
    for T in (1, 4):
        x = to_dev_bits(synth.to_f16_bits(synth.tokens_f32(96, T, d, 1 / 16)), "f16")
        ws = moe.new_workspace(moe.workspace_size(moe.OP_EXPERT, T, d, f))
        ws.fill_(0xFF)
        moe.workspace_init(ws)          # zero-fill kernel: makes any buffer usable
        ys = [moe.expert_forward_sparse(ex, x, ws=ws) for _ in range(3)]
        y_ref = moe.expert_forward_sparse(ex, x)
        torch.cuda.synchronize()
        for yy in ys:                   # the workspace stays usable call after call
            torch.testing.assert_close(yy, y_ref, rtol=1e-5, atol=1e-7)


def test_mixtral_graph_replay_launch_config(mixtral):
    """The benchmark's launch configuration: batch-1 calls at 90% sparsity
    sharing one workspace, captured in a HIP graph and replayed.  Every replay
    must reproduce the eager outputs bit for bit (the partial-row reduction
    has a fixed order), and the eager outputs match the oracle."""
    hx, thr, c = mixtral
    ex = hx.to_device(thr[0.9])
    x_bits = synth.to_f16_bits(synth.tokens_f32(synth.CFG_MIXTRAL, 6, c["d"], c["x_scale"],
                                                tensor_id=synth.T_NOISE))
    x = to_dev_bits(x_bits, "f16")
    n = 12
    ws = moe.new_workspace(moe.workspace_size(moe.OP_EXPERT, 1, hx.d, hx.f))
    ys = torch.zeros((n, 1, hx.d), dtype=torch.float32, device=DEV)
    masks = torch.zeros((n, 1, hx.f), dtype=torch.uint8, device=DEV)
    for i in range(n):
        moe.expert_forward_sparse(ex, x[i % 6:i % 6 + 1], y=ys[i], ws=ws, mask_out=masks[i])
    torch.cuda.synchronize()
    y_eager, m_eager = ys.cpu().numpy().copy(), masks.cpu().numpy().copy()
    for i in (0, 5):
        v_ref, _, _ = hx.oracle_forward(x_bits[i:i + 1], thr[0.9])
        check_mask(m_eager[i], v_ref, thr[0.9], f"graph config token {i}")
        _, _, y_ref = hx.oracle_forward(x_bits[i:i + 1], thr[0.9], mask_in=m_eager[i])
        check_y(y_eager[i], y_ref, 2e-3, f"graph config token {i}")
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(n):
            moe.expert_forward_sparse(ex, x[i % 6:i % 6 + 1], y=ys[i], ws=ws, mask_out=masks[i])
    for rep in range(3):
        ys.fill_(7.0)
        masks.fill_(9)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        stream.synchronize()
        assert np.array_equal(ys.cpu().numpy(), y_eager), f"replay {rep}"
        assert np.array_equal(masks.cpu().numpy(), m_eager), f"replay {rep}"
        # eager work on the same workspace between replays
        moe.expert_forward_sparse(ex, x[3:4], y=ys[0], ws=ws)
    say("graph replays reproduce the eager outputs bit for bit")

"""GPU parity of the expert with the up projection at 8, 4 and 1 bits per code
(FloE review, "敏感度分析") against the fp64 oracle, through the C ABI: the
device packer bit-exact, v within fp32 rounding, the mask exact outside the
threshold band, y against the oracle fed the GPU's mask."""
import numpy as np
import pytest
import torch

import activation_sparse_expert_amd as moe
import oracle
import synth
from gpu_helpers import (DEV, TORCH_DT, Guarded, bits_to_f64, check_bits_exports, check_mask,
                         check_y, dev_bits, guarded_workspace, say,
                         to_dev_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def host_expert(cfg, d, f, bits, wdt):
    g, u, dn = synth.expert_weights_f32(cfg, 0, 0, d, f, 0.02)
    up_q, up_sz = oracle.pack_up_bits(u, bits)
    return dict(u=u, up_q=up_q, up_sz=up_sz, gate=synth.to_bits(g, wdt),
                down=synth.to_bits(dn, wdt), d=d, f=f, bits=bits, wdt=wdt)


def device_expert(h, thr):
    return moe.Expert(torch.from_numpy(h["up_q"]).to(DEV),
                      torch.from_numpy(h["up_sz"].view(np.int16)).to(DEV),
                      to_dev_bits(h["gate"], h["wdt"]), to_dev_bits(h["down"], h["wdt"]),
                      float(thr))


def threshold_for(h, x_bits, sparsity):
    W = oracle.dequant_up_bits(h["up_q"], h["up_sz"], h["d"], h["bits"])
    v = bits_to_f64(x_bits, h["wdt"]) @ W.T
    return oracle.calibrate_threshold(np.abs(v), sparsity)


def run_and_check(h, ex, x_bits, thr, what, scale=None):
    T, d, f = x_bits.shape[0], h["d"], h["f"]
    x = to_dev_bits(x_bits, h["wdt"])
    gm = Guarded((T, f), torch.uint8)
    gv = Guarded((T, f), torch.float32)
    gb = Guarded((T, f // 64), torch.int64)
    gn = Guarded((T,), torch.int32)
    gy = Guarded((T, d), torch.float32)
    gw = guarded_workspace(moe.workspace_size(moe.OP_EXPERT_BITS, T, d, f))
    sc = None if scale is None else torch.from_numpy(scale.astype(np.float32)).to(DEV)
    moe.expert_forward_sparse_bits(ex, h["bits"], x, y=gy.t, mask_out=gm.t, v_out=gv.t,
                                   mask_bits=gb.t, nnz=gn.t, token_scale=sc, ws=gw.t)
    torch.cuda.synchronize()
    for g, n in ((gm, "mask"), (gv, "v"), (gb, "mask_bits"), (gn, "nnz"), (gy, "y"),
                 (gw, "workspace")):
        g.check(f"{what} {n}")
    m, v, y = gm.t, gv.t, gy.t
    check_bits_exports(m.cpu().numpy(), gb.t, gn.t, what)
    v_ref, _, _ = oracle.expert_forward(x_bits, h["wdt"], h["up_q"], h["up_sz"], h["gate"],
                                        h["down"], h["wdt"], thr, bits=h["bits"])
    vg = v.cpu().numpy().astype(np.float64)
    scale_v = np.abs(v_ref).max()
    assert np.abs(vg - v_ref).max() <= 1e-5 * scale_v + 1e-7, f"{what}: v"
    mg = m.cpu().numpy()
    nd = check_mask(mg, v_ref, thr, what)
    _, _, y_ref = oracle.expert_forward(x_bits, h["wdt"], h["up_q"], h["up_sz"], h["gate"],
                                        h["down"], h["wdt"], thr, mask_in=mg,
                                        scale=None if scale is None else scale.astype(np.float64),
                                        bits=h["bits"])
    err = check_y(y.cpu().numpy(), y_ref, what=what)
    say(f"{what}: active {mg.mean():.3f}, mask diffs in band {nd}, max relL2 {err:.2e}")
    return y, mg


@pytest.mark.parametrize("bits", [8, 4, 1])
@pytest.mark.parametrize("d,f,wdt", [(512, 320, "f16"), (1024, 192, "bf16"), (2048, 448, "f16")])
def test_pack_bits_matches_oracle_bit_exact(bits, d, f, wdt):
    u = synth.normal_f32(synth.seed_of(20, 0, bits, 1), (f, d), 0.02)
    ub = synth.to_bits(u, wdt)
    uf = bits_to_f64(ub, wdt).astype(np.float32)        # what the device reads
    q_ref, sz_ref = oracle.pack_up_bits(uf, bits)
    q, sz = moe.pack_up_bits(to_dev_bits(ub, wdt), bits)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sz.cpu().numpy().view(np.uint16), sz_ref)


@pytest.mark.parametrize("bits", [8, 4, 1])
@pytest.mark.parametrize("d,f,T,wdt,sp", [(512, 320, 1, "f16", 0.9), (1024, 192, 3, "bf16", 0.7),
                                          (2048, 448, 8, "f16", 0.8), (4096, 256, 2, "bf16", 0.5),
                                          (1024, 576, 13, "f16", 0.7), (2048, 128, 1, "bf16", 0.0),
                                          # between the geometries' widths
                                          (768, 128, 2, "f16", 0.7), (3584, 128, 1, "bf16", 0.9)])
def test_expert_bits_small(bits, d, f, T, wdt, sp):
    h = host_expert(30 + bits, d, f, bits, wdt)
    x_bits = synth.to_bits(synth.normal_f32(synth.seed_of(31, 0, bits, 4), (T, d), 1 / 16), wdt)
    thr = threshold_for(h, x_bits, sp)
    ex = device_expert(h, thr)
    run_and_check(h, ex, x_bits, thr, f"bits={bits} d={d} f={f} T={T} {wdt}")


def test_expert_bits_degenerate_thresholds_scale_and_two_bits():
    d, f, T = 1024, 256, 2
    h = host_expert(40, d, f, 4, "f16")
    x_bits = synth.to_bits(synth.normal_f32(41, (T, d), 1 / 16), "f16")
    # t < 0: every channel; t = inf: none, y exactly 0
    y_all, m_all = run_and_check(h, device_expert(h, -1.0), x_bits, -1.0, "bits=4 t<0")
    assert m_all.all()
    ex = device_expert(h, float("inf"))
    y = moe.expert_forward_sparse_bits(ex, 4, to_dev_bits(x_bits, "f16"))
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0
    # token scale, accumulate and the 16-bit outputs
    thr = threshold_for(h, x_bits, 0.8)
    ex = device_expert(h, thr)
    run_and_check(h, ex, x_bits, thr, "bits=4 scaled", scale=np.array([0.5, -2.0]))
    x = to_dev_bits(x_bits, "f16")
    y1 = moe.expert_forward_sparse_bits(ex, 4, x)
    y2 = y1.clone()
    moe.expert_forward_sparse_bits(ex, 4, x, y=y2, accumulate=True)
    yh = moe.expert_forward_sparse_bits(ex, 4, x, out_dtype=torch.float16)
    torch.cuda.synchronize()
    assert torch.equal(y2, y1 + y1)
    assert torch.equal(yh, y1.half())
    # repeatable bit for bit
    y3 = moe.expert_forward_sparse_bits(ex, 4, x)
    torch.cuda.synchronize()
    assert torch.equal(y1, y3)
    # bits = 2 is the INT2 entry point
    h2 = host_expert(42, d, f, 2, "f16")
    e2 = device_expert(h2, thr)
    ya = moe.expert_forward_sparse_bits(e2, 2, x)
    yb = moe.expert_forward_sparse(e2, x)
    torch.cuda.synchronize()
    assert torch.equal(ya, yb)


@pytest.mark.parametrize("bits", [8, 4, 1])
def test_mixtral_expert_bits(bits):
    """One Mixtral-8x7B-shaped expert (d=4096, f=14336) drawn and packed on the
    device, 90% sparsity, T = 1 and 4; the packer checked bit-exact on sampled
    rows, y on every token against the oracle."""
    d, f = 4096, 14336
    u = synth.device_normal(synth.seed_of(2, 0, 0, synth.T_UP), (f, d), 0.02, DEV)
    g = synth.device_normal(synth.seed_of(2, 0, 0, synth.T_GATE), (f, d), 0.02, DEV, torch.float16)
    dn = synth.device_normal(synth.seed_of(2, 0, 0, synth.T_DOWN), (f, d), 0.02, DEV, torch.float16)
    up_q, up_sz = moe.pack_up_bits(u, bits)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 777, 8191, f - 1])
    q_ref, sz_ref = oracle.pack_up_bits(u[rows].cpu().numpy(), bits)
    assert np.array_equal(up_q[rows].cpu().numpy(), q_ref)
    assert np.array_equal(up_sz[rows].cpu().numpy().view(np.uint16), sz_ref)
    h = dict(up_q=up_q.cpu().numpy(), up_sz=up_sz.cpu().numpy().view(np.uint16),
             gate=dev_bits(g), down=dev_bits(dn), d=d, f=f, bits=bits, wdt="f16")
    del u
    for T in (1, 4):
        x_bits = synth.to_bits(synth.normal_f32(synth.seed_of(2, 0, 0, synth.T_X) + T, (T, d), 1 / 64),
                               "f16")
        thr = threshold_for(h, x_bits, 0.9)
        ex = moe.Expert(up_q, up_sz, g, dn, float(thr))
        run_and_check(h, ex, x_bits, thr, f"mixtral bits={bits} T={T}")

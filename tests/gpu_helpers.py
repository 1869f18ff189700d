"""Shared pieces of the GPU parity tests: seeded experts and layers built on the
host (INT2 bytes from the oracle's packer) or on the device (large shapes), and
the acceptance checks (mask exact outside the threshold band, relative L2 of y
against the oracle fed the GPU's mask)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import activation_sparse_expert_amd as moe
import oracle
import synth

DEV = "cuda"
TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}
REL_L2 = 2e-3           # per token, y against the oracle fed the GPU mask
BAND = 1e-4             # mask entries with ||v| - t| <= BAND * t may differ


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------------------
# Canary-guarded device buffers: every output and workspace handed to the
# library sits between two runs of canary bytes, checked after the call, so a
# write past either end of a buffer fails the test.
# ---------------------------------------------------------------------------
CANARY = 0xA5
GUARD = 4096            # bytes on each side (keeps every alignment the library asks for)


class Guarded:
    """A device tensor of `shape` and `dtype` inside a canary-filled buffer."""

    def __init__(self, shape, dtype, fill=None):
        shape = tuple(int(s) for s in shape)
        esz = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) * esz
        self.n = n
        self.buf = torch.full((GUARD + n + GUARD,), CANARY, dtype=torch.uint8, device=DEV)
        self.t = self.buf[GUARD:GUARD + n].view(dtype).view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def check(self, what=""):
        b = self.buf.cpu().numpy()
        lo, hi = b[:GUARD], b[GUARD + self.n:]
        assert (lo == CANARY).all(), f"{what}: {int((lo != CANARY).sum())} bytes written before the buffer"
        assert (hi == CANARY).all(), f"{what}: {int((hi != CANARY).sum())} bytes written past the buffer"


def guarded_workspace(nbytes):
    """A workspace of exactly `nbytes` (the library's stated size) between canaries."""
    return Guarded((nbytes,), torch.uint8, fill=None)


def bits_of(mask_u8: np.ndarray) -> np.ndarray:
    """[..][f] 0/1 bytes -> [..][f/64] uint64 words, channel 64 i + l at bit l of word i."""
    m = np.ascontiguousarray(mask_u8 != 0)
    packed = np.packbits(m, axis=-1, bitorder="little")          # 8 channels per byte
    return packed.view(np.uint64) if packed.shape[-1] % 8 == 0 else None


def check_bits_exports(mask_u8, bits_dev, nnz_dev, what=""):
    """The bitmask and nnz exports are the byte mask in another form, bit for bit."""
    b = bits_dev.cpu().numpy().view(np.uint64)
    assert np.array_equal(b, bits_of(mask_u8)), f"{what}: bitmask differs from the byte mask"
    assert np.array_equal(nnz_dev.cpu().numpy(), (mask_u8 != 0).sum(-1)), f"{what}: nnz"


def to_dev_bits(bits: np.ndarray, dt: str):
    """uint16 bit patterns -> device tensor of dtype dt (same bytes)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy())
    return t.view(TORCH_DT[dt]).to(DEV)


def dev_bits(t) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class HostExpert:
    """A seeded expert generated on the host; INT2 packing by the oracle."""

    def __init__(self, cfg, layer, e, d, f, wdt="f16", std=0.02):
        g, u, dn = synth.expert_weights_f32(cfg, layer, e, d, f, std)
        self.d, self.f, self.wdt = d, f, wdt
        self.up_q, self.up_sz = oracle.pack_up_int2(u)
        self.gate = synth.to_bits(g, wdt)
        self.down = synth.to_bits(dn, wdt)

    def to_device(self, thr):
        return moe.Expert(
            torch.from_numpy(self.up_q).to(DEV),
            torch.from_numpy(self.up_sz.view(np.int16)).to(DEV),
            to_dev_bits(self.gate, self.wdt), to_dev_bits(self.down, self.wdt), float(thr))

    def calibrate(self, cfg, scale, sparsity, layer=0, expert=0):
        """Threshold at the `sparsity` quantile of |v| over the 64 seeded
        calibration vectors (v from the oracle's dequantised weights)."""
        xc = synth.to_bits(synth.calibration_f32(cfg, self.d, scale, layer, expert), self.wdt)
        xd = bits_to_f64(xc, self.wdt)
        W = oracle.dequant_up(self.up_q, self.up_sz, self.d)
        v = xd @ W.T
        return oracle.calibrate_threshold(np.abs(v), sparsity)

    def oracle_forward(self, x_bits, thr, mask_in=None, scale=None):
        return oracle.expert_forward(x_bits, self.wdt, self.up_q, self.up_sz, self.gate,
                                     self.down, self.wdt, thr, scale=scale, mask_in=mask_in)


def bits_to_f64(bits, dt):
    if dt == "f16":
        return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(
        np.float32).astype(np.float64)


def check_mask(m_gpu, v_oracle, thr, what=""):
    """Mask bit-exact except inside the band around the threshold."""
    m_ref = (np.abs(v_oracle) > float(np.float32(thr))).astype(np.uint8)
    diff = m_gpu != m_ref
    if np.isfinite(thr) and thr > 0:
        band = np.abs(np.abs(v_oracle) - float(thr)) <= BAND * float(thr)
    else:
        band = np.zeros_like(diff)
    bad = diff & ~band
    assert not bad.any(), f"{what}: {int(bad.sum())} mask entries differ outside the band"
    return int(diff.sum())


def rel_l2_rows(y_gpu, y_ref):
    """Per-row relative L2 error; rows whose reference is exactly 0 must be 0."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    out = []
    for a, b in zip(y_gpu, y_ref):
        nb = np.linalg.norm(b)
        if nb == 0.0:
            assert np.all(a == 0.0), "reference row is 0 but the GPU row is not"
            out.append(0.0)
        else:
            out.append(np.linalg.norm(a - b) / nb)
    return np.array(out)


def check_y(y_gpu, y_ref, tol=REL_L2, what=""):
    e = rel_l2_rows(y_gpu, y_ref)
    assert e.max() <= tol, f"{what}: max relative L2 {e.max():.3e} > {tol}"
    return float(e.max())


def check_route(x_bits, xdt, R_bits, rdt, E, k, renorm, bias, out, what):
    """Top-k bit-exact against the oracle except at fp32-vs-fp64 near-ties,
    where it must equal the stable top-k of the GPU's own fp32 logits."""
    ref = oracle.route_topk(x_bits, xdt, R_bits, rdt, E, k, renormalize=renorm, bias=bias)
    idx = out["topk_idx"].cpu().numpy()
    lg = out["logits"].cpu().numpy().astype(np.float64)
    X = bits_to_f64(x_bits, xdt) if xdt != "f32" else np.asarray(x_bits, np.float64)
    Rm = bits_to_f64(R_bits, rdt) if rdt != "f32" else np.asarray(R_bits, np.float64)
    mag = np.abs(X) @ np.abs(Rm).T                     # sum_k |x_k R_ek|
    L = ref["logits"]
    srt = np.sort(L, axis=1)[:, ::-1]
    gap = srt[:, k - 1] - (srt[:, k] if k < E else -np.inf)
    near = gap <= 2.0 ** -16 * mag.max(axis=1)
    own = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    for t in range(idx.shape[0]):
        if near[t]:
            assert np.array_equal(idx[t], own[t]), f"{what}: token {t} near-tie"
        else:
            assert np.array_equal(idx[t], ref["topk_idx"][t]), f"{what}: token {t}"
    np.testing.assert_allclose(lg, L, rtol=1e-4, atol=1e-5 * mag.max())
    w = out["topk_w"].cpu().numpy()
    ok = ~near
    np.testing.assert_allclose(w[ok], ref["topk_w"][ok], rtol=2e-5, atol=1e-6)
    # grouping is fixed exactly by the GPU's own top-k
    flat = idx.ravel()
    cnt = np.bincount(flat, minlength=E)
    assert np.array_equal(out["expert_count"].cpu().numpy(), cnt)
    assert np.array_equal(out["expert_offset"].cpu().numpy(), np.concatenate([[0], np.cumsum(cnt)]))
    assert np.array_equal(out["pair_by_expert"].cpu().numpy(), np.argsort(flat, kind="stable"))
    say(f"{what}: near-ties {int(near.sum())}/{len(near)}")


def run_layer(L, x, path, want_masks=True):
    """One layer call with every output, export and the workspace canary-
    guarded; the bitmask and nnz exports are checked against the byte masks."""
    T = x.shape[0]
    g = dict(topk_idx=Guarded((T, L.k), torch.int32),
             topk_w=Guarded((T, L.k), torch.float32),
             logits=Guarded((T, L.E), torch.float32),
             expert_count=Guarded((L.E,), torch.int32))
    sparse = want_masks and path == moe.PATH_SPARSE
    if sparse:
        g["masks"] = Guarded((T, L.k + L.S, L.f), torch.uint8)
        g["mask_bits"] = Guarded((T, L.k + L.S, L.f // 64), torch.int64)
        g["nnz"] = Guarded((T, L.k + L.S), torch.int32)
    y = Guarded((T, L.d), torch.float32)
    ws = guarded_workspace(L.workspace_bytes(T))
    moe.layer_forward(L, x, path=path, y=y.t, ws=ws.t, trace={k: v.t for k, v in g.items()})
    torch.cuda.synchronize()
    for k, v in g.items():
        v.check(f"layer export {k}")
    y.check("layer y")
    ws.check("layer workspace")
    tr = {k: v.t.cpu().numpy() for k, v in g.items()}
    if sparse:
        check_bits_exports(tr["masks"], g["mask_bits"].t, g["nnz"].t, "layer masks")
    return y.t.cpu().numpy(), tr


# ---------------------------------------------------------------------------
# Full-size layers generated on the device.  torch draws the weights; the INT2
# bytes come from the library's packer, which the tests hold bit-exact against
# the oracle's packer on every expert the oracle later reads, so the oracle is
# always fed its own packing of the same fp32 draws.
# ---------------------------------------------------------------------------

def device_draws(cfg, layer, e, d, f, wdt, std=0.02):
    """(gate_t, up_t fp32, down) drawn on the device for one expert."""
    g = synth.device_normal(synth.seed_of(cfg, layer, e, synth.T_GATE), (f, d), std, DEV,
                            TORCH_DT[wdt])
    u = synth.device_normal(synth.seed_of(cfg, layer, e, synth.T_UP), (f, d), std, DEV)
    dn = synth.device_normal(synth.seed_of(cfg, layer, e, synth.T_DOWN), (f, d), std, DEV,
                             TORCH_DT[wdt])
    return g, u, dn


def torch_dequant(up_q, up_sz, d):
    """fp32 [f][d] = s (q - z) from the INT2 bytes, in torch on the device
    (calibration only).  Word i of a row holds input 16i+2m+h at bits 16h+2m."""
    f = up_q.shape[0]
    w = up_q.view(torch.int32).reshape(f, d // 16, 1)
    j = torch.arange(16, device=up_q.device, dtype=torch.int32)
    shift = 16 * (j % 2) + 2 * (j // 2)
    q = ((w >> shift) & 3).reshape(f, d).float()
    sz = up_sz.view(torch.float16).float()
    s = sz[..., 0].repeat_interleave(64, dim=1)
    z = sz[..., 1].repeat_interleave(64, dim=1)
    return s * (q - z)


def torch_threshold(up_q, up_sz, cfg, layer, e, d, wdt, xscale, sparsity):
    """Threshold at the `sparsity` quantile of |x_c . w'| over the 64 seeded
    calibration vectors, w' the dequantised INT2 up weights (torch fp32).  It
    only places the realised sparsity; parity never depends on it."""
    xc = torch.from_numpy(synth.calibration_f32(cfg, d, xscale, layer, e)).to(TORCH_DT[wdt])
    v = xc.to(DEV).float() @ torch_dequant(up_q, up_sz, d).T
    return oracle.calibrate_threshold(v.abs().cpu().numpy(), sparsity)


class DeviceLayer:
    """E routed + S shared experts of one layer, stacked on the device."""

    def __init__(self, cfg, layer, E, S, k, d, f, wdt, xscale, sparsity, router_std=0.02,
                 bias=None, dense=False):
        self.cfg, self.layer, self.E, self.S, self.k = cfg, layer, E, S, k
        self.d, self.f, self.wdt = d, f, wdt
        n = E + S
        up_q = torch.empty((n, f, d // 4), dtype=torch.uint8, device=DEV)
        up_sz = torch.empty((n, f, d // 64, 2), dtype=torch.int16, device=DEV)
        gate = torch.empty((n, f, d), dtype=TORCH_DT[wdt], device=DEV)
        down = torch.empty((n, f, d), dtype=TORCH_DT[wdt], device=DEV)
        thr = np.zeros(n, dtype=np.float32)
        for e in range(n):
            g, u, dn = device_draws(cfg, layer, e, d, f, wdt)
            gate[e].copy_(g)
            down[e].copy_(dn)
            del g, dn
            moe.pack_up_int2(u, up_q=up_q[e], up_sz=up_sz[e])
            del u
            thr[e] = torch_threshold(up_q[e], up_sz[e], cfg, layer, e, d, wdt, xscale,
                                     sparsity)
        self.thr = thr
        self.R_bits = synth.to_bits(synth.router_f32(cfg, layer, E, d, router_std), wdt)
        self.bias = bias
        self.L = moe.Layer(d=d, f=f, E=E, S=S, k=k, renormalize=True,
                           router_w=to_dev_bits(self.R_bits, wdt), up_q=up_q, up_sz=up_sz,
                           gate_t=gate, down=down, thresholds=torch.from_numpy(thr).to(DEV),
                           router_bias=None if bias is None else torch.from_numpy(bias).to(DEV))
        if dense:
            # dense path: up weights in the layer's type and W^down transposed
            # (the 256 x 256-tile MFMA kernels)
            self.L.up_dense = torch.empty((n, f, d), dtype=TORCH_DT[wdt], device=DEV)
            for e in range(n):
                moe.materialize_up(up_q[e], up_sz[e], d, TORCH_DT[wdt], out=self.L.up_dense[e])
            self.L.down_dense = moe.transpose_down(down)
        torch.cuda.synchronize()

    def host_weights(self, experts):
        """Host copies for the oracle: the oracle's own INT2 packing of the
        regenerated fp32 up draws (asserted bit-exact against the device
        packing) and the gate/down bit patterns.  Experts not listed are left
        zero; the oracle reads only the experts it is fed."""
        n = self.E + self.S
        d, f = self.d, self.f
        uq = np.zeros((n, f, d // 4), np.uint8)
        us = np.zeros((n, f, d // 64, 2), np.uint16)
        g = np.zeros((n, f, d), np.uint16)
        dn = np.zeros((n, f, d), np.uint16)
        for e in sorted(set(int(x) for x in experts)):
            _, u, _ = device_draws(self.cfg, self.layer, e, d, f, self.wdt)
            q_ref, sz_ref = oracle.pack_up_int2(u.cpu().numpy())
            del u
            assert np.array_equal(self.L.up_q[e].cpu().numpy(), q_ref), f"pack codes e={e}"
            assert np.array_equal(self.L.up_sz[e].cpu().numpy().view(np.uint16), sz_ref), \
                f"pack scales e={e}"
            uq[e], us[e] = q_ref, sz_ref
            g[e] = dev_bits(self.L.gate_t[e])
            dn[e] = dev_bits(self.L.down[e])
        return uq, us, g, dn

    def free(self):
        self.L = None
        torch.cuda.empty_cache()


def check_layer_tokens(lay: DeviceLayer, x_bits, y, tr, tokens, dense, what):
    """Oracle check of a layer's output on the listed tokens, fed the GPU's
    top-k (and masks on the sparse path); each mask against the oracle's v."""
    k, S, E = lay.k, lay.S, lay.E
    used = set(range(E, E + S))
    for t in tokens:
        used.update(int(e) for e in tr["topk_idx"][t])
    uq, us, g, dn = lay.host_weights(used)
    sub = x_bits[tokens]
    masks_in = None if dense else tr["masks"][tokens]
    y_ref, _, w_ref, _ = oracle.layer_forward(
        sub, lay.wdt, lay.R_bits, lay.wdt, lay.bias, E, k, S, True, uq, us, g, dn, lay.wdt,
        lay.thr, dense=dense, topk_in=tr["topk_idx"][tokens], masks_in=masks_in)
    np.testing.assert_allclose(tr["topk_w"][tokens], w_ref, rtol=2e-5, atol=1e-6)
    ndiff = 0
    if not dense:
        for i, t in enumerate(tokens):
            for s in range(k + S):
                e = int(tr["topk_idx"][t, s]) if s < k else E + (s - k)
                v_ref, _, _ = oracle.expert_forward(x_bits[t:t + 1], lay.wdt, uq[e], us[e], g[e],
                                                    dn[e], lay.wdt, np.inf)
                ndiff += check_mask(tr["masks"][t, s][None], v_ref, lay.thr[e],
                                    f"{what} t={t} slot={s}")
    err = check_y(y[tokens], y_ref, REL_L2, what)
    say(f"{what}: tokens {list(tokens)} band-diffs={ndiff} max relL2={err:.2e}")
    return err

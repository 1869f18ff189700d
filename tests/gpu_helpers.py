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

"""The allocation-free entry point (moe_expert_forward_sparse_noalloc) against
moe_expert_forward_sparse with a caller workspace, through the C ABI: the same
kernels on the same inputs, so every output must agree bit for bit.  Two calls
in a row on the library's static scratch, the second with a smaller input
(fewer tokens, a smaller expert), so stale scratch contents from the first call
would show."""
import ctypes as C

import numpy as np
import pytest
import torch

import activation_sparse_expert_amd as moe
import synth
from gpu_helpers import DEV, Guarded, HostExpert, say, to_dev_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def outputs(hx, T):
    return dict(y=Guarded((T, hx.d), torch.float32), mask_out=Guarded((T, hx.f), torch.uint8),
                v_out=Guarded((T, hx.f), torch.float32),
                mask_bits=Guarded((T, hx.f // 64), torch.int64), nnz=Guarded((T,), torch.int32))


def run_both(hx, thr, x_bits, what):
    ex = hx.to_device(thr)
    x = to_dev_bits(x_bits, hx.wdt)
    T = x.shape[0]
    ref, got = outputs(hx, T), outputs(hx, T)
    ws = moe.new_workspace(moe.workspace_size(moe.OP_EXPERT, T, hx.d, hx.f))
    moe.expert_forward_sparse(ex, x, ws=ws, **{k: v.t for k, v in ref.items()})
    moe.expert_forward_sparse_noalloc(ex, x, **{k: v.t for k, v in got.items()})
    torch.cuda.synchronize()
    for k in ref:
        got[k].check(f"{what} noalloc {k}")
        a, b = ref[k].t.cpu().numpy(), got[k].t.cpu().numpy()
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{what}: {k} differs"
    say(f"{what}: noalloc == workspace path bit for bit "
        f"(nnz {got['nnz'].t.cpu().numpy().tolist()})")


def test_noalloc_matches_workspace_path_twice_second_smaller():
    big = HostExpert(synth.CFG_MIXTRAL, 3, 0, 4096, 14336)
    thr = big.calibrate(synth.CFG_MIXTRAL, 1 / 64, 0.9, layer=3)
    x4 = synth.to_f16_bits(synth.tokens_f32(97, 4, 4096, 1 / 64))
    run_both(big, thr, x4, "d=4096 f=14336 T=4")
    run_both(big, thr, x4[2:3], "d=4096 f=14336 T=1")
    small = HostExpert(98, 0, 0, 1024, 512, wdt="bf16")
    ts = small.calibrate(98, 1 / 64, 0.7)
    x1 = synth.to_bits(synth.tokens_f32(99, 1, 1024, 1 / 64), "bf16")
    run_both(small, ts, x1, "d=1024 f=512 bf16 T=1")


def test_noalloc_rejects_what_does_not_fit():
    L = moe.lib()
    assert L.moe_noalloc_scratch_bytes() == 32 << 20
    v = moe.ExpertView(0x10000, 0x10000, 0x10000, 0x10000, 0.1)
    # 512 tokens at d = 16384 need far more than the static scratch: refused
    # on the host before anything is enqueued
    st = L.moe_expert_forward_sparse_noalloc(C.byref(v), 16384, 4096, 0, 0x10000, 0, 512, None, 0,
                                             0x10000, 2, None, None, None, None, None)
    assert st == -2

"""Child process of test_layer_mixed_first_call_under_capture (run alone, not
collected): the process's first MOE_PATH_MIXED call is made under graph
capture, where the library cannot create its second stream, so the captured
call runs the sparse kernel and the GEMMs in order on the capturing stream.
Its replays must equal the eager calls made afterwards, which fork onto the
library stream.  Prints one line and exits 0 on success."""
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import activation_sparse_expert_amd as moe  # noqa: E402
import synth  # noqa: E402
from gpu_helpers import DEV, to_dev_bits  # noqa: E402
from test_parity_layer_gpu import build_host_layer, device_layer  # noqa: E402


def main():
    E, S, k, d, f, T = 16, 1, 4, 512, 256, 64
    experts, thr = build_host_layer(70, E, S, d, f, "f16", 0.7, 1.0, layer=d)
    R_bits = synth.to_bits(synth.router_f32(70, d, E, d), "f16")
    bias = synth.zipf_bias(71, d, E, 1.1)
    L = device_layer(experts, thr, R_bits, "f16", E, S, k, bias=bias, dense="gemm")
    L.density = 0.3
    assert 1 < L.mixed_dense_min(T) <= T
    x = to_dev_bits(synth.to_bits(synth.tokens_f32(90, T, d, 1.0, layer=d), "f16"), "f16")
    ws = moe.new_workspace(L.workspace_bytes(T))
    y = torch.zeros((T, d), dtype=torch.float32, device=DEV)
    # the sparse path once, so that the graph capture below is not the first
    # GPU work of the process (the library stream is still absent)
    moe.layer_forward(L, x, path=moe.PATH_SPARSE, y=y, ws=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        moe.layer_forward(L, x, path=moe.PATH_MIXED, y=y, ws=ws)
    replays = []
    for _ in range(3):
        y.fill_(7.0)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        stream.synchronize()
        replays.append(y.cpu().numpy().copy())
    eager = []
    for _ in range(2):                  # these create and use the library stream
        y2 = moe.layer_forward(L, x, path=moe.PATH_MIXED, ws=ws)
        torch.cuda.synchronize()
        eager.append(y2.cpu().numpy())
    for i, r in enumerate(replays):
        assert np.array_equal(r, eager[0]), f"replay {i} differs from the forked eager call"
    assert np.array_equal(eager[0], eager[1])
    print("mixed first call under capture: serial replays equal the forked eager calls", flush=True)


if __name__ == "__main__":
    main()

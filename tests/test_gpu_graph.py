"""HIP graph capture of the library's calls (through torch.cuda.graph on the
caller's stream): the global-scale pre-pass (which zeroes its accumulator with
a fill kernel, not hipMemsetAsync), the fused quantize with per-expert
scales, the dequantize, the compact SwiGLU pass and the grouped GEMM with
the fused epilogue. The graph is replayed
several times with eager work and synchronizations between the replays, and
every replay must reproduce the eager results bit for bit, also after the
input changes in place."""
import numpy as np
import pytest
import torch

from moe_swiglu_epilogue_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu]", *a, flush=True)


def test_graph_replays_match_eager():
    import moe_swiglu_epilogue_amd as M
    assert torch.cuda.is_available()
    dev = torch.device("cuda:0")
    rows, inter, experts = 300, 1040, 7
    x = torch.from_numpy(W.random_fused(rows, inter, 81, 2.0).view(np.int16)).to(dev).view(torch.bfloat16)
    offs = torch.from_numpy(W.random_offsets(rows, experts, 81, empty=2)).to(dev)
    gw = W.moe_gemm(83, 300, 128, 256, experts)
    gx = torch.from_numpy(gw.x.view(np.int16)).to(dev).view(torch.bfloat16)
    gwt = torch.from_numpy(gw.w1.view(np.int16)).to(dev).view(torch.bfloat16)

    def outputs():
        return dict(gs=torch.empty(experts, dtype=torch.float32, device=dev),
                    p=torch.empty((rows, inter // 2), dtype=torch.uint8, device=dev),
                    s=torch.empty((rows, inter // 16), dtype=torch.uint8, device=dev),
                    dq=torch.empty((rows, inter), dtype=torch.float32, device=dev),
                    yb=torch.empty((rows, inter), dtype=torch.bfloat16, device=dev),
                    gp=torch.empty((300, 128), dtype=torch.uint8, device=dev),
                    gsc=torch.empty((300, 16), dtype=torch.uint8, device=dev))

    def run(o):
        M.swiglu_nvfp4_global_scale(x, offs, gs=o["gs"])
        M.swiglu_nvfp4_quantize(x, o["gs"], offs, packed=o["p"], scales=o["s"])
        M.nvfp4_dequantize(o["p"], o["s"], o["gs"], offs, out=o["dq"])
        M.swiglu_bf16(x, out=o["yb"])
        M.moe_l1_gemm_swiglu_nvfp4(gx, gwt, offs, o["gs"], packed=o["gp"], scales=o["gsc"])

    def snapshot(o):
        torch.cuda.synchronize()
        return {k: v.view(torch.uint8).cpu().numpy().copy() for k, v in o.items()}

    eager = outputs()
    run(eager)
    want = snapshot(eager)

    cap = outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up outside capture, as torch advises
        run(cap)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(cap)
    for r in range(3):
        for v in cap.values():                 # eager work between replays
            v.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        say("graph replay", r)
        g.replay()
        got = snapshot(cap)
        for k in want:
            assert np.array_equal(got[k], want[k]), (r, k)
    # new input in place: the graph reads the same buffer
    x.view(torch.int16).copy_(torch.from_numpy(W.random_fused(rows, inter, 82, 0.5).view(np.int16)).to(dev))
    run(eager)
    want = snapshot(eager)
    for r in range(2):
        for v in cap.values():
            v.view(torch.uint8).fill_(0x5A)
        say("graph replay on new input", r)
        g.replay()
        got = snapshot(cap)
        for k in want:
            assert np.array_equal(got[k], want[k]), ("new input", r, k)

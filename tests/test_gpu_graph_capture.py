"""The entry points can be captured in a HIP graph (they allocate nothing,
synchronize nothing and record no memset) and replayed: every replay, with
eager work and synchronizations in between, equals the eager call's bits."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import DEV, dev_bf16, dev_f32, dev_u8, host_bits, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qh():
    import quantized_weight_decode_amd as m

    assert torch.cuda.is_available()
    return m


def test_graph_replays_match_eager(qh):
    V, H = 4096, 2048
    wf = synth.weight_rows_f32(synth.FP8_8192X1024, 0, V, vocab=V, hidden=H)
    w, s = oracle.prep_fp8_rows(wf)
    g = oracle.nvfp4_global(float(np.abs(wf).max()))
    wp, bs = oracle.prep_nvfp4_rows(wf, g)
    blocks = oracle.prep_q6k_rows(wf)
    wd, sd, wpd, bsd, bld = dev_u8(w), dev_f32(s), dev_u8(wp), dev_u8(bs), dev_u8(blocks)
    x = dev_bf16(synth.activations_bf16(synth.FP8_8192X1024, 20, hidden=H, max_rows=20))
    gate_h, up_h = synth.gate_up_bf16(synth.SILU_DOWN_7168X18432, 20, hidden=H, max_rows=20)
    gate, up = dev_bf16(gate_h), dev_bf16(up_h)
    ws8 = qh.w8a8_workspace(H, DEV)
    ws6 = torch.empty((qh.q6k_workspace_bytes(H),), dtype=torch.uint8, device=DEV)
    outs = {k: torch.empty((20, V), dtype=torch.bfloat16, device=DEV)
            for k in ("fp8", "w8a8", "nvfp4", "q6k", "silu")}

    def calls():
        qh.fp8_rowscale(wd, sd, x, out=outs["fp8"])
        qh.w8a8(wd, sd, x, out=outs["w8a8"], workspace=ws8)
        qh.nvfp4(wpd, bsd, x, g, out=outs["nvfp4"])
        qh.q6k(bld, x, out=outs["q6k"], workspace=ws6)
        qh.w8a8_silu(wd, sd, gate, up, out=outs["silu"], workspace=ws8)

    calls()
    torch.cuda.synchronize()
    eager = {k: host_bits(v) for k, v in outs.items()}

    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        calls()
    torch.cuda.synchronize()
    for rep in range(4):
        log(f"[case] graph replay {rep}")
        for v in outs.values():
            v.zero_()                                  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert np.array_equal(host_bits(v), eager[k]), (k, rep)

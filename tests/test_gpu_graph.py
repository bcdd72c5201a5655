"""The library's calls inside a captured HIP graph.

The entry points only enqueue kernels on the caller's stream (no allocation,
no memset, no host synchronization), so a serving loop can capture them.  A
captured decode step (W4A16 GEMVs and the tied-table lookup), a prefill GEMM
with split-K partials in a workspace, W8A16 GEMMs (K-sliced and mixed-size
launches), a W8A8 GEMM and the MoE are replayed
several times, with eager work and synchronizations in between, and every
replay must equal the eager result bit for bit (the kernels are
deterministic: fixed summation orders, split-K slices summed in order)."""
import numpy as np
import pytest
import torch

import synth_inputs as si
import weight_only_quantized_w8a16_amd as qg
from helpers import BF16, FP16, to_dev

pytestmark = pytest.mark.gpu


def _w4(n, k, g, tag, dtype=BF16, bias=False):
    packed, s, z, b = si.w4_weights(n, k, g, si.seed_of(tag, n, k, g), dtype,
                                    bias_dtype=FP16 if bias else 0)
    return (qg.repack_w4(to_dev(packed)), to_dev(s, dtype), to_dev(z, dtype),
            to_dev(b, FP16) if bias else None)


def test_captured_calls_replay_bit_exact():
    dev = "cuda"
    K = 2048
    # decode: M = 1 GEMVs at two widths and a lookup from the wider table
    w_small, w_wide = _w4(3072, K, 64, "g-small"), _w4(13312, K, 64, "g-wide")
    a1 = to_dev(si.activations(1, K, 3), BF16)
    ids = to_dev(np.array([5, 13311, 0, 77], dtype=np.int32))
    # prefill with split-K partials (M = 128 on the 64 x 64 tile)
    wp = _w4(3072, K, 64, "g-pre", bias=True)
    a128 = to_dev(si.activations(128, K, 4), BF16)
    ws = torch.empty(max(qg.gemm_workspace_size(128, 3072, K, 64, 4), 256), dtype=torch.uint8,
                     device=dev)
    assert qg.gemm_workspace_size(128, 3072, K, 64, 4) > 0
    # prefill on the dequantize-then-dense path (M = 512: the weight dequantized
    # into the workspace, then the dense tile)
    a512 = to_dev(si.activations(512, K, 6), BF16)
    wsd = torch.empty(qg.gemm_workspace_size(512, 3072, K, 64, 4), dtype=torch.uint8, device=dev)
    assert wsd.numel() == 3072 * K * 2
    # W8A16 (K = 3584): M = 128 on the code-converting tile in K slices (its
    # partials in a workspace), M = 1024 on the mixed 256 / 128 launch (one
    # scale per channel) and on the mixed fused 256 x 256 / 256 x 128 launch
    # (group 128)
    K8 = 3584
    c8a, s8a, _ = si.w8_weights(3584, K8, -1, si.seed_of("g-w8a", K8))
    c8b, s8b, _ = si.w8_weights(18944, K8, -1, si.seed_of("g-w8b", K8))
    c8c, s8c, _ = si.w8_weights(18944, K8, 128, si.seed_of("g-w8c", K8))
    b8a, b8b, b8c = (qg.repack_w8(to_dev(c)) for c in (c8a, c8b, c8c))
    s8a, s8b, s8c = (to_dev(x, FP16) for x in (s8a, s8b, s8c))
    a8_128 = to_dev(si.activations(128, K8, 8, FP16), FP16)
    a8_1024 = to_dev(si.activations(1024, K8, 9, FP16), FP16)
    ws8s = torch.empty(qg.gemm_workspace_size(128, 3584, K8, -1, 8), dtype=torch.uint8, device=dev)
    assert ws8s.numel() == 4 * 128 * 3584 * 4
    # W8A8
    p8 = si.w8a8_problem(64, 1024, 1024, True, True, tag="g-w8a8")
    A8, B8 = torch.from_numpy(p8.A).to(dev), torch.from_numpy(p8.B).to(dev)
    r8, c8 = torch.from_numpy(p8.alpha_row).to(dev), torch.from_numpy(p8.alpha_col).to(dev)
    ws8 = torch.empty(max(qg.w8a8_workspace_size(64, 1024, 1024), 256), dtype=torch.uint8, device=dev)
    # MoE
    m = si.moe_problem(64, 256, 256, 8, 2, 64, tag="g-moe")
    mx, ml = to_dev(m.x, BF16), torch.from_numpy(m.logits).to(dev)
    w1 = torch.stack([qg.repack_w4(to_dev(m.w1[e])) for e in range(8)])
    w2 = torch.stack([qg.repack_w4(to_dev(m.w2[e])) for e in range(8)])
    s1, z1, s2, z2 = (to_dev(a, BF16) for a in (m.s1, m.z1, m.s2, m.z2))
    mws = torch.empty(qg.moe_workspace_size(64, 256, 256, 8, 2), dtype=torch.uint8, device=dev)

    outs = {
        "g_small": torch.empty((1, 3072), dtype=torch.bfloat16, device=dev),
        "g_wide": torch.empty((1, 13312), dtype=torch.bfloat16, device=dev),
        "pre": torch.empty((128, 3072), dtype=torch.bfloat16, device=dev),
        "dense": torch.empty((512, 3072), dtype=torch.bfloat16, device=dev),
        "w8a8": torch.empty((64, 1024), dtype=torch.float16, device=dev),
        "w8_split": torch.empty((128, 3584), dtype=torch.float16, device=dev),
        "w8_wx": torch.empty((1024, 18944), dtype=torch.float16, device=dev),
        "w8_dx": torch.empty((1024, 18944), dtype=torch.float16, device=dev),
    }
    state = {}

    def step():
        qg.gemm_w4a16(a1, w_small[0], w_small[1], w_small[2], None, 64, out=outs["g_small"])
        qg.gemm_w4a16(a1, w_wide[0], w_wide[1], w_wide[2], None, 64, out=outs["g_wide"])
        state["emb"] = qg.embed_w4(ids, w_wide[0], w_wide[1], w_wide[2], 64)
        qg.gemm_w4a16(a128, wp[0], wp[1], wp[2], wp[3], 64, out=outs["pre"], workspace=ws)
        qg.gemm_w4a16(a512, wp[0], wp[1], wp[2], wp[3], 64, out=outs["dense"], workspace=wsd)
        qg.gemm_w8a16(a8_128, b8a, s8a, None, -1, out=outs["w8_split"], workspace=ws8s)
        qg.gemm_w8a16(a8_1024, b8b, s8b, None, -1, out=outs["w8_wx"])
        qg.gemm_w8a16(a8_1024, b8c, s8c, None, 128, out=outs["w8_dx"])
        qg.gemm_w8a8(A8, B8, r8, c8, out=outs["w8a8"], workspace=ws8)
        state["moe"] = qg.moe_grouped(mx, ml, w1, s1, z1, w2, s2, z2, 2, 64, workspace=mws)

    step()                      # eager: also sets the kernels' one-time attributes
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    eager["emb"], eager["moe"] = state["emb"].clone(), state["moe"].clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    graph_out = dict(outs, emb=state["emb"], moe=state["moe"])
    for rep in range(4):
        for v in graph_out.values():
            v.zero_()           # eager work between replays (a fill kernel)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in graph_out.items():
            assert torch.equal(v, eager[k]), (rep, k)

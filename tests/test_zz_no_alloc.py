"""The allocation-free MoE entry point (qmoe_grouped_noalloc), called through
the C ABI: its workspace is the library's device scratch, so two calls in a
row -- the second on a smaller problem, over the first one's leftovers --
must each match qmoe_grouped with a caller workspace bit for bit (same
kernels, same plan), and the routing must equal the oracle's."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import weight_only_quantized_w8a16_amd as qg
from helpers import BF16, TOL, rel_err, to_dev

pytestmark = pytest.mark.gpu

def _noalloc():
    return qg.lib().qmoe_grouped_noalloc      # the C entry point itself


def _inputs(T, H, I, E, k, g, tag):
    p = si.moe_problem(T, H, I, E, k, g, tag=tag)
    dev = "cuda"
    t = dict(x=to_dev(p.x, BF16), logits=torch.from_numpy(p.logits).to(dev),
             w1=torch.stack([qg.repack_w4(to_dev(p.w1[e])) for e in range(E)]),
             w2=torch.stack([qg.repack_w4(to_dev(p.w2[e])) for e in range(E)]))
    for nm in ("s1", "z1", "s2", "z2"):
        t[nm] = to_dev(getattr(p, nm), BF16)
    return p, t


def _call_noalloc(t, T, H, I, E, k, g):
    out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    ids = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    wts = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    st = _noalloc()(t["x"].data_ptr(), t["logits"].data_ptr(), t["w1"].data_ptr(),
                    t["s1"].data_ptr(), t["z1"].data_ptr(), t["w2"].data_ptr(), t["s2"].data_ptr(),
                    t["z2"].data_ptr(), out.data_ptr(), T, H, I, E, k, g, 1, ids.data_ptr(),
                    wts.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, qg.lib().qg_strerror(st)
    return out, ids, wts


def _call_ws(t, T, H, I, E, k, g):
    return qg.moe_grouped(t["x"], t["logits"], t["w1"], t["s1"], t["z1"], t["w2"], t["s2"],
                          t["z2"], k, g, return_routing=True)


@pytest.mark.parametrize("shapes", [
    [(256, 512, 384, 16, 4, 64, "na-a"), (37, 512, 384, 16, 4, 64, "na-b")],
    [(1024, 2048, 1408, 64, 6, 64, "na-c"), (64, 2048, 1408, 64, 6, 64, "na-d")],
])
def test_noalloc_matches_workspace_call_twice(shapes):
    for (T, H, I, E, k, g, tag) in shapes:
        p, t = _inputs(T, H, I, E, k, g, tag)
        out, ids, wts = _call_noalloc(t, T, H, I, E, k, g)
        ref_out, ref_ids, ref_w = _call_ws(t, T, H, I, E, k, g)
        torch.cuda.synchronize()
        assert torch.equal(ids, ref_ids) and torch.equal(wts, ref_w)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), tag
        toks = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(T).integers(0, T, 14)]))
        ref, rids, _ = oracle.moe(p.x, p.logits, p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, k, g,
                                  tokens=toks)
        assert np.array_equal(ids.cpu().numpy(), rids)
        assert rel_err(out.float().cpu().numpy()[toks], ref) <= TOL[BF16]
        # the binding of the same entry point
        out2 = torch.empty_like(out)
        qg.moe_grouped_noalloc(t["x"], t["logits"], t["w1"], t["s1"], t["z1"], t["w2"], t["s2"],
                               t["z2"], k, g, out2)
        torch.cuda.synchronize()
        assert torch.equal(out2.view(torch.int16), ref_out.view(torch.int16))


def test_noalloc_rejects_problems_beyond_the_scratch():
    # 2048 tokens of the 64-expert workload need about 81 MiB of workspace,
    # more than the 64 MiB scratch: refused before any launch, outputs untouched.
    T, H, I, E, k, g = 2048, 2048, 1408, 64, 6, 64
    assert qg.moe_workspace_size(T, H, I, E, k) > 64 << 20
    _, t = _inputs(T, H, I, E, k, g, "na-big")
    out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    st = _noalloc()(t["x"].data_ptr(), t["logits"].data_ptr(), t["w1"].data_ptr(),
                    t["s1"].data_ptr(), t["z1"].data_ptr(), t["w2"].data_ptr(), t["s2"].data_ptr(),
                    t["z2"].data_ptr(), out.data_ptr(), T, H, I, E, k, g, 1, None, None,
                    torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 6                                      # QG_ERR_WORKSPACE
    assert bool(torch.isnan(out.float()).all())

"""GPU parity, part 3: the top-k MoE against the CPU oracle.

Routing ids must equal the oracle's exactly (same fp32 comparisons, ties to
the lower expert); weights and outputs within tolerance."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import weight_only_quantized_w8a16_amd as qg
from helpers import BF16, FP16, TOL, rel_err, to_dev

pytestmark = pytest.mark.gpu


def run_moe(p):
    dev = "cuda"
    x = to_dev(p.x, p.dtype)
    lg = torch.from_numpy(p.logits).to(dev)
    w1 = torch.stack([qg.repack_w4(to_dev(p.w1[e])) for e in range(p.experts)])
    w2 = torch.stack([qg.repack_w4(to_dev(p.w2[e])) for e in range(p.experts)])
    s1, z1, s2, z2 = (to_dev(a, p.dtype) for a in (p.s1, p.z1, p.s2, p.z2))
    out, ids, w = qg.moe_grouped(x, lg, w1, s1, z1, w2, s2, z2, p.topk, p.group,
                                 return_routing=True)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


def check(p, tokens=None, tol=TOL[BF16]):
    out, ids, w = run_moe(p)
    ref, rids, rw = oracle.moe(p.x, p.logits, p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, p.topk,
                               p.group, p.dtype, tokens=tokens)
    assert np.array_equal(ids, rids)
    np.testing.assert_allclose(w, rw, rtol=2e-6, atol=1e-7)
    sel = np.arange(p.tokens) if tokens is None else np.asarray(tokens)
    err = rel_err(out[sel], ref)
    assert err <= tol, err
    return out


@pytest.fixture(params=["default", "S"])
def moe_tile(request):
    """Run a test on the default grouped-GEMM tile and on the 128 x 128 one."""
    if request.param == "S":
        qg.set_override(moe_tile="S")
    return request.param


@pytest.mark.parametrize("T,H,I,E,k,g", [
    (4, 128, 128, 4, 2, 64), (33, 256, 256, 16, 4, 64), (1, 256, 128, 8, 8, 128),
    (64, 256, 384, 8, 1, 64), (200, 128, 128, 64, 6, 64), (130, 384, 256, 4, 2, 128),
    (512, 256, 256, 4, 2, 64), (300, 512, 640, 8, 3, 128),
])
def test_moe_small_full(T, H, I, E, k, g, moe_tile):
    p = si.moe_problem(T, H, I, E, k, g, tag="moe-small")
    check(p)


def test_moe_more_routing_workgroups_than_plan_workgroups(moe_tile):
    # 3000 tokens x top-6 = 18000 expert rows from 188 routing workgroups of
    # 16 tokens: more than the plan's 128 workgroups, so each plan workgroup
    # places the rows of two routing workgroups (the second from counts
    # carried over from the first; checked on a sample of tokens, routing in
    # full).
    p = si.moe_problem(3000, 256, 256, 8, 6, 64, tag="moe-many-rows")
    assert -(-p.tokens // 16) > 128
    toks = np.unique(np.concatenate([[0, 1, 2999], np.random.default_rng(7).integers(0, 3000, 256)]))
    check(p, tokens=toks)


def test_moe_expert_tiles_exactly_full(moe_tile):
    # 256 tokens all routed to experts 5 and 2: two experts of exactly 256 rows.
    p = si.moe_problem(256, 256, 256, 8, 2, 64, tag="moe-full-tiles")
    p.logits[:] = 0.0
    p.logits[:, 5] = 3.0
    p.logits[:, 2] = 2.0
    check(p)


def test_moe_expert_row_counts_cover_every_partial_tile(moe_tile):
    # Top-1 routes with chosen expert sizes: every number of filled 32-row
    # blocks in each half of a 256-row expert tile, exact multiples of 32 and
    # their neighbours, experts longer than one tile, and an empty expert.
    counts = [1, 31, 32, 33, 64, 96, 127, 128, 129, 160, 191, 192, 193, 224, 255, 256, 257,
              300, 0]
    E, T = len(counts), sum(counts)
    p = si.moe_problem(T, 256, 128, E, 1, 64, tag="moe-counts")
    owner = np.repeat(np.arange(E), counts)
    np.random.default_rng(7).shuffle(owner)
    p.logits[:] = 0.0
    p.logits[np.arange(T), owner] = 4.0
    assert np.array_equal(np.bincount(owner, minlength=E), counts)
    check(p)


def test_moe_fp16(moe_tile):
    p = si.moe_problem(48, 256, 256, 8, 2, 64, tag="moe-f16", dtype=FP16)
    check(p, tol=TOL[FP16])


def test_moe_identical_experts_give_dense_ffn():
    p = si.moe_problem(40, 256, 128, 8, 3, 64, tag="moe-same")
    for a in (p.w1, p.s1, p.z1, p.w2, p.s2, p.z2):
        a[1:] = a[0]
    out, _, _ = run_moe(p)
    ref, _, _ = oracle.moe(p.x, p.logits, p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, 3, 64)
    assert rel_err(out, ref) <= TOL[BF16]


def test_moe_forced_routes_and_empty_experts():
    p = si.moe_problem(16, 128, 128, 8, 2, 64, tag="moe-forced")
    p.logits[:] = 0.0
    p.logits[:, 5] = 3.0           # every token picks 5 first
    p.logits[:, 2] = 2.0           # then 2; experts 0,1,3,4,6,7 receive no rows
    out, ids, w = run_moe(p)
    assert (ids[:, 0] == 5).all() and (ids[:, 1] == 2).all()
    check(p)


def test_moe_full_size_sampled_tokens(moe_tile):
    # 2048 tokens, hidden 2048, inter 1408, 64 experts, top-6, g=64: every
    # output row written (NaN-filled output comes back finite), routing of
    # all tokens exact, 128 sampled tokens against the oracle.
    p = si.moe_problem(2048, 2048, 1408, 64, 6, 64, tag="cfg4")
    dev = "cuda"
    w1 = torch.stack([qg.repack_w4(to_dev(p.w1[e])) for e in range(p.experts)])
    w2 = torch.stack([qg.repack_w4(to_dev(p.w2[e])) for e in range(p.experts)])
    s1, z1, s2, z2 = (to_dev(a, p.dtype) for a in (p.s1, p.z1, p.s2, p.z2))
    out = torch.full((2048, 2048), float("nan"), dtype=torch.bfloat16, device=dev)
    qg.moe_grouped(to_dev(p.x, p.dtype), torch.from_numpy(p.logits).to(dev), w1, s1, z1, w2, s2,
                   z2, 6, 64, out=out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    toks = np.unique(np.concatenate([[0, 1, 2047], np.random.default_rng(4).integers(0, 2048, 125)]))
    check(p, tokens=toks)


def test_moe_route_neg_inf_selection_logits():
    # Selection logits with -inf entries, top-6 of 8 with as few as no finite
    # entry in a row: every chosen expert is distinct, ids equal the
    # oracle's (the untaken -inf experts in index order), weights from the
    # finite gating logits.
    T, E, k = 40, 8, 6
    p = si.moe_problem(T, 128, 128, E, k, 64, tag="moe-neginf")
    sel = p.logits.copy()
    rng = np.random.default_rng(3)
    for t in range(T):
        sel[t, rng.permutation(E)[t % 7:]] = -np.inf       # 0 .. 6 finite entries
    out, ids, w = run_moe_ex(p, None, None, sel, None, True)
    ref, rids, rw = oracle.moe(p.x, p.logits, p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, k, 64, BF16,
                               sel_logits=sel)
    assert all(len(set(r)) == k for r in ids.tolist())
    assert np.array_equal(ids, rids)
    np.testing.assert_allclose(w, rw, rtol=2e-6, atol=1e-7)
    assert rel_err(out, ref) <= TOL[BF16]


@pytest.mark.parametrize("E,k", [(65, 6), (96, 8), (128, 6), (200, 16), (256, 64), (64, 64)])
def test_moe_route_many_experts(E, k):
    # Routing over 65 .. 256 experts (a lane holds up to four, the last slot
    # partly filled) and top-k up to 64 (every expert of 64): ids equal the
    # oracle's, weights and outputs within tolerance.
    p = si.moe_problem(40, 128, 128, E, k, 64, tag="moe-wide")
    out, ids, w = run_moe_ex(p, None, None, None, None, True)
    ref, rids, rw = oracle.moe(p.x, p.logits, p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, k, 64, BF16)
    assert all(len(set(r)) == k for r in ids.tolist())
    assert np.array_equal(ids, rids)
    np.testing.assert_allclose(w, rw, rtol=2e-6, atol=1e-7)
    assert rel_err(out, ref) <= TOL[BF16]


@pytest.mark.parametrize("E", [64, 200])
def test_moe_route_ties_go_to_the_lower_expert(E):
    # Logits on a coarse grid (many exact ties, -0.0 beside 0.0): every
    # choice takes the lowest expert id among equal values, as the oracle's
    # strict-greater scan does, also across a lane's four slots.
    T, k = 64, 6
    p = si.moe_problem(T, 128, 128, E, k, 64, tag="moe-ties")
    lg = np.round(p.logits * 2.0).astype(np.float32) / 2.0
    lg[lg == 0.0] = np.where(np.arange((lg == 0.0).sum()) % 2 == 0, 0.0, -0.0).astype(np.float32)
    p = dataclasses.replace(p, logits=lg)
    out, ids, w = run_moe_ex(p, None, None, None, None, True)
    ref, rids, rw = oracle.moe(p.x, p.logits, p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, k, 64, BF16)
    assert np.array_equal(ids, rids)
    np.testing.assert_allclose(w, rw, rtol=2e-6, atol=1e-7)
    assert rel_err(out, ref) <= TOL[BF16]


# -- optional parts of runMoe: biased selection logits, finished rows, fc1 / fc2
# expert biases, normalization mode -------------------------------------------------

def run_moe_ex(p, b1, b2, sel, fin, renormalize):
    dev = "cuda"
    x = to_dev(p.x, p.dtype)
    lg = torch.from_numpy(p.logits).to(dev)
    w1 = torch.stack([qg.repack_w4(to_dev(p.w1[e])) for e in range(p.experts)])
    w2 = torch.stack([qg.repack_w4(to_dev(p.w2[e])) for e in range(p.experts)])
    s1, z1, s2, z2 = (to_dev(a, p.dtype) for a in (p.s1, p.z1, p.s2, p.z2))
    kw = dict(renormalize=renormalize)
    if b1 is not None:
        kw["b1"] = to_dev(b1, p.dtype)
    if b2 is not None:
        kw["b2"] = to_dev(b2, p.dtype)
    if sel is not None:
        kw["sel_logits"] = torch.from_numpy(sel).to(dev)
    if fin is not None:
        kw["finished"] = torch.from_numpy(fin.astype(bool)).to(dev)
    out, ids, w = qg.moe_grouped(x, lg, w1, s1, z1, w2, s2, z2, p.topk, p.group,
                                 return_routing=True, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("parts", ["biases", "selection", "finished", "no_renorm", "all"])
@pytest.mark.parametrize("T,H,I,E,k,g", [(37, 256, 256, 8, 2, 64), (300, 512, 384, 16, 4, 128)])
def test_moe_optional_parts(parts, T, H, I, E, k, g, moe_tile):
    p = si.moe_problem(T, H, I, E, k, g, tag="moe-extras")
    b1, b2, sel, fin = si.moe_extras(p)
    use = dict(b1=b1 if parts in ("biases", "all") else None,
               b2=b2 if parts in ("biases", "all") else None,
               sel=sel if parts in ("selection", "all") else None,
               fin=fin if parts in ("finished", "all") else None,
               renormalize=parts not in ("no_renorm", "all"))
    out, ids, w = run_moe_ex(p, **use)
    ref, rids, rw = oracle.moe(p.x, p.logits, p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, p.topk, p.group,
                               p.dtype, b1=use["b1"], b2=use["b2"], sel_logits=use["sel"],
                               finished=use["fin"], renormalize=use["renormalize"])
    assert np.array_equal(ids, rids)
    np.testing.assert_allclose(w, rw, rtol=2e-6, atol=1e-7)
    assert rel_err(out, ref) <= TOL[BF16]
    if use["fin"] is not None:
        assert fin.any() and (out[fin == 1] == 0).all() and (ids[fin == 1] == -1).all()


def test_moe_all_rows_finished():
    p = si.moe_problem(16, 128, 128, 4, 2, 64, tag="moe-allfin")
    out, ids, w = run_moe_ex(p, None, None, None, np.ones(16, np.uint8), True)
    assert (out == 0).all() and (ids == -1).all() and (w == 0).all()


def test_moe_optional_parts_full_size_sampled():
    # The 2048-token, 64-expert workload with every optional part on.
    p = si.moe_problem(2048, 2048, 1408, 64, 6, 64, tag="cfg4")
    b1, b2, sel, fin = si.moe_extras(p)
    out, ids, w = run_moe_ex(p, b1, b2, sel, fin, False)
    toks = np.unique(np.concatenate([[0, 2047], np.flatnonzero(fin)[:3],
                                     np.random.default_rng(9).integers(0, 2048, 16)]))
    ref, rids, rw = oracle.moe(p.x, p.logits, p.w1, p.s1, p.z1, p.w2, p.s2, p.z2, 6, 64, BF16,
                               tokens=toks, b1=b1, b2=b2, sel_logits=sel, finished=fin,
                               renormalize=False)
    assert np.array_equal(ids, rids)
    np.testing.assert_allclose(w, rw, rtol=2e-6, atol=1e-7)
    assert rel_err(out[toks], ref) <= TOL[BF16]

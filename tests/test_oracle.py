"""Pins of the oracle to things other than itself (CPU only).

Each pin checks the oracle against what the pages or the mathematics fix:
a library routine (torch's fp64 dense scaled-dot-product attention with the
block mask expanded to elements, and its autograd gradients — the page's own
reference), finite differences, closed forms, invariants, a special case that
reduces to dense attention, the pages' two-pass statistics route, and the
values the pages print (tests/golden). The planted-mistake test at the end
shows that a plausible slip anywhere in the oracle fails at least one pin.
"""
import json
import math
import shutil
import subprocess
from pathlib import Path

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as W

GOLDEN = Path(__file__).resolve().parent / "golden"
B = W.BLOCK


def _rel(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-30))


def _inputs(b, h, s, d, seed=0, dtype="fp32"):
    q, k, v, do = W.make_inputs(b, h, s, d, dtype, seed)
    return [t.double().numpy() for t in (q, k, v, do)]


def _elem_mask(bm, block=B):
    t = torch.from_numpy(np.asarray(bm, dtype=bool))
    return t.repeat_interleave(block, 0).repeat_interleave(block, 1)


def dense_reference(q, k, v, do, bm, scale=None, block=B):
    """torch fp64 SDPA with the element mask + autograd: (O, lse, dQ, dK, dV)."""
    qt, kt, vt = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    em = _elem_mask(bm, block)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=em, scale=scale)
    o.backward(torch.from_numpy(do))
    sc = (scale if scale is not None else 1.0 / math.sqrt(q.shape[-1]))
    scores = (torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2)) * sc
    scores = scores.masked_fill(~em, float("-inf"))
    lse = torch.logsumexp(scores, dim=-1)
    rmax = torch.amax(scores, dim=-1)
    return (o.detach().numpy(), lse.numpy(), rmax.numpy(), qt.grad.numpy(), kt.grad.numpy(),
            vt.grad.numpy())


STRUCTS = [
    ("local", 4, None),
    ("global", 4, None),
    ("dilated", 4, None),
    ("dilated_pages", 8, None),
    ("random", 5, 0.3),
    ("full", 3, None),
]


# ---------------------------------------------------------------------------
# Library routine: dense fp64 SDPA with the expanded block mask (the page's own
# reference computation) and its autograd gradients.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kind,nb,dens", STRUCTS)
def test_fwd_matches_dense_sdpa(oracle_mod, kind, nb, dens):
    bm = W.block_mask(kind, nb, density=dens)
    rp, ci = W.bsr_from_block_mask(bm)
    q, k, v, do = _inputs(1, 2, nb * B, 32, seed=3)
    o, m, l_ = oracle_mod.fwd(q, k, v, rp, ci)
    o_ref, lse_ref, max_ref, *_ = dense_reference(q, k, v, do, bm)
    assert _rel(o, o_ref) < 1e-12
    assert _rel(m, max_ref) < 1e-13
    assert _rel(m + np.log(l_), lse_ref) < 1e-13


@pytest.mark.parametrize("kind,nb,dens", STRUCTS)
def test_bwd_matches_dense_autograd(oracle_mod, kind, nb, dens):
    bm = W.block_mask(kind, nb, density=dens)
    rp, ci = W.bsr_from_block_mask(bm)
    q, k, v, do = _inputs(1, 2, nb * B, 32, seed=4)
    dq, dk, dv = oracle_mod.bwd(q, k, v, do, rp, ci)
    *_, dq_r, dk_r, dv_r = dense_reference(q, k, v, do, bm)
    assert _rel(dq, dq_r) < 1e-11
    assert _rel(dk, dk_r) < 1e-11
    assert _rel(dv, dv_r) < 1e-11


def test_custom_scale(oracle_mod):
    bm = W.block_mask("global", 4)
    rp, ci = W.bsr_from_block_mask(bm)
    q, k, v, do = _inputs(1, 1, 4 * B, 16, seed=5)
    o, m, l_ = oracle_mod.fwd(q, k, v, rp, ci, scale=0.37)
    dq, dk, dv = oracle_mod.bwd(q, k, v, do, rp, ci, scale=0.37)
    o_r, lse_r, max_r, dq_r, dk_r, dv_r = dense_reference(q, k, v, do, bm, scale=0.37)
    for x, r in ((o, o_r), (m, max_r), (m + np.log(l_), lse_r), (dq, dq_r), (dk, dk_r), (dv, dv_r)):
        assert _rel(x, r) < 1e-11


# ---------------------------------------------------------------------------
# Finite differences of L = <O, dO> (the pages' gradcheck: fp64, seq 256).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kind", ["diagonal", "lower", "full"])
def test_finite_differences(oracle_mod, kind):
    nb = 2
    if kind == "lower":
        bm = np.tril(np.ones((nb, nb), dtype=bool))
    else:
        bm = W.block_mask(kind, nb)
    rp, ci = W.bsr_from_block_mask(bm)
    q, k, v, do = _inputs(1, 1, nb * B, 16, seed=6)
    dq, dk, dv = oracle_mod.bwd(q, k, v, do, rp, ci)

    def loss(qq, kk, vv):
        o, _, _ = oracle_mod.fwd(qq, kk, vv, rp, ci)
        return float(np.sum(o * do))

    rng = np.random.default_rng(0)
    eps = 1e-6
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        # a few single entries (one in each block) and one random direction
        for _ in range(3):
            idx = (0, 0, int(rng.integers(0, nb * B)), int(rng.integers(0, 16)))
            args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
            args[name][idx] += eps
            lp = loss(args["q"], args["k"], args["v"])
            args[name][idx] -= 2 * eps
            lm = loss(args["q"], args["k"], args["v"])
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(grad[idx])), (name, idx, fd, grad[idx])
        direction = rng.standard_normal(q.shape)
        args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
        args[name] = args[name] + eps * direction
        lp = loss(args["q"], args["k"], args["v"])
        args[name] = args[name] - 2 * eps * direction
        lm = loss(args["q"], args["k"], args["v"])
        fd = (lp - lm) / (2 * eps)
        an = float(np.sum(grad * direction))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


# ---------------------------------------------------------------------------
# Closed forms, special cases and invariants.
# ---------------------------------------------------------------------------
def test_diagonal_mask_is_per_block_dense_attention(oracle_mod):
    nb = 3
    bm = W.block_mask("diagonal", nb)
    rp, ci = W.bsr_from_block_mask(bm)
    q, k, v, do = _inputs(1, 2, nb * B, 16, seed=7)
    o, _, _ = oracle_mod.fwd(q, k, v, rp, ci)
    for blk in range(nb):
        sl = slice(blk * B, (blk + 1) * B)
        ref = F.scaled_dot_product_attention(*(torch.from_numpy(x[:, :, sl]) for x in (q, k, v)))
        assert _rel(o[:, :, sl], ref.numpy()) < 1e-12


def test_zero_queries_give_uniform_attention(oracle_mod):
    """Q = 0: every attended score is 0, so row_max = 0, row_denom = number of
    attended keys and O is the mean of the attended values."""
    bm = W.block_mask("global", 5)
    rp, ci = W.bsr_from_block_mask(bm)
    _, k, v, _ = _inputs(1, 1, 5 * B, 16, seed=8)
    q = np.zeros_like(k)
    o, m, l_ = oracle_mod.fwd(q, k, v, rp, ci)
    for r in range(5 * B):
        cols = ci[rp[r // B]:rp[r // B + 1]]
        keys = np.concatenate([np.arange(c * B, (c + 1) * B) for c in cols])
        assert m[0, 0, r] == 0.0
        assert l_[0, 0, r] == len(keys)
        np.testing.assert_allclose(o[0, 0, r], v[0, 0, keys].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_forward_invariants(oracle_mod):
    bm = W.block_mask("random", 6, density=0.3, seed=2)
    rp, ci = W.bsr_from_block_mask(bm)
    q, k, v, do = _inputs(2, 2, 6 * B, 24, seed=9)
    q = q * 3.0  # sharper softmax
    o, m, l_ = oracle_mod.fwd(q, k, v, rp, ci)
    n_att = np.repeat((rp[1:] - rp[:-1]) * B, B)
    # 1 <= row_denom <= number of attended keys
    assert np.all(l_ >= 1.0 - 1e-12) and np.all(l_ <= n_att[None, None, :] + 1e-9)
    # row_max bounds every attended score; O lies in the box of attended values
    scale = 1.0 / math.sqrt(24)
    for r in range(0, 6 * B, 37):
        cols = ci[rp[r // B]:rp[r // B + 1]]
        keys = np.concatenate([np.arange(c * B, (c + 1) * B) for c in cols])
        s = scale * (k[0, 1, keys] @ q[0, 1, r])
        assert np.all(s <= m[0, 1, r] + 1e-12)
        vk = v[0, 1, keys]
        assert np.all(o[0, 1, r] <= vk.max(axis=0) + 1e-12)
        assert np.all(o[0, 1, r] >= vk.min(axis=0) - 1e-12)
    # constant V -> O equals that constant (softmax rows sum to one)
    vc = np.full_like(v, 0.75)
    o2, _, _ = oracle_mod.fwd(q, k, vc, rp, ci)
    np.testing.assert_allclose(o2, 0.75, rtol=0, atol=1e-13)


def test_backward_invariants(oracle_mod):
    bm = W.block_mask("random", 6, density=0.3, seed=2)
    rp, ci = W.bsr_from_block_mask(bm)
    q, k, v, do = _inputs(1, 2, 6 * B, 24, seed=10)
    dq, dk, dv = oracle_mod.bwd(q, k, v, do, rp, ci)
    # sum_c dS_rc = 0 for every row  =>  sum over keys of dK = 0 per head
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-11)
    # rows of P sum to one  =>  sum over keys of dV = sum over rows of dO
    np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=1e-12, atol=1e-11)
    # scores depend on Q K^T only: <Q, dQ> = <K, dK> per head
    np.testing.assert_allclose((q * dq).sum(axis=(2, 3)), (k * dk).sum(axis=(2, 3)), rtol=1e-10)
    # dO = 0 -> every gradient is zero
    z = oracle_mod.bwd(q, k, v, np.zeros_like(do), rp, ci)
    for g in z:
        assert np.all(g == 0.0)
    # constant V -> O does not depend on Q or K -> dQ = dK = 0
    dq2, dk2, _ = oracle_mod.bwd(q, k, np.full_like(v, -1.25), do, rp, ci)
    np.testing.assert_allclose(dq2, 0.0, atol=1e-12)
    np.testing.assert_allclose(dk2, 0.0, atol=1e-12)


def test_empty_rows_and_columns(oracle_mod):
    """A block row with no stored block: O = 0, row_max = -inf, row_denom = 0,
    dQ = 0; keys no row attends to: dK = dV = 0."""
    bm = np.zeros((3, 3), dtype=bool)
    bm[0, 0] = bm[2, 0] = bm[2, 2] = True  # row 1 empty, column 1 unreferenced
    rp, ci = W.bsr_from_block_mask(bm)
    q, k, v, do = _inputs(1, 1, 3 * B, 16, seed=11)
    o, m, l_ = oracle_mod.fwd(q, k, v, rp, ci)
    dq, dk, dv = oracle_mod.bwd(q, k, v, do, rp, ci)
    sl = slice(B, 2 * B)
    assert np.all(o[:, :, sl] == 0) and np.all(np.isneginf(m[:, :, sl])) and np.all(l_[:, :, sl] == 0)
    assert np.all(dq[:, :, sl] == 0) and np.all(dk[:, :, sl] == 0) and np.all(dv[:, :, sl] == 0)
    # the non-empty rows still agree with dense attention
    o_r, _, _, dq_r, dk_r, dv_r = dense_reference(q, k, v, do, bm)
    keep = np.r_[0:B, 2 * B:3 * B]
    assert _rel(o[:, :, keep], o_r[:, :, keep]) < 1e-12
    assert _rel(dq[:, :, keep], dq_r[:, :, keep]) < 1e-11
    assert _rel(dk[:, :, keep], dk_r[:, :, keep]) < 1e-11
    assert _rel(dv[:, :, keep], dv_r[:, :, keep]) < 1e-11


def test_two_pass_statistics_route(oracle_mod):
    """The pages' two-pass route: per stored block (tile_max, tile_sumexp),
    then a log-sum-exp reduction per row, gives the same row statistics."""
    bm = W.block_mask("global", 5)
    rp, ci = W.bsr_from_block_mask(bm)
    q, k, v, _ = _inputs(1, 1, 5 * B, 16, seed=12)
    _, m, l_ = oracle_mod.fwd(q, k, v, rp, ci)
    scale = 1.0 / 4.0
    for I in range(5):
        tiles = []
        for J in ci[rp[I]:rp[I + 1]]:
            s = scale * q[0, 0, I * B:(I + 1) * B] @ k[0, 0, J * B:(J + 1) * B].T
            tmax = s.max(axis=1)
            tiles.append((tmax, np.exp(s - tmax[:, None]).sum(axis=1)))
        gmax = np.max([t[0] for t in tiles], axis=0)
        gsum = np.sum([t[1] * np.exp(t[0] - gmax) for t in tiles], axis=0)
        np.testing.assert_allclose(m[0, 0, I * B:(I + 1) * B], gmax, rtol=1e-14)
        np.testing.assert_allclose(l_[0, 0, I * B:(I + 1) * B], gsum, rtol=1e-12)


def test_sampled_entry_points_match_full(oracle_mod):
    bm = W.block_mask("global", 4)
    rp, ci = W.bsr_from_block_mask(bm)
    q, k, v, do = _inputs(1, 2, 4 * B, 16, seed=13)
    S = 4 * B
    o, m, l_ = oracle_mod.fwd(q, k, v, rp, ci)
    dq, dk, dv = oracle_mod.bwd(q, k, v, do, rp, ci)
    rows = np.array([0, 5, 127, 128, S + 300, 2 * S - 1])
    o_s, m_s, l_s = oracle_mod.fwd_rows(q, k, v, rp, ci, rows)
    dq_s = oracle_mod.bwd_rows(q, k, v, do, rp, ci, rows)
    dk_s, dv_s = oracle_mod.bwd_cols(q, k, v, do, rp, ci, rows)
    flat = lambda x: x.reshape(-1, x.shape[-1]) if x.ndim == 4 else x.reshape(-1)
    assert np.array_equal(o_s, flat(o)[rows]) and np.array_equal(m_s, flat(m)[rows])
    assert np.array_equal(l_s, flat(l_)[rows]) and np.array_equal(dq_s, flat(dq)[rows])
    np.testing.assert_allclose(dk_s, flat(dk)[rows], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dv_s, flat(dv)[rows], rtol=1e-13, atol=1e-15)


def test_batch_and_heads_are_independent(oracle_mod):
    bm = W.block_mask("local", 3)
    rp, ci = W.bsr_from_block_mask(bm)
    q, k, v, do = _inputs(2, 3, 3 * B, 16, seed=14)
    o, m, l_ = oracle_mod.fwd(q, k, v, rp, ci)
    o1, m1, l1 = oracle_mod.fwd(q[1:2, 2:3], k[1:2, 2:3], v[1:2, 2:3], rp, ci)
    assert np.array_equal(o[1, 2], o1[0, 0]) and np.array_equal(m[1, 2], m1[0, 0])


# ---------------------------------------------------------------------------
# Values the pages print or define (tests/golden).
# ---------------------------------------------------------------------------
def test_golden_page_masks():
    g = json.loads((GOLDEN / "pages_masks.json").read_text())
    for name, mat in g["masks"].items():
        kind, nb = name.rsplit("_nb", 1)
        assert np.array_equal(W.block_mask(kind, int(nb)), np.array(mat, dtype=bool)), name


def test_golden_stats_array_size():
    g = json.loads((GOLDEN / "pages_masks.json").read_text())["stats_array"]
    nb = g["seq_len"] // g["block_size"]
    rp, ci = W.bsr_from_block_mask(W.block_mask(g["mask"], nb))
    assert len(ci) * g["block_size"] * g["bytes_per_value"] == g["stats_bytes"]
    assert g["seq_len"] ** 2 * g["bytes_per_value"] == g["dense_score_bytes"]


def test_config_block_counts():
    """Closed-form block counts of the benchmark masks."""
    assert len(W.bsr_from_block_mask(W.block_mask("local", 4))[1]) == 3 * 4 - 2
    # global at nb: row 0 (nb) + column 0 (nb - 1) + band blocks outside both
    for nb in (4, 16, 64):
        band = 3 * nb - 2
        expect = nb + (nb - 1) + band - 3
        assert W.block_mask("global", nb).sum() == expect
    assert W.block_mask("global", 64).sum() == 314
    # dilated (benchmark form) at nb = 16: band 46, plus lower stride-4 blocks off the band
    nb = 16
    extra = sum(1 for i in range(nb) for j in range(nb) if i - j >= 4 and (i - j) % 4 == 0)
    assert W.block_mask("dilated", nb).sum() == (3 * nb - 2) + extra == 70
    # random: k drawn blocks plus the diagonal
    m = W.block_mask("random", 64, density=0.10, seed=0)
    assert m.sum() >= 410 and np.all(np.diag(m))


# ---------------------------------------------------------------------------
# Planted mistakes: each must fail at least one pin.
# ---------------------------------------------------------------------------
MUTANTS = [
    ("drop_scale", "const double s = pb->scale * dot(", "const double s = 1.0 * dot("),
    ("denominator_not_shifted", "l += exp(rr->p[i] - m);", "l += exp(rr->p[i]);"),
    ("output_from_keys", "const double *vc = vb + rr->keys[i] * D;", "const double *vc = kb + rr->keys[i] * D;"),
    ("diagonal_only_keys", "for (int64_t c = J * b; c < (J + 1) * b; ++c)", "for (int64_t c = I * b; c < (I + 1) * b; ++c)"),
    ("ds_sign", "rr->ds[i] = rr->p[i] * (dp - rr->delta);", "rr->ds[i] = rr->p[i] * (rr->delta - dp);"),
    ("delta_wrong_operand", "rr->delta = dot(dor, rr->o, D);", "rr->delta = dot(dor, dor, D);"),
    ("dq_from_values", "const double *kc = kall + (bh * S + rr.keys[i]) * D;", "const double *kc = pb.v + (bh * S + rr.keys[i]) * D;"),
    ("dk_no_scale", "dkc[d] += scale * rr.ds[i] * qr[d];", "dkc[d] += rr.ds[i] * qr[d];"),
    ("dv_from_ds", "dvc[d] += rr.p[i] * dor[d];", "dvc[d] += rr.ds[i] * dor[d];"),
    ("transposed_structure", "if (!block_stored(&pb, I, J)) continue;", "if (!block_stored(&pb, J, I)) continue;"),
    ("denominator_as_log", "rr->l = l;", "rr->l = log(l);"),
]


def _pins_pass(orc) -> bool:
    """A compact battery of the pins above, on an asymmetric structure."""
    bm = W.block_mask("dilated", 6)  # asymmetric: (4, 0) and (5, 1) stored, transposes not
    assert not np.array_equal(bm, bm.T)
    rp, ci = W.bsr_from_block_mask(bm)
    q, k, v, do = _inputs(1, 1, 6 * B, 16, seed=21)
    o, m, l_ = orc.fwd(q, k, v, rp, ci)
    dq, dk, dv = orc.bwd(q, k, v, do, rp, ci)
    o_r, lse_r, max_r, dq_r, dk_r, dv_r = dense_reference(q, k, v, do, bm)
    ok = True
    for x, r in ((o, o_r), (m, max_r), (m + np.log(np.maximum(l_, 1e-300)), lse_r),
                 (dq, dq_r), (dk, dk_r), (dv, dv_r)):
        ok &= bool(np.all(np.isfinite(x))) and _rel(x, r) < 1e-10
    return ok


def test_unmodified_oracle_passes_battery(oracle_mod):
    assert _pins_pass(oracle_mod.default())


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name,find,replace", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, find, replace):
    src = oracle.SOURCE.read_text()
    assert src.count(find) == 1, f"mutation anchor for {name} not found exactly once"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(find, replace))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(mutated), "-o",
                    str(lib), "-lm"], check=True)
    assert not _pins_pass(oracle.Oracle(lib)), f"planted mistake {name} passed every pin"


# ---------------------------------------------------------------------------
# Block-sparse times dense (C = A B over the stored blocks)
# ---------------------------------------------------------------------------
def _densify(bm_shape_nb, row_ptr, col_idx, blocks, b=128):
    """Dense A from its stored blocks, placed one by one (independent of the
    oracle's loop order)."""
    nb = bm_shape_nb
    a = np.zeros((nb * b, nb * b))
    for I in range(nb):
        for p in range(row_ptr[I], row_ptr[I + 1]):
            J = col_idx[p]
            a[I * b:(I + 1) * b, J * b:(J + 1) * b] = blocks[p]
    return a


@pytest.mark.parametrize("kind,nb,n", [("random", 4, 128), ("global", 3, 64), ("dilated", 6, 32), ("local", 2, 200)])
def test_spmm_equals_dense_matmul(oracle_mod, kind, nb, n):
    """The plain definition against a library dense product of the densified A."""
    bm = W.block_mask(kind, nb, density=0.4, seed=2)
    rp, ci = W.bsr_from_block_mask(bm)
    rng = np.random.default_rng(4)
    blocks = rng.standard_normal((len(ci), 128, 128))
    b_dense = rng.standard_normal((nb * 128, n))
    c = oracle_mod.spmm(blocks, b_dense, rp, ci)
    ref = _densify(nb, rp, ci, blocks) @ b_dense
    assert np.abs(c - ref).max() <= 1e-10 * np.abs(ref).max()


def test_spmm_identity_blocks_and_empty_rows(oracle_mod):
    """Identity blocks on the diagonal reproduce B; an empty block row gives zeros;
    a single off-diagonal block moves B's block row."""
    nb, n = 3, 16
    bm = np.zeros((nb, nb), dtype=bool)
    bm[0, 0] = bm[2, 1] = True  # block row 1 empty
    rp, ci = W.bsr_from_block_mask(bm)
    blocks = np.stack([np.eye(128), np.eye(128)])
    b_dense = np.random.default_rng(1).standard_normal((nb * 128, n))
    c = oracle_mod.spmm(blocks, b_dense, rp, ci)
    assert np.array_equal(c[:128], b_dense[:128])
    assert np.all(c[128:256] == 0)
    assert np.array_equal(c[256:], b_dense[128:256])
    empty = oracle_mod.spmm(np.zeros((0, 128, 128)), b_dense, np.zeros(nb + 1, dtype=np.int32),
                            np.zeros(0, dtype=np.int32))
    assert np.all(empty == 0)


def test_spmm_transposed_block_would_fail(oracle_mod):
    """A plausible mistake (blocks used transposed) disagrees with the dense
    product, so the dense comparison above pins the orientation."""
    bm = W.block_mask("random", 3, density=0.5, seed=5)
    rp, ci = W.bsr_from_block_mask(bm)
    rng = np.random.default_rng(6)
    blocks = rng.standard_normal((len(ci), 128, 128))
    b_dense = rng.standard_normal((3 * 128, 8))
    ref = _densify(3, rp, ci, blocks) @ b_dense
    wrong = oracle_mod.spmm(np.ascontiguousarray(blocks.transpose(0, 2, 1)), b_dense, rp, ci)
    assert np.abs(wrong - ref).max() > 1.0

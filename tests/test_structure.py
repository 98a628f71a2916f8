"""Host-side tests of the C ABI (CPU only, no GPU call is ever made).

The library loads and exports every function the header declares; the
structure builder validates its input, builds the BSC transpose, covers every
stored block exactly once in the row and the column schedules, splits long
lines into balanced segments and packs the documented plan; fwd/bwd reject
bad arguments before launching anything.
"""
import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

import workloads as W

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "bsr_attn.h"

bsr = pytest.importorskip("block_sparse_attention_bsr_amd")


@pytest.fixture(scope="module")
def lib():
    if not bsr.LIBRARY_PATH.exists():
        pytest.fail("libbsr_attn.so is not built (run __graft_entry__.build())")
    return bsr.library()


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsr_attn_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert "bsr_attn_build_structure" in names and "bsr_attn_fwd" in names and "bsr_attn_bwd" in names
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"


def _build_raw(lib, nb, row_ptr, col_idx, block=128, split=0):
    rp = np.ascontiguousarray(np.asarray(row_ptr, dtype=np.int32))
    ci = np.ascontiguousarray(np.asarray(col_idx, dtype=np.int32))
    h = ctypes.c_void_p()
    st = lib.bsr_attn_build_structure(nb, rp.ctypes.data, ci.ctypes.data if ci.size else None, block, split,
                                      ctypes.byref(h))
    if st == 0:
        lib.bsr_attn_destroy_structure(h)
    return st, lib.bsr_attn_last_error().decode()


@pytest.mark.parametrize("case,nb,rp,ci,block,status", [
    ("block_size", 2, [0, 1, 2], [0, 1], 64, 2),
    ("nb_zero", 0, [0], [], 128, 1),
    ("row_ptr_start", 2, [1, 2, 3], [0, 1, 0], 128, 1),
    ("row_ptr_decreasing", 3, [0, 2, 1, 3], [0, 1, 2], 128, 1),
    ("col_out_of_range", 2, [0, 1, 2], [0, 2], 128, 1),
    ("col_negative", 2, [0, 1, 2], [-1, 1], 128, 1),
    ("col_duplicate", 2, [0, 2, 3], [1, 1, 0], 128, 1),
    ("col_unsorted", 2, [0, 2, 3], [1, 0, 0], 128, 1),
    ("row_too_long", 2, [0, 3, 3], [0, 1, 1], 128, 1),
])
def test_build_rejects_malformed_structures(lib, case, nb, rp, ci, block, status):
    st, msg = _build_raw(lib, nb, rp, ci, block)
    assert st == status, (case, st, msg)
    assert msg


def test_build_rejects_negative_split(lib):
    st, msg = _build_raw(lib, 2, [0, 1, 2], [0, 1], 128, split=-1)
    assert st == 1 and "split" in msg


def test_empty_structure_is_valid():
    s = bsr.bsr_attn_build_structure([0, 0, 0], [])
    assert s.info["nnzb"] == 0
    assert s.info["n_row_items"] == 2 and s.info["n_col_items"] == 2  # one empty item per line


def _parse_plan(s):
    return _parse_plan_array(s.plan)


def _parse_plan_array(p):
    hdr = p[:24]
    assert hdr[0] == 0x42535241 and hdr[1] == 5
    nb, nnzb, nri, nci, nrm, ncm, nrs, ncs = hdr[2:10]
    oc, orow, ori, oci, orm, ocm, orp, ocp, orq, ocq, obb = hdr[10:21]
    ofine = int(hdr[21])
    assert ofine % 4 == 0 and list(hdr[22:24]) == [0, 0]
    for off in (oc, orow, ori, oci, orm, ocm, orp, ocp, orq, ocq, obb):
        assert off % 4 == 0  # int4-aligned

    def queues(table, n_items):
        out = {}
        for lv in range(7):
            n, off = 1 << lv, int(p[table + lv])
            assert off % 4 == 0
            offs = p[off:off + n + 1]
            out[n] = [list(p[off + n + 1 + offs[j]:off + n + 1 + offs[j + 1]]) for j in range(n)]
            assert offs[0] == 0 and offs[n] == n_items
        assert p[table + 7] == 0
        return out
    return {
        "row_queues": queues(orq, nri), "col_queues": queues(ocq, nci),
        "nb": nb, "nnzb": nnzb, "row_ptr": p[orp:orp + nb + 1], "col_ptr": p[ocp:ocp + nb + 1],
        "col_idx": p[oc:oc + nnzb], "row_idx": p[orow:orow + nnzb],
        "row_items": p[ori:ori + 4 * nri].reshape(-1, 4), "col_items": p[oci:oci + 4 * nci].reshape(-1, 4),
        "row_merges": p[orm:orm + 4 * nrm].reshape(-1, 4), "col_merges": p[ocm:ocm + 4 * ncm].reshape(-1, 4),
        "n_row_slots": nrs, "n_col_slots": ncs, "bsc_block": p[obb:obb + nnzb],
        "fine_offset": ofine,
    }


def _check_schedule(items, merges, lines_ptr, n_slots, T, nb):
    """Every block of every line covered exactly once; segments <= T and balanced;
    longest first; slots consecutive per split line in segment order."""
    covered = {}
    for line, first, end, slot in items:
        assert 0 <= line < nb and lines_ptr[line] <= first <= end <= lines_ptr[line + 1]
        assert end - first <= T
        covered.setdefault(line, []).append((first, end, slot))
    lens = [e - f for _, f, e, _ in items]
    assert lens == sorted(lens, reverse=True)
    merged = {int(m[0]): m for m in merges}
    used_slots = []
    for line in range(nb):
        segs = sorted(covered.get(line, []))
        n = lines_ptr[line + 1] - lines_ptr[line]
        if n == 0:
            assert segs == [(lines_ptr[line], lines_ptr[line], -1)]
            continue
        assert segs[0][0] == lines_ptr[line] and segs[-1][1] == lines_ptr[line + 1]
        for a, b in zip(segs, segs[1:]):
            assert a[1] == b[0]
        if n <= T:
            assert len(segs) == 1 and segs[0][2] == -1 and line not in merged
        else:
            m = merged[line]
            assert m[2] == len(segs) == -(-n // T)
            assert [sg[2] for sg in segs] == list(range(m[1], m[1] + m[2]))
            sizes = [sg[1] - sg[0] for sg in segs]
            assert max(sizes) - min(sizes) <= 1
            used_slots += [sg[2] for sg in segs]
    assert sorted(used_slots) == list(range(n_slots))


def _check_queues(items, queues):
    """Each schedule holds every item once, in the greedy longest-first
    assignment: item i goes to the queue with the least work so far (an
    empty line counts 1), lowest index on ties."""
    work = [max(1, int(e - f)) for _, f, e, _ in items]
    for n, qs in queues.items():
        assert sorted(i for q in qs for i in q) == list(range(len(items)))
        load = [0] * n
        expect = [[] for _ in range(n)]
        for i, wk in enumerate(work):
            j = min(range(n), key=lambda x: (load[x], x))
            expect[j].append(i)
            load[j] += wk
        assert qs == expect
        # the greedy bound: no queue exceeds the mean by more than one item
        assert max(load) <= sum(work) / n + max(work)


@pytest.mark.parametrize("kind,nb,dens,split", [
    ("global", 64, None, 0), ("global", 64, None, 8), ("global", 16, None, 3), ("dilated", 16, None, 0),
    ("random", 64, 0.10, 0), ("random", 64, 0.5, 0), ("random", 33, 0.2, 5), ("local", 4, None, 1),
    ("full", 7, None, 2), ("diagonal", 9, None, 0),
])
def test_plan_bsc_and_schedule(kind, nb, dens, split):
    bm = W.block_mask(kind, nb, density=dens, seed=1)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=split)
    T = s.info["split_threshold"]
    if split:
        assert T == split
    else:
        assert T >= 4
    pl = _parse_plan(s)
    assert pl["nb"] == nb and pl["nnzb"] == len(ci) == s.info["nnzb"]
    assert np.array_equal(pl["col_idx"], ci)
    assert np.array_equal(pl["row_ptr"], rp)
    # BSC: the same blocks, column by column, rows ascending
    col_ptr = np.concatenate([[0], np.cumsum(bm.sum(axis=0))])
    assert np.array_equal(pl["col_ptr"], col_ptr)
    for c in range(nb):
        rows = pl["row_idx"][col_ptr[c]:col_ptr[c + 1]]
        assert np.array_equal(rows, np.nonzero(bm[:, c])[0])
        # each BSC entry points at the same block's BSR position
        for q in range(col_ptr[c], col_ptr[c + 1]):
            b = pl["bsc_block"][q]
            r = pl["row_idx"][q]
            assert rp[r] <= b < rp[r + 1] and ci[b] == c
    _check_schedule(pl["row_items"], pl["row_merges"], rp, pl["n_row_slots"], T, nb)
    _check_schedule(pl["col_items"], pl["col_merges"], col_ptr, pl["n_col_slots"], T, nb)
    _check_queues(pl["row_items"], pl["row_queues"])
    _check_queues(pl["col_items"], pl["col_queues"])
    assert s.info["max_row_blocks"] == bm.sum(axis=1).max()
    assert s.info["max_col_blocks"] == bm.sum(axis=0).max()


@pytest.mark.parametrize("kind,nb,dens", [("local", 4, None), ("global", 64, None), ("random", 64, 0.10),
                                          ("dilated", 16, None), ("diagonal", 3, None), ("random", 64, 0.5)])
def test_fine_split_plan(kind, nb, dens):
    """With the automatic threshold the structure also carries a finer split
    (threshold max(1, ceil(nnzb / 256)) when smaller), embedded in the plan at
    off_fine_plan as the complete plan of that explicit threshold; launches
    with batch * heads * row items <= 64 run on it, and the workspace a
    problem needs follows that choice."""
    lib = bsr.library()
    bm = W.block_mask(kind, nb, density=dens, seed=1)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci)
    nnzb = len(ci)
    fine_T = max(1, -(-nnzb // 256))
    plan = _parse_plan(s)
    if fine_T >= s.info["split_threshold"]:
        assert plan["fine_offset"] == 0 and s.info["fine_split_threshold"] == 0
        return
    assert s.info["fine_split_threshold"] == fine_T
    off = plan["fine_offset"]
    assert off > 0 and off % 4 == 0
    explicit = bsr.bsr_attn_build_structure(rp, ci, split_threshold=fine_T)
    assert np.array_equal(s.plan[off:], explicit.plan)
    assert _parse_plan_array(s.plan[off:])["fine_offset"] == 0
    assert s.info["fine_n_row_items"] == explicit.info["n_row_items"]
    # the workspace follows the split the launch runs on
    S = nb * 128
    for BH in (1, 2, 8, 64):
        p = _problem(1, BH, S, 64, 1)
        runs_fine = BH * s.info["n_row_items"] <= 64
        ref = explicit if runs_fine else bsr.bsr_attn_build_structure(rp, ci, split_threshold=s.info["split_threshold"])
        for kind_ in (0, 1):
            assert lib.bsr_attn_workspace_bytes(s.handle, ctypes.byref(p), kind_) == \
                lib.bsr_attn_workspace_bytes(ref.handle, ctypes.byref(p), kind_)


def test_plan_binding(lib):
    """fwd/bwd/spmm accept only device plans bound to the structure they get:
    a plan of another structure is rejected before any launch."""
    a = bsr.bsr_attn_build_structure(*W.bsr_from_block_mask(W.block_mask("local", 4)))
    b = bsr.bsr_attn_build_structure(*W.bsr_from_block_mask(W.block_mask("global", 4)))
    pa, pb = FAKE, FAKE + 4096
    nbytes = lib.bsr_attn_structure_plan_bytes(a.handle)
    assert lib.bsr_attn_structure_bind_plan(a.handle, pa, nbytes - 4) == 1  # wrong size
    assert lib.bsr_attn_structure_bind_plan(a.handle, pa + 8, nbytes) == 1  # misaligned
    assert lib.bsr_attn_structure_bind_plan(a.handle, pa, nbytes) == 0
    assert lib.bsr_attn_structure_bind_plan(a.handle, pa, nbytes) == 0  # again: no-op
    assert lib.bsr_attn_structure_bind_plan(b.handle, pb, lib.bsr_attn_structure_plan_bytes(b.handle)) == 0
    p = _problem()
    # b's plan passed with a: rejected as not bound, before the (fake) launch
    assert _fwd(lib, a, p, plan=pb) == 1
    assert "bound" in lib.bsr_attn_last_error().decode()
    args = [FAKE] * 10
    assert lib.bsr_attn_bwd(a.handle, pb, ctypes.byref(p), *args, FAKE, 1 << 30, None) == 1
    p16 = _problem(dtype=1)
    assert lib.bsr_attn_bwd_ds(a.handle, pb, ctypes.byref(p16), *args, FAKE, 1 << 30, None) == 1
    assert lib.bsr_spmm(a.handle, pb, 1, 128, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert "bound" in lib.bsr_attn_last_error().decode()
    # unbinding: a's own plan is then rejected too
    assert lib.bsr_attn_structure_unbind_plan(a.handle, pa) == 0
    assert lib.bsr_attn_structure_unbind_plan(a.handle, pa) == 1
    assert lib.bsr_attn_fwd(a.handle, pa, ctypes.byref(p), *([FAKE] * 6), FAKE, 1 << 30, None) == 1
    assert "bound" in lib.bsr_attn_last_error().decode()


def test_binding_validates_structure_arrays():
    """The binding checks what the C builder cannot see: array ranks and
    col_idx's length against row_ptr[-1] (the builder reads exactly
    row_ptr[nb] entries)."""
    with pytest.raises(ValueError):
        bsr.bsr_attn_build_structure([0, 2, 3], [0, 1])  # short col_idx
    with pytest.raises(ValueError):
        bsr.bsr_attn_build_structure([0, 1, 2], [0, 1, 1])  # extra entry
    with pytest.raises(ValueError):
        bsr.bsr_attn_build_structure(np.array([[0, 1, 2]]), [0, 1])
    with pytest.raises(ValueError):
        bsr.bsr_attn_build_structure([0], [])


def test_global_mask_schedule_splits_row_and_column_zero():
    bm = W.block_mask("global", 64)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=8)
    assert s.info["nnzb"] == 314
    assert s.info["n_row_merges"] == 1 and s.info["n_col_merges"] == 1
    assert s.info["n_row_slots"] == 8 and s.info["n_col_slots"] == 8
    assert s.info["n_row_items"] == 63 + 8


def _problem(B=1, H=2, S=512, D=64, dtype=0, scale=0.125):
    return bsr._Problem(B, H, S, D, dtype, scale)


def test_workspace_sizes(lib):
    bm = W.block_mask("global", 4)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci, split_threshold=2)
    B, H, S, D = 2, 3, 512, 64
    p = _problem(B, H, S, D)
    fwd = lib.bsr_attn_workspace_bytes(s.handle, ctypes.byref(p), 0)
    bwd = lib.bsr_attn_workspace_bytes(s.handle, ctypes.byref(p), 1)
    rs, cs = s.info["n_row_slots"], s.info["n_col_slots"]
    counts_r, counts_c = bm.sum(axis=1), bm.sum(axis=0)
    assert rs == sum(-(-n // 2) for n in counts_r if n > 2)
    assert cs == sum(-(-n // 2) for n in counts_c if n > 2)
    assert fwd >= rs * B * H * 128 * (D + 2) * 4
    assert bwd >= 2 * B * H * S * 4 + (rs + 2 * cs) * B * H * 128 * D * 4
    assert lib.bsr_attn_workspace_bytes(s.handle, ctypes.byref(_problem(S=256)), 0) == 0
    nosplit = bsr.bsr_attn_build_structure(rp, ci, split_threshold=64)
    assert lib.bsr_attn_workspace_bytes(nosplit.handle, ctypes.byref(p), 0) == 0


FAKE = 1 << 20  # an aligned, non-null address; never dereferenced: every call below fails validation


def _bind(lib, s, ptr=FAKE):
    """Bind a (fake) device plan address to s: host bookkeeping only."""
    assert lib.bsr_attn_structure_bind_plan(s.handle, ptr, lib.bsr_attn_structure_plan_bytes(s.handle)) == 0
    return ptr


def _fwd(lib, s, p, ptrs=None, ws=None, ws_bytes=0, plan=FAKE):
    ptrs = ptrs or [FAKE] * 6
    if s is not None and plan == FAKE:
        _bind(lib, s)
    return lib.bsr_attn_fwd(s.handle if s else None, plan, ctypes.byref(p) if p else None, *ptrs, ws, ws_bytes,
                            None)


@pytest.mark.parametrize("field,value,status", [
    ("seq_len", 384, 1), ("head_dim", 8, 2), ("head_dim", 40, 2), ("head_dim", 272, 2), ("head_dim", 512, 2),
    ("dtype", 7, 1), ("batch", 0, 1),
    ("heads", -1, 1), ("scale", 0.0, 1), ("scale", float("nan"), 1), ("scale", float("inf"), 1),
])
def test_fwd_rejects_bad_problem(lib, field, value, status):
    s = bsr.bsr_attn_build_structure(*W.bsr_from_block_mask(W.block_mask("local", 4)))
    p = _problem()
    setattr(p, field, value)
    assert _fwd(lib, s, p) == status
    assert lib.bsr_attn_last_error().decode()


def test_fp32_head_dim_256_is_unsupported(lib):
    s = bsr.bsr_attn_build_structure(*W.bsr_from_block_mask(W.block_mask("local", 4)))
    assert _fwd(lib, s, _problem(D=256, dtype=0)) == 2
    assert _fwd(lib, s, _problem(D=144, dtype=0)) == 2  # past the widest fp32 instance (128)


def _align256(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("dtype,D,width", [(1, 16, 32), (1, 48, 64), (1, 96, 128), (1, 112, 128), (1, 192, 256),
                                           (0, 16, 32), (0, 80, 128), (2, 160, 256)])
def test_padded_head_dim_workspace(lib, dtype, D, width):
    """A head dim without an instance of its own runs at the next instantiated
    width: its workspace is that width's own, then zero-padded copies of
    4 (forward) or 8 (backward) [B*H*S, width] tensors."""
    bm = W.block_mask("global", 4)
    s = bsr.bsr_attn_build_structure(*W.bsr_from_block_mask(bm), split_threshold=2)
    B, H, S = 2, 3, 512
    e = 4 if dtype == 0 else 2
    pad = _align256(B * H * S * width * e)
    for backward, n in ((0, 4), (1, 8)):
        native = lib.bsr_attn_workspace_bytes(s.handle, ctypes.byref(_problem(B, H, S, width, dtype)), backward)
        padded = lib.bsr_attn_workspace_bytes(s.handle, ctypes.byref(_problem(B, H, S, D, dtype)), backward)
        assert padded == _align256(native) + n * pad


def test_head_dim_512_workspace(lib):
    """head_dim 512 (16-bit): the forward needs only the fp32 partials of its
    split rows (O, reference max, sum, row max), as at the other widths; the
    backward materialises P and dS blocks and needs delta and lse2 plus fp32
    partials of the split rows and columns; 400 pads to 512 and adds its
    operand copies."""
    bm = W.block_mask("global", 4)
    s = bsr.bsr_attn_build_structure(*W.bsr_from_block_mask(bm), split_threshold=2)
    B, H, S, D = 1, 2, 512, 512
    nnzb, rs, cs = s.info["nnzb"], s.info["n_row_slots"], s.info["n_col_slots"]
    blocks = B * H * nnzb * 128 * 128
    a = _align256
    part_rows = B * H * rs * 128
    fwd = a(part_rows * D * 4) + 3 * a(part_rows * 4) if rs else 0
    bwd = 2 * a(B * H * S * 4) + a(blocks * 2) + a(blocks * 2) + \
        a(B * H * rs * 128 * D * 4) + a(B * H * cs * 128 * D * 4)
    for dtype in (1, 2):
        assert lib.bsr_attn_workspace_bytes(s.handle, ctypes.byref(_problem(B, H, S, D, dtype)), 0) == fwd
        assert lib.bsr_attn_workspace_bytes(s.handle, ctypes.byref(_problem(B, H, S, D, dtype)), 1) == bwd
        assert lib.bsr_attn_workspace_bytes(s.handle, ctypes.byref(_problem(B, H, S, D, dtype)), 2) == bwd
        assert lib.bsr_attn_workspace_bytes(s.handle, ctypes.byref(_problem(B, H, S, 400, dtype)), 0) == \
            a(fwd) + 4 * a(B * H * S * 512 * 2)
    assert _fwd(lib, s, _problem(D=528, dtype=1)) == 2  # past 512


def test_ds_backward_workspace_and_dtypes(lib):
    """The dS-storing backward needs the backward's workspace, then the dS
    blocks: B*H*nnzb blocks of 128 x 128 in the operand dtype; it takes no
    fp32 (workspace 0, status unsupported)."""
    bm = W.block_mask("global", 4)
    s = bsr.bsr_attn_build_structure(*W.bsr_from_block_mask(bm), split_threshold=2)
    B, H, S = 2, 3, 512
    nnzb = s.info["nnzb"]
    for dtype, e in ((1, 2), (2, 2)):
        for D in (64, 256):
            p = _problem(B, H, S, D, dtype)
            bwd = lib.bsr_attn_workspace_bytes(s.handle, ctypes.byref(p), 1)
            assert lib.bsr_attn_workspace_bytes(s.handle, ctypes.byref(p), 2) == \
                _align256(bwd) + B * H * nnzb * 128 * 128 * e
    p = _problem(B, H, S, 64, 0)
    assert lib.bsr_attn_workspace_bytes(s.handle, ctypes.byref(p), 2) == 0
    assert lib.bsr_attn_workspace_bytes(s.handle, ctypes.byref(p), 3) == 0
    _bind(lib, s)
    args = [FAKE] * 10
    assert lib.bsr_attn_bwd_ds(s.handle, FAKE, ctypes.byref(p), *args, FAKE, 1 << 30, None) == 2
    assert "bf16 or fp16" in lib.bsr_attn_last_error().decode()


def test_fp16_is_a_dtype_and_unknown_dtypes_are_invalid(lib):
    s = bsr.bsr_attn_build_structure(*W.bsr_from_block_mask(W.block_mask("local", 4)))
    assert _fwd(lib, s, _problem(D=40, dtype=2)) == 2  # valid dtype, unsupported head_dim
    assert _fwd(lib, s, _problem(D=64, dtype=3)) == 1


def test_fwd_rejects_null_and_misaligned(lib):
    s = bsr.bsr_attn_build_structure(*W.bsr_from_block_mask(W.block_mask("local", 4)))
    p = _problem()
    assert _fwd(lib, None, p) == 1
    assert _fwd(lib, s, None) == 1
    assert _fwd(lib, s, p, plan=None) == 1
    for i in range(6):
        ptrs = [FAKE] * 6
        ptrs[i] = None
        assert _fwd(lib, s, p, ptrs, ws=FAKE, ws_bytes=1 << 30) == 1
        ptrs[i] = FAKE + 4
        assert _fwd(lib, s, p, ptrs, ws=FAKE, ws_bytes=1 << 30) == 1
        assert "aligned" in lib.bsr_attn_last_error().decode()


def test_fwd_rejects_small_workspace(lib):
    s = bsr.bsr_attn_build_structure(*W.bsr_from_block_mask(W.block_mask("global", 4)), split_threshold=2)
    p = _problem()
    need = lib.bsr_attn_workspace_bytes(s.handle, ctypes.byref(p), 0)
    assert need > 0
    assert _fwd(lib, s, p, ws=FAKE, ws_bytes=need - 1) == 3
    assert _fwd(lib, s, p, ws=None, ws_bytes=need) == 1


def test_bwd_rejects_bad_arguments(lib):
    s = bsr.bsr_attn_build_structure(*W.bsr_from_block_mask(W.block_mask("local", 4)))
    p = _problem()
    need = lib.bsr_attn_workspace_bytes(s.handle, ctypes.byref(p), 1)
    assert need > 0  # delta and log-sum-exp rows at least
    _bind(lib, s)
    args = [FAKE] * 10
    assert lib.bsr_attn_bwd(s.handle, FAKE, ctypes.byref(p), *args, FAKE, need - 1, None) == 3
    for i in range(10):
        bad = list(args)
        bad[i] = None
        assert lib.bsr_attn_bwd(s.handle, FAKE, ctypes.byref(p), *bad, FAKE, need, None) == 1
    p.head_dim = 40
    assert lib.bsr_attn_bwd(s.handle, FAKE, ctypes.byref(p), *args, FAKE, need, None) == 2


def test_binding_rejects_cpu_tensors():
    import torch
    s = bsr.bsr_attn_build_structure(*W.bsr_from_block_mask(W.block_mask("local", 4)))
    q = torch.zeros(1, 1, 512, 64)
    with pytest.raises(ValueError):
        bsr.bsr_attn_fwd(s, q, q, q)


@pytest.mark.parametrize("name,expect_split", [
    ("c5_bf16_rand01", False),  # mean 1.6 -> 4, longest line 5: one block over, no split
    ("c5_bf16_rand05", True),   # mean 4.1 -> 8, longest line 10: split
    ("c3_bf16_global", True),   # mean 4.9 -> 8, longest line 64: split
    ("c2_bf16_dilated", False), # mean 4.4 -> 8, longest line 6
])
def test_automatic_split_threshold(name, expect_split):
    bm = np.asarray(W.config_mask(name)).astype(bool)
    rp, ci = W.bsr_from_block_mask(bm)
    s = bsr.bsr_attn_build_structure(rp, ci)
    info = s.info
    nb = bm.shape[0]
    base = max(4, -(-3 * -(-len(ci) // nb) // 2))
    longest = int(max(bm.sum(axis=0).max(), bm.sum(axis=1).max()))
    T = info["split_threshold"]
    assert T == (longest if longest <= base + 1 and longest > base else base)
    has_merges = info["n_row_merges"] + info["n_col_merges"] > 0
    assert has_merges == expect_split == (longest > T)


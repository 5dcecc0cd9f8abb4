"""CPU-only checks of the MMQ launch plan (qmm_mmq_plan, qmm_mmq_plan_work): host
arithmetic that decides how the output tiles map onto work-groups and which
tiles are split along the inner dimension.  Over thousands of seeded shapes and
GPU sizes the plan must cover every output tile exactly once, split only a tail
that runs in one wave, give every k-group of every slice at least one
super-block, and keep its partials inside the scratch -- properties that a wrong
plan breaks without any GPU in the loop (a division by zero in the planner
first surfaced as a crash on the GPU)."""
import os
import re

import numpy as np
import pytest

import quant_q8_gemm_amd as qmm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TYPES = [qmm.Q4_K, qmm.Q6_K, qmm.Q4_K_PACKED]
CUS = [1, 2, 7, 32, 80, 104, 120, 228, 256, 304]


def _cases(n, seed):
    """Seeded shapes: rows, inner and tokens log-uniform over the whole range the
    library accepts (tokens and rows capped so one launch holds the tiles)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        type_ = TYPES[int(rng.integers(0, 3))]
        od = int(np.exp(rng.uniform(0, np.log(qmm_max_od()))))
        id_ = 256 * int(np.exp(rng.uniform(0, np.log(4096))))
        n_tok = int(np.exp(rng.uniform(0, np.log(20000))))
        cus = CUS[int(rng.integers(0, len(CUS)))]
        out.append((type_, od, id_, n_tok, cus))
    return out


def qmm_max_od():
    return 1 << 21


def _edge_cases():
    """Row counts that put the tile count at and around whole waves (one to seven
    of them) for every tile height/width and residency the planner uses, on MI355X
    and other GPU sizes: exactly k full waves, one row tile more or fewer, single
    tiles, one super-block."""
    out = []
    for cus in (256, 304, 1, 3):
        for type_ in TYPES:
            for n_tok in (1, 64, 128, 129, 512, 2048, 3314, 4096):
                ods = {1, cus * 64, cus * 128 + 1}
                for waves in (1, 2, 3, 4, 7):
                    for per_cu in (1, 2, 4):
                        for tile_tokens in (64, 128):
                            rows = waves * cus * per_cu // -(-n_tok // tile_tokens) * 64
                            ods |= {rows - 64, rows - 1, rows, rows + 1, rows + 64}
                for od in sorted(o for o in ods if 1 <= o <= qmm_max_od()):
                    for id_ in (256, 512, 4096, 11008 // 256 * 256):
                        out.append((type_, od, id_, n_tok, cus))
    return out


def _check_plan(type_, od, id_, n_tok, cus):
    p = qmm.mmq_plan(type_, od, id_, n_tok, cus)
    nsb = id_ // 256
    assert p.nsb == nsb
    # the tiles cover the output, with no tile of padding only
    assert p.row_tiles == -(-od // p.tile_rows) and p.tok_tiles == -(-n_tok // p.tile_tokens)
    # 16 waves of 64 lanes per compute unit in every geometry
    assert p.threads == 64 * (p.tile_rows // 32) * (p.tile_tokens // 32) * p.k_groups
    assert p.per_cu * p.threads == 1024
    tiles = p.row_tiles * p.tok_tiles
    slots = cus * p.per_cu
    assert p.n_tail == (p.row_tiles - p.dp_row_tiles) * p.tok_tiles
    assert p.work_groups == p.dp_row_tiles * p.tok_tiles + p.n_tail * p.split
    assert (p.split == 1) == (p.n_tail == 0)
    if p.n_tail:
        assert p.split >= 2
        assert p.split * p.k_groups <= nsb, "a k-group of a slice without a super-block"
        assert p.n_tail * p.split <= slots, "the split tail must run in one wave"
        assert tiles % slots != 0, "whole waves are never split"
        # the data-parallel part: the whole waves, rounded down to whole row tiles
        assert p.dp_row_tiles == (tiles // slots) * slots // p.tok_tiles
        assert p.scratch_bytes == p.n_tail * p.split * p.tile_rows * p.tile_tokens * 4
    else:
        assert p.dp_row_tiles == p.row_tiles and p.scratch_bytes == 0
    assert p.scratch_bytes <= cus * 64 * 1024
    if cus == 256:
        assert p.scratch_bytes <= 16 << 20, "qmm_mmq_noalloc's static scratch must hold every MI355X plan"
    assert p.work_groups * p.threads < 1 << 32
    return p


def test_plan_struct_matches_header():
    hdr = open(os.path.join(ROOT, "include", "qmm.h")).read()
    end = hdr.index("} qmm_plan;")
    body = hdr[hdr.rindex("typedef struct {", 0, end) + len("typedef struct {"):end]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    assert re.findall(r"(\w+)\s*;", body) == [f[0] for f in qmm.Plan._fields_]
    consts = dict(re.findall(r"#define (QMM_[A-Z0-9_]+) \(?(-?\d+)\)?", hdr))
    assert int(consts["QMM_MAX_CUS"]) == qmm.MAX_CUS


def test_plan_invariants_random_shapes():
    tails = 0
    for case in _cases(6000, seed=5):
        tails += _check_plan(*case).n_tail > 0
    assert tails > 200, "the sweep must reach split tails"


def test_plan_invariants_around_whole_waves():
    kinds = set()
    for case in _edge_cases():
        p = _check_plan(*case)
        tiles, slots = p.row_tiles * p.tok_tiles, case[4] * p.per_cu
        kinds.add((p.many, p.n_tail > 0, tiles % slots == 0, tiles > 2 * slots))
    # both geometries, with and without a tail, exact multiples, and tails behind several waves
    assert {(1, True, False, True), (1, False, True, True), (0, True, False, False), (0, False, False, False)} <= kinds


def _coverage(type_, od, id_, n_tok, cus):
    p = _check_plan(type_, od, id_, n_tok, cus)
    nsb = id_ // 256
    whole = np.zeros((p.row_tiles, p.tok_tiles), np.int32)
    slices = {}
    for wg in range(p.work_groups):
        rt, tt, s0, s1 = qmm.mmq_plan_work(p, wg)
        assert 0 <= rt < p.row_tiles and 0 <= tt < p.tok_tiles
        if wg < p.dp_row_tiles * p.tok_tiles:
            assert rt < p.dp_row_tiles and (s0, s1) == (0, nsb)
            whole[rt, tt] += 1
        else:
            assert rt >= p.dp_row_tiles
            # each k-group of the slice gets at least one super-block
            assert s1 - s0 >= p.k_groups
            slices.setdefault((rt, tt), []).append((s0, s1))
    assert (whole[:p.dp_row_tiles] == 1).all(), "a data-parallel tile computed twice or never"
    assert (whole[p.dp_row_tiles:] == 0).all()
    assert len(slices) == p.n_tail
    for key, sl in slices.items():
        assert len(sl) == p.split
        # consecutive work-groups take consecutive slices that partition [0, nsb)
        assert sl[0][0] == 0 and sl[-1][1] == nsb
        assert all(a[1] == b[0] for a, b in zip(sl, sl[1:])), f"slices of {key} leave a gap or overlap"
    return p


@pytest.mark.parametrize("case", [
    (qmm.Q6_K, 4096, 11008 // 256 * 256, 3314, 256),   # short last wave behind three full ones
    (qmm.Q6_K, 4097, 11008 // 256 * 256, 509, 256),    # ragged second wave (few tiles)
    (qmm.Q4_K, 11008, 4096, 512, 256),                 # ragged second wave (many tiles)
    (qmm.Q4_K, 4096, 4096, 3314, 256),                 # several waves, no split
    (qmm.Q4_K_PACKED, 512, 3072, 300, 256),            # every tile a tail tile
    (qmm.Q6_K, 4096, 3072, 3072, 256),                 # whole waves exactly
    (qmm.Q4_K, 1, 256, 1, 256),                        # one tile, one super-block
    (qmm.Q6_K, 70000, 256, 1, 256),                    # one super-block: nothing to split
    (qmm.Q4_K, 5000, 7424, 995, 304),
    (qmm.Q6_K, 3000, 2048, 700, 7),
    (qmm.Q4_K, 2000, 1024, 3000, 1),
])
def test_plan_work_covers_every_tile_once(case):
    _coverage(*case)


def test_plan_work_covers_random_tail_shapes():
    done = 0
    for case in _cases(3000, seed=23):
        p = qmm.mmq_plan(*case)
        if p.n_tail and p.work_groups <= 20000:
            _coverage(*case)
            done += 1
            if done == 40:
                break
    assert done == 40
    # and a few without a tail
    for case in [c for c in _cases(200, seed=3) if qmm.mmq_plan(*c).work_groups <= 5000][:10]:
        _coverage(*case)


def test_plan_empty_batch():
    p = qmm.mmq_plan(qmm.Q4_K, 4096, 4096, 0, 256)
    assert p.work_groups == 0 and p.scratch_bytes == 0 and p.nsb == 16


@pytest.mark.parametrize("args", [
    (5, 4096, 4096, 512, 256), (qmm.Q4_K, 0, 4096, 512, 256), (qmm.Q4_K, 4096, 255, 512, 256),
    (qmm.Q4_K, 4096, 4096, -1, 256), (qmm.Q4_K, 4096, 4096, 512, 0), (qmm.Q4_K, 4096, 4096, 512, qmm.MAX_CUS + 1),
    (qmm.Q4_K, (1 << 21) + 1, 4096, 512, 256), (qmm.Q4_K, 4096, 4096, (1 << 20) + 1, 256),
    # more tiles than one launch holds
    (qmm.Q4_K, 1 << 21, 256, 1 << 20, 256)])
def test_plan_rejects_bad_arguments(args):
    with pytest.raises(qmm.QmmError) as e:
        qmm.mmq_plan(*args)
    assert e.value.code == qmm.EINVAL


def test_plan_work_rejects_bad_arguments():
    import ctypes
    p = qmm.mmq_plan(qmm.Q6_K, 4096, 11008 // 256 * 256, 3314, 256)
    assert p.n_tail > 0
    for wg in (-1, p.work_groups):
        with pytest.raises(qmm.QmmError):
            qmm.mmq_plan_work(p, wg)
    for field, value in [("split", 1), ("work_groups", p.work_groups + 1), ("n_tail", p.n_tail + 1),
                         ("tok_tiles", 0), ("nsb", 0), ("split", p.nsb + 1), ("dp_row_tiles", -1)]:
        bad = qmm.Plan.from_buffer_copy(p)
        setattr(bad, field, value)
        with pytest.raises(qmm.QmmError):
            qmm.mmq_plan_work(bad, 0)
    i = ctypes.c_int32()
    assert qmm._lib.qmm_mmq_plan_work(None, 0, ctypes.byref(i), ctypes.byref(i), ctypes.byref(i),
                                      ctypes.byref(i)) == qmm.EINVAL
    assert qmm._lib.qmm_mmq_plan(qmm.Q4_K, 4096, 4096, 512, 256, None) == qmm.EINVAL


# Shapes the GPU parity suite relies on for a given launch plan on MI355X's 256
# compute units: (type, od, id, n_tok) -> (many-tile geometry, tail tiles, slices).
PARITY_PLANS = {
    (qmm.Q4_K, 4160, 1024, 512): (0, 4, 2),                 # ragged second wave, split
    (qmm.Q6_K, 4200, 768, 500): (0, 0, 1),                  # ragged, but 3 super-blocks: whole
    (qmm.Q6_K, 4097, 2048, 509): (0, 4, 4),                 # the stream tests' split tail
    (qmm.Q6_K, 512, 2816, 300): (0, 24, 5),                 # every tile split
    (qmm.Q4_K, 512, 3072, 300): (0, 24, 6),
    (qmm.Q4_K, 512, 1024, 300): (0, 24, 2),
    (qmm.Q6_K, 4160, 2048, 512): (0, 4, 4),
    (qmm.Q6_K, 1000, 512, 4100): (1, 33, 2),                # many tiles, split tail
    (qmm.Q6_K, 2100, 256, 4000): (1, 0, 1),                 # one super-block: nothing to split
    (qmm.Q6_K, 4097, 1024, 3199): (1, 100, 4),              # short last wave behind three full ones
    (qmm.Q6_K, 4096, 1024, 3072): (1, 0, 1),                # exactly three full waves
    (qmm.Q4_K, 2527, 4352, 1572): (0, 13, 8),
    (qmm.Q4_K, 70000, 256, 1): (1, 0, 1),
    (qmm.Q4_K, 96, 512, 40): (0, 0, 1),
    (qmm.Q6_K, 4096, 11008 // 256 * 256, 3314): (1, 130, 3),  # the layer's ffn_down
    (qmm.Q4_K, 11008, 4096, 512): (1, 352, 2),               # gate/up at 512 tokens: 1376 tiles on 1024 slots
}


@pytest.mark.parametrize("shape", list(PARITY_PLANS), ids=[f"{t}-{o}x{i}-T{n}" for t, o, i, n in PARITY_PLANS])
def test_parity_shapes_reach_their_plans(shape):
    p = _check_plan(*shape, 256)
    assert (p.many, p.n_tail, p.split) == PARITY_PLANS[shape]

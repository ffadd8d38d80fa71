"""Property tests of the host layout algebra (canonicalize, merge, injectivity) against brute
force: for random layouts, the canonical shard tc_plan reports must enumerate exactly the same
(source offset, destination offset) pairs as the original layouts, and a destination that maps
two logical indices to one element must be rejected."""

import itertools
from collections import Counter

import numpy as np
from hypothesis import given, settings, strategies as st

import layout_permuting_copy_amd as L
from oracle import ref as R


def _pairs(shape, ss, so, ds, do):
    out = Counter()
    for idx in itertools.product(*[range(e) for e in shape]):
        out[(so + sum(i * s for i, s in zip(idx, ss)), do + sum(i * d for i, d in zip(idx, ds)))] += 1
    return out


@st.composite
def layouts(draw):
    rank = draw(st.integers(1, 4))
    shape = draw(st.lists(st.integers(1, 6), min_size=rank, max_size=rank))
    # destination: a permuted dense row-major layout (injective), sometimes with a zeroed or
    # repeated stride (non-injective), modes maybe walked backwards; source: permuted, stepped,
    # maybe negative or zero strides (the planner may reverse modes: the pairs stay the same)
    perm_d = draw(st.permutations(range(rank)))
    ds, acc = [0] * rank, 1
    for k in reversed(perm_d):
        ds[k] = acc
        acc *= shape[k]
    if draw(st.integers(0, 9)) == 0:
        k = draw(st.integers(0, rank - 1))
        ds[k] = draw(st.sampled_from([0, ds[(k + 1) % rank]]))
    # destination modes walked backwards (a flipped or rotated view)
    flips = draw(st.lists(st.booleans(), min_size=rank, max_size=rank))
    ds = [-d if f else d for d, f in zip(ds, flips)]
    perm_s = draw(st.permutations(range(rank)))
    steps = draw(st.lists(st.sampled_from([1, 1, 2, 3, -1]), min_size=rank, max_size=rank))
    ss, acc = [0] * rank, 1
    for k in reversed(perm_s):
        ss[k] = acc * steps[k]
        acc *= shape[k] * abs(steps[k])
    if draw(st.integers(0, 9)) == 0:
        ss[draw(st.integers(0, rank - 1))] = 0  # broadcast read
    so = acc + draw(st.integers(0, 7))  # room for negative strides
    do = int(np.prod(shape)) + draw(st.integers(0, 7))
    # insert extent-1 modes with arbitrary strides on either side
    if draw(st.booleans()):
        pos = draw(st.integers(0, rank))
        shape_s = shape[:pos] + [1] + shape[pos:]
        ss = ss[:pos] + [draw(st.integers(-50, 50))] + ss[pos:]
    else:
        shape_s = shape
    return shape, tuple(shape_s), tuple(ss), so, tuple(ds), do


@settings(max_examples=400, deadline=None)
@given(layouts(), st.sampled_from([1, 2, 4, 8, 16]))
def test_canonical_shard_enumerates_the_same_pairs(lay, eb):
    shape, shape_s, ss, so, ds, do = lay
    dt = {1: L.TC_I8, 2: L.TC_BF16, 4: L.TC_F32, 8: L.TC_F64, 16: L.TC_B128}[eb]
    p = L.tc_plan((shape_s, ss, so), (shape, ds, do), dt, raise_on_error=False)
    # the two sides' non-unit modes, paired in order (equal extents by construction)
    src_nu = [(e, s) for e, s in zip(shape_s, ss) if e != 1]
    dst_nu = [(e, d) for e, d in zip(shape, ds) if e != 1]
    ext = [e for e, _ in dst_nu]
    assert ext == [e for e, _ in src_nu]
    want = _pairs(ext, [s for _, s in src_nu], so, [d for _, d in dst_nu], do)
    dst_offsets = Counter()
    for (_, d), n in want.items():
        dst_offsets[d] += n
    if max(dst_offsets.values()) > 1:
        assert p["status"] == L.TC_E_NONINJECTIVE, (lay, p["error"])
        return
    assert p["status"] == L.TC_OK, (lay, p["error"])
    got = _pairs(p["extent"], p["src_stride"], p["src_offset"], p["dst_stride"], p["dst_offset"])
    assert got == want, (lay, p["extent"], p["src_stride"], p["dst_stride"])
    # and the oracle's joint modes (its own reading of the two layouts) agree
    modes = R.common_modes(R.layout(shape_s, ss, so), R.layout(shape, ds, do))
    assert Counter({k: v for k, v in _pairs([e for e, _, _ in modes], [s for _, s, _ in modes], so,
                                             [d for _, _, d in modes], do).items()}) == want

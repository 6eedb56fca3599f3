"""The streaming decode-attention form's split of the work, modelled on the CPU.

The streaming form (csrc/vq_attention.hip) cuts the attended tokens of every
(sequence, kv head) segment into 64-token slices, lays them end to end in
(sequence, kv head, slice) order, gives workgroup i of G the slices
[U i / G, U (i+1) / G) of the U in total, and writes the partial of each
(workgroup, segment) pair it touches to slot i + sigma, sigma = b Hkv + h,
recording the first and the last workgroup of every segment for the merge.
This models that integer arithmetic (not the floating point) on random
length sets and checks what the kernel and its merge rely on: every slice
goes to exactly one workgroup, the slots are distinct and below
G + B Hkv - 1, the recorded first and last workgroups bound exactly the
workgroups that touch a segment, and the host's workspace bound holds.
"""
import numpy as np
import pytest

SLICE = 64
CHUNK = 256


def seq_slices(L, window):
    first = max(0, L - window) if window > 0 else 0
    return -(-(L - first) // SLICE)


def parts(lengths, Hkv, G, window=0):
    """(workgroup, sequence, head, j0, j1) for every part, in the kernel's
    order, following its loop: find the sequence of s_begin, then walk."""
    ns = [seq_slices(int(L), window) for L in lengths]
    U = Hkv * sum(ns)
    out = []
    for wg in range(G):
        s_begin, s_end = U * wg // G, U * (wg + 1) // G
        if s_begin >= s_end:
            continue
        seq0, b = 0, 0
        while not (ns[b] > 0 and seq0 <= s_begin < seq0 + Hkv * ns[b]):
            seq0 += Hkv * ns[b]
            b += 1
        pos = s_begin
        while pos < s_end and b < len(lengths):
            span = Hkv * ns[b]
            if pos >= seq0 + span:
                seq0 += span
                b += 1
                continue
            r = pos - seq0
            h = r // ns[b]
            j0 = r - h * ns[b]
            j1 = min(ns[b], s_end - seq0 - h * ns[b])
            out.append((wg, b, h, j0, j1))
            pos = seq0 + h * ns[b] + j1
    return ns, out


@pytest.mark.parametrize("seed", range(12))
def test_every_slice_once_and_distinct_slots(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 700))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    S = int(rng.integers(1, 5000))
    window = int(rng.choice([0, 0, int(rng.integers(1, 3000))]))
    lengths = rng.integers(0, S + 1, size=B)
    lengths[rng.random(B) < 0.1] = 0
    G = int(rng.integers(1, 1000))
    ns, ps = parts(lengths, Hkv, G, window)
    seen = {}
    slots = set()
    first, last = {}, {}
    for wg, b, h, j0, j1 in ps:
        assert 0 <= j0 < j1 <= ns[b]
        sigma = b * Hkv + h
        for j in range(j0, j1):
            assert (sigma, j) not in seen, "a slice taken twice"
            seen[(sigma, j)] = wg
        slot = wg + sigma
        assert slot not in slots, "two parts share a slot"
        assert slot < G + B * Hkv - 1
        slots.add(slot)
        if j0 == 0:
            first[sigma] = wg
        if j1 == ns[b]:
            last[sigma] = wg
    for b in range(B):
        for h in range(Hkv):
            sigma = b * Hkv + h
            if ns[b] == 0:
                assert sigma not in first and sigma not in last
                continue
            assert all((sigma, j) in seen for j in range(ns[b])), "a slice left out"
            touching = sorted({seen[(sigma, j)] for j in range(ns[b])})
            # the merge reads slots first..last: exactly the workgroups that
            # touch the segment, which are consecutive
            assert touching == list(range(first[sigma], last[sigma] + 1))


def test_parts_follow_the_workgroup_order():
    # lengths of mixed sizes, the ranges cut segments in the middle
    ns, ps = parts([700, 1, 0, 4096, 333], 4, 37)
    assert [p[0] for p in ps] == sorted(p[0] for p in ps)
    assert sum(j1 - j0 for _, _, _, j0, j1 in ps) == 4 * sum(ns)


@pytest.mark.parametrize("B,Hq,Hkv,D,S,per_cu", [
    (128, 12, 4, 256, 4096, 3), (2048, 2, 1, 64, 1024, 3), (260, 16, 2, 256, 2048, 2),
    (640, 8, 2, 128, 2048, 3), (96, 12, 4, 256, 4096, 3), (1, 1, 1, 64, 300, 3)])
def test_workspace_bound_of_the_streaming_form(B, Hq, Hkv, D, S, per_cu):
    """The host runs the streaming form with G = per_cu x CUs workgroups only
    when there are at least 32 slices per workgroup and the partials plus the
    segment table fit in the chunked form's workspace."""
    cus = 256
    g = Hq // Hkv
    segs = B * Hkv
    row = g * (D + 2)
    avail = B * Hq * -(-S // CHUNK) * (D + 2)          # floats of the workspace
    gmax = (avail - 2 * segs) // row - segs + 1
    G = per_cu * cus
    slices = segs * -(-S // SLICE)
    runs = slices >= 32 * G and G <= gmax
    if runs:
        assert (G + segs - 1) * row + 2 * segs <= avail
    expect = (B, S) in {(128, 4096), (2048, 1024), (260, 2048), (640, 2048), (96, 4096)}
    assert runs == expect

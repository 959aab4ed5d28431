"""The work split of fwd_causal_wide_kernel, modelled on the CPU: every key step of both
query tiles of a tile pair is merged exactly once, into its own tile.

The kernel pairs query tile A = T-1-i (T - i causal key steps) with tile B = i (i + 1 key
steps), so a pair has S = T + 1 steps, A's first. Its ns workgroups of NW = 8 waves cut them
into NW * ns runs with boundaries rounded up, ceil(r S / (NW ns)) for run r. A run that
reaches the end of A parks A's partial in a separate crossing record and goes on with B; at
the end every wave parks its last partial in slot w. Then tile A gathers the slots of the
runs that end within A plus the crossing record (when a run crosses), and tile B the slots
of the runs that end after A. These are the rules the kernel's run_start, crossing test and
merge flags implement; the GPU parity cases check the kernel itself on several T and ns.
"""
NW = 8


def run_start(sw, r, S, ns):
    return -((-(sw * NW + r) * S) // (NW * ns))  # ceil


def merged_steps(T, i, ns):
    """{tile: list of key steps merged into it} over all ns workgroups of tile pair i,
    following the kernel's rules; raises AssertionError where a rule is broken."""
    nA, S = T - i, T + 1
    out = {"A": [], "B": []}
    for sw in range(ns):
        slot, crossrec = {}, None
        for w in range(NW):
            st, en = run_start(sw, w, S, ns), run_start(sw, w + 1, S, ns)
            cur = []
            for n in range(st, en):
                cur.append(n)
                if n + 1 == nA and n + 1 < en:  # the run continues into B
                    assert crossrec is None, "two runs cross in one workgroup"
                    crossrec, cur = cur, []
            slot[w] = cur
        for tile in ("A", "B"):
            mergeA = tile == "A"
            inc, cross = [], False
            for p in range(NW):
                sp, ep = run_start(sw, p, S, ns), run_start(sw, p + 1, S, ns)
                inc.append(sp < ep and (ep <= nA) == mergeA)
                cross |= sp < nA < ep
            for p in range(NW):
                if inc[p]:
                    out[tile] += slot[p]
                else:  # a slot left out holds only the other tile's steps, or none
                    assert all((n < nA) != mergeA for n in slot[p]), (T, i, ns, sw, p)
            if cross and mergeA:
                out[tile] += crossrec
    return out


def test_every_step_merged_once_into_its_tile():
    checked = 0
    for T in range(2, 257, 2):
        for ns in (1, 2, 4, 8):
            for i in range(T // 2):
                nA, S = T - i, T + 1
                got = merged_steps(T, i, ns)
                assert sorted(got["A"]) == list(range(nA)), (T, i, ns)
                assert sorted(got["B"]) == list(range(nA, S)), (T, i, ns)
                checked += 1
    assert checked == 4 * sum(T // 2 for T in range(2, 257, 2))


def test_longer_run_comes_first():
    """Rounded up, the runs with an extra step are the first ones: at T = 64 (one share)
    run 0 has 9 steps and starts at A's first key step, so it never crosses into B."""
    S = 65
    lens = [run_start(0, r + 1, S, 1) - run_start(0, r, S, 1) for r in range(NW)]
    assert lens == [9, 8, 8, 8, 8, 8, 8, 8]
    for i in range(32):
        assert run_start(0, 1, S, 1) <= 64 - i  # run 0 ends within A

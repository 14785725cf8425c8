"""Workload labels that the profile summaries give to a run's kernel dispatches (host logic only).

Counter runs report only the flattened grid size, so two token counts can share a kernel and
grid; an expand dispatch then takes the token count of the shrink dispatched right before it.
"""
import bench_profiles as bp

SH = "shrink_kernel<1, 1, 1, 8, 2, true, true>"
LDS = "shrink_lds_kernel<1, 2, 3, 6, 2>"
EX = "expand_kernel<1, 4, 1, 2, true, true, false>"
EXS = "expand_shared_kernel<1, 1, true>"
PAIR = "pair_kernel<1, true, true>"

# (token count, shrink dispatch, expand dispatch, single-launch dispatch or None), with grids
# flattened as in a counter run: 512 and 1024 tokens share the shrink's grid, 1024 and 4096 the
# expand's.
CASES = [
    (50, (SH, (192, 1)), (EX, (216, 1)), (PAIR, (312, 1))),
    (128, (SH, (288, 1)), (EX, (324, 1)), (PAIR, (468, 1))),
    (256, (SH, (240, 1)), (EX, (300, 1)), (PAIR, (420, 1))),
    (512, (SH, (216, 1)), (EXS, (612, 1)), (PAIR, (468, 1))),
    (1024, (SH, (216, 1)), (EXS, (1020, 1)), None),
    (2048, (LDS, (72, 1)), (EXS, (972, 1)), None),
    (4096, (LDS, (136, 1)), (EXS, (1020, 1)), None),
    (6144, (LDS, (200, 1)), (EXS, (900, 1)), None),
    (8192, (LDS, (176, 1)), (EXS, (1188, 1)), None),
]


def _run():
    disp, want = [], []
    for t, s, e, _ in CASES:  # separate calls
        disp += [s, e]
        want += [f"shrink_tok{t}", f"expand_tok{t}"]
    for _ in range(2):  # one single-launch call per case
        for t, s, e, p in CASES:
            if p is not None:
                disp.append(p)
                want.append(f"pair_tok{t}")
            else:
                disp += [s, e]
                want += [f"shrink_tok{t}", f"expand_tok{t}"]
    return disp, want


def test_coinciding_expand_grids_take_the_preceding_shrink_token_count():
    disp, want = _run()
    got = bp.label_dispatches(disp)
    assert len(got) == len(want)
    for g, w in zip(got, want):
        if w.startswith("expand_tok"):
            assert g == w
        else:
            # shrinks and single launches that share a grid keep the joint label
            assert w in g.split(" / ")
    assert "shrink_tok512 / shrink_tok1024" in got
    assert "pair_tok128 / pair_tok512" in got


def test_expand_after_an_unrelated_shrink_keeps_the_joint_label():
    disp, _ = _run()
    # an expand with the shared grid, preceded by the 2048-token shrink: no unique token count
    disp.append((LDS, (72, 1)))
    disp.append((EXS, (1020, 1)))
    got = bp.label_dispatches(disp)
    assert got[-1] == "expand_tok1024 / expand_tok4096"

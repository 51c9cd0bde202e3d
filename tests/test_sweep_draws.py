"""The random GPU sweep's draws (host only): the same cases every run, and
the shapes its docstring promises are among them."""
from tests.test_gpu_sweep import (draw_prefix_case, draw_suffix_case, draw_tree_case,
                                  draw_window_case)


def test_draws_are_fixed_and_cover_the_edges():
    s = [draw_suffix_case(i) for i in range(24)]
    assert s == [draw_suffix_case(i) for i in range(24)]
    assert {c["dtype"] for c in s} == {"bf16", "f32"}
    assert {c["d"] for c in s if c["dtype"] == "f32"} == {64, 128}
    assert any(c["p"] == 0 for c in s) and any(c["p"] % 32 and c["p"] > 32 for c in s)
    assert any(0 in c["lens"] for c in s) and any(1 in c["lens"] for c in s)
    assert any(len(c["lens"]) >= 4 for c in s)
    assert any(c["qmap"] is not None for c in s)
    assert {c["hq"] // c["hkv"] for c in s} >= {1, 2, 3, 4}
    assert any(c["scale_q"] > 1 for c in s) and any(c["min_ws"] for c in s)
    assert all(sum(c["lens"]) > 0 for c in s)
    assert {c["softmax_scale"] for c in s} == {0.0, 0.05, 0.2}
    assert len({c["softmax_scale"] for c in (draw_prefix_case(i) for i in range(10))}) > 1
    for c in s:
        if c["qmap"] is not None:
            group = c["hq"] // c["hkv"]
            assert sorted(c["qmap"]) == sorted(list(range(c["hkv"])) * group)
    p = [draw_prefix_case(i) for i in range(10)]
    assert any(not c["with_do"] for c in p) and any(c["min_ws"] for c in p)
    assert min(c["p"] for c in p) <= 2 and max(c["p"] for c in p) > 256
    w = [draw_window_case(i) for i in range(10)]
    assert any(c["node"] == 0 for c in w) and any(c["node"] > 0 for c in w)
    assert {c["dtype"] for c in w} == {"bf16", "f32"} and any(c["min_ws"] for c in w)
    t = [draw_tree_case(i) for i in range(10)]
    assert {c["dtype"] for c in t} == {"bf16", "f32"} and any(c["min_ws"] for c in t)
    assert any(c["n"] == 1 for c in t) and max(c["n"] for c in t) >= 16
    assert any(c["qmap"] is not None for c in t) and any(c["softmax_scale"] for c in t)

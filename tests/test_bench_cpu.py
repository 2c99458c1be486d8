"""bench.py on the host: its command-line contract (a request for more than
one GPU ends at once with a one-line JSON error and exit status 2, since the
fused kernels emulate the peer ranks on one device), and the host logic of its
ECT comparisons (link-paced block schedules, row-block views, alternating
timing passes)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = r.stdout.strip().splitlines()[-1]
    assert "one GPU" in json.loads(line)["error"]


def test_help_lists_the_switches():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--no-ect", "--no-cold", "--no-cpu-baseline",
                 "--copy-probe"):
        assert flag in r.stdout


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_link_schedule_whole_chunks_match_the_link_times():
    b = _bench()
    t = 82200
    seq, times = b.link_schedule(list(range(8)), 1, t, "direct")
    assert seq == list(range(8)) and times == [0] + [t] * 7
    seq, times = b.link_schedule(list(range(8)), 1, t, "ring")
    assert seq == list(range(8)) and times == [a * t for a in range(8)]


def test_link_schedule_blocks_land_in_order():
    """Block q of a chunk lands (q+1)/parts of a link time after its chunk's
    transfer began; the local chunk's blocks are in place at 0; the sequence
    is sorted by arrival (the paced signal needs non-decreasing times) and
    names every block once."""
    b = _bench()
    t, n = 82200, 8
    for parts in (2, 4):
        for kind in ("direct", "ring"):
            order = [3, 0, 1, 2, 4, 5, 6, 7]          # chunk 3 local, then the rest
            seq, times = b.link_schedule(order, parts, t, kind)
            assert sorted(seq) == list(range(n * parts))
            assert times == sorted(times)
            at = dict(zip(seq, times))
            for a, c in enumerate(order):
                for q in range(parts):
                    start = 0 if kind == "direct" else (a - 1) * t
                    want = 0 if a == 0 else start + (q + 1) * t // parts
                    assert at[c * parts + q] == want, (kind, parts, c, q)
            # the last block of every peer chunk lands where its whole chunk did
            whole = dict(zip(*b.link_schedule(order, 1, t, kind)))
            for c in order[1:]:
                assert at[c * parts + parts - 1] == whole[c]


def test_part_views_are_row_blocks_in_chunk_order():
    import numpy as np
    b = _bench()
    chunks = [np.arange(c * 100, c * 100 + 8).reshape(8, 1) for c in range(3)]
    views = b.part_views(chunks, 4)
    assert len(views) == 12
    for c in range(3):
        for q in range(4):
            assert views[c * 4 + q].tolist() == chunks[c][2 * q:2 * q + 2].tolist()


def test_time_rounds_takes_turns_and_the_median(monkeypatch):
    b = _bench()
    calls = []
    fake = {"a": iter([5.0, 1.0, 3.0]), "b": iter([2.0, 9.0, 4.0])}

    def time_loop(fn, iters, warmup):
        name = fn()
        calls.append(name)
        return next(fake[name]), 0.0

    monkeypatch.setattr(b, "time_loop", time_loop)
    med = b.time_rounds([("a", lambda: "a"), ("b", lambda: "b")], iters=1, rounds=3)
    assert calls == ["a", "b"] * 3
    assert med == {"a": 3.0, "b": 4.0}

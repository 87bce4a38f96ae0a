"""Host logic of the benchmark's serving clock (two 80 ms steps per 160 ms
beat, p99 per beat, late session-beats: the Nemotron VoiceChat case
study's measurement notes), driven by a stub context and a stub clock, so
the percentile and late-beat accounting is checked without a GPU."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_beat_stats_percentiles_and_late_count():
    lat = [10.0] * 98 + [170.0, 200.0]
    st = bench.beat_stats(lat, [9.0] * 100, n_active=56)
    assert st["p50_ms"] == 10.0
    assert st["p99_ms"] == 170.0          # nearest rank of 100 beats
    assert st["max_ms"] == 200.0
    assert st["late_beats"] == 2
    assert st["late_session_beats"] == 2 * 56
    assert st["gpu_p99_ms"] == 9.0
    # exactly at the deadline is on time
    assert bench.beat_stats([160.0, 160.0], [], n_active=3)["late_beats"] == 0
    assert bench.beat_stats([160.0001], [], n_active=3)["late_session_beats"] == 3


class _Clock:
    def __init__(self):
        self.t = 100.0

    def __call__(self):
        return self.t

    def sleep(self, dt):
        assert dt >= 0
        self.t += dt


class _StubCtx:
    """The slot calls run_beats makes, with fd_step's position rules."""

    def __init__(self, slots, window):
        self.max_slots, self.window = slots, window
        self.active, self.pos = [0] * slots, [0] * slots
        self.steps = 0

    def fd_slot_state(self, s):
        return self.active[s], self.pos[s]

    def fd_free(self, ids):
        assert len(set(ids)) == len(ids)
        for s in ids:
            assert self.active[s], "freeing a free slot"
            self.active[s] = 0

    def fd_alloc_slots(self, n):
        free = [s for s in range(self.max_slots) if not self.active[s]]
        assert len(free) >= n
        for s in free[:n]:
            self.active[s], self.pos[s] = 1, 0
        return free[:n]

    def fd_set_position(self, s, p):
        assert self.active[s] and 0 <= p <= self.window
        self.pos[s] = p

    def step(self):
        for s in range(self.max_slots):
            if self.active[s]:
                assert self.pos[s] < self.window, "stepping a full window (FD_E_CTXFULL)"
                self.pos[s] += 1
        self.steps += 1


@pytest.mark.parametrize("slow_beat", [None, 7])
def test_run_beats_churn_and_late_beats(slow_beat):
    """40 beats x 2 runs, 12 of 16 slots active in a 30-frame window (so
    sessions end and new ones are admitted every few beats); one beat may
    take 200 ms of a 160 ms budget."""
    clock = _Clock()
    ctx = _StubCtx(16, 30)
    beat = {"n": 0}

    def two_steps():
        ctx.step()
        ctx.step()
        b = beat["n"]
        beat["n"] += 1
        # the first call of each run is its warm-up pair
        dur = 0.200 if (slow_beat is not None and b == slow_beat + 1) else 0.012
        clock.t += dur
        assert sum(ctx.active) == 12, "the active count changes only by churn"
        return dur * 1e3

    out = bench.run_beats(ctx, two_steps, beats=40, runs=2, n_active=12, max_context=30,
                          seed=3, clock=clock, sleep=clock.sleep)
    assert out["session_beats"] == 12 * 40 * 2
    assert out["admissions"] == out["retirements"] > 0
    assert ctx.steps == 2 * (40 + 1) * 2
    if slow_beat is None:
        assert out["late_beats"] == 0 and out["late_session_beats"] == 0
        assert out["max_ms"][0] == pytest.approx(12.0)
    else:
        # only the slow beat misses: the next starts 40 ms behind its
        # schedule and still finishes within 160 ms of it
        assert out["late_beats"] == 1 and out["late_session_beats"] == 12
        assert out["max_ms"][0] == pytest.approx(200.0)
        assert out["p99_ms"][0] == pytest.approx(200.0)
    assert all(p <= 30 for p in ctx.pos)


def test_attention_trace_summary_phases():
    """Stamps in 10 ns ticks: two workgroups, one entering 1 us late."""
    stamps = [[1000, 1100, 1500, 1520],
              [1100, 1150, 1400, 1410],
              [0, 0, 0, 0]]  # a row no workgroup wrote
    t = bench.attention_trace_summary(stamps, concurrent=2)
    assert t["workgroups"] == 2
    assert t["span_us"] == pytest.approx(5.2)
    assert t["last_entry_us"] == pytest.approx(1.0)
    assert t["prologue_us"]["max"] == pytest.approx(1.0)
    assert t["stream_us"]["p50"] == pytest.approx(4.0)
    assert t["epilogue_us"]["sum"] == pytest.approx(0.3)
    assert t["busy_frac"] == pytest.approx((5.2 + 3.1) / (5.2 * 2))


def test_summarize_launches_groups_step_kernels(tmp_path):
    """Setup kernels are dropped; step kernels group by name and grid."""
    f = tmp_path / "k.csv"
    f.write_text(
        "Kernel_Name,Grid_Size_X,Start_Timestamp,End_Timestamp\n"
        '"void fd::pack_kernel<1>(fd::PackArgs)",1024,0,5000\n'
        '"void fd::gemm_kernel<1, 6, 5, 3, 1, 0>(fd::GemmArgs)",65536,100,2100\n'
        '"void fd::attn_kernel<1, 1, 128, 1>(fd::AttnArgs)",655360,2200,12200\n'
        '"void fd::gemm_kernel<1, 6, 5, 3, 1, 0>(fd::GemmArgs)",65536,13000,17000\n'
        '"void fd::gemm_kernel<1, 6, 5, 3, 1, 0>(fd::GemmArgs)",60160,18000,19000\n')
    out = bench.summarize_launches(str(f), "cmd", "t")
    rows = [l for l in out.splitlines() if l.startswith("| `")]
    assert len(rows) == 3
    assert rows[0].startswith("| `fd::gemm_kernel<1, 6, 5, 3, 1, 0>` | 65536 | 2 | 3.00 |")
    assert "attn_kernel" in rows[1] and "| 10.00 |" in rows[1]
    assert "pack_kernel" not in out


def test_summarize_pmc_separates_grids_and_scales_by_the_copy(tmp_path):
    """Counter passes scale by the 1 GiB copy's reading; the 80-slot
    attention launches are kept apart from a largest-S run's."""
    hdr = "Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n"
    copy = '"void at::native::elementwise_kernel<MulFunctor<float>>(x)",1024,{c},{v}\n'
    a80 = '"void fd::attn_kernel<1, 1, 128, 1>(fd::AttnArgs)",655360,{c},{v}\n'
    a709 = '"void fd::attn_kernel<1, 1, 128, 1>(fd::AttnArgs)",5808128,{c},{v}\n'
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    fetch.write_text(hdr + copy.format(c="FETCH_SIZE", v=524288) + a80.format(c="FETCH_SIZE", v=480000)
                     + a80.format(c="FETCH_SIZE", v=482000) + a709.format(c="FETCH_SIZE", v=4e6))
    write.write_text(hdr + copy.format(c="WRITE_SIZE", v=1048576) + a80.format(c="WRITE_SIZE", v=2000)
                     + a80.format(c="WRITE_SIZE", v=2000) + a709.format(c="WRITE_SIZE", v=9000))
    cpath = tmp_path / "counters.json"
    md = bench.summarize_pmc(str(fetch), str(write), "7b_s80_p1499", "cmd", counters_path=str(cpath))
    import json
    e = json.loads(cpath.read_text())["attention@7b_s80_p1499"]
    # copy: 1 GiB read shows as 512 MiB fetched -> fetch scale 2, write scale 1
    assert e["scale_fetch"] == pytest.approx(2.0) and e["scale_write"] == pytest.approx(1.0)
    assert e["fetch_kib"] == pytest.approx(481000)
    assert e["hbm_bytes_per_launch"] == pytest.approx(481000 * 1024 * 2 + 2000 * 1024)
    assert "| 5808128 |" in md and "| 655360 |" in md

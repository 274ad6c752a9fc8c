"""Host logic of the progressive tracer: ordered-log comparison, level and
window filtering, and the trace file round trip (no GPU)."""
from bitwise_deterministic_moe_amd.trace import LEVELS, Record, Tracer, first_divergence


def _r(step, phase, name, fp, op="op"):
    return Record(step, phase, op, name, "f32", [2, 3], 6, fp)


def test_first_divergence_finds_the_earliest_differing_record():
    a = [_r(0, "forward", "y", "01"), _r(0, "backward", "dx", "02"), _r(1, "forward", "y", "03")]
    b = [_r(0, "forward", "y", "01"), _r(0, "backward", "dx", "ff"), _r(1, "forward", "y", "04")]
    i, ra, rb = first_divergence(a, b)
    assert i == 1 and ra.name == "dx" and rb.fp == "ff"
    assert first_divergence(a, list(a)) is None


def test_first_divergence_sees_missing_and_reshaped_records():
    a = [_r(0, "forward", "y", "01"), _r(0, "backward", "dx", "02")]
    i, ra, rb = first_divergence(a, a[:1])
    assert i == 1 and ra is a[1] and rb is None
    c = [_r(0, "forward", "y", "01"), Record(0, "backward", "op", "dx", "f32", [3, 2], 6, "02")]
    assert first_divergence(a, c)[0] == 1          # same bits, different shape


def test_levels_and_window():
    t = Tracer("phases", window=range(2, 3))
    assert t._on(0, 0) and t._on(5, 0)             # metrics: every step
    assert not t._on(1, 1) and t._on(2, 1)         # phases: the window only
    assert not t._on(2, 2)                         # ops: above the level
    assert Tracer("ops")._on(7, 2)
    assert LEVELS["metrics"] < LEVELS["phases"] < LEVELS["ops"]


def test_metric_records_hold_exact_bits_and_round_trip(tmp_path):
    t = Tracer("metrics")
    t.metric(0, "loss", 0.1)
    t.metric(0, "loss", 0.1 + 2 ** -56)            # one ulp away: a different record
    assert t.records[0].fp != t.records[1].fp
    p = tmp_path / "trace.jsonl"
    t.save(str(p))
    back = Tracer.load(str(p))
    assert [r.__dict__ for r in back] == [r.__dict__ for r in t.records]

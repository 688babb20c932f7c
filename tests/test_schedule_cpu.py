"""Host logic of precision scheduling (mixed-precision neural-operator page, "Tiivistelmä":
training moves from mixed to full precision): which precision each step takes."""
import pytest

from fno_spectral_convolution_amd.stack import PrecisionSchedule, SPECTRAL_PRECISIONS


@pytest.mark.parametrize("half", ["bf16", "f16"])
def test_switch_is_one_way_at_the_step(half):
    s = PrecisionSchedule(3, half)
    assert [s.precision_at(i) for i in range(6)] == [half] * 3 + ["f32"] * 3


def test_switch_at_zero_is_fp32_throughout():
    s = PrecisionSchedule(0)
    assert {s.precision_at(i) for i in range(5)} == {"f32"}


def test_from_fraction_floors():
    assert PrecisionSchedule.from_fraction(10, 0.75).switch_step == 7
    assert PrecisionSchedule.from_fraction(8, 0.5, "f16").switch_step == 4
    assert PrecisionSchedule.from_fraction(8, 1.0).precision_at(7) == "bf16"
    assert PrecisionSchedule.from_fraction(8, 0.0).precision_at(0) == "f32"


@pytest.mark.parametrize("args", [(-1,), (1.5,), (True,), (2, "fp8"), (2, "f32")])
def test_rejects_bad_schedules(args):
    with pytest.raises(ValueError):
        PrecisionSchedule(*args)


def test_rejects_bad_fraction_and_step():
    with pytest.raises(ValueError):
        PrecisionSchedule.from_fraction(10, 1.5)
    with pytest.raises(ValueError):
        PrecisionSchedule(2).precision_at(-1)


def test_every_scheduled_precision_is_a_plan_precision():
    for half in ("bf16", "f16"):
        s = PrecisionSchedule(1, half)
        assert {s.precision_at(0), s.precision_at(1)} <= set(SPECTRAL_PRECISIONS)

"""Host-side recipe logic (no device): the sample-and-hold refresh schedule
("UE5M3 FP4 Block Scaling for Stable Language Model Pretraining", §5.1: the
tensor maximum is re-sampled every D steps and held in between) and the
per-operand targets (§5.2)."""
import pytest

from fp4_block_scaled_fp4q_amd.recipe import Fp4Recipe, is_refresh


def test_refresh_every_d_steps():
    assert [s for s in range(12) if is_refresh(s, 5)] == [0, 5, 10]
    assert all(is_refresh(s, 1) for s in range(5))            # D = 1: current scaling
    assert [s for s in range(200) if is_refresh(s, 50)] == [0, 50, 100, 150]
    with pytest.raises(ValueError):
        is_refresh(0, 0)


def test_targets():
    r = Fp4Recipe()
    assert (r.refresh_period, r.target, r.t_dy_wgrad()) == (50, 448.0, 448.0)
    r2 = Fp4Recipe(target_dy_wgrad=2048)
    assert r2.t_dy_wgrad() == 2048.0 and r2.target == 448.0
    # the page's headroom figures follow from the largest UE5M3 scale
    assert round(61440 / 448) == 137 and 61440 / 2048 == 30

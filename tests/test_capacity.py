"""The capacity policy on synthetic latency curves (RealtimeWAM §3: the upper
end of the latency plateau holding the required token count)."""
import pytest

from sparse_kv_refresh_amd.capacity import plateau_capacity

ROWS = [32 * i for i in range(1, 21)]           # 32 .. 640


def _steps(r):
    # flat within 128-row tiles, +10 per tile, small noise-free
    return 100.0 + 10.0 * ((r + 127) // 128)


def test_rounds_up_to_the_end_of_the_tile_plateau():
    ms = [_steps(r) for r in ROWS]
    assert plateau_capacity(ROWS, ms, 130) == 256
    assert plateau_capacity(ROWS, ms, 256) == 256
    assert plateau_capacity(ROWS, ms, 257) == 384
    assert plateau_capacity(ROWS, ms, 1) == 128


def test_tolerance_merges_small_steps():
    ms = [_steps(r) for r in ROWS]
    # 10/110 = 9 % steps: a 10 % tolerance spans one more tile
    assert plateau_capacity(ROWS, ms, 130, tol=0.10) == 384
    assert plateau_capacity(ROWS, ms, 130, tol=0.0) == 256


def test_beyond_profile_and_noise():
    ms = [_steps(r) for r in ROWS]
    assert plateau_capacity(ROWS, ms, 700) == 700          # beyond the profile: unchanged
    noisy = list(ms)
    noisy[5] *= 1.05                                      # a spike inside the first plateau
    assert plateau_capacity(ROWS, noisy, 130) == 160       # stops before the spike
    assert plateau_capacity(ROWS, ms, 0) == 128


def test_never_below_k_and_validates():
    ms = [_steps(r) for r in ROWS]
    for k in range(0, 640, 7):
        assert plateau_capacity(ROWS, ms, k) >= k
    with pytest.raises(ValueError):
        plateau_capacity([64, 32], [1.0, 1.0], 10)
    with pytest.raises(ValueError):
        plateau_capacity([32], [1.0, 2.0], 10)

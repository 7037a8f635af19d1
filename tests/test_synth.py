"""Input generator: known-answer vectors and distribution checks (CPU)."""
import numpy as np
import pytest

from synth import synth, workloads


# Known-answer vectors published with the Random123 library for
# Philox4x32 with 10 rounds (counter, key) -> output.
PHILOX_KAT = [
    ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
    ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
    ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
     [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
]


@pytest.mark.parametrize("ctr,key,want", PHILOX_KAT)
def test_philox_known_answers(ctr, key, want):
    assert list(synth.philox_block(ctr, key)) == want


def test_irwin_hall_moments():
    z = synth.std_normal(123, synth.STREAM_W, 0, 2_000_000)
    assert abs(z.mean()) < 3e-3
    assert abs(z.var() - 1.0) < 5e-3
    assert np.abs(z).max() <= 6.0
    # Irwin-Hall(12) excess kurtosis is -0.1
    k = ((z - z.mean()) ** 4).mean() / z.var() ** 2 - 3
    assert abs(k + 0.1) < 0.02
    # exact construction: every value is an integer multiple of 2^-32
    assert np.all(np.ldexp(z, 32) == np.round(np.ldexp(z, 32)))


def test_weights_rows_are_addressable():
    full = synth.weights(77, 96, 0, 10, 0.02, nthreads=3)
    part = synth.weights(77, 96, 4, 5, 0.02, nthreads=1)
    assert np.array_equal(full[4:9], part)
    # fp32 value is one rounding of isum * sigma * 2^-32
    z = synth.std_normal(77, synth.STREAM_W, 4 * 96, 96)
    want = (z * 0.02).astype(np.float32)
    assert np.array_equal(part[0], want)


def test_outliers_rate_and_scale():
    K, n = 1024, 400
    base = synth.weights(5, K, 0, n, 0.02)
    w = synth.weights(5, K, 0, n, 0.02, outlier_thresh=workloads.OUTLIER_THRESH)
    mask = synth.outlier_mask(5, 0, n * K, workloads.OUTLIER_THRESH).reshape(n, K).astype(bool)
    rate = mask.mean()
    assert 0.0007 < rate < 0.0013
    assert np.array_equal(w[~mask], base[~mask])
    want = (base[mask].astype(np.float64) * 20.0).astype(np.float32)
    assert np.array_equal(w[mask], want)


def test_x_fp16_deterministic():
    a = synth.x_fp16(9, 3, 256)
    b = synth.x_fp16(9, 3, 256)
    assert a.dtype == np.float16 and np.array_equal(a.view(np.uint16), b.view(np.uint16))
    z = synth.std_normal(9, synth.STREAM_X, 0, 3 * 256).reshape(3, 256)
    assert np.array_equal(a, z.astype(np.float16))


def test_workload_shapes():
    w4 = workloads.workload(4)
    assert len(w4.matrices) == 256 and w4.Ms == [48]
    wb = sum(workloads.weight_bytes(m.bits, m.N, m.K) for m in w4.matrices)
    assert abs(wb / 1e9 - 11.89) < 0.01
    w5 = workloads.workload(5)
    wb5 = sum(workloads.weight_bytes(m.bits, m.N, m.K) for m in w5.matrices)
    assert abs(wb5 / 1e9 - 14.53) < 0.01
    w2 = workloads.workload(2)
    m = w2.matrices[0]
    assert abs(workloads.weight_bytes(m.bits, m.N, m.K) / 1e6 - 100.27) < 0.01
    for M in w5.Ms:
        slots = workloads.ragged_slots(M)
        assert sum(slots) == M and all(1 <= s <= 7 for s in slots)


def test_weight_bytes_of_every_format_match_the_packed_size():
    """For tile-aligned shapes the packed buffer holds exactly the algorithmic
    code, scale and zero-point bytes."""
    from oracle import oracle

    for fmt in (4, 5, workloads.FMT_G64, workloads.FMT_ZP):
        for N, K in [(34816, 5120), (5120, 17408), (16, 128)]:
            assert workloads.weight_bytes(fmt, N, K) == oracle.packed_bytes(fmt, N, K)

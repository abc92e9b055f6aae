"""The clock stamps behind the bench line's clock_observed (kd_clock_stamp,
kd_wall_clock_khz): every compute unit writes a stamp, the identity words name each of
the eight accelerator complexes, and the per-unit clock over some work is a plausible
shader clock."""
import numpy as np
import pytest

import bench
import output_head_kl_amd as kd

pytestmark = pytest.mark.gpu


def test_every_compute_unit_stamps_and_clocks_are_plausible(torch_cuda):
    torch = torch_cuda
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    stamps = torch.zeros((2, 3 * bench.CLOCK_GROUPS), dtype=torch.int64, device="cuda")
    x = torch.randn(4096, 4096, device="cuda")

    def work():
        y = x
        for _ in range(20):
            y = torch.tanh(y @ y)
        return y

    # The cycle counters advance at the clock the units actually run, idle included, so
    # the stamps must bracket GPU work only: the first call (library loading) comes first.
    work()
    torch.cuda.synchronize()
    print(f"clock stamps: {bench.CLOCK_GROUPS} workgroups, {n_cu} compute units", flush=True)
    kd.clock_stamp(stamps[0])
    work()
    kd.clock_stamp(stamps[1])
    torch.cuda.synchronize()
    khz = kd.wall_clock_khz()
    assert khz > 0
    rec = stamps.cpu().numpy().reshape(2, -1, 3)
    xcc = set(((rec[:, :, 0] >> 32) & 15).ravel().tolist())
    assert xcc == set(range(8)), xcc
    units = {(int(i >> 32) & 15, int(i >> 8) & 0xFF) for i in rec[0, :, 0]}
    assert len(units) == n_cu
    mhz = bench.unit_clocks(rec[0].ravel(), rec[1].ravel(), khz)
    print(f"per-unit clock MHz: median {np.median(mhz):.1f}, min {mhz.min():.1f}, "
          f"max {mhz.max():.1f}", flush=True)
    assert mhz.size == n_cu
    assert 300.0 < mhz.min() and mhz.max() < 3000.0
    # the constant counter advanced by the same time on every unit (one device clock)
    ticks = rec[1, :, 2] - rec[0, :, 2]
    assert ticks.min() > 0 and ticks.max() - ticks.min() < 0.01 * ticks.max()
    with pytest.raises(ValueError):
        kd.clock_stamp(torch.zeros(5, dtype=torch.int64, device="cuda"))

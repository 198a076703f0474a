"""Host arithmetic of the per-workgroup stamp summary (``stamps.summarize``)
on hand-made stamps, no GPU."""
import pytest
import torch

from dense_fp32_gemm_f32_amd.stamps import summarize


def test_summary_of_hand_made_stamps():
    # 16 workgroups; workgroup w starts at tick 100 + w (100 MHz: 10 ns a
    # tick), loops 1000 + 9 w ticks at 2.4 shader cycles per ns, stores 100
    st = torch.zeros(16, 6, dtype=torch.int64)
    for w in range(16):
        r0 = 100 + w
        r1 = r0 + 1000 + 9 * w
        st[w] = torch.tensor([r0, r1, r1 + 100, 7, 7 + 24 * (r1 - r0), 0])
    s = summarize(st, 100_000)
    assert s["start_spread_us"] == pytest.approx(0.15)
    loops = [10.0 + 0.09 * w for w in range(16)]
    assert s["loop_us_mean"] == pytest.approx(sum(loops) / 16, abs=1e-3)
    assert s["loop_us_max"] == pytest.approx(loops[-1], abs=1e-3)
    # XCD x holds workgroups x and x + 8
    assert s["loop_us_by_xcd"] == [pytest.approx((loops[x] + loops[x + 8]) / 2, abs=0.006)
                                   for x in range(8)]
    assert s["store_us_mean"] == pytest.approx(1.0)
    assert s["span_us"] == pytest.approx((115 + 1000 + 135 + 100 - 100) * 0.01)
    assert s["ghz"] == pytest.approx(2.4)

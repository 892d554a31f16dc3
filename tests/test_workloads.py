"""Seeded input generation: determinism, shapes, dtypes and the row sample.
CPU only."""

import torch

from workloads import WORKLOADS, make_inputs, sample_rows, workload_inputs


def test_inputs_are_deterministic_and_rounded():
    a = make_inputs(1, 2, 5, 7, 8, "bf16", seed=3, amp=0.5, with_dO=True)
    b = make_inputs(1, 2, 5, 7, 8, "bf16", seed=3, amp=0.5, with_dO=True)
    assert [x.shape for x in a] == [(1, 2, 5, 8), (1, 2, 7, 8), (1, 2, 7, 8), (1, 2, 5, 8)]
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and torch.equal(x, y)
    c = make_inputs(1, 2, 5, 7, 8, "bf16", seed=4)
    assert not torch.equal(a[0], c[0])


def test_amplitude_is_exact_scaling_before_rounding():
    g = torch.Generator().manual_seed(9)
    ref = (torch.randn(1, 1, 4, 8, generator=g) * 0.5).to(torch.bfloat16)
    q = make_inputs(1, 1, 4, 4, 8, "bf16", seed=9, amp=0.5)[0]
    assert torch.equal(q, ref)


def test_sample_rows():
    r = sample_rows(H=8, L=32768, n=256, seed=3)
    assert r.shape == (1, 8, 256)
    for h in range(8):
        rows = r[0, h].tolist()
        assert len(set(rows)) == 256 and rows[0] == 0 and rows[1] == 32767
        assert min(rows) >= 0 and max(rows) < 32768
    assert torch.equal(r, sample_rows(H=8, L=32768, n=256, seed=3))


def test_workload_table():
    assert set(WORKLOADS) == {
        "fwd_f32_B1H1L128d64", "fwd_bf16_B4H16L1024d64", "fwd_bf16_causal_B1H32L4096d128",
        "fwd_bf16_causal_B1H8L32768d128", "bwd_bf16_causal_B2H16L2048d128",
        "decode_bf16_B8H32Lq1Lk16384d128"}
    w = WORKLOADS["fwd_f32_B1H1L128d64"]
    q, k, v = workload_inputs(w)
    assert q.dtype == torch.float32 and q.shape == (1, 1, 128, 64)


def test_window_block_mask():
    from workloads import window_block_mask
    m = window_block_mask(6, window=2)
    assert m.dtype == torch.uint8 and m.shape == (6, 6)
    assert m.tolist() == [[1, 0, 0, 0, 0, 0], [1, 1, 0, 0, 0, 0], [1, 1, 1, 0, 0, 0],
                          [1, 0, 1, 1, 0, 0], [1, 0, 0, 1, 1, 0], [1, 0, 0, 0, 1, 1]]
    assert window_block_mask(3, window=1, first=False).tolist() == [[1, 0, 0], [0, 1, 0], [0, 0, 1]]

"""Seeded inputs and physical layouts (CPU)."""
import numpy as np
import pytest
import torch

from invariant_rmsnorm_backward_amd import inputs, layouts


def test_vector_hash_matches_scalar_definition():
    keys = [inputs.pack_key(inputs.TAG_X, s, p, h, c)
            for s, p, h, c in [(0, 0, 0, 0), (5, 13, 3, 4095), (1023, 262143, 63, 65535), (7, 1, 0, 9)]]
    seed = 0x1A7E0002
    want = [inputs.hash64(seed, k) for k in keys]
    t = torch.tensor([inputs._signed(k ^ inputs.seed_mix(seed)) for k in keys], dtype=torch.int64)
    got = [int(v) & inputs.MASK64 for v in inputs.mix64_t(t)]
    assert got == want
    # published SplitMix64 first output for seed 0 (state advanced by the golden gamma)
    assert inputs.mix64(0x9E3779B97F4A7C15) == 0xE220A8397B1DCDAF


def test_bf16_rounding_matches_torch_conversion():
    f = torch.randn(100000, dtype=torch.float32) * 1000
    f[:4] = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0])  # ties, zero
    ours = inputs._bits_to_bf16_tensor(inputs._f32_to_bf16_bits(f))
    ref = f.to(torch.bfloat16)
    assert torch.equal(ours.view(torch.int16), ref.view(torch.int16))


def test_generation_is_deterministic_and_row_addressable():
    wl = inputs.scaled(inputs.workload_h4096(), "small", hidden=256, lengths=[40, 25])
    x1 = inputs.gen_x(wl)
    x2 = inputs.gen_x(wl, chunk=7)
    assert torch.equal(x1.view(torch.int16), x2.view(torch.int16))
    rows = np.array([3, 64, 0, 41])
    xs = inputs.gen_x(wl, rows)
    assert torch.equal(xs.view(torch.int16), x1[rows].view(torch.int16))
    dy = inputs.gen_dy(wl)
    assert torch.equal(inputs.gen_dy(wl, rows).view(torch.int16), dy[rows].view(torch.int16))


def test_distributions():
    wl = inputs.scaled(inputs.workload_h4096(), "small", hidden=512, lengths=[300, 212])
    x = inputs.gen_x(wl).float()
    assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 1.0) < 0.01
    assert float(x.abs().max()) <= 3.47
    w = inputs.gen_w(wl).float()
    assert float(w.min()) >= 0.5 and float(w.max()) <= 1.5
    dy = inputs.gen_dy(wl).double()
    n = wl.n_tokens
    assert float(dy.abs().max()) <= 1.0 / n * 1.004
    assert abs(float(dy.mean())) < 0.01 / n


def test_mask_and_denominator():
    wl = inputs.scaled(inputs.workload_h5120(), "small", hidden=64, lengths=[100, 60, 40], pad_rows=30)
    s, p, _ = inputs.logical_keys(wl)
    act = inputs.active_mask(wl, s, p)
    assert 0.35 < act.mean() < 0.65
    assert inputs.n_active(wl) == int(act.sum())
    dy = inputs.gen_dy(wl).float()
    assert torch.all(dy[torch.from_numpy(~act)] == 0)
    assert torch.all(dy[torch.from_numpy(act)].abs().sum(dim=1) > 0)


def test_workload_shapes():
    w3 = inputs.workload_h8192()
    assert len(w3.lengths) == 16 and all(512 <= n <= 8192 for n in w3.lengths)
    w5 = inputs.workload_h5120()
    assert w5.n_tokens == 98304 and len(w5.lengths) == 64 and min(w5.lengths) > 0
    assert sum(inputs.pad_run_lengths(w5)) == 32768 and w5.n_tokens + w5.pad_rows == 131072
    q, k = inputs.workload_qk("q"), inputs.workload_qk("k")
    assert q.n_logical == 16384 * 32 and k.n_logical == 16384 * 8
    assert inputs.workload_h4096().n_logical == 32768


def _coverage(cell):
    seen = np.zeros(cell.n_logical, dtype=np.int64)
    for c in cell.calls:
        rl = np.arange(c.rows) if c.row_logical is None else c.row_logical
        real = rl[rl >= 0]
        np.add.at(seen, real, 1)
    return seen


def test_page_matrix_structure_h8():
    """Call counts and row shapes of the hidden=8 matrix printed on the page."""
    wl = inputs.workload_h8()
    cells = {c.name: c for c in layouts.page_matrix(wl)}
    assert cells["BN/full"].call_shapes == [59]
    assert cells["BN/chunked"].call_shapes == [7, 4, 7, 7, 2, 7, 6, 7, 7, 5]
    assert cells["BN/chunked_per_sample"].call_shapes == [7, 4, 7, 7, 2, 7, 6, 7, 7, 5]
    assert cells["B1-singleton_aggregate/full"].call_shapes[0] == 11        # s0
    assert cells["B1-singleton_aggregate/full"].call_shapes == [11, 7, 13, 9, 5, 14]
    assert cells["BN/padded_right"].call_shapes == [80]
    assert cells["BN/padded_left"].call_shapes == [80]
    assert cells["BN/permuted"].call_shapes == [59]
    for c in cells.values():
        assert np.all(_coverage(c) == 1), c.name
    pr = cells["BN/padded_right"].calls[0].row_logical
    pl = cells["BN/padded_left"].calls[0].row_logical
    assert np.all(pr[59:] == -1) and np.all(pl[:21] == -1)
    perm = cells["BN/permuted"].calls[0].row_logical
    assert not np.array_equal(perm, np.arange(59))


def test_per_head_layouts_and_packed_padding():
    q = inputs.scaled(inputs.workload_qk("q"), "q_small", lengths=[5, 3])
    cell = layouts.chunked_per_sample(q, chunk=2)
    assert cell.call_shapes == [2 * 32, 2 * 32, 1 * 32, 2 * 32, 1 * 32]
    assert np.all(_coverage(cell) == 1)
    rl = cell.calls[1].row_logical
    assert list(rl[:3]) == [2 * 32 + 0, 2 * 32 + 1, 2 * 32 + 2]
    w5 = inputs.scaled(inputs.workload_h5120(), "p_small", hidden=64, lengths=[10, 20, 5], pad_rows=9)
    pk = layouts.packed_with_padding(w5)
    assert pk.call_shapes == [44] and pk.calls[0].n_pad == 9
    assert np.all(_coverage(pk) == 1)


def test_gather_physical():
    wl = inputs.workload_h8()
    logical = np.arange(59 * 2).reshape(59, 2)
    cell = layouts.padded(wl, 80, "left")
    phys = layouts.gather_physical(logical, cell.calls[0], pad_value=-7)
    assert np.all(phys[:21] == -7) and np.array_equal(phys[21:], logical)

"""Host checks of the two weight relayouts the device paths read (synth.device):
the column-block layout of the TEAL projections and of the step's down
projection, and the step-major tile layout of the batched matrix-core path.
Each is checked element by element against its definition, with ragged
edges (padding zero)."""

import numpy as np
import torch

from synth import device as sdev


def _w(rows, cols, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(rows, cols, generator=g)


def test_column_blocks_hold_each_output_column_of_each_input_channel():
    d_out, d_in = 300, 7  # the last block holds 44 real columns
    w = _w(d_out, d_in, 1)
    wb = sdev.teal_blocked(w)
    assert wb.shape == (3, d_in, 128)
    for b in range(3):
        for j in range(d_in):
            for c in range(128):
                o = b * 128 + c
                want = w[o, j] if o < d_out else 0.0
                assert wb[b, j, c] == want
    # one channel's piece of one block is 128 contiguous values
    flat = wb.flatten()
    assert torch.equal(flat[(1 * d_in + 4) * 128:(1 * d_in + 5) * 128], w[128:256, 4])


def test_down_column_blocks_come_from_the_transposed_down_rows():
    # the step's down copy: W_down [d, d_ff] in column blocks, built from
    # w_down_t [d_ff, d]; block b, input channel j, column c = w_down_t[j, 128 b + c]
    d, d_ff = 256, 40
    w_down_t = _w(d_ff, d, 2)
    wb = sdev.teal_blocked(w_down_t.t())
    assert wb.shape == (2, d_ff, 128)
    assert torch.equal(wb[0], w_down_t[:, :128])
    assert torch.equal(wb[1], w_down_t[:, 128:])
    # y = W_down h through the blocks equals the row form sum_j h_j w_down_t[j]
    h = _w(d_ff, 1, 3)[:, 0].double()
    y_blocks = torch.cat([(wb[b].double() * h[:, None]).sum(0) for b in range(2)])
    y_rows = (w_down_t.double() * h[:, None]).sum(0)
    assert torch.allclose(y_blocks, y_rows, rtol=0, atol=1e-12)


def test_matrix_core_tiles_follow_the_lane_order():
    rows, d_in = 37, 70  # 3 tiles (11 padding rows), 3 steps (26 padding channels)
    w = _w(rows, d_in, 4)
    t = sdev.mma_tiles(w)
    assert t.shape == (3, 3, 4, 16, 8)  # [step, tile, q, r, e]
    rng = np.random.default_rng(0)
    for _ in range(400):
        step, tile, q, r, e = (int(rng.integers(n)) for n in t.shape)
        row, ch = tile * 16 + r, step * 32 + q * 8 + e
        want = w[row, ch] if row < rows and ch < d_in else 0.0
        assert t[step, tile, q, r, e] == want
    # lane l of a (tile, step) fragment: row l % 16, channels 8 (l // 16) .. + 7
    frag = t[1, 2].reshape(64, 8)
    for lane in range(64):
        row, c0 = 32 + lane % 16, 32 + 8 * (lane // 16)
        for e in range(8):
            want = w[row, c0 + e] if row < rows and c0 + e < d_in else 0.0
            assert frag[lane, e] == want

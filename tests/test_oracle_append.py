"""Cache append rows of the oracle against the draft pass's own block keys:
layer l's row at a position must equal the [c | k_pe] that the attention of
layer l computes for a block token whose layer input is the fc output of the
same captured states (the attention code path, traced), at every layer."""
import numpy as np

from oracle import dspark as O
from synth import configs as C, gen


def test_cache_rows_equal_block_keys_of_each_layer_on_the_fc_output():
    wl = C.CFG1.replace(kv_lens=(5, 17), fixture_gains=True)
    m = wl.model
    stored = gen.make_weights(wl)
    inp = gen.make_inputs(wl)
    W = O.Weights(stored)
    _, _, per_layer = O.backbone(m, W, inp, wl.formats.kv_cache, wl.formats.captured, keep_layers=True)
    x_fc = per_layer[0]
    caches = [np.asarray(c, np.float64) for c in inp.caches]
    n_seq, B = wl.n_seq, m.block
    # the captured states of every block row, [n_seq * B, n_captured, H], and their positions
    cap = np.asarray(inp.captured).transpose(0, 2, 1, 3).reshape(n_seq * B, m.n_captured, m.hidden)
    pos = np.concatenate([np.diff(inp.kv_offsets)[s] + np.arange(B) for s in range(n_seq)])
    rows = O.cache_rows(m, W, cap, pos, wl.formats.captured)
    assert rows.shape == (m.n_layers, n_seq * B, m.latent)
    for l in range(m.n_layers):
        tr = {}
        O.layer(m, W, l, x_fc, caches, inp.kv_offsets, trace=tr)
        for s in range(n_seq):
            want = np.concatenate([tr[s]["c"], tr[s]["kp"]], axis=1)
            np.testing.assert_allclose(rows[l, s * B:(s + 1) * B], want, rtol=1e-12, atol=1e-12)


def test_cache_rows_rope_at_position_zero_is_identity():
    wl = C.CFG1.replace(kv_lens=(3,))
    m = wl.model
    W = O.Weights(gen.make_weights(wl))
    cap = np.repeat(gen.normal((1, m.n_captured, m.hidden), 4, 0), 2, axis=0)  # one state, twice
    r0 = O.cache_rows(m, W, cap, [0, 0], "f32")
    r1 = O.cache_rows(m, W, cap, [0, 1], "f32")
    # same row content; position 0 leaves k_pe unrotated, position 1 rotates it
    np.testing.assert_array_equal(r0[:, 0], r0[:, 1])
    np.testing.assert_array_equal(r1[:, 0, :m.kv_lora], r1[:, 1, :m.kv_lora])
    assert not np.allclose(r1[:, 0, m.kv_lora:], r1[:, 1, m.kv_lora:])
    # rotation keeps the norm of every pair
    a, b = r1[:, 0, m.kv_lora:], r1[:, 1, m.kv_lora:]
    np.testing.assert_allclose(a[..., 0::2] ** 2 + a[..., 1::2] ** 2, b[..., 0::2] ** 2 + b[..., 1::2] ** 2,
                               rtol=1e-12)

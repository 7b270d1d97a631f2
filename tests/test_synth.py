"""The shared input generator: Philox known answers, determinism, slices,
rotary embedding properties and the planted structure.  CPU only."""
import ctypes
import json
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        ctr = (ctypes.c_uint32 * 4)(*[int(x, 16) for x in c["ctr"]])
        key = (ctypes.c_uint32 * 2)(*[int(x, 16) for x in c["key"]])
        out = (ctypes.c_uint32 * 4)()
        synth.lib().syn_philox(ctr, key, out)
        assert ["%08x" % v for v in out] == c["out"]


def test_normal_rope_deterministic_and_sliceable():
    a = synth.normal_rope(5, synth.T_K, 2, 0, 300, 4, 64, 1e4, 0, "f32")
    b = synth.normal_rope(5, synth.T_K, 2, 0, 300, 4, 64, 1e4, 0, "f32")
    np.testing.assert_array_equal(a, b)
    part = synth.normal_rope(5, synth.T_K, 2, 120, 50, 4, 64, 1e4, 120, "f32")
    np.testing.assert_array_equal(part, a[120:170])
    c = synth.normal_rope(5, synth.T_K, 3, 0, 300, 4, 64, 1e4, 0, "f32")
    assert not np.array_equal(a, c)


def test_normal_statistics():
    x = synth.normal_rope(9, synth.T_V, 0, 0, 20000, 8, 64, 0.0, 0, "f32").astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3
    assert abs(((x - x.mean()) ** 4).mean() / x.var() ** 2 - 3.0) < 0.05   # kurtosis


def test_rope_rotates_pairs():
    D, half = 64, 32
    raw = synth.normal_rope(4, synth.T_Q, 0, 0, 64, 2, D, 0.0, 0, "f32").astype(np.float64)
    rot = synth.normal_rope(4, synth.T_Q, 0, 0, 64, 2, D, 1e4, 0, "f32").astype(np.float64)
    # pair norms are preserved
    np.testing.assert_allclose(raw[..., :half] ** 2 + raw[..., half:] ** 2,
                               rot[..., :half] ** 2 + rot[..., half:] ** 2, rtol=1e-5, atol=1e-6)
    # position 0 is not rotated; position t rotates pair i by t * base^(-2i/D)
    np.testing.assert_allclose(rot[0], raw[0], rtol=0, atol=1e-7)
    t, i = 17, 3
    ang = t * 1e4 ** (-2.0 * i / D)
    want = raw[t, 0, i] * np.cos(ang) - raw[t, 0, i + half] * np.sin(ang)
    assert abs(rot[t, 0, i] - want) < 1e-5


def test_bf16_storage_rounding():
    x = np.asarray([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], np.float32)
    np.testing.assert_array_equal(synth.to_bf16(x), [0x3F80, 0x3F80, 0x3F82, 0xC020])
    np.testing.assert_array_equal(synth.from_bf16(synth.to_bf16(x[[0, 3]])), x[[0, 3]])


def test_projection_selector_and_noise():
    Wq, Wk = synth.projections(11, 6, 128, "f32")
    assert Wq.shape == (6, 128, 16)
    dims = synth.low_freq_dims(128)
    sel = Wq[:, dims, np.arange(16)]
    assert np.all(np.abs(sel - 1.0) < 0.15)
    off = np.delete(Wq.reshape(6, -1), (dims * 16 + np.arange(16)), axis=1)
    assert abs(off.std() - 0.02) < 1e-3
    assert not np.array_equal(Wq, Wk)


def test_small_workloads_shapes_and_structure():
    w = synth.small(2)
    assert w.kind == "decode" and w.q.shape == (3, 32, 128) and w.q.dtype == np.uint16
    assert [k.shape for k in w.k] == [(6000, 8, 128), (9001, 8, 128), (4097, 8, 128)]
    assert len(w.ret_heads) == 6 and w.ret_heads == sorted(w.ret_heads)
    c = synth.small(3)
    assert c.kind == "chunk" and c.n_tok == 300 and c.chunk_pos0 == 5000 - 300
    assert c.row_pos(0) == 4700 and c.row_pos(299) == 4999
    r = synth.small(5)
    assert len(set(r.seq_lens.tolist())) == len(r.seq_lens)
    assert set(r.top_p.tolist()) <= set(np.asarray([0.8, 0.9, 0.95, 0.99], np.float32).tolist())


def test_amplitude_formula():
    # share of the mass of n cluster keys at score a^2 against L background
    # keys with scores ~ N(0, a^2): n e^{s a^2} / (n e^{s a^2} + L e^{s^2 a^2/2})
    a = synth.amplitude(16, 131072, 0.25)
    s = 0.25
    share = 16 * np.exp(s * a * a) / (16 * np.exp(s * a * a) + 131072 * np.exp(s * s * a * a / 2))
    assert abs(share - 0.999) < 1e-9 and 8.4 < a < 8.6


def test_shared_kv_clusters():
    # grouped retrieval heads share their KV head's planted cluster: the same
    # size, and the first head's planted keys score high for the second head's
    # query too; without the option the heads draw independent clusters, and the
    # option leaves every other draw (and the ungrouped heads) unchanged
    kw = dict(seed=41, lens=(5000, 7000), Hq=32, Hkv=8, D=128, n_ret=3, p=0.9, window=256, sinks=8,
              rope=1e4, size_dist=("loguniform", 64, 256), ret_heads=[4, 5, 20])
    a = synth.cluster_decode(shared_kv=True, **kw)
    b = synth.cluster_decode(shared_kv=False, **kw)
    for bq in range(2):
        assert a.info["sizes"][(bq, 4)] == a.info["sizes"][(bq, 5)]
        assert a.info["sizes"][(bq, 20)] == b.info["sizes"][(bq, 20)]
    np.testing.assert_array_equal(a.k[0][:, 5, :], b.k[0][:, 5, :])      # KV head 5 (head 20) untouched
    np.testing.assert_array_equal(a.q[:, 4], b.q[:, 4])                  # the group's first head as before
    assert not np.array_equal(a.q[:, 5], b.q[:, 5])                      # the second head follows the shared cluster
    # head 5's query, projected on the planted low-frequency coordinates,
    # points along head 4's: both were planted along the same direction
    dims = synth.low_freq_dims(128)
    for bq in range(2):
        u4 = synth.as_f32(a.q[bq, 4])[dims]
        u5 = synth.as_f32(a.q[bq, 5])[dims]
        cos = float(u4 @ u5 / np.linalg.norm(u4) / np.linalg.norm(u5))
        assert cos > 0.9, cos

"""Input generators: SplitMix64 against its published output, bf16 rounding, blob
placement and distributions."""
import numpy as np

import synth


def test_splitmix64_published_sequence():
    # SplitMix64 seeded with 0 (Steele, Lea & Flood 2014; the widely published
    # reference implementation) starts with these outputs.
    w = synth.words(0, 0, 4)
    assert [int(v) for v in w] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                   0x06C45D188009454F, 0xF88BB8A8724C81EC]
    # counter-based: any window equals the same slice of the full stream
    assert np.array_equal(synth.words(0, 2, 2), w[2:])


def test_bf16_round_to_nearest_even():
    f = np.array([1.0, 0x3F808000, 0x3F818000, 0x3F80C000, -2.5], dtype=np.float64)
    bits = np.array([0x3F800000, 0x3F808000, 0x3F818000, 0x3F80C000], dtype=np.uint32).view(np.float32)
    got = synth.f32_to_bf16_rne(np.concatenate([bits, np.array([-2.5], np.float32)]))
    assert [int(v) for v in got] == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020]
    del f


def test_blob_planes_and_distributions():
    H, I, bits = 512, 256, 4
    b = synth.expert_blob(123, 0, 5, H, I, bits)
    off, tot = synth.blob_layout(H, I, bits)
    sizes = synth.plane_sizes(H, I, bits)
    assert b.size == tot == 221_184
    # code plane bytes are the raw stream bytes
    key = synth.stream_key(123, 0, 5, synth.T_UP_CODES)
    assert np.array_equal(b[off[2]:off[2] + sizes[2]], synth.random_bytes(key, sizes[2]))
    # sb plane: scales in [0.002, 0.02], biases in [-0.1, 0.1], bf16 exact
    for t in (1, 3, 5):
        sb = b[off[t]:off[t] + sizes[t]].view(np.uint16).reshape(-1, 2)
        s, bb = synth.bf16_to_f32(sb[:, 0]), synth.bf16_to_f32(sb[:, 1])
        assert s.min() >= 0.002 - 1e-5 and s.max() <= 0.02 + 6.2e-5   # bf16 half-ulp at 0.02
        assert bb.min() >= -0.1001 and bb.max() <= 0.1001
        assert abs(s.mean() - 0.011) < 0.001 and abs(bb.mean()) < 0.01
    # uniform codes
    codes = b[off[0]:off[0] + sizes[0]]
    nib = np.concatenate([codes & 15, codes >> 4])
    assert np.abs(np.bincount(nib, minlength=16) / nib.size - 1 / 16).max() < 0.005
    # different experts, layers and seeds give different bytes
    assert not np.array_equal(b, synth.expert_blob(123, 0, 6, H, I, bits))
    assert not np.array_equal(b, synth.expert_blob(123, 1, 5, H, I, bits))


def test_tiered_and_zipf_inputs():
    wl = synth.WORKLOADS[2]
    bits = wl.expert_bits()
    assert (bits == 4).sum() == 128 and (bits == 2).sum() == 384
    perm, p = synth.zipf_prior(wl.seed, wl.E)
    assert abs(p.sum() - 1) < 1e-12 and p[perm[0]] > p[perm[1]] > p[perm[-1]]
    assert np.array_equal(np.sort(perm[:128]), synth.hot_set(wl.seed, wl.E))
    lb = wl.logit_bias()
    assert lb.dtype == np.float32 and np.argmax(lb) == perm[0]

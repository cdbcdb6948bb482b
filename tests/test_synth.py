"""The seeded input generator: published Philox known answers, determinism,
shape of the distribution (CPU only)."""

import numpy as np
import pytest

import synth

# Known-answer vectors of Philox4x32-10 published with the Random123 library
# that accompanies Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3".
KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(ctr, key, want):
    assert synth.philox4x32_10(ctr, key) == want


def test_fill_equals_gather_and_offsets():
    st = synth.peer_stream(3, 1, 5)
    a = synth.normal_bf16(7, st, 10_000, 1e-3)
    idx = np.array([0, 1, 17, 9_999, 4_321])
    assert np.array_equal(synth.normal_bf16_at(7, st, idx, 1e-3), a[idx])
    b = synth.normal_bf16(7, st, 100, 1e-3, i0=500)
    assert np.array_equal(b, a[500:600])
    f = synth.normal_f32(7, synth.master_stream(0), 4096, 0.02)
    assert np.array_equal(synth.normal_f32_at(7, synth.master_stream(0), idx[idx < 4096], 0.02),
                          f[idx[idx < 4096]])


def test_streams_differ():
    n = 4096
    base = synth.normal_bf16(1, synth.peer_stream(1, 0, 0), n, 1e-3)
    for other in (synth.peer_stream(2, 0, 0), synth.peer_stream(1, 1, 0),
                  synth.peer_stream(1, 0, 1), synth.tensor_stream(1, 0, 0, 0)):
        assert not np.array_equal(base, synth.normal_bf16(1, other, n, 1e-3))
    assert not np.array_equal(base, synth.normal_bf16(2, synth.peer_stream(1, 0, 0), n, 1e-3))


def test_normal_shape():
    x = synth.normal_f32(11, synth.master_stream(0), 1 << 20, 0.02).astype(np.float64)
    assert abs(x.mean()) < 5 * 0.02 / np.sqrt(x.size)
    assert abs(x.std() / 0.02 - 1) < 0.01
    # Irwin-Hall with 8 terms: support +-sqrt(24) sigma
    assert np.abs(x).max() <= np.sqrt(24) * 0.02 * (1 + 1e-6)
    g = synth.normal_bf16(11, synth.peer_stream(1, 0, 0), 1 << 18, 1e-3)
    gf = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(gf.std() / 1e-3 - 1) < 0.02


def test_tokens_range():
    c = [synth.tokens(5, t, r) for t in range(1, 20) for r in range(8)]
    assert min(c) >= synth.TOKENS_LO and max(c) <= synth.TOKENS_HI
    assert len(set(c)) > 100


def test_workload_sizes():
    w = synth.WORKLOADS
    assert w["tiny_mlp"].psi == 525_568
    assert w["gpt2_small"].psi == 124_439_808 and len(w["gpt2_small"].params) == 148
    assert w["llama3_8b"].psi == 8_030_261_248 and len(w["llama3_8b"].params) == 291
    assert w["gpt_7b5"].psi == 6_648_963_072 and len(w["gpt_7b5"].params) == 387
    assert w["llama3_8b_dp"].psi == w["llama3_8b"].psi

"""Seeded input generators: storage conversions against torch's casts, and
the workload recipes (shapes, determinism, planted needles)."""
import numpy as np
import torch

from long_context_mean_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(50000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 50000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38], np.float32)]).astype(np.float32)
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-448, 448, 50000), rng.standard_normal(50000) * 0.01,
                        rng.standard_normal(5000) * 1e-3]).astype(np.float32)
    # midpoints between neighbouring codes exercise ties-to-even
    pos = synth._E4M3_POS
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids]).astype(np.float32)
    ours = synth.f64_to_e4m3_codes(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_quantization_scale():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((3, 50, 128)).astype(np.float32)
    k[1, 7] = 0.0
    codes, scale = synth.quantize_e4m3(k)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    assert scale[1, 7] == 1.0 and np.all(codes[1, 7] == 0)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy() * scale[..., None]
    assert np.max(np.abs(dec - k)) <= np.max(np.abs(k)) / 16        # 3 mantissa bits
    amax = np.abs(torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()).max(-1)
    assert np.all((amax == 448.0) | (scale == 1.0))


def test_generators_are_deterministic_and_shaped():
    a = synth.make("c1")
    b = synth.make("c1")
    assert np.array_equal(a.k, b.k) and np.array_equal(a.q, b.q) and np.array_equal(a.w, b.w)
    assert a.k.shape == (1, 4096, 64) and a.q.shape == (1, 16, 64) and a.k.dtype == np.float32
    assert (a.B, a.h, a.topk) == (64, 4, 256)
    c = synth.make("c1", seed=7)
    assert not np.array_equal(a.k, c.k)


def test_needles_are_planted():
    p = synth.make("c4", L=4096, n_needles=32)
    q = synth.bf16_bits_to_f32(p.q)
    k = synth.bf16_bits_to_f32(p.k)
    for n in range(p.N):
        pos, heads = p.needles[n, :, 0], p.needles[n, :, 1]
        assert len(set(pos.tolist())) == 32
        expect = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(3.0 * q[n, heads]))
        assert np.array_equal(k[p.q_seq[n], pos], expect)


def test_prefill_positions():
    p = synth.make("c3", L=8192, q_pos=np.arange(8192 - 256, 8192, dtype=np.int32),
                   q_seq=np.zeros(256, np.int32), N=256)
    assert p.N == 256 and p.q_pos[0] == 8192 - 256 and p.q_pos[-1] == 8191
    assert p.tokens_indexed() == int(np.arange(8192 - 255, 8193).sum())


def test_fp8_prefill_workload_quantizes_the_bf16_draws():
    """The fp8 prefill chunk stores the same fp32 draws as the bf16 one: q per
    head and k per token as e4m3 codes with an absmax/448 scale."""
    over = dict(L=4096, N=64, q_seq=np.zeros(64, np.int32),
                q_pos=np.arange(4096 - 64, 4096, dtype=np.int32))
    p8 = synth.make("c3f8", **over)
    pb = synth.make("c3", **over)
    assert p8.q.dtype == np.uint8 and p8.k.dtype == np.uint8
    assert p8.q_scale.shape == (64, 64) and p8.k_scale.shape == (1, 4096)
    q8 = torch.from_numpy(p8.q.copy()).view(torch.float8_e4m3fn).float().numpy()
    assert np.all(np.abs(q8).max(-1) == 448.0)
    qd = q8 * p8.q_scale[..., None]
    qb = synth.bf16_bits_to_f32(pb.q)
    assert np.max(np.abs(qd - qb)) <= np.abs(qb).max() / 8
    assert np.array_equal(synth.e4m3_codes_to_f32(p8.q, p8.q_scale), qd)

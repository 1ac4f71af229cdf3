"""Pins of the weight-quantised GEMM oracle (CPU): the INT4 quantiser by closed forms and round-half-to-even ties, the FP8 quantiser against torch's own
e4m3 cast, and the GEMM against brute force and one-hot rows."""
import numpy as np
import pytest
import torch

from oracle import codec, wgemm


def _bf16(a):
    return codec.bf16_from_f32(np.asarray(a, dtype=np.float32))


def test_int4_exact_multiples_and_ties():
    K = 128
    # group 0: multiples of 0.25 up to 7 * 0.25 -> scale exactly 0.25, codes are the integers
    ints = np.tile(np.arange(-7, 8), 9)[:K].astype(np.float32)
    ints[0] = 7.0
    # group 1 (second row): absmax 7 -> scale 1; halves round to even
    ties = np.zeros(K, dtype=np.float32)
    ties[:8] = [7.0, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, -6.5]
    w = _bf16(np.stack([ints * 0.25, ties]))
    q, s = wgemm.quantize_w4(w)
    assert codec.f32_from_bf16(s).tolist() == [[0.25], [1.0]]
    assert np.array_equal(q[0], ints.astype(np.int8))
    assert q[1, :8].tolist() == [7, 2, 4, -2, 0, 2, 0, -6]
    assert not q[1, 8:].any()


def test_int4_zero_group_and_bounds():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((48, 512)).astype(np.float32)
    w[7, 128:256] = 0.0
    wb = _bf16(w)
    q, s = wgemm.quantize_w4(wb)
    assert s[7, 1] == 0 and not q[7, 128:256].any()
    assert q.min() >= -8 and q.max() <= 7
    # each group's largest element maps to +-7 and the reconstruction is within half a step
    wf = codec.f64_from_bf16(wb)
    sf = codec.f64_from_bf16(s)
    deq = wgemm.dequant_w4(q, s)
    for n in range(48):
        for g in range(4):
            blk = wf[n, 128 * g:128 * g + 128]
            if not blk.any():
                continue
            i = np.argmax(np.abs(blk))
            assert abs(q[n, 128 * g + i]) == 7
            assert np.max(np.abs(deq[n, 128 * g:128 * g + 128] - blk)) <= 0.5 * sf[n, g] * (1 + 2 ** -6)


def test_int4_matches_torch_rounding():
    rng = np.random.default_rng(4)
    w = _bf16(rng.standard_normal((32, 384)).astype(np.float32) * 0.02)
    q, s = wgemm.quantize_w4(w)
    wt = torch.from_numpy(codec.f32_from_bf16(w)).reshape(32, 3, 128)
    amax = wt.abs().amax(dim=2)
    st = (amax / 7.0).to(torch.bfloat16).to(torch.float32)
    inv = torch.where(st > 0, 1.0 / st, torch.zeros_like(st))
    qt = torch.clamp(torch.round(wt * inv[:, :, None]), -8, 7).to(torch.int8).reshape(32, 384)
    assert np.array_equal(q, qt.numpy())
    assert np.array_equal(s, st.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_fp8_quantiser_matches_torch_cast():
    rng = np.random.default_rng(5)
    w = _bf16(rng.standard_normal((32, 256)).astype(np.float32) * 3.0)
    c, s = wgemm.quantize_w8(w)
    wt = torch.from_numpy(codec.f32_from_bf16(w)).reshape(32, 2, 128)
    st = (wt.abs().amax(dim=2) / 448.0).to(torch.bfloat16).to(torch.float32)
    ct = (wt * (1.0 / st)[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(32, 256)
    assert np.array_equal(c, ct.numpy())


def test_gemm_one_hot_and_brute_force():
    rng = np.random.default_rng(6)
    N, K, M = 16, 128, 3
    w = _bf16(rng.standard_normal((N, K)).astype(np.float32))
    q, s = wgemm.quantize_w4(w)
    W = wgemm.dequant_w4(q, s)
    x = np.zeros((M, K), dtype=np.float32)
    x[0, 5] = 1.0
    x[1, 127] = -2.0
    x[2] = rng.standard_normal(K)
    xb = _bf16(x)
    y = wgemm.gemm(xb, W)
    assert np.array_equal(y[0], W[:, 5]) and np.array_equal(y[1], -2.0 * W[:, 127])
    xf = codec.f64_from_bf16(xb)
    for n in range(N):
        acc = 0.0
        for k in range(K):
            acc += float(xf[2, k]) * float(codec.f64_from_bf16(s[n, k // 128])) * float(q[n, k])
        assert y[2, n] == pytest.approx(acc, rel=1e-12, abs=1e-12)

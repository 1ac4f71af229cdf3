"""Weight-quantised decode GEMM on the GPU against the oracle (Cloudflare post, section "Compressed
model weights"): the library's INT4 and FP8 quantisers are bit-exact to the oracle's (codes in the
packed layout, scales), and y = x W^T matches the fp64 GEMM over the dequantised weights within the
bf16-output tolerance, for M = 1..64, several split counts (ragged last split included) and, at the
8192 x 8192 size the benchmark streams, on sampled output tiles."""
import numpy as np
import pytest
import torch

import fp8_paged_kv_append_amd as kv
from kvsynth import weights as wsyn
from oracle import codec, wgemm
from tests import layout
from tests.gpu_util import dev, host, note

pytestmark = pytest.mark.gpu

TOL = 1e-2          # max |y - ref| / max |ref| per output row, bf16 result


def _quantize_dev(w_bits, bits):
    n, k = w_bits.shape
    packed = torch.empty(n * k // (2 if bits == 4 else 1), dtype=torch.uint8, device="cuda")
    scales = torch.empty(n * k // 128, dtype=torch.int16, device="cuda")
    (kv.w4_quantize_bf16 if bits == 4 else kv.w8_quantize_bf16)(dev(w_bits), packed, scales)
    torch.cuda.synchronize()
    return packed, scales


def _oracle_codes(w_bits, bits):
    """The oracle's codes [N][K] and scales [N][K/128] in logical order, and the weights they stand for."""
    if bits == 4:
        q, s = wgemm.quantize_w4(w_bits)
        return q, s, wgemm.dequant_w4(q, s)
    c, s = wgemm.quantize_w8(w_bits)
    return c, s, wgemm.dequant_w8(c, s)


def _device_codes(packed_bytes, scales_bits, n, k, bits):
    """Device codes and scales mapped from the library's packed layout to logical order."""
    codes = (layout.unpack_w4 if bits == 4 else layout.unpack_w8)(packed_bytes, n, k)
    return codes, layout.unpack_scales(scales_bits, n, k)


def _row_err(y_bits, ref):
    y = codec.f64_from_bf16(y_bits)
    den = np.maximum(np.max(np.abs(ref), axis=1), 1e-30)
    return float(np.max(np.max(np.abs(y - ref), axis=1) / den))


def _gemm(bits, x, packed, scales, n, k, splits=0):
    m = x.shape[0]
    y = torch.empty((m, n), dtype=torch.int16, device="cuda")
    s = splits or kv.wgemm_auto_splits(m, n, k)
    nb = kv.wgemm_workspace_bytes(m, n, k, s)
    ws = torch.zeros(max(nb, 16) // 4 + 4, dtype=torch.float32, device="cuda")   # counter words start at zero
    (kv.w4a16_gemm if bits == 4 else kv.w8a16_gemm)(x, packed, scales, n, k, y, num_splits=splits, workspace=ws)
    torch.cuda.synchronize()
    return host(y, np.uint16)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("shape", ["tiny", "ragged"])
def test_quantiser_bit_exact(bits, shape):
    note(f"quantiser w{bits} {shape}")
    sh = wsyn.SHAPES[shape]
    w = wsyn.weights(sh)
    w[3, 128:256] = 0                      # an all-zero group: scale 0, codes 0
    packed, scales = _quantize_dev(w, bits)
    o_codes, o_scales, _ = _oracle_codes(w, bits)
    g_codes, g_scales = _device_codes(host(packed, np.uint8), host(scales, np.uint16), sh.n, sh.k, bits)
    assert np.array_equal(g_codes, o_codes)
    assert np.array_equal(g_scales, o_scales)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("m", [1, 5, 16, 17, 40, 64])
def test_gemm_matches_oracle(bits, m):
    sh = wsyn.SHAPES["ragged"]                       # N = 320 (5 column blocks, the last one partly idle)
    note(f"gemm w{bits} ragged m={m}")
    w = wsyn.weights(sh)
    packed, scales = _quantize_dev(w, bits)
    o_codes, _, W = _oracle_codes(w, bits)
    assert np.array_equal(_device_codes(host(packed, np.uint8), host(scales, np.uint16), sh.n, sh.k, bits)[0], o_codes)
    x = wsyn.activations(sh, m)
    ref = wgemm.gemm(x, W)
    dx = dev(x)
    for splits in (0, 1, 2, 3, 5):                   # K = 1280: 5 chunks; 2 and 3 splits leave a short last one
        err = _row_err(_gemm(bits, dx, packed, scales, sh.n, sh.k, splits), ref)
        note(f"  splits={splits}: row error {err:.2e}")
        assert err <= TOL


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("m", [1, 3, 16])
def test_gemm_in_block_k_split(bits, m):
    """N = 4096 output channels and one split: the four waves of a block cut K = 1280 (10 groups) into
    3 + 3 + 3 + 1 groups and add their results through LDS; also with an explicit second split."""
    sh = wsyn.SHAPES["wide"]
    note(f"gemm w{bits} wide m={m}")
    w = wsyn.weights(sh)
    packed, scales = _quantize_dev(w, bits)
    _, _, W = _oracle_codes(w, bits)
    x = wsyn.activations(sh, m)
    ref = wgemm.gemm(x, W)
    dx = dev(x)
    assert kv.wgemm_auto_splits(m, sh.n, sh.k) == 1
    for splits in (0, 2):
        err = _row_err(_gemm(bits, dx, packed, scales, sh.n, sh.k, splits), ref)
        note(f"  splits={splits}: row error {err:.2e}")
        assert err <= TOL


@pytest.mark.parametrize("bits", [4, 8])
def test_gemm_tiny_and_zero_rows(bits):
    """K = 256 (one chunk, one split), an all-zero activation row and an all-zero weight group."""
    sh = wsyn.SHAPES["tiny"]
    note(f"gemm w{bits} tiny")
    w = wsyn.weights(sh)
    w[5, :128] = 0
    packed, scales = _quantize_dev(w, bits)
    _, _, W = _oracle_codes(w, bits)
    x = wsyn.activations(sh, 3)
    x[1] = 0
    y = _gemm(bits, dev(x), packed, scales, sh.n, sh.k)
    assert not y[1].any()
    ref = wgemm.gemm(x, W)
    assert _row_err(y[[0, 2]], ref[[0, 2]]) <= TOL


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("m", [1, 3, 8, 16, 64])
def test_gemm_full_size_sampled(bits, m):
    """8192 x 8192 weights (one matrix of the benchmark's stack), the library's split choice at the
    benchmark's row counts and M=3 (the in-block K split at M <= 4, the split form with its staging sized to
    8 rows and to 16, the chunked form at 64): the codes of sampled 16-row tiles bit-exact to the oracle's,
    and y on those tiles' columns within tolerance."""
    sh = wsyn.SHAPES["stack_8k"]
    note(f"gemm w{bits} 8192x8192 m={m}")
    w = wsyn.weights(sh, layer=0)
    packed, scales = _quantize_dev(w, bits)
    x = wsyn.activations(sh, m)
    y = _gemm(bits, dev(x), packed, scales, sh.n, sh.k)
    hp, hs = host(packed, np.uint8), host(scales, np.uint16)
    KG = sh.k // 128
    tile_bytes = KG * 64 * (16 if bits == 4 else 32)
    for t in (0, 137, 511):
        o_codes, o_scales, W = _oracle_codes(w[16 * t:16 * t + 16], bits)
        g_codes, g_scales = _device_codes(hp[t * tile_bytes:(t + 1) * tile_bytes], hs[t * KG * 16:(t + 1) * KG * 16],
                                          16, sh.k, bits)
        assert np.array_equal(g_codes, o_codes), t
        assert np.array_equal(g_scales, o_scales), t
        ref = wgemm.gemm(x, W)
        err = _row_err(y[:, 16 * t:16 * t + 16], ref)
        note(f"  tile {t}: row error {err:.2e}")
        assert err <= TOL


@pytest.mark.parametrize("bits", [4, 8])
def test_workspace_reuse_and_graph_replay(bits):
    """One workspace serves calls of different shapes and split counts back to back with the same
    results, and a captured graph of two GEMMs replays bit-identically to the eager calls."""
    note(f"gemm w{bits} workspace reuse + graph")
    shapes = [(wsyn.SHAPES["ragged"], 5, 5), (wsyn.SHAPES["ragged"], 33, 2), (wsyn.SHAPES["tiny"], 1, 1),
              (wsyn.SHAPES["ragged"], 1, 3)]
    ws = torch.zeros(1 << 20, dtype=torch.float32, device="cuda")
    cases = []
    for sh, m, splits in shapes:
        w = wsyn.weights(sh)
        packed, scales = _quantize_dev(w, bits)
        _, _, W = _oracle_codes(w, bits)
        x = wsyn.activations(sh, m)
        cases.append((sh, dev(x), packed, scales, splits, wgemm.gemm(x, W)))
    f = kv.w4a16_gemm if bits == 4 else kv.w8a16_gemm
    outs = []
    for rep in range(2):
        for sh, dx, packed, scales, splits, ref in cases:
            y = torch.empty((dx.shape[0], sh.n), dtype=torch.int16, device="cuda")
            f(dx, packed, scales, sh.n, sh.k, y, num_splits=splits, workspace=ws)
            torch.cuda.synchronize()
            assert _row_err(host(y, np.uint16), ref) <= TOL, (sh.name, dx.shape[0], splits, rep)
            outs.append(y)
    for a_, b_ in zip(outs[:len(cases)], outs[len(cases):]):
        assert torch.equal(a_, b_)
    # graph of the first two cases
    ys = [torch.empty((c[1].shape[0], c[0].n), dtype=torch.int16, device="cuda") for c in cases[:2]]

    def run():
        for (sh, dx, packed, scales, splits, _), y in zip(cases[:2], ys):
            f(dx, packed, scales, sh.n, sh.k, y, num_splits=splits, workspace=ws)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        run()
    junk = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for i in range(4):
        for y in ys:
            y.fill_(0x5555)
        junk.normal_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, want in zip(ys, outs[:2]):
            assert torch.equal(y, want), i

"""GPU parity, bit-exact: weight packing (q8, q4) and per-token activation
quantization against the oracle, on exhaustive fp16 grids, tie-laden and
degenerate inputs, ragged shapes and the DiT-width weights."""
import numpy as np
import pytest

import oracle
import synthetic_inputs as si
from tests.gpu_util import dev, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import quantized_diffusion_transformer_qlinear_amd as m
    return m


ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)
FINITE = ALL[np.isfinite(ALL.view(np.float16))]


def _pack_both(q, w, bits):
    wq, s = q.qpack(bits, dev(w))
    ref_q, ref_s = oracle.qpack8(w) if bits == 8 else oracle.qpack4(w, 32)
    gq, gs = host(wq), host(s)
    assert gq.shape == ref_q.shape and gs.shape == ref_s.shape
    assert np.array_equal(gs.view(np.uint16), ref_s.view(np.uint16)), "scales differ"
    assert np.array_equal(gq.view(np.uint8), ref_q.view(np.uint8)), "packed weights differ"


@pytest.mark.parametrize("bits", [8, 4])
# N % 8 == 0 takes the 16-byte tiled kernels, any other N the channel-strip
# ones: both with K tails past a tile (K % 128, K % 64 != 0) and partial
# channel blocks
@pytest.mark.parametrize("K,N", [(32, 1), (64, 3), (96, 65), (160, 130), (256, 64), (544, 97),
                                 (32, 8), (96, 72), (160, 136), (544, 200), (1056, 24)])
def test_pack_ragged(q, bits, K, N):
    log(f"qpack{bits} K={K} N={N}")
    rng = np.random.default_rng(K * 1000 + N)
    w = (rng.standard_normal((K, N)) * np.exp2(rng.integers(-12, 4, N))[None, :]).astype(np.float16)
    w[:, 0] = 0                       # an all-zero channel
    if K >= 64:
        w[32:64, -1] = 0              # an all-zero group
    _pack_both(q, w, bits)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("mult8", [True, False])
def test_pack_fp16_grid(q, bits, mult8):
    """Every finite fp16 value appears as a weight, under many scales (columns
    with different absmax, including subnormal scales and exact ties); with a
    channel count that is a multiple of 8 (16-byte tiled kernels) and one that
    is not."""
    vals = FINITE.view(np.float16)
    K = 1024
    cols = []
    for a in (np.float16(1.0), np.float16(15.875), np.float16(7.0), np.float16(2.0 ** -14),
              np.float16(65504.0), np.float16(0.3333), np.float16(1e-6)):
        sel = vals[np.abs(vals.astype(np.float64)) <= float(a)]
        for i in range(0, sel.size, K - 1):
            c = np.zeros(K, np.float16)
            chunk = sel[i:i + K - 1]
            c[:chunk.size] = chunk
            c[-1] = a                  # absmax of the channel (and of its last group)
            cols.append(c)
    while (len(cols) % 8 == 0) != mult8:
        cols.append(np.zeros(K, np.float16))
    w = np.stack(cols, axis=1)
    log(f"qpack{bits} grid K={K} N={w.shape[1]}")
    _pack_both(q, w, bits)


def test_pack_identity(q):
    K = N = 256
    perm = np.random.default_rng(5).permutation(N)
    w = np.zeros((K, N), np.float16)
    w[perm, np.arange(N)] = 1.0
    _pack_both(q, w, 8)
    _pack_both(q, w, 4)


@pytest.mark.parametrize("bits", [8, 4])
def test_pack_dit_width(q, bits):
    log(f"qpack{bits} 1536x6144 (MLP-up weights)")
    _pack_both(q, si.mlp_up_w8a16().w, bits)


def _actquant_both(q, x):
    xq, sa = q.quant_act(dev(x))
    rq, rs = oracle.quant_act(x)
    assert np.array_equal(host(sa).view(np.uint16), rs.view(np.uint16)), "token scales differ"
    assert np.array_equal(host(xq), rq), "int8 activations differ"


@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (5, 512), (7, 544), (64, 256), (130, 1536),
                                 (9, 6144), (4, 8192), (2, 16384)])
def test_actquant_ragged(q, M, K):
    log(f"actquant M={M} K={K}")
    rng = np.random.default_rng(M * 7 + K)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-10, 6, M))[:, None]).astype(np.float16)
    x[0] = 0                                           # an all-zero token
    _actquant_both(q, x)


@pytest.mark.parametrize("K", [64, 1536, 6144])
def test_actquant_max_in_every_lane(q, K):
    """Row m holds its largest magnitude in the k that lane m % 64 of the
    row's wave loads (element c * 512 + lane * 8 + e): the wave-wide maximum
    must reach every lane, whichever 16-lane row of the wave it starts in.
    Signs alternate so that a reduction over signed values would also fail."""
    rng = np.random.default_rng(K)
    M = 128
    x = (rng.standard_normal((M, K)) * 0.5).astype(np.float16)
    for m in range(M):
        lane, c, e = m % 64, (m // 64) % max(1, K // 512), m % 8
        k = min(c * 512 + lane * 8 + e, K - 1)
        x[m, k] = np.float16((-1) ** m * (8.0 + m / 16))
    log(f"actquant max in every lane K={K}")
    _actquant_both(q, x)


def test_actquant_fp16_grid(q):
    """Every finite fp16 value is quantized under scales with ties, subnormal
    scales and the largest input."""
    vals = FINITE.view(np.float16)
    K = 4096
    rows = []
    for a in (np.float16(1.0), np.float16(15.875), np.float16(7.0), np.float16(2.0 ** -14),
              np.float16(65504.0), np.float16(127.0 / 64.0)):
        sel = vals[np.abs(vals.astype(np.float64)) <= float(a)]
        for i in range(0, sel.size, K - 1):
            r = np.zeros(K, np.float16)
            chunk = sel[i:i + K - 1]
            r[:chunk.size] = chunk
            r[-1] = -a
            rows.append(r)
    x = np.stack(rows)
    log(f"actquant grid M={x.shape[0]} K={K}")
    _actquant_both(q, x)


def test_actquant_dit_shapes(q):
    x = si.dit_block()["h"]
    log("actquant 2048x1536")
    _actquant_both(q, x)
    x2 = si.normal_f16((2048, 6144), 1.0, 999)
    log("actquant 2048x6144")
    _actquant_both(q, x2)


@pytest.mark.parametrize("M,W,col0,ncols", [(1, 96, 64, 32), (77, 4608, 3072, 1536), (2048, 4608, 3072, 1536),
                                            (130, 1024, 8, 512)])
def test_quant_act_columns(q, M, W, col0, ncols):
    """The row-strided act-quant of a column block read in place equals the
    oracle's quantization of that block, bit for bit."""
    rng = np.random.default_rng(M + W + col0)
    x = (rng.standard_normal((M, W)) * 3).astype(np.float16)
    log(f"quant_act_columns M={M} W={W} cols {col0}+{ncols}")
    xq, sa = q.quant_act_columns(dev(x), col0, ncols)
    xq_ref, sa_ref = oracle.quant_act(np.ascontiguousarray(x[:, col0:col0 + ncols]))
    assert np.array_equal(host(xq), xq_ref)
    assert np.array_equal(host(sa).view(np.uint16), sa_ref.view(np.uint16))

"""bloom_linear: the decoder's linear layers as a standalone call, at the 176B shapes, on
every kernel the plans choose (vector-ALU GEMV up to 4 rows, the MFMA GEMM's decode
tiles up to 128 rows, its prompt tiles from 256 rows), for each weight type and
activation storage.

One-hot rows pin the layout bit for bit: row m of x is c * e_k(m), so y[m][n] is the
single product c * W[n][k(m)] (times the int8 row scale, plus the bias), which the
kernels form with at most one rounding, the same one as float32 of the exact value
(with fp16 activations the MFMA GEMM multiplies fp16 copies of the bf16 weights, exact
from 2^-14 in magnitude, so there W[n][k] is its nearest fp16 value);
a wrong weight row or column, scale index, bias index, tile origin or split-K
reduction shows as a mismatch.  Random rows are compared with oracle.linear on the
same stored inputs (bf16 / fp16 rounding, or int8_rows for W8A8, whose float32
decisions both sides take on the same float32 values).
"""
import dataclasses

import numpy as np
import pytest
import torch

import bloom_inputs as bi
import oracle
import transformer_bloom_decode_amd as tb

pytestmark = pytest.mark.gpu

_W = {}


def _weights(wdt, N, K):
    """Seeded weights on the device: bf16 N(0, 0.02) or int8 codes with fp16 scales,
    and a bf16 bias."""
    key = (wdt, N, K)
    if key not in _W:
        _W.clear()
        torch.cuda.empty_cache()
        g = torch.Generator(device="cuda").manual_seed(N * 7 + K)
        if wdt == "bf16":
            w = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
            s = None
        else:
            w = torch.randint(-127, 128, (N, K), generator=g, device="cuda", dtype=torch.int8)
            s = (torch.rand((N,), generator=g, device="cuda") * 1e-3 + 1e-4).to(torch.float16)
        b = (torch.randn((N,), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        _W[key] = (w, s, b)
    return _W[key]


def _cfg(wdt, act):
    shape = bi.BLOOM_176B_INT8 if wdt == "int8" else bi.BLOOM_176B_TP8_RANK0
    return tb.make_config(dataclasses.replace(shape, activations=act))


def _run(cfg, x, w, s, b, N):
    M, K = x.shape
    y = torch.full((M, N), float("nan"), device="cuda")
    ws = torch.empty(max(1, tb.bloom_linear_workspace_bytes(cfg, M, N, K)), dtype=torch.uint8,
                     device="cuda")
    tb.bloom_linear(cfg, M, N, K, x, w, s, b, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


CASES = [("bf16", "bf16", 14336, 1792), ("bf16", "f32", 14336, 1792), ("bf16", "f16", 5376, 14336),
         ("bf16", "bf16", 5376, 14336), ("int8", "bf16", 14336, 14336),
         ("int8", "f16", 43008, 14336), ("int8", "int8", 14336, 14336),
         ("int8", "int8", 43008, 14336)]


@pytest.mark.parametrize("M", [1, 3, 16, 64, 128, 256])
@pytest.mark.parametrize("wdt, act, N, K", CASES)
def test_one_hot_rows_return_weight_columns(wdt, act, N, K, M):
    w, s, b = _weights(wdt, N, K)
    cfg = _cfg(wdt, act)
    ks = (np.arange(M) * 7919 + 5) % K
    # W8A8: c = 127 / 8, so the row's scale is 1/8 and the code of c is 127 (both exact);
    # no bias there (its addition would be a second rounding after the scale products)
    c = 127.0 / 8 if act == "int8" else 1.0
    bias = None if act == "int8" else b
    x = torch.zeros((M, K), device="cuda")
    x[torch.arange(M), torch.from_numpy(ks).cuda()] = c
    y = _run(cfg, x, w, s, bias, N)
    col = w[:, torch.from_numpy(ks).cuda()].t().float().cpu().numpy()  # [M][N]
    if act == "f16" and wdt == "bf16" and M > 4:
        col = col.astype(np.float16)        # the fp16 MFMA's copy of the weights
    col = col.astype(np.float64)
    exact = col * (127.0 if act == "int8" else 1.0)
    if act == "int8":
        exact = exact / 8
    if s is not None:
        exact = exact * s.float().cpu().numpy().astype(np.float64)[None, :]
    if bias is not None:
        exact = exact + bias.float().cpu().numpy().astype(np.float64)[None, :]
    np.testing.assert_array_equal(y.view(np.uint32), exact.astype(np.float32).view(np.uint32))


def _stored(x, act):
    """The values the path stores for float32 inputs x (oracle side); float32
    activations reach the MFMA GEMM as two bf16 planes of the float32 value."""
    if act == "bf16":
        return oracle.round_bf16(x)
    if act == "f16":
        return x.astype(np.float16).astype(np.float64)
    if act == "int8":
        return oracle.int8_rows(x)
    return x.astype(np.float64)


@pytest.mark.parametrize("M", [2, 16, 128, 256])
@pytest.mark.parametrize("wdt, act, N, K", [CASES[1], CASES[2], CASES[4], CASES[5], CASES[6]])
def test_random_rows_match_oracle_linear(wdt, act, N, K, M):
    """Gaussian rows with a few large entries (outliers set the int8 row scales):
    relative L2 error <= 2e-6 against oracle.linear of the stored inputs (float32
    accumulation), 1e-4 where the MFMA GEMM reads two bf16 planes (2^-17)."""
    w, s, b = _weights(wdt, N, K)
    cfg = _cfg(wdt, act)
    rng = np.random.default_rng(M * 31 + N)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.integers(0, K, 4)] *= 9.0
    y = _run(cfg, torch.from_numpy(x).cuda(), w, s, b, N)
    if wdt == "int8":
        W = oracle.Int8RowScale(w.cpu().numpy(), s.float().cpu().numpy())
    else:
        W = w.float().cpu().numpy()
        if act == "f16" and M > 4:
            W = W.astype(np.float16)        # the fp16 MFMA's copy of the weights
    ref = oracle.linear(_stored(x, act), W, b.float().cpu().numpy())
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    print(f"linear {wdt} x {act} {N}x{K} M{M}: rel {rel:.2e}")
    assert rel <= (1e-4 if act == "f32" and M > 4 else 2e-6)

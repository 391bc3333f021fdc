"""bloom_sample_tokens_static (the library's per-GPU scratch array, no workspace and
no allocation) against bloom_sample_tokens (caller workspace) through the C ABI: the
same tokens, bit for bit, on two calls in a row (the second with fewer rows and a
shorter vocabulary, so stale partials of the first call are present in the array),
and rows that need more scratch than the array holds are rejected before any launch."""
import numpy as np
import pytest
import torch

import bloom_inputs as bi
import transformer_bloom_decode_amd as tb

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _both(B, V, seed):
    logits, T, P, u = bi.sampling_inputs(B, V, seed=seed)
    T[0] = 0.0                      # a greedy row
    P[1] = 1.0                      # every token kept
    lg, Td, Pd, ud = _dev(logits), _dev(T), _dev(P), _dev(u)
    ref = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    got = torch.full((B,), -9, dtype=torch.int32, device="cuda")
    tb.bloom_sample_tokens(lg, B, V, Td, Pd, ud, ref)
    tb.bloom_sample_tokens_static(lg, B, V, Td, Pd, ud, got)
    torch.cuda.synchronize()
    return got.cpu().numpy(), ref.cpu().numpy()


def test_static_scratch_matches_the_workspace_entry_point_twice():
    for B, V, seed in ((48, 250880, 31), (5, 4099, 32)):
        fits, _ = tb.bloom_sample_scratch_limit(B, V)
        assert fits
        got, ref = _both(B, V, seed)
        np.testing.assert_array_equal(got, ref)
        assert np.all((got >= 0) & (got < V))


def test_static_scratch_rejects_rows_beyond_its_size():
    B, V = 4096, 250880
    fits, nbytes = tb.bloom_sample_scratch_limit(B, V)
    assert not fits and nbytes == 16 << 20
    assert tb.bloom_sample_workspace_bytes(B, V) > nbytes
    x = torch.zeros(1, dtype=torch.float32, device="cuda")
    # rejected on the host before any launch (the 1-element buffers are never read)
    rc = tb.lib.bloom_sample_tokens_static(x.data_ptr(), B, V, x.data_ptr(), x.data_ptr(),
                                           x.data_ptr(), x.data_ptr(), None)
    assert rc == tb.BLOOM_EWORKSPACE

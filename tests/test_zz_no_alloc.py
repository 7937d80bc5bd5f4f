"""The allocation-free permutation entry point (moe_permute_noalloc).

It runs the permutation with its count tables in the library's static device
array instead of a caller workspace. Its outputs must equal moe_permute's bit
for bit (moe_permute is tied to the oracle by the stage tests), on calls in a
row that share the one array, the later ones smaller, covering the one-block,
multi-block and separate-scan placement paths and the row gather; calls past
the array's limit are refused before anything is enqueued.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import to_i64

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def g():
    import gated_mlp_transformer_amd as mod
    return mod


def ids(T, E, k, seed):
    r = np.random.default_rng(seed)
    a = np.sort(np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]), axis=1) \
        if T else np.zeros((0, k), dtype=np.int64)
    return torch.from_numpy(a.astype(np.int32)).to(DEV)


def outputs(T, k, ec, d=None):
    i32 = torch.int32
    o = dict(counts=torch.full((ec,), -7, dtype=i32, device=DEV),
             offsets=torch.full((ec + 1,), -7, dtype=i32, device=DEV),
             src_token=torch.full((T * k,), -7, dtype=i32, device=DEV),
             inv_pos=torch.full((T, k), -7, dtype=i32, device=DEV))
    o["x_perm"] = None if d is None else torch.zeros((T * k, d), dtype=torch.bfloat16, device=DEV)
    return o


def same(a, b, S):
    assert torch.equal(a.counts, b.counts)
    assert torch.equal(a.offsets, b.offsets)
    assert torch.equal(a.src_token[:S], b.src_token[:S])
    assert torch.equal(a.inv_pos, b.inv_pos)


# (T, E, k, e_begin, e_count, with rows): 79 blocks x 256 experts take the
# separate scan pass, 33 x 32 the self-scanning placement, one block the
# single-launch path; each call is smaller than the one before
CALLS = [(20000, 256, 8, 0, 256, False), (8192, 256, 8, 0, 32, True), (200, 64, 6, 8, 24, True),
         (1, 16, 8, 0, 16, False)]


def test_noalloc_equals_workspace_permute_on_calls_in_a_row(g):
    for n, (T, E, k, eb, ec, rows) in enumerate(CALLS):
        print(f"noalloc call {n}: T={T} E={E} k={k} experts [{eb}, {eb + ec}) rows={rows}",
              flush=True)
        idx = ids(T, E, k, seed=100 + n)
        x = synth.normal((T, 128), name="t.noalloc.x", sub=n, device=DEV) if rows else None
        ref = g.moe_permute(idx, eb, ec, x)
        got = g.moe_permute_noalloc(idx, eb, ec, x, **outputs(T, k, ec, 128 if rows else None))
        torch.cuda.synchronize()
        S = int(ref.offsets[-1])
        same(got, ref, S)
        if rows:
            assert torch.equal(got.x_perm[:S], ref.x_perm[:S])
        # and the integers are the oracle's
        counts, offsets, src, inv, _ = oracle.permute(to_i64(idx), eb, ec)
        assert np.array_equal(to_i64(got.offsets), offsets)
        assert np.array_equal(to_i64(got.src_token)[:S], src)
        assert np.array_equal(to_i64(got.inv_pos), inv)


def test_noalloc_refuses_calls_past_its_array(g):
    T, k, ec = 65537, 8, 256   # 257 token blocks x 256 experts > 65536 table entries
    idx = torch.zeros((T, k), dtype=torch.int32, device=DEV)
    with pytest.raises(g.MoEFFNError) as e:
        g.moe_permute_noalloc(idx, 0, ec, None, **outputs(T, k, ec))
    assert e.value.status == -2

"""Shared helpers for the GPU tests: device transfer of the seeded inputs and
comparison with the oracle.  Imports the binding lazily so CPU-only
collection never loads the HIP library."""
import numpy as np
import torch

from oracle import formats as OF


def fp4q():
    from block_scaled_fp4_mxfp4_amd import fp4q as m
    return m


DEV = "cuda:0"


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(DEV).view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def packed(codes_unpacked):
    return OF.pack_nibbles(codes_unpacked)


def assert_bytes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.nonzero(got != want)
    if bad[0].size:
        idx = tuple(b[0] for b in bad)
        raise AssertionError(f"{what}: {bad[0].size} mismatches, first at {idx}: got {got[idx]} want {want[idx]}")


def sample_rows(n_rows, k=48, seed=0):
    rng = np.random.default_rng(seed)
    rows = set([0, n_rows - 1]) | set(rng.choice(n_rows, size=min(k, n_rows), replace=False).tolist())
    return np.array(sorted(rows))

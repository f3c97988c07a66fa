"""Checkpoint and resume of the looped re-quantization ("Looped Transformer
quantization", sections 2.1-2.2: the chain's state between accesses is the
residue r_k alone; section 2 for the stochastic form, whose words depend
only on the access index), through the C ABI.  A chain stopped after k
accesses, its residue saved to host memory and restored into fresh device
memory, must continue bit for bit as the uninterrupted chain and as the
oracle's chain resumed from the same residue."""
import numpy as np
import pytest
import torch

from oracle import nvfp4 as ONV, sigma_delta as OSD
from block_scaled_fp4_mxfp4_amd import synth
from gpu_util import fp4q, dev_f32, host, packed, assert_bytes_equal

pytestmark = pytest.mark.gpu
SHAPES = [(48, 64), (16, 128), (7, 32)]


def _segments(ws, banks=1):
    L = fp4q()
    segs = []
    for w in ws:
        wd = dev_f32(w)
        _, sc, ts = L.quantize_nvfp4(wd)
        rows, cols = w.shape
        segs.append({"w": wd, "scales": sc, "tensor_scale": ts,
                     "residue": torch.zeros((rows, cols), dtype=torch.float32, device=wd.device),
                     "codes": torch.empty((banks, rows, cols // 2), dtype=torch.uint8, device=wd.device)})
    return segs


def test_sigma_delta_checkpoint_resume_single_steps():
    ws = [synth.normal_f32(810 + i, shp, 0.02) for i, shp in enumerate(SHAPES)]
    L = fp4q()
    print("sigma-delta: 12 steps uninterrupted vs 5 + checkpoint + 7", flush=True)
    full, part = _segments(ws), _segments(ws)
    want_codes = []
    for k in range(12):
        L.sigma_delta_requant(full, steps=1)
        want_codes.append([host(s["codes"][0]).copy() for s in full])
    for k in range(5):
        L.sigma_delta_requant(part, steps=1)
    saved = [host(s["residue"]).copy() for s in part]            # checkpoint: the residues only
    for s, r in zip(part, saved):
        s["residue"] = torch.from_numpy(r).to(s["w"].device)      # fresh device memory
    for k in range(5, 12):
        L.sigma_delta_requant(part, steps=1)
        for j, s in enumerate(part):
            assert_bytes_equal(host(s["codes"][0]), want_codes[k][j], f"step {k} segment {j}")
    for a, b in zip(full, part):
        assert_bytes_equal(host(b["residue"]).view(np.uint32), host(a["residue"]).view(np.uint32), "final residue")
    # the oracle resumed from the saved residue
    for j, (w, r0, s) in enumerate(zip(ws, saved, part)):
        st = ONV.tensor_scale_from_amax(np.abs(w).max())
        ref = OSD.sigma_delta_nvfp4(w, 7, r0=r0, tensor_scale=st)
        assert_bytes_equal(host(s["codes"][0]), packed(ref["codes"][-1]), f"oracle resume segment {j}")
        assert_bytes_equal(host(s["residue"]).view(np.uint32), ref["residues"][-1].view(np.uint32), "oracle residue")


def test_sigma_delta_multi_bank_resumes_from_saved_residue():
    ws = [synth.normal_f32(820 + i, shp, 0.02) for i, shp in enumerate(SHAPES)]
    L = fp4q()
    print("sigma-delta: 3 single steps, checkpoint, then one 6-bank launch", flush=True)
    segs = _segments(ws)
    for _ in range(3):
        L.sigma_delta_requant(segs, steps=1)
    saved = [host(s["residue"]).copy() for s in segs]
    stride = -(-max(w.size // 2 for w in ws) // 16) * 16
    multi = _segments(ws)
    for s, r in zip(multi, saved):
        s["residue"] = torch.from_numpy(r).to(s["w"].device)
        s["codes"] = torch.empty((6, stride), dtype=torch.uint8, device=s["w"].device)
    L.sigma_delta_requant(multi, steps=6, bank_stride=stride)
    for j, (w, r0, s) in enumerate(zip(ws, saved, multi)):
        st = ONV.tensor_scale_from_amax(np.abs(w).max())
        ref = OSD.sigma_delta_nvfp4(w, 6, r0=r0, tensor_scale=st)
        got = host(s["codes"])
        for k in range(6):
            assert_bytes_equal(got[k, :w.size // 2].reshape(w.shape[0], -1), packed(ref["codes"][k]), f"bank {k} segment {j}")
        assert_bytes_equal(host(s["residue"]).view(np.uint32), ref["residues"][-1].view(np.uint32), "final residue")


def test_stochastic_rounding_resume_at_any_access():
    ws = [synth.normal_f32(830 + i, shp, 0.02) for i, shp in enumerate(SHAPES)]
    L = fp4q()
    print("stochastic rounding: accesses 0..7 in one launch vs 5..7 resumed", flush=True)
    stride = -(-max(w.size // 2 for w in ws) // 16) * 16
    one, tail = _segments(ws), _segments(ws)
    for s in one:
        s["codes"] = torch.empty((8, stride), dtype=torch.uint8, device=s["w"].device)
    for s in tail:
        s["codes"] = torch.empty((3, stride), dtype=torch.uint8, device=s["w"].device)
    L.stochastic_round_requant(one, 8, seed=1234, step0=0, bank_stride=stride)
    L.stochastic_round_requant(tail, 3, seed=1234, step0=5, bank_stride=stride)
    for j, (a, b, w) in enumerate(zip(one, tail, ws)):
        n = w.size // 2                                  # bytes past n in a bank are not written
        assert_bytes_equal(host(b["codes"])[:, :n], host(a["codes"])[5:8, :n], f"segment {j}")

"""GPU parity of the per-row fp8 quantiser (indexer_quant_fp8) against the oracle.

Codes are compared byte for byte and scales bit for bit: both sides decide
every code from the same float32 value x * float32(448 / amax).
"""

import ctypes
import json
import os

import numpy as np
import pytest
import torch

import fp8_mqa_logits_amd as F
import oracle.indexer_oracle as O
from workloads.generate import quant_inputs, ragged_inputs
from tests.parity import assert_logits_close

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def _gpu(x: np.ndarray):
    c, s = F.indexer_quant_fp8(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda())
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def _assert_same(x, what=""):
    gc, gs = _gpu(x)
    oc, os_ = O.quant_fp8_rows(x)
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), f"{what}: scales differ"
    bad = np.argwhere(gc != oc)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first {bad[:3].tolist()} " \
                          f"gpu {gc[tuple(bad[0])]:#x} oracle {oc[tuple(bad[0])]:#x}"


@pytest.mark.parametrize("rows,D", [(1, 4), (300, 4), (19, 8), (45, 16), (70, 32), (7, 64), (33, 128),
                                    (1001, 128), (5, 132), (40, 256), (9, 512), (6, 1000), (3, 2048)])
def test_random_rows_bit_exact(rows, D):
    _assert_same(quant_inputs(rows, D, seed=rows * 1000 + D), f"{rows}x{D}")


def test_edge_rows_bit_exact():
    pins = json.load(open(os.path.join(HERE, "golden", "e4m3fn_encoder_pins.json")))
    D = 128
    rows = []
    # amax = 448: y = x exactly, so the page's tie / subnormal points are encoded directly
    r = np.zeros(D, np.float32)
    vals = [448.0] + [p["x"] for p in pins["ties"] + pins["subnormals"]]
    r[:len(vals)] = vals
    rows.append(r)
    rows.append(np.zeros(D, np.float32))                                   # zero row
    r = np.linspace(-3.0, 1.0, D).astype(np.float32); rows.append(r)     # negative maximum
    r = np.full(D, 0.7, np.float32); rows.append(r)                      # all equal
    r = np.zeros(D, np.float32); r[0] = 1.0; r[1:] = np.float32(2.0 ** -14) * np.arange(1, D); rows.append(r)
    r = -np.zeros(D, np.float32); r[5] = 2.5; r[6] = -1e-30; rows.append(r)  # -0.0 and tiny negatives
    # every representable y half-step (ties between neighbouring codes) at amax = 448
    tab = O.e4m3fn_value_table()
    pos = np.sort(tab[np.isfinite(tab) & (tab >= 0)])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    for i in range(0, len(mids), D - 1):
        r = np.zeros(D, np.float32); r[0] = 448.0
        chunk = mids[i:i + D - 1]
        r[1:1 + len(chunk)] = chunk
        rows.append(r.copy())
        rows.append(-r)
    _assert_same(np.stack(rows), "edge rows")


def test_strided_rows_through_the_c_abi():
    rows, D, ld_x, ld_c = 37, 128, 136, 144
    x = quant_inputs(rows, ld_x, seed=5)
    xd = torch.from_numpy(x).cuda()
    codes = torch.full((rows, ld_c), 0xAB, dtype=torch.uint8, device="cuda")
    scale = torch.empty(rows, dtype=torch.float32, device="cuda")
    L = F.load_library()
    st = L.indexer_quant_fp8(xd.data_ptr(), ld_x, rows, D, codes.data_ptr(), ld_c, scale.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    oc, os_ = O.quant_fp8_rows(x[:, :D])
    c = codes.cpu().numpy()
    assert np.array_equal(c[:, :D], oc)
    assert np.all(c[:, D:] == 0xAB), "bytes past D were written"
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), os_.view(np.uint32))


@pytest.mark.parametrize("shape", [(65536, 128), (8192 * 32, 128)], ids=["kv_n65536", "q_m8192_h32"])
def test_full_size_sampled(shape):
    rows, D = shape
    x = quant_inputs(rows, D, seed=rows)
    gc, gs = _gpu(x)
    # every row: the scale is amax / 448 and the largest magnitude lands on +-448
    amax = np.abs(x).max(axis=1)
    assert np.array_equal(gs, (amax / np.float32(448.0)).astype(np.float32))
    assert np.all((gc & 0x7F).max(axis=1) == 0x7E)
    sample = np.linspace(0, rows - 1, 256).astype(np.int64)
    oc, os_ = O.quant_fp8_rows(x[sample])
    assert np.array_equal(gc[sample], oc)
    assert np.array_equal(gs[sample].view(np.uint32), os_.view(np.uint32))


def test_quantised_inputs_feed_the_logits_kernel():
    # quantise float32 q (per row and head) and kv (per token) on the GPU, then the logits
    # of those codes and scales must match the oracle's logits on the oracle's own codes
    m, n, H, D = 24, 700, 32, 128
    qf = quant_inputs(m * H, D, seed=77, spread=1.0)
    kf = quant_inputs(n, D, seed=78, spread=1.0)
    qc, qs = _gpu(qf)
    kc, ksc = _gpu(kf)
    oqc, oqs = O.quant_fp8_rows(qf)
    okc, oks = O.quant_fp8_rows(kf)
    assert np.array_equal(qc, oqc) and np.array_equal(kc, okc)
    # the q scale multiplies every head's score, so it folds into the head weights
    rng = np.random.default_rng(1)
    w = rng.random((m, H)).astype(np.float32) * oqs.reshape(m, H)
    ks = np.zeros(m, np.int32)
    ke = np.full(m, n, np.int32)
    got = F.indexer_logits_ragged(torch.from_numpy(qc.reshape(m, H, D)).cuda(), torch.from_numpy(kc).cuda(),
                                  torch.from_numpy(ksc).cuda(), torch.from_numpy(w).cuda(),
                                  torch.from_numpy(ks).cuda(), torch.from_numpy(ke).cuda(), clean=True)
    torch.cuda.synchronize()
    ref = O.mqa_logits(oqc.reshape(m, H, D), okc, oks, w, ks, ke)
    assert_logits_close(got.cpu().numpy(), ref, ks, ke, True, what="quantised inputs")

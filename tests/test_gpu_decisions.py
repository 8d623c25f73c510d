"""Bit-exact integer decisions of the HIP kernels on identical float inputs,
and the fp8 decoder, against the oracle.  Runs through the C ABI."""
import numpy as np
import pytest

import dllm_inputs as di
from oracle import dllm_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    return t


def _stream(torch):
    return torch.cuda.current_stream().cuda_stream


def test_fp8_decode_every_code(torch):
    from masked_block_diffusion_amd import binding as B
    codes = torch.arange(256, dtype=torch.uint8, device="cuda")
    out = torch.empty(256, dtype=torch.float32, device="cuda")
    assert B.dllm_debug_decode_fp8(codes.data_ptr(), 256, out.data_ptr(), _stream(torch)) == 0
    got = out.cpu().numpy().astype(np.float64)
    ref = O.e4m3fn_to_f64(np.arange(256, dtype=np.uint8))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.all(np.isnan(got[~fin]))


@pytest.mark.parametrize("n,E,k", [(1, 16, 2), (37, 256, 8), (512, 256, 8), (64, 32, 4), (5, 16, 16)])
def test_route_bit_exact(torch, n, E, k):
    from masked_block_diffusion_amd import binding as B
    rng = np.random.default_rng(n * 1000 + E + k)
    logits = (rng.standard_normal((n, E)) * 2).astype(np.float32)
    logits[:, 3] = logits[:, 5]                       # exact ties between experts
    if n > 2:
        logits[2, :] = 0.25                           # a token with all-equal logits
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    bias[7] = 5.0 if E > 8 else bias[7]               # planted bias forces expert 7
    lt = torch.from_numpy(logits).cuda()
    bt = torch.from_numpy(bias).cuda()
    idx = torch.empty((n, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((n, k), dtype=torch.float32, device="cuda")
    assert B.dllm_debug_route(lt.data_ptr(), bt.data_ptr(), n, E, k, idx.data_ptr(), gates.data_ptr(),
                              _stream(torch)) == 0
    gi, gg = idx.cpu().numpy(), gates.cpu().numpy()
    _, s, key = O.route_keys(np.zeros((n, 1)), np.zeros((E, 1)), bias)   # shapes only
    s = O.sigmoid_f32(logits.astype(np.float64))
    key = (s + bias[None, :]).astype(np.float32)
    for i in range(n):
        ref = O.topk_desc(key[i], k)
        assert list(gi[i]) == list(ref), i
        assert np.allclose(gg[i], O.gates_from(s[i], ref), rtol=1e-6, atol=0)
        if E > 8:
            assert 7 in gi[i]


@pytest.mark.parametrize("strategy", [0, 1, 2])
@pytest.mark.parametrize("n_seq,LB,V", [(1, 32, 4096), (4, 32, 1000), (16, 32, 300), (3, 7, 257)])
def test_unmask_bit_exact(torch, strategy, n_seq, LB, V):
    from masked_block_diffusion_amd import binding as B
    rng = np.random.default_rng(strategy * 7 + n_seq + V)
    mask = 99999
    ids = rng.integers(0, V, size=(n_seq, LB)).astype(np.int32)
    for s in range(n_seq):
        ids[s, rng.permutation(LB)[: max(1, LB // 2 + s % 3)]] = mask
    logits = (rng.standard_normal((n_seq, LB, V)) * 3).astype(np.float32)
    logits[0, :, 5] = logits[0, :, 9] = 40.0           # exact argmax tie: lower id wins
    steps, lo = 8, 123
    for t, thr in ((0, 0), (3, 0), (7, 0), (0, 1)):
        it = torch.from_numpy(ids).cuda()
        lt = torch.from_numpy(logits).cuda()
        out = torch.empty_like(it)
        rem = torch.empty(n_seq, dtype=torch.int32, device="cuda")
        conf = torch.empty((n_seq, LB), dtype=torch.float32, device="cuda")
        xh = torch.empty((n_seq, LB), dtype=torch.int32, device="cuda")
        assert B.dllm_debug_unmask(it.data_ptr(), lt.data_ptr(), n_seq, LB, V, lo, mask, steps, t,
                                   strategy, thr, 0.5, out.data_ptr(), rem.data_ptr(), conf.data_ptr(),
                                   xh.data_ptr(), _stream(torch)) == 0
        go, gr, gc, gx = out.cpu().numpy(), rem.cpu().numpy(), conf.cpu().numpy(), xh.cpu().numpy()
        for s in range(n_seq):
            mpos = np.nonzero(ids[s] == mask)[0]
            xi, ci = O.confidence(logits[s, mpos].astype(np.float64), strategy)
            assert np.array_equal(gx[s, mpos], xi + lo)
            assert np.allclose(gc[s, mpos], ci, rtol=2e-5, atol=1e-6)
            xfull = np.zeros(LB, np.int64)
            cfull = np.full(LB, -np.inf)
            xfull[mpos] = xi + lo
            # decision in the kernel's precision: the float32 confidences
            cfull[mpos] = gc[s, mpos]
            ref, info = O.select_commit(ids[s], mask, xfull, cfull, steps, t, bool(thr), 0.5)
            assert np.array_equal(go[s], ref), (s, t)
            assert gr[s] == int(np.sum(ref == mask))


@pytest.mark.parametrize("rows,P,ratio", [(1, 1024, 0.5), (2, 4160, 0.5), (3, 100, 0.8), (1, 7, 0.3),
                                          (1, 2048, 1.0), (2, 3000, 0.01)])
def test_retention_bit_exact(torch, rows, P, ratio):
    from masked_block_diffusion_amd import binding as B
    rng = np.random.default_rng(P + rows)
    mass = rng.random((rows, P)).astype(np.float32) * 50
    mass[:, ::7] = mass[:, 3:4]                        # many exact ties
    mass[0, :5] = 0.0
    mt = torch.from_numpy(mass).cuda()
    kept = torch.full((rows, P), -1, dtype=torch.int32, device="cuda")
    cnt = torch.empty(rows, dtype=torch.int32, device="cuda")
    assert B.dllm_debug_retention(mt.data_ptr(), rows, P, ratio, kept.data_ptr(), cnt.data_ptr(),
                                  _stream(torch)) == 0
    gk, gc = kept.cpu().numpy(), cnt.cpu().numpy()
    for r in range(rows):
        ref = O.retention_select(mass[r].astype(np.float64), ratio)
        assert gc[r] == len(ref)
        assert np.array_equal(gk[r, : gc[r]], ref)

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
    assert B.dllm_debug_retention(mt.data_ptr(), rows, P, ratio, 0, 0, 0, 0.0, 0.0, kept.data_ptr(),
                                  cnt.data_ptr(), _stream(torch)) == 0
    gk, gc = kept.cpu().numpy(), cnt.cpu().numpy()
    for r in range(rows):
        ref = O.retention_select(mass[r].astype(np.float64), ratio)
        assert gc[r] == len(ref)
        assert np.array_equal(gk[r, : gc[r]], ref)


@pytest.mark.parametrize("rows,P,r_img,r_txt", [(1, 4160, 0.8, 1.0), (2, 1000, 0.5, 0.5), (3, 97, 0.3, 0.7),
                                                (1, 5, 1.0, 0.2), (2, 2048, 0.01, 1.0)])
def test_retention_pools_bit_exact(torch, rows, P, r_img, r_txt):
    """Per-modality pools: visual ids [vis_lo, vis_hi) keep their own top
    ceil(r_img P_img), the rest ceil(r_txt P_txt); ties to the lower position."""
    from masked_block_diffusion_amd import binding as B
    rng = np.random.default_rng(P * 3 + rows)
    score = (np.round(rng.random((rows, P)) * 64) / 8).astype(np.float32)   # many exact ties
    vis_lo, vis_hi = 1000, 1500
    ids = rng.integers(0, 2000, size=(rows, P)).astype(np.int32)
    ids[0, : min(P, 64)] = 2000                       # [MASK] ids count as text
    if rows > 1:
        ids[1] = rng.integers(vis_lo, vis_hi, size=P)  # a row that is all visual
    st = torch.from_numpy(score).cuda()
    it = torch.from_numpy(ids).cuda()
    kept = torch.full((rows, P), -1, dtype=torch.int32, device="cuda")
    cnt = torch.empty(rows, dtype=torch.int32, device="cuda")
    assert B.dllm_debug_retention(st.data_ptr(), rows, P, 0.5, it.data_ptr(), vis_lo, vis_hi, r_img, r_txt,
                                  kept.data_ptr(), cnt.data_ptr(), _stream(torch)) == 0
    gk, gc = kept.cpu().numpy(), cnt.cpu().numpy()
    for r in range(rows):
        pool = ((ids[r] >= vis_lo) & (ids[r] < vis_hi)).astype(np.int64)
        ref = O.retention_select(score[r].astype(np.float64), 0.5, pool, (r_txt, r_img))
        assert gc[r] == len(ref)
        assert np.array_equal(gk[r, : gc[r]], ref)


@pytest.mark.parametrize("dt,np_dt,es", [("bf16", np.uint16, 1), ("fp8", np.uint8, 2), ("f32", np.float32, 0)])
def test_pack_gate_up_layout(torch, dt, np_dt, es):
    """The packed fragment layout: fragment (t, c) of each [F][D] matrix holds
    lane l's KL elements W[16 t + l % 16][KC c + KL (l / 16) + j] at KL l + j
    (KL = 16 for fp8, else 8; KC = 4 KL)."""
    from masked_block_diffusion_amd import binding as B
    L, E, F, D = 2, 3, 48, 192
    KL = 16 if dt == "fp8" else 8
    rng = np.random.default_rng(es)
    src = rng.integers(0, 255, size=(L, E, F, D)).astype(np_dt)
    m = di.ModelConfig(n_layers=L, hidden=D, n_heads=1, head_dim=32, n_experts=E, top_k=1, n_shared=0,
                       expert_ffn=F, shared_ffn=F, vocab_text=10, vocab_image=0,
                       act_dtype="f32" if dt == "f32" else "bf16", expert_dtype=dt)
    cfg = B.model_config_struct(m)
    st = torch.from_numpy(src.view(np.int16) if np_dt == np.uint16 else src).cuda()
    dst = torch.empty_like(st)
    assert B.dllm_pack_gate_up(cfg, st.data_ptr(), dst.data_ptr(), _stream(torch)) == 0
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np_dt).reshape(-1)
    ref = src.reshape(L * E, F // 16, 16, D // (4 * KL), 4, KL).transpose(0, 1, 3, 4, 2, 5).reshape(-1)
    assert np.array_equal(got, ref)
    assert B.dllm_pack_gate_up(cfg, st.data_ptr(), st.data_ptr(), _stream(torch)) == B.DLLM_ERR_INVALID_ARG

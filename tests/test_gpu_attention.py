"""Block-wise attention alone (dllm_debug_block_attention: the step's kernels
and launch plan) against the oracle's plain definition, element by element:
softmax(q k^T / sqrt(d) + block mask) v over the cached prefix (or its
retained subset) and the block's own keys.  Covers each kernel the plan
picks: the streaming kernel with one key range per (row, head) at the
batched thinking shape (16 rows x 16 heads, 2048- and 6112-key prefixes) and
with several ranges plus the merge, the 128-key gather kernel (a prefix that
is not a multiple of 32, a retained subset), the float32 kernel, partial
tiles and an empty prefix.  Runs through the C ABI."""
import numpy as np
import pytest

from oracle import dllm_oracle as O

pytestmark = pytest.mark.gpu

F32, BF16 = 0, 1
STREAM, GATHER, FLOAT = 2, 1, 0


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    return t


def _dev(torch, x, dt):
    """Host float array -> device tensor of the act dtype, and the float64
    values the device holds (bf16 rounding of the inputs is input preparation)."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    if dt == BF16:
        t = t.to(torch.bfloat16)
    return t, t.float().cpu().numpy().astype(np.float64)


def _run(torch, dt, rows, H, dh, LB, P, seed, kept=None, cap=None, sample_rows=None):
    """Random q / K / V (N(0, 1), so the scaled scores spread about 1), the
    library's attention on the GPU, and the oracle on the sampled rows."""
    from masked_block_diffusion_amd import binding as B
    cap = cap or max(P, 1)
    rng = np.random.default_rng(seed)
    q, qh = _dev(torch, rng.standard_normal((rows, H, LB, dh)), dt)
    kc, kch = _dev(torch, rng.standard_normal((rows, H, cap, dh)), dt)
    vc, vch = _dev(torch, rng.standard_normal((rows, H, cap, dh)), dt)
    bk, bkh = _dev(torch, rng.standard_normal((rows, H, LB, dh)), dt)
    bv, bvh = _dev(torch, rng.standard_normal((rows, H, LB, dh)), dt)
    out = torch.empty((rows, LB, H * dh), dtype=torch.float32 if dt == F32 else torch.bfloat16, device="cuda")
    lse = torch.empty((rows, H, LB), dtype=torch.float32, device="cuda")
    kp = nk = 0
    if kept is not None:
        kt = np.full((rows, cap), -1, np.int32)
        for r, kr in enumerate(kept):
            kt[r, : len(kr)] = kr
        kept_d = torch.from_numpy(kt).cuda()
        nkept_d = torch.tensor([len(kr) for kr in kept], dtype=torch.int32, device="cuda")
        kp, nk = kept_d.data_ptr(), nkept_d.data_ptr()
    st, plan = B.dllm_debug_block_attention(dt, q.data_ptr(), kc.data_ptr() if P else 0, vc.data_ptr() if P else 0,
                                            cap, bk.data_ptr(), bv.data_ptr(), kp, nk, rows, H, dh, LB, P,
                                            out.data_ptr(), lse.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, st
    go = out.float().cpu().numpy().astype(np.float64)
    gl = lse.cpu().numpy().astype(np.float64)
    pos = P + np.arange(LB)
    errs, lerrs = [], []
    for r in (range(rows) if sample_rows is None else sample_rows):
        ppos = np.arange(P) if kept is None else np.asarray(kept[r])
        kk = np.concatenate([kch[r][:, ppos], bkh[r]], axis=1).transpose(1, 0, 2)   # [nk, H, dh]
        vv = np.concatenate([vch[r][:, ppos], bvh[r]], axis=1).transpose(1, 0, 2)
        kpos = np.concatenate([ppos, pos])
        o, _ = O.attention(qh[r].transpose(1, 0, 2), kk, vv, pos, kpos, LB)             # [LB, H, dh]
        ref = o.reshape(LB, H * dh)
        errs.append(np.max(np.abs(go[r] - ref)) / np.max(np.abs(ref)))
        # log-sum-exp of the scaled, masked scores of each (head, query)
        s = np.einsum("hqd,khd->hqk", qh[r], kk) / np.sqrt(dh)
        s = np.where(O.block_visible(pos, kpos, LB)[None], s, -np.inf)
        m = np.max(s, axis=-1)
        ref_l = m + np.log(np.sum(np.exp(s - m[..., None]), axis=-1))
        lerrs.append(np.max(np.abs(gl[r] - ref_l)))
    print(f"[attention] dtype={dt} rows={rows} H={H} dh={dh} LB={LB} P={P} kept={kept is not None} "
          f"plan={plan} out max-abs-rel {max(errs):.2e} lse max-abs {max(lerrs):.2e}", flush=True)
    return max(errs), max(lerrs), plan


def _tol(dt):
    # bf16: the probabilities enter the PV product as bf16 and the output is
    # stored as bf16 (relative steps of 2^-9); float32: accumulation order only
    return (1e-2, 2e-3) if dt == BF16 else (1e-5, 1e-5)


def test_stream_one_range_per_unit_first_block(torch):
    """The batched thinking step at the first block: 16 rows x 16 heads,
    2048 cached keys + 32 block keys, one workgroup per (row, head) covering
    every key (17 tiles of 128 keys), output written without a merge."""
    err, lerr, plan = _run(torch, BF16, 16, 16, 128, 32, 2048, 1, sample_rows=[0, 7, 15])
    assert plan[0] == STREAM and plan[2] == 1 and plan[1] >= 2080, plan
    assert err < _tol(BF16)[0] and lerr < _tol(BF16)[1], (err, lerr)


def test_stream_one_range_per_unit_last_block(torch):
    """The last block of the thinking generation: 6112 cached keys."""
    err, lerr, plan = _run(torch, BF16, 16, 16, 128, 32, 6112, 2, sample_rows=[0, 15])
    assert plan[0] == STREAM and plan[2] == 1, plan
    assert err < _tol(BF16)[0] and lerr < _tol(BF16)[1], (err, lerr)


@pytest.mark.parametrize("rows,H,dh,P", [(1, 16, 128, 4160), (4, 8, 32, 2048), (2, 4, 64, 8192)])
def test_stream_several_ranges_merged(torch, rows, H, dh, P):
    """Few (row, head) units: the key range splits over several workgroups of
    384 keys (three 128-key tiles each), and the partials are merged."""
    err, lerr, plan = _run(torch, BF16, rows, H, dh, 32, P, rows * 100 + P)
    assert plan[0] == STREAM and plan[2] >= 2 and plan[1] > 128, plan
    assert err < _tol(BF16)[0] and lerr < _tol(BF16)[1], (err, lerr)


@pytest.mark.parametrize("P,LB", [(48, 16), (1000, 8)])
def test_gather_kernel_prefix_not_multiple_of_32(torch, P, LB):
    """Whole blocks of 16 or 8 positions whose prefix ends inside a 32-key
    tile: the 128-key gather kernel."""
    err, lerr, plan = _run(torch, BF16, 2, 4, 128, LB, P, P)
    assert plan[0] == GATHER, plan
    assert err < _tol(BF16)[0] and lerr < _tol(BF16)[1], (err, lerr)


def test_gather_kernel_retained_prefix(torch):
    """A retained subset of a 4160-key prefix, different sizes per row (one
    row keeps everything, one a single key), through the kept-index gather."""
    rng = np.random.default_rng(9)
    P = 4160
    kept = [np.sort(rng.choice(P, 2080, replace=False)), np.arange(P), np.array([17])]
    err, lerr, plan = _run(torch, BF16, 3, 4, 128, 32, P, 9, kept=kept)
    assert plan[0] == GATHER and plan[2] >= 2, plan
    assert err < _tol(BF16)[0] and lerr < _tol(BF16)[1], (err, lerr)


@pytest.mark.parametrize("dh,P,LB", [(32, 96, 32), (64, 0, 32), (128, 48, 16)])
def test_float32_kernel(torch, dh, P, LB):
    err, lerr, plan = _run(torch, F32, 2, 4, dh, LB, P, dh + P, cap=max(P, 1))
    assert plan[0] == FLOAT, plan
    assert err < _tol(F32)[0] and lerr < _tol(F32)[1], (err, lerr)


@pytest.mark.parametrize("LB,P", [(16, 64), (16, 48), (32, 0), (8, 1024)])
def test_block_lengths_and_empty_prefix(torch, LB, P):
    """Blocks shorter than a 32-key tile (keys that end inside a tile) and the
    block as the whole context."""
    err, lerr, plan = _run(torch, BF16, 2, 8, 64, LB, P, LB * 7 + P)
    assert err < _tol(BF16)[0] and lerr < _tol(BF16)[1], (err, lerr, plan)


def test_invalid_arguments(torch):
    from masked_block_diffusion_amd import binding as B
    s = torch.cuda.current_stream().cuda_stream
    t = torch.empty(1 << 16, dtype=torch.float32, device="cuda")
    buf = t.data_ptr()
    bad = [(2, 64, 32, 0), (BF16, 48, 32, 0), (BF16, 64, 65, 0), (BF16, 64, 32, 9)]   # dtype, dh, LB, P > cap
    for dt, dh, LB, P in bad:
        st, _ = B.dllm_debug_block_attention(dt, buf, buf, buf, 8, buf, buf, 0, 0, 1, 2, dh, LB, P, buf, 0, s)
        assert st == -1, (dt, dh, LB, P, st)
    st, _ = B.dllm_debug_block_attention(BF16, buf, 0, 0, 64, buf, buf, 0, 0, 1, 2, 64, 32, 32, buf, 0, s)
    assert st == -1                                     # a prefix without cache pointers
    st, _ = B.dllm_debug_block_attention(BF16, buf, buf, buf, 64, buf, buf, 0, 0, 1, 2, 64, 32, 48, buf, 0, s)
    assert st == -1                                     # a prefix that is not whole blocks

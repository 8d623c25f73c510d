"""Oracle parity at the full-size shapes the bench times, on sampled
sequences: the GPU runs every sequence in the bench's launch configuration,
and the oracle follows a subset of them (sequences are independent: each has
its own rows, cache, routing and commits).  Slow: the oracle runs float64
layers at hidden 2048 with 256 experts."""
import numpy as np
import pytest

import dllm_inputs as di
from masked_block_diffusion_amd import binding as B
from tests import _parity as PA

pytestmark = pytest.mark.gpu


def test_think_fp8_layer_full_size_sampled_sequences():
    """The batched thinking layer: 16 sequences x 2048-token prefixes, fp8
    experts at hidden 2048 / width 512 (4 chunks per gate/up wavefront, 4
    batches of 2 in the down kernel), the single-split streaming attention
    over 2080 keys per (row, head) (17 tiles of 128 keys per workgroup,
    written without a merge), the LDS-tiled LM head over 157,184 ids, and the
    prefill as 8 append passes of 256 tokens per row (4096 model-row tokens
    each; all but the first at P > 0).  The oracle follows sequences 0 and 15: hidden states, router
    logits and head logits within the fp8 tolerance, commits exact."""
    wl = di.workload("think_fp8_layer")
    g = wl.gen
    res = PA.run(wl, seed=0, rows=[0, g.n_seq - 1], max_steps=2, keep_experts=True)
    PA.check(res, wl)
    kind, split, n_splits = res.plans[0]
    assert kind == B.ATTN_STREAM and split >= wl.prefix_len and n_splits == 1, res.plans


def test_think_fp8_two_layers_full_size_sampled_sequences():
    """Two stacked layers of the batched thinking shape (16 sequences x
    2048-token prefixes, fp8 experts, 157,184-id head): layer 1 runs on
    what layer 0's combine and norm hand it (bf16 expert outputs summed in
    float32, the next layer's normalised rows), in prefill and in the step.
    The oracle follows sequences 0 and 15 for one step."""
    wl = di.workload("think_fp8_layer")
    wl.model.n_layers = 2
    g = wl.gen
    res = PA.run(wl, seed=5, rows=[0, g.n_seq - 1], max_steps=1, keep_experts=True)
    PA.check(res, wl)


@pytest.mark.parametrize("keep,n_keep", [(0.5, 2080), (0.33, 1373)])
def test_und_layer_sprint_full_size(keep, n_keep):
    """The understanding layer with SPRINT: one sequence, 4096 visual + 64
    text prefix ids (5 append passes, 4 at P > 0), threshold 0.9, retention
    by attention mass.  Step 0 scores the full prefix and keeps ceil(r P)
    positions, which are copied into the compacted K/V (1373 kept: 11 leading
    zero rows masked out); steps 1 and 2 stream them as a contiguous prefix
    over several key ranges merged.  Mass, kept set, hidden states and
    logits over the 157,184-id text sub-vocabulary against the oracle."""
    wl = di.workload("und_layer")
    g = wl.gen
    g.use_sprint, g.keep_ratio, g.cache_warmup_steps = True, keep, 1
    g.use_threshold, g.threshold = True, 0.9
    res = PA.run(wl, seed=0, max_steps=3, keep_experts=True)
    PA.check(res, wl)
    assert res.mass_err
    n_kept = res.session.debug(B.DEBUG_NKEPT, 0, np.int32, (1,))
    assert n_kept[0] == n_keep
    kind, split, n_splits = res.plans[1]
    assert kind == B.ATTN_STREAM and n_splits >= 2, res.plans

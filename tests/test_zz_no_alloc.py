"""moe_align_noalloc (the entry point that allocates nothing) against
moe_align, through the C ABI: two calls in a row, the second with a smaller
input, must give moe_align's tables byte for byte; sizes past the static
scratch array are refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

mx = pytest.importorskip("mixture_experts_routed_moe_amd")

KEYS = ("group_sizes", "group_offsets", "group_padded_offsets", "group_idx_for_bx", "sorted_pair", "pair_to_row")


def _ids(T, k, E, seed, d):
    rng = np.random.default_rng(seed)
    rows = np.stack([rng.permutation(E)[:k] for _ in range(101)]).astype(np.int32)
    return torch.from_numpy(rows[rng.integers(0, 101, T)]).to(d).contiguous()


def test_noalloc_matches_moe_align_twice_shrinking():
    d = dev()
    cfg = moe_synth.CONFIGS["dsv3_prefill"]
    ids_big, _ = mx.moe_topk_softmax(moe_synth.router_logits(cfg, d), cfg.top_k,
                                     expert_bias=moe_synth.expert_bias(cfg, d))
    # a larger first call (about 1 MiB of the 4 MiB array), then a smaller one
    cases = [("big", _ids(131071, 8, 256, 1, d), 256), ("dsv3", ids_big, cfg.E), ("small", _ids(37, 3, 20, 2, d), 20)]
    for name, ids, E in cases:
        say("noalloc", name, tuple(ids.shape), E)
        ref = mx.moe_align(ids, E, 128, 128)
        got = mx.moe_align_noalloc(ids, E, 128, 128)
        torch.cuda.synchronize()
        for key in KEYS:
            assert torch.equal(got[key], ref[key]), (name, key)
    # and against the oracle for the last one
    ids = cases[-1][1]
    tab = oracle.dispatch_tables(host(ids), 20, 128, 128)
    for key in KEYS:
        assert np.array_equal(host(got[key]), tab[key]), key


def test_noalloc_preallocated_tables_and_limit():
    d = dev()
    cap = mx.moe_align_noalloc_max_scratch_bytes()
    assert cap == 4 << 20
    ids = _ids(4096, 8, 256, 3, d)
    tb = mx.alloc_tables(4096 * 8, 256, 128, 128, d)
    for _ in range(2):
        mx.moe_align_noalloc(ids, 256, 128, 128, tb)
    ref = mx.moe_align(ids, 256, 128, 128)
    torch.cuda.synchronize()
    for key in KEYS:
        assert torch.equal(tb[key], ref[key]), key
    # one chunk (1024 pairs) of histogram per 4*E bytes: past the array, refused on the host
    E = 1000
    T = (cap // (4 * E) + 1) * 1024
    big = torch.zeros(T, 1, dtype=torch.int32, device=d)
    with pytest.raises(mx.MoeError) as ei:
        mx.moe_align_noalloc(big, E, 128, 128)
    assert ei.value.code == -2 and "scratch" in str(ei.value)

"""GPU parity of the top-K loss across the number of cached entries K: one
entry; the pages' K = 100 with a partial-mass teacher and every option; and
the largest supported lists over a 16384-word vocabulary: KD_MAX_K = 8192
entries, or 8191 plus a cross-entropy label (a label is one more entry and
K + 1 may not exceed KD_MAX_K).  Those are the prep kernel's largest sort and
put hits in every epilogue round, past the cursor's window of two entries.
"""
import pytest
import torch

import chunked_kl_loss_logit_amd as kd
import kdinputs as G
from tests.gpu_util import say
from tests.test_parity_options import check, run_opts

pytestmark = pytest.mark.gpu


def test_single_cached_entry():
    inp = G.make_topk(300, 256, 1288, 1, torch.bfloat16, tau=1.0, mask="random10", number=51, g="normal")
    say("K=1 T=300 d=256 V=1288")
    check(run_opts(inp, chunk_rows=256), inp, torch.bfloat16)


@pytest.mark.parametrize("one_call", [False, True])
def test_k100_partial_mass_every_option(one_call):
    inp = G.make_topk(700, 384, 2568, 100, torch.bfloat16, tau=1.0, mask="random10", number=52, g="normal")
    inp = G.add_topk_options(inp, tau_rows=True, partial_mass=True, labels=True, ce_weight=0.3, number=52)
    say(f"K=100 every option T=700 d=384 V=2568 one_call={one_call}")
    check(run_opts(inp, chunk_rows=256, one_call=one_call), inp, torch.bfloat16)


@pytest.mark.parametrize("label", [False, True])
def test_max_k(label):
    K = kd.KD_MAX_K - 1 if label else kd.KD_MAX_K
    inp = G.make_topk(260, 128, 16384, K, torch.bfloat16, tau=1.2, number=53, g="normal")
    if label:
        inp = G.add_topk_options(inp, labels=True, ce_weight=0.2, number=53)
    say(f"K={K} T=260 d=128 V=16384 label={label}")
    check(run_opts(inp), inp, torch.bfloat16)

"""GPU: the per-bucket tile tuner of the fp8-activation stages (SM90 fused-MoE page,
Parameters: profile the legal tiles per token bucket, cache the winner). Whatever
family wins, the layer must still match the oracle; clearing the table restores the
built-in rule bit for bit."""
import numpy as np
import pytest
import torch

import mixture_experts_expert_softmax_amd as M
import moe_synth as S
from parity import assert_close_bf16
from test_gpu_mx import MX_MAX_ABS, MX_REL, _dev, _fwd, _oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("wfmt,T", [("mxfp4", 24), ("mxfp8", 200), ("fp8", 48)])
def test_tuned_choice_keeps_parity_and_clear_restores(wfmt, T):
    c = S.w4a8_moe(seed=61, T=T, H=512, I=512, E=8, top_k=2, wfmt=wfmt)
    d = _dev(c)
    ids, w = M.moe_route(torch.from_numpy(c.logits).to(DEV), c.top_k)
    M.moe_tune_clear()
    before = _fwd(c, d, ids, w, d["w1"], d["w1_sf"], d["w2"], d["w2_sf"])
    choice = M.moe_tune_mx(d["x"], d["x_sf"], ids, w, d["w1"], d["w1_sf"], d["w2"], d["w2_sf"],
                           c.num_experts, act_scale=d.get("act_scale"))
    assert all(ch in (0, 1) for ch in choice)
    tuned = _fwd(c, d, ids, w, d["w1"], d["w1_sf"], d["w2"], d["w2_sf"])
    assert_close_bf16(tuned, _oracle(c, ids, w), MX_MAX_ABS, MX_REL, what=f"tuned {wfmt} {choice}")
    M.moe_tune_clear()
    after = _fwd(c, d, ids, w, d["w1"], d["w1_sf"], d["w2"], d["w2_sf"])
    torch.cuda.synchronize()
    assert torch.equal(before, after)

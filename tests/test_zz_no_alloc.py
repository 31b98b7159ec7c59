"""GPU test of tr_gdn_replay_noalloc, the replay entry point that allocates nothing: its results
equal tr_gdn_replay's (same kernels; the split schedule's records in the library's static
device scratch instead of a caller's workspace) on two calls in a row, the second smaller,
and a request whose records would exceed the scratch is rejected before anything runs."""
import pytest
import torch

import synthetic
from linear_attention_state_amd import (TailReplayError, gdn_replay, gdn_replay_noalloc, gdn_replay_workspace_size,
                                        get_gdn_schedule, set_gdn_schedule)
from linear_attention_state_amd import _lib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("schedule", ["auto", "fused"])
def test_noalloc_equals_workspace_entry_point(schedule):
    prev = get_gdn_schedule()
    set_gdn_schedule(schedule)
    try:
        # few heads: "auto" takes the split schedule (records in the static scratch)
        for i, (lens, Hqk, Hv) in enumerate((([700, 5, 300, 64], 2, 4), ([65, 1], 1, 2))):
            inp = synthetic.gdn_inputs(lens, Hqk, Hv, 128, 128, seed=90 + i).to("cuda")
            need = gdn_replay_workspace_size(inp.cu_seqlens, Hqk, Hv, 128, 128, torch.bfloat16)
            assert (need > 0) == (schedule == "auto")
            assert need <= _lib.TR_NOALLOC_SCRATCH_BYTES
            s_in = torch.randn((len(lens), Hv, 128, 128), generator=torch.Generator().manual_seed(i)).cuda() * 0.2
            S1, o1 = gdn_replay(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, q_scale=0.9, state_in=s_in)
            S2 = torch.full_like(S1, float("nan"))
            o2 = torch.full_like(o1, float("nan"))
            cu_dev = inp.cu_seqlens.cuda()
            gdn_replay_noalloc(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, cu_dev, S2, o2, q_scale=0.9,
                               state_in=s_in)
            torch.cuda.synchronize()
            print("noalloc %s call %d: %d sequences, %d records bytes, equal %s"
                  % (schedule, i, len(lens), need, torch.equal(S1, S2) and torch.equal(o1, o2)), flush=True)
            assert torch.equal(S1, S2) and torch.equal(o1, o2)
            # state only
            S3 = torch.empty_like(S1)
            gdn_replay_noalloc(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, cu_dev, S3, None, q_scale=0.9,
                               state_in=s_in)
            torch.cuda.synchronize()
            assert torch.equal(S3, S1)
    finally:
        set_gdn_schedule(prev)


def test_noalloc_rejects_requests_beyond_the_scratch():
    prev = get_gdn_schedule()
    set_gdn_schedule("split")
    try:
        lens = [2000] * 8
        inp = synthetic.gdn_inputs(lens, 8, 16, 128, 128, seed=99).to("cuda")
        need = gdn_replay_workspace_size(inp.cu_seqlens, 8, 16, 128, 128, torch.bfloat16)
        assert need > _lib.TR_NOALLOC_SCRATCH_BYTES
        S = torch.zeros((len(lens), 16, 128, 128), device="cuda")
        with pytest.raises(TailReplayError) as err:
            gdn_replay_noalloc(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, inp.cu_seqlens.cuda(), S, None)
        assert err.value.status == _lib.TR_ERR_WORKSPACE and "scratch" in str(err.value)
        torch.cuda.synchronize()
        assert not S.any()                      # nothing ran
    finally:
        set_gdn_schedule(prev)

"""still_prefill_noalloc (static scratch, no workspace) gives exactly what
still_prefill gives with a caller workspace, on two calls in a row, the
second with a smaller input, through the C ABI."""
import pytest
import torch

from linear_attention_still_amd import still
from linear_attention_still_amd.inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _run_both(wl):
    x = {k: v.cuda() for k, v in make_inputs(wl).items()}
    L = wl.seq_len
    p = still.params_for(wl)
    ref = still.PrefillBuffers(p, L)
    still.run_prefill(p, x, ref)
    got = still.PrefillBuffers(p, L)
    got.out.fill_(3.0)
    got.score.fill_(3.0)
    still.still_prefill_noalloc(p, L, x["q"], x["k"], x["v"], x["fmap_w"], x["gate"], got.out,
                                got.sel if got.sel.numel() else None, got.score, got.state)
    torch.cuda.synchronize()
    print("  noalloc %s L=%d" % (wl.name, L), flush=True)
    assert torch.equal(got.out, ref.out)
    assert torch.equal(got.sel, ref.sel)
    assert torch.equal(got.score, ref.score)
    assert torch.equal(got.state, ref.state)


def test_noalloc_matches_workspace_entry_twice_second_smaller():
    big = Workload("na_big", "bf16", 2, 8, 2, 128, 2000, 64, 64, 64 + 8 * 32, 32,
                   sigma=0.5, outlier_frac=0.01, seed=21)
    small = Workload("na_small", "bf16", 1, 4, 1, 64, 300, 32, 32, 32 + 5 * 10, 10,
                     sigma=0.5, outlier_frac=0.01, seed=22)
    assert still.still_workspace_bytes(still.params_for(big), big.seq_len) > \
        still.still_workspace_bytes(still.params_for(small), small.seq_len)
    _run_both(big)
    _run_both(small)


def test_noalloc_rejects_problems_beyond_its_scratch():
    wl = Workload("na_huge", "bf16", 4, 32, 8, 128, 65536, 128, 128, 1024, 512)
    p = still.params_for(wl)
    assert still.still_workspace_bytes(p, wl.seq_len) > still.still_noalloc_scratch_bytes()
    t = torch.zeros(64, dtype=torch.bfloat16, device="cuda")  # never read: rejected first
    g = torch.zeros(32, dtype=torch.float32, device="cuda")
    with pytest.raises(still.StillError) as e:
        still.still_prefill_noalloc(p, wl.seq_len, t, t, t, t, g, t, None, None, t)
    assert e.value.rc == still.STILL_ESCRATCH

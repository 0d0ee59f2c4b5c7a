"""dflash_block_forward_noalloc, the forward for callers that cannot allocate: its partials
live in the library's static per-device scratch array instead of the context's buffers.
Through the C ABI it must give exactly what dflash_block_forward gives (same kernels, same
sums: bit for bit, stricter than the parity bar), on consecutive calls that shrink (the array
keeps the previous call's contents), and it must refuse a forward whose partials exceed the
array, before anything changes."""
import numpy as np
import pytest
import torch

import synth
from block_diffusion_draft_02_amd import binding as B
from gpu_util import DEV, dev_weights

pytestmark = pytest.mark.gpu
SEED = 1601


def _both(d, seqs, bonus, gamma, qpos=None):
    """(tokens, logits) of the regular forward and of the no-allocation forward, same inputs."""
    out = []
    V = d.m["vocab"]
    for f in (d.dflash_block_forward, d.dflash_block_forward_noalloc):
        t = torch.full((len(seqs), gamma - 1), -1, dtype=torch.int32, device=DEV)
        lg = torch.empty((len(seqs) * (gamma - 1), V), dtype=torch.float32, device=DEV)
        f(seqs, bonus, t, lg, q_rope_pos=qpos, gamma=gamma)
        torch.cuda.synchronize()
        out.append((t.cpu().numpy(), lg.cpu().numpy()))
    return out


def _hd128_model():
    m = synth.model("qwen3-L8-h2048")
    m.update(num_layers=2, hidden=512, num_q_heads=16, num_kv_heads=4, head_dim=128, intermediate=1024,
             vocab=2048, num_taps=2, target_hidden=512)
    return m


def test_noalloc_matches_forward_tiny_two_calls_shrinking():
    m = synth.model("tiny-L2-h256")
    W = dev_weights(synth.gen_weights(m, SEED))
    d = B.Drafter(m, W, 256, 4)
    for s, n in enumerate([64, 17, 200, 1]):
        d.dflash_ctx_kv_append(s, torch.from_numpy(synth.gen_hidden(m, SEED, n, s).view(np.int16)).to(DEV)
                               .view(torch.bfloat16))
    calls = [([0, 1, 2, 3], 16, None), ([2, 0], 9, [300, 7])]   # the second call is smaller
    for i, (seqs, gamma, qpos) in enumerate(calls):
        bonus = synth.gen_bonus(m, SEED, len(seqs), index=i)
        (t0, l0), (t1, l1) = _both(d, seqs, bonus, gamma, qpos)
        assert np.array_equal(t0, t1), f"call {i}: drafts differ"
        assert np.array_equal(l0.view(np.uint32), l1.view(np.uint32)), f"call {i}: logits differ"
        assert t0.min() >= 0 and t0.max() < m["vocab"]
    d.close()


def test_noalloc_matches_forward_both_attention_paths_then_refuses_oversize():
    """A head_dim-128 drafter (4 kv heads) made for 32 sequences (bands past 2048 keys take the
    LDS path, 12 chunks at 24000 keys): 16 bands of 24000 keys need ~49 MiB of attention
    partials (fits), then 2 bands (smaller); 32 such bands need ~97 MiB, more than the 64 MiB
    array, and are refused with ERANGE, changing nothing."""
    m = _hd128_model()
    W = dev_weights(synth.gen_weights(m, SEED))
    n_long, C = 32, 24000
    d = B.Drafter(m, W, C + 64, n_long)
    H = torch.from_numpy(synth.gen_hidden(m, SEED, 2048, 0).view(np.int16)).to(DEV).view(torch.bfloat16)
    for s in range(n_long):
        for r0 in range(0, C, 2048):
            d.dflash_ctx_kv_append(s, H[:min(2048, C - r0)])
    print(f"appended {n_long} x {C} rows", flush=True)
    calls = [(list(range(16)), 16), ([3, 1], 5)]
    for i, (seqs, gamma) in enumerate(calls):
        bonus = synth.gen_bonus(m, SEED, len(seqs), index=10 + i)
        (t0, l0), (t1, l1) = _both(d, seqs, bonus, gamma)
        assert np.array_equal(t0, t1), f"call {i}: drafts differ"
        assert np.array_equal(l0.view(np.uint32), l1.view(np.uint32)), f"call {i}: logits differ"
    before = [d.dflash_seq_info(s) for s in range(n_long)]
    t = torch.empty((n_long, 15), dtype=torch.int32, device=DEV)
    with pytest.raises(B.DflashError) as e:
        d.dflash_block_forward_noalloc(list(range(n_long)), [5] * n_long, t)
    assert e.value.code == B.DFLASH_ERANGE and "no-allocation limit" in str(e.value)
    assert [d.dflash_seq_info(s) for s in range(n_long)] == before
    # the regular forward still serves the same call
    d.dflash_block_forward(list(range(n_long)), [5] * n_long, t)
    torch.cuda.synchronize()
    assert int(t.min()) >= 0 and int(t.max()) < m["vocab"]
    d.close()

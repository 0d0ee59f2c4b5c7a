"""The attention merge (k_attn_combine) in both of its launch forms. A call whose bands, kv heads
and four-row query blocks add up to 2048 or more gives each merge workgroup four blocks; a
smaller call gives it one. The form changes how many loads a thread has in flight, not what
any output element adds in which order. Here 32 bands at gamma 9 on a 32:4-head drafter have
72 query rows per kv head (18 blocks; the fifth block of a four-block workgroup holds 8 real
rows and 8 past the end), so the 32-band call takes the four-block form and a one-band call
the one-block form:
  * the 32-band call against the oracle;
  * bands of it bit for bit against the same bands forwarded alone."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import Agreement, Pair, DEV

pytestmark = pytest.mark.gpu
SEED = 3101


@pytest.mark.parametrize("hd", [32, 128])
def test_combine_row_blocks_ragged(hd):
    m = dict(synth.model("tiny-L2-h256"), num_q_heads=32, num_kv_heads=4, head_dim=hd)
    W = synth.gen_weights(m, SEED)
    nb, gamma = 32, 9
    pair = Pair(m, W, 700, nb)
    lens = [100 + (53 * s) % 500 for s in range(nb)]   # 1-3 attention chunks a band
    for s in range(nb):
        pair.append(s, synth.gen_hidden(m, SEED, lens[s], 10 + s))
    agree = Agreement()
    bonus = synth.gen_bonus(m, SEED, nb, index=7)
    toks, logits, ref = pair.forward(list(range(nb)), bonus, gamma=gamma)
    agree.add(toks, logits, ref)
    agree.check(min_positions=nb * (gamma - 1) // 2)
    V = m["vocab"]
    for s in (0, 17, 31):
        t1 = torch.empty((1, gamma - 1), dtype=torch.int32, device=DEV)
        l1 = torch.empty((gamma - 1, V), dtype=torch.float32, device=DEV)
        pair.gpu.dflash_block_forward([s], [bonus[s]], t1, l1, gamma=gamma)
        torch.cuda.synchronize()
        assert np.array_equal(t1[0].cpu().numpy(), toks[s]), f"band {s} drafts"
        assert np.array_equal(l1.cpu().numpy().astype(np.float64), logits[s]), f"band {s} logits"
    pair.close()

"""Per-layer parity at the benchmark's full shape (8 layers, hidden 2048, GQA 32:4, head_dim
128, ff 6144, vocab 151936; a 4096-row context, batch 1, gamma 16), through the library's
debug seam (the per-layer dumps of memra_engine/dflash.rs, DflashDraft::forward_block): the
context features of the last append chunk, and for every layer Q after q_norm and RoPE, the
block's cached K and V, the attention output, the residual after attention and the layer's
output, each element against the oracle's intermediates.

Bar per (layer, tensor): max |gpu - oracle| <= 3e-2 * max |oracle| (the logits' bar applied to
each intermediate); the context features, computed from exact bf16 inputs in fp32 and carried
as two bf16 terms, to 1e-3 * max."""
import numpy as np
import pytest
import torch

import synth
from block_diffusion_draft_02_amd import binding as B
from oracle import dflash_oracle as O
from gpu_util import Agreement, Pair, read_slot_kv

pytestmark = pytest.mark.gpu
LAYER_TOL = 3e-2
FEAT_TOL = 1e-3


def _read(gpu, buf, n, dtype):
    t = torch.empty(n, dtype=dtype)
    gpu.dflash_debug_copy(buf, t)
    return t.numpy()


def _bf16_pair(gpu, hi, lo, n):
    h = _read(gpu, hi, n, torch.int16).view(np.uint16)
    l_ = _read(gpu, lo, n, torch.int16).view(np.uint16)
    return O.widen(h) + O.widen(l_)


def _close(got, want, tol, what, report):
    err = np.abs(got - want).max()
    scale = np.abs(want).max()
    report.append(f"{what} {err / scale:.2e}")
    assert err <= tol * scale, f"{what}: max |d| {err:.4g} > {tol} * {scale:.4g}"


def test_per_layer_intermediates_full_shape():
    w = synth.workload("qwen3-L8-h2048-ctx4096-b1")
    m, seed = w["model_cfg"], w["seed"]
    W = synth.gen_weights(m, seed)
    L, h, qd, gamma = m["num_layers"], m["hidden"], m["num_q_heads"] * m["head_dim"], m["gamma_max"]
    C = w["ctx"][0]
    pair = Pair(m, W, w["max_seq_len"], 1)
    H = synth.gen_hidden(m, seed, C, 0)
    for r0 in range(0, C, 2048):
        pair.append(0, H[r0:r0 + 2048])
    report = []
    F_gpu = _bf16_pair(pair.gpu, B.DFLASH_BUF_CTX_FEAT, B.DFLASH_BUF_CTX_FEAT_LO, 2048 * h).reshape(2048, h)
    F_ref = pair.ora.d.ctx_features(H[C - 2048:C])
    _close(F_gpu, F_ref, FEAT_TOL, "ctx features", report)

    pair.gpu.dflash_debug_capture(True)
    rows = w["max_batch"] * gamma           # per-layer stride of the capture buffers
    agree = Agreement()
    for call, (bonus, qpos) in enumerate([(int(synth.gen_bonus(m, seed, 1, index=900)[0]), None), (77, C + 40)]):
        toks, logits, _ = pair.forward([0], [bonus], q_rope_pos=None if qpos is None else [qpos])
        ref = pair.ora.block_forward([0], [bonus], q_rope_pos=None if qpos is None else [qpos], capture=True)
        agree.add(toks, logits, ref)
        caps = ref["layers"][0]
        Q = _bf16_pair(pair.gpu, B.DFLASH_BUF_LAYER_Q, B.DFLASH_BUF_LAYER_Q_LO, L * rows * qd).reshape(L, rows, qd)
        A = _bf16_pair(pair.gpu, B.DFLASH_BUF_LAYER_ATTN, B.DFLASH_BUF_LAYER_ATTN_LO, L * rows * qd).reshape(L, rows, qd)
        X1 = _read(pair.gpu, B.DFLASH_BUF_LAYER_X1, L * rows * h, torch.float32).reshape(L, rows, h)
        X = _read(pair.gpu, B.DFLASH_BUF_LAYER_X, L * rows * h, torch.float32).reshape(L, rows, h)
        kv_len = pair.gpu.dflash_seq_info(0)[0]
        slots = pair.ora.pool.slots(0, range(kv_len, kv_len + gamma))
        for l in range(L):
            c = caps[l]
            _close(Q[l, :gamma], c["q"].reshape(gamma, qd), LAYER_TOL, f"call {call} layer {l} q", report)
            K, V = read_slot_kv(pair.gpu, l, slots)
            _close(O.widen(K), c["k"], LAYER_TOL, f"call {call} layer {l} block k", report)
            _close(O.widen(V), c["v"], LAYER_TOL, f"call {call} layer {l} block v", report)
            _close(A[l, :gamma], c["attn"], LAYER_TOL, f"call {call} layer {l} attn", report)
            _close(X1[l, :gamma].astype(np.float64), c["x1"], LAYER_TOL, f"call {call} layer {l} x1", report)
            _close(X[l, :gamma].astype(np.float64), c["x"], LAYER_TOL, f"call {call} layer {l} x", report)
    agree.check(min_positions=20)
    print("max |d| / max |oracle|: " + "; ".join(report))
    pair.close()

"""Pins for the CPU oracle: closed forms, textbook identities, brute force on tiny
inputs and invariants of the method. None of these re-runs the oracle's own formula
through the same code; each would fail on a plausible mistake in it (a dropped term, a
wrong sign or index, a transposed operand, an offset-form norm, interleaved RoPE pairs,
a wrong GQA head map, a causal mask, a wrong lm_head row)."""
import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import dflash_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 widening

def test_widen_known_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x4049, 0x7F7F], dtype=np.uint16)
    want = [1.0, -2.0, 1.0078125, 0.0, -0.0, 3.140625, 3.3895313892515355e38]
    got = O.widen(bits)
    assert got.tolist() == want


def test_bf16_rounding_of_generator_is_rne():
    # 1 + 2^-8 lies exactly between two bf16 values; RNE keeps the even one (1.0)
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.5], dtype=np.float32)
    assert synth.f32_to_bf16_bits(x).tolist() == [0x3F80, 0x3F82, 0xBFC0]


# ---------------------------------------------------------------- RMSNorm

def test_rms_norm_hand_value_and_vanilla_form():
    x = np.array([[3.0, 4.0]])
    w = np.array([2.0, 1.0])
    y = O.rms_norm(x, w, 0.0)
    r = math.sqrt((9 + 16) / 2)
    assert np.allclose(y, [[6 / r, 4 / r]], rtol=0, atol=1e-15)


def test_rms_norm_closed_form_unit_weight():
    g = np.random.default_rng(0)
    x = g.standard_normal((7, 64)) * 0.01
    eps = 1e-6
    y = O.rms_norm(x, np.ones(64), eps)
    ms = np.mean(x * x, axis=1)
    assert np.allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-12)


def test_rms_norm_is_not_offset_form():
    # with w ~ 1 + N(0, 0.02) the vanilla form keeps output RMS ~ 1; the offset form
    # x * (1 + w) would give ~ 2
    g = np.random.default_rng(1)
    x = g.standard_normal((4, 512))
    w = 1 + 0.02 * g.standard_normal(512)
    y = O.rms_norm(x, w, 1e-6)
    rms = np.sqrt(np.mean(y * y, axis=1))
    assert np.all(np.abs(rms - 1.0) < 0.01)


# ---------------------------------------------------------------- RoPE / YaRN

def test_inv_freq_plain_closed_form():
    f = O.inv_freq_plain(1e6, 128)
    assert f.shape == (64,)
    assert f[0] == 1.0
    assert math.isclose(f[1], 10 ** (-6 / 64), rel_tol=1e-14)
    assert math.isclose(f[63], 1e6 ** (-126 / 128), rel_tol=1e-14)


def test_rope_hand_example():
    # hd = 4, theta = 100 -> inv_freq = [1, 0.1]; pairs (0, 2) and (1, 3)
    x = np.array([1.0, 0.0, 0.0, 1.0])
    y = O.rope_neox(x[None], np.array([1]), O.inv_freq_plain(100.0, 4))[0]
    want = [math.cos(1), -math.sin(0.1), math.sin(1), math.cos(0.1)]
    assert np.allclose(y, want, atol=1e-15)


def test_rope_equals_complex_rotation_of_half_pairs():
    # textbook: rotate-half RoPE multiplies z_j = x_j + i x_{j+d/2} by exp(i pos w_j)
    g = np.random.default_rng(2)
    d = 16
    x = g.standard_normal((5, d))
    pos = np.array([0, 1, 7, 1000, 34815])
    w = O.inv_freq_plain(1e6, d)
    y = O.rope_neox(x, pos, w)
    z = (x[:, : d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * pos[:, None] * w[None, :])
    assert np.allclose(y[:, : d // 2], z.real, atol=1e-12)
    assert np.allclose(y[:, d // 2:], z.imag, atol=1e-12)


def test_rope_norm_and_relative_angle():
    g = np.random.default_rng(3)
    d = 32
    a, b = g.standard_normal(d), g.standard_normal(d)
    w = O.inv_freq_plain(1e4, d)
    ra = O.rope_neox(a[None], np.array([37]), w)[0]
    rb = O.rope_neox(b[None], np.array([101]), w)[0]
    assert math.isclose(np.linalg.norm(ra), np.linalg.norm(a), rel_tol=1e-13)
    # <R(p)a, R(q)b> = <a, R(q - p) b>
    rb2 = O.rope_neox(b[None], np.array([101 - 37]), w)[0]
    assert math.isclose(ra @ rb, a @ rb2, rel_tol=1e-11, abs_tol=1e-12)


def test_yarn_constants_match_golden():
    gd = json.load(open(os.path.join(GOLD, "yarn_wide_drafter.json")))
    low, high = O.yarn_bounds(gd["head_dim"], gd["rope_theta"], gd["factor"], gd["orig"],
                              gd["beta_fast"], gd["beta_slow"])
    assert (low, high) == (gd["low"], gd["high"])
    assert math.isclose(O.yarn_mscale(gd["factor"]), gd["mscale"], rel_tol=1e-15)
    f = O.inv_freq_yarn(gd["head_dim"], gd["rope_theta"], gd["factor"], gd["orig"],
                        gd["beta_fast"], gd["beta_slow"])
    base = np.array([1e6 ** (-j / 64) for j in range(64)])
    # pairs at or below `low` keep the plain frequency, pairs at or above `high` are
    # divided by the factor, and the ramp between is linear in j
    assert np.allclose(f[:18], base[:18], rtol=1e-14)
    assert np.allclose(f[34:], base[34:] / 32.0, rtol=1e-14)
    j = 25
    r = (j - 17) / 17
    assert math.isclose(f[j], base[j] * (1 - r) + base[j] / 32 * r, rel_tol=1e-14)


# ---------------------------------------------------------------- attention

def _attn_brute(q, qp, k, v, kp, scale, window):
    T, nh, d = q.shape
    Tk, nkv, _ = k.shape
    G = nh // nkv
    out = np.zeros_like(q)
    for i in range(T):
        for h in range(nh):
            kh = h // G
            s = []
            for j in range(Tk):
                if window > 0 and not (qp[i] - kp[j] < window):
                    continue
                s.append((j, sum(q[i, h, t] * k[j, kh, t] for t in range(d)) * scale))
            mx = max(val for _, val in s)
            den = sum(math.exp(val - mx) for _, val in s)
            for j, val in s:
                out[i, h, :] += math.exp(val - mx) / den * v[j, kh, :]
    return out


@pytest.mark.parametrize("window", [0, 3])
def test_attention_brute_force(window):
    g = np.random.default_rng(4)
    q = g.standard_normal((3, 4, 5))
    k = g.standard_normal((7, 2, 5))
    v = g.standard_normal((7, 2, 5))
    qp = np.array([5, 6, 7])
    kp = np.array([0, 1, 2, 3, 5, 6, 7])
    a = O.gqa_attention(q, qp, k, v, kp, 0.4, window)
    b = _attn_brute(q, qp, k, v, kp, 0.4, window)
    assert np.allclose(a, b, atol=1e-13)


def test_attention_single_key_and_zero_query():
    g = np.random.default_rng(5)
    k = g.standard_normal((6, 1, 4))
    v = g.standard_normal((6, 1, 4))
    # single visible key (window 1 and only key 5 shares the query's position) -> its V
    q = g.standard_normal((1, 2, 4))
    a = O.gqa_attention(q, np.array([9]), k, v, np.array([0, 1, 2, 3, 4, 9]), 1.0, 1)
    assert np.allclose(a[0, 0], v[5, 0]) and np.allclose(a[0, 1], v[5, 0])
    # zero query -> uniform weights -> mean of V
    a = O.gqa_attention(np.zeros((1, 1, 4)), np.array([0]), k, v, np.arange(6), 1.0, 0)
    assert np.allclose(a[0, 0], v[:, 0].mean(axis=0))


def test_gqa_equals_mha_with_repeated_kv():
    g = np.random.default_rng(6)
    nh, nkv, d = 8, 2, 6
    q = g.standard_normal((4, nh, d))
    k = g.standard_normal((9, nkv, d))
    v = g.standard_normal((9, nkv, d))
    qp, kp = np.arange(4) + 9, np.arange(9)
    a = O.gqa_attention(q, qp, k, v, kp, 0.3, 0)
    kr, vr = np.repeat(k, nh // nkv, axis=1), np.repeat(v, nh // nkv, axis=1)
    b = O.gqa_attention(q, qp, kr, vr, kp, 0.3, 0)
    assert np.allclose(a, b, atol=1e-14)
    # and each head is plain single-head attention against its group's kv head
    for h in range(nh):
        c = O.gqa_attention(q[:, h:h + 1], qp, k[:, h // 4:h // 4 + 1], v[:, h // 4:h // 4 + 1], kp, 0.3, 0)
        assert np.allclose(a[:, h], c[:, 0], atol=1e-14)


def test_window_equals_truncation():
    g = np.random.default_rng(7)
    q = g.standard_normal((4, 2, 8))
    k = g.standard_normal((30, 1, 8))
    v = g.standard_normal((30, 1, 8))
    kp = np.arange(30)
    qp = np.array([26, 27, 28, 29])
    W = 10
    a = O.gqa_attention(q, qp, k, v, kp, 0.35, W)
    for i in range(4):
        keep = kp > qp[i] - W
        b = O.gqa_attention(q[i:i + 1], qp[i:i + 1], k[keep], v[keep], kp[keep], 0.35, 0)
        assert np.allclose(a[i], b[0], atol=1e-14)


def test_attention_is_non_causal():
    # a key placed after the query still contributes
    q = np.ones((1, 1, 2))
    k = np.array([[[0.0, 0.0]], [[5.0, 5.0]]])
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    a = O.gqa_attention(q, np.array([0]), k, v, np.array([0, 1]), 1.0, 0)
    assert a[0, 0, 1] > 0.99


# ---------------------------------------------------------------- silu / argmax

def test_silu_and_argmax():
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert math.isclose(O.silu(np.array([1.0]))[0], 1 / (1 + math.exp(-1)), rel_tol=1e-15)
    assert math.isclose(O.silu(np.array([40.0]))[0], 40.0, rel_tol=1e-15)
    assert O.argmax_lowest(np.array([[1.0, 3.0, 3.0, 2.0]]))[0] == 1


# ---------------------------------------------------------------- the page model

def test_pool_sizing_golden():
    gd = json.load(open(os.path.join(GOLD, "pool_sizing.json")))
    for c in gd["cases"]:
        assert O.pool_pages(c["max_seq_len"], c["gamma"], c["max_batch"]) == (c["per_seq"], c["pool"])


def test_page_model_brute_force():
    order = synth.gen_page_order(O.pool_pages(64, 16, 2)[1] - 1, 9)
    p = O.PagePool(64, 16, 2, order)
    assert p.num_pages == 13 and sorted(p.free) == list(range(1, 13))
    p.ensure(0, 20)          # 2 pages
    p.ensure(1, 5)           # 1 page
    p.ensure(0, 33)          # 1 more
    assert p.bt[0] == list(order[:2]) + [order[3]] and p.bt[1] == [order[2]]
    sl = p.slots(0, [0, 15, 16, 32])
    bt = p.bt[0]
    assert sl.tolist() == [bt[0] * 16, bt[0] * 16 + 15, bt[1] * 16, bt[2] * 16]
    assert sl.dtype == np.int64
    # slots of distinct positions never collide, and never touch page 0
    allsl = np.concatenate([p.slots(0, range(48)), p.slots(1, range(16))])
    assert len(set(allsl.tolist())) == 64 and allsl.min() >= 16
    freed = list(p.bt[0])
    p.reset(0)
    assert p.free[-3:] == freed and p.bt[0] == []
    with pytest.raises(O.PoolError):
        p.ensure(1, 16 * 20)


# ---------------------------------------------------------------- the drafter

def _micro_model(**kw):
    m = dict(num_layers=1, hidden=8, num_q_heads=4, num_kv_heads=2, head_dim=4,
             intermediate=6, vocab=11, num_taps=2, target_hidden=5, gamma_max=3,
             mask_token_id=4, rms_eps=1e-6, rope_theta=100.0, rope_type="plain",
             sliding_window=0, layer_sliding=None)
    m.update(kw)
    return m


def _micro_brute(m, Wf, taps, ctx_pos, bonus, q_pos, gamma):
    """Scalar-loop re-derivation of the micro drafter from the definitions:
    y[o] = sum_k W[o][k] x[k] for every [out, in] weight, rotate-half RoPE as a complex
    rotation, softmax attention over (context keys, block keys)."""
    h, nh, nkv, d, ff = m["hidden"], m["num_q_heads"], m["num_kv_heads"], m["head_dim"], m["intermediate"]
    eps = m["rms_eps"]
    G = nh // nkv

    def lin(W, x):
        return [sum(W[o][k] * x[k] for k in range(len(x))) for o in range(len(W))]

    def norm(x, w):
        r = math.sqrt(sum(t * t for t in x) / len(x) + eps)
        return [x[i] / r * w[i] for i in range(len(x))]

    def rope(x, p):
        half = d // 2
        out = list(x)
        for j in range(half):
            a = p * m["rope_theta"] ** (-2.0 * j / d)
            z = complex(x[j], x[j + half]) * complex(math.cos(a), math.sin(a))
            out[j], out[j + half] = z.real, z.imag
        return out

    L = Wf
    # context features and keys
    ctx = []
    for r in range(len(taps)):
        f = norm(lin(L["fc"], list(taps[r])), L["hidden_norm"])
        ctx.append(f)
    layers_kv = []
    for l in range(m["num_layers"]):
        p = f"layers.{l}."
        ks, vs = [], []
        for r, f in enumerate(ctx):
            kr = lin(L[p + "k_proj"], f)
            vr = lin(L[p + "v_proj"], f)
            ks.append([rope(norm(kr[g * d:(g + 1) * d], L[p + "k_norm"]), ctx_pos[r]) for g in range(nkv)])
            vs.append([vr[g * d:(g + 1) * d] for g in range(nkv)])
        layers_kv.append((ks, vs))
    toks = [bonus] + [m["mask_token_id"]] * (gamma - 1)
    x = [list(L["embed_tokens"][t]) for t in toks]
    bpos = [q_pos + i for i in range(gamma)]
    for l in range(m["num_layers"]):
        p = f"layers.{l}."
        xn = [norm(r, L[p + "input_layernorm"]) for r in x]
        qs = [lin(L[p + "q_proj"], r) for r in xn]
        kb = [lin(L[p + "k_proj"], r) for r in xn]
        vb = [lin(L[p + "v_proj"], r) for r in xn]
        qh = [[rope(norm(qs[i][hh * d:(hh + 1) * d], L[p + "q_norm"]), bpos[i]) for hh in range(nh)] for i in range(gamma)]
        kbh = [[rope(norm(kb[i][g * d:(g + 1) * d], L[p + "k_norm"]), bpos[i]) for g in range(nkv)] for i in range(gamma)]
        vbh = [[vb[i][g * d:(g + 1) * d] for g in range(nkv)] for i in range(gamma)]
        ks = layers_kv[l][0] + kbh
        vs = layers_kv[l][1] + vbh
        new_x = []
        for i in range(gamma):
            att = []
            for hh in range(nh):
                g = hh // G
                sc = [sum(qh[i][hh][t] * ks[j][g][t] for t in range(d)) / math.sqrt(d) for j in range(len(ks))]
                mx = max(sc)
                e = [math.exp(s - mx) for s in sc]
                z = sum(e)
                att += [sum(e[j] / z * vs[j][g][t] for j in range(len(ks))) for t in range(d)]
            o = lin(L[p + "o_proj"], att)
            x1 = [x[i][t] + o[t] for t in range(h)]
            n1 = norm(x1, L[p + "post_attention_layernorm"])
            gg = lin(L[p + "gate_proj"], n1)
            uu = lin(L[p + "up_proj"], n1)
            a = [gg[t] / (1 + math.exp(-gg[t])) * uu[t] for t in range(ff)]
            dn = lin(L[p + "down_proj"], a)
            new_x.append([x1[t] + dn[t] for t in range(h)])
        x = new_x
    y = [norm(r, L["norm"]) for r in x]
    return [lin(L["lm_head"], y[i]) for i in range(1, gamma)]


def test_micro_drafter_brute_force():
    """Non-square micro shapes so that any transposed weight or wrong head slicing fails."""
    m = _micro_model()
    W = synth.gen_weights(m, 77)
    # inflate the weights so that every term matters at fp64 precision
    Wbig = {}
    for k, v in W.items():
        a = O.widen(v)
        Wbig[k] = synth.f32_to_bf16_bits((a if a.ndim == 1 else a * 25.0).astype(np.float32))
    taps = synth.gen_hidden(m, 77, 5)
    ctx_pos = np.array([0, 1, 2, 4, 7])
    eng = O.Engine(m, Wbig, max_seq_len=16, max_batch=1, kv_bf16=False)
    eng.ctx_kv_append(0, taps, positions=ctx_pos)
    res = eng.block_forward([0], [9], q_rope_pos=[8], gamma=3)
    Wf = {k: O.widen(v).tolist() for k, v in Wbig.items()}
    want = _micro_brute(m, Wf, O.widen(taps).tolist(), ctx_pos.tolist(), 9, 8, 3)
    assert np.allclose(res["logits"][0], np.array(want), rtol=1e-10, atol=1e-10)
    assert res["tokens"][0].tolist() == np.argmax(np.array(want), axis=1).tolist()


@pytest.fixture(scope="module")
def tiny():
    m = synth.model("tiny-L2-h256")
    W = synth.gen_weights(m, 1001)
    return m, W


def _engine_with_ctx(m, W, n=64, seed=1001, positions=None, **kw):
    eng = O.Engine(m, W, max_seq_len=kw.pop("max_seq_len", 128), max_batch=kw.pop("max_batch", 1), **kw)
    eng.ctx_kv_append(0, synth.gen_hidden(m, seed, n), positions=positions)
    return eng


def test_position_shift_invariance_plain(tiny):
    m, W = tiny
    e1 = _engine_with_ctx(m, W, kv_bf16=False)
    e2 = _engine_with_ctx(m, W, positions=np.arange(64) + 5000, kv_bf16=False)
    a = e1.block_forward([0], [17], gamma=16)
    b = e2.block_forward([0], [17], q_rope_pos=[5064], gamma=16)
    assert np.allclose(a["logits"], b["logits"], atol=1e-9)


def test_position_shift_invariance_yarn_and_window(tiny):
    m, W = tiny
    m = dict(m, rope_type="yarn", yarn_factor=4.0, yarn_orig_max_pos=64.0, yarn_beta_fast=32.0,
             yarn_beta_slow=1.0, sliding_window=24, layer_sliding=[True, False])
    e1 = _engine_with_ctx(m, W, kv_bf16=False)
    e2 = _engine_with_ctx(m, W, positions=np.arange(64) + 777, kv_bf16=False)
    a = e1.block_forward([0], [3], gamma=16)
    b = e2.block_forward([0], [3], q_rope_pos=[777 + 64], gamma=16)
    assert np.allclose(a["logits"], b["logits"], atol=1e-9)
    # and a yarn drafter is not the plain one
    c = _engine_with_ctx(dict(m, rope_type="plain"), W).block_forward([0], [3], gamma=16)
    assert np.abs(a["logits"] - c["logits"]).max() > 1e-3


def test_non_causal_permutation(tiny):
    """Permuting block rows 1..T-1 together with their positions permutes the outputs."""
    m, W = tiny
    e = _engine_with_ctx(m, W)
    s = e.seqs[0]
    toks = np.array([17] + [m["mask_token_id"]] * 15)
    bpos = 64 + np.arange(16)
    y = e.d.block_hidden(s["k"], s["v"], s["pos"], toks, bpos)
    perm = np.concatenate([[0], 1 + np.random.default_rng(8).permutation(15)])
    yp = e.d.block_hidden(s["k"], s["v"], s["pos"], toks[perm], bpos[perm])
    assert np.allclose(yp, y[perm], atol=1e-11)
    # all block rows at one position: the 15 mask rows are identical
    ye = e.d.block_hidden(s["k"], s["v"], s["pos"], toks, np.full(16, 70))
    assert np.allclose(ye[1:], ye[1], atol=1e-12)
    assert np.abs(ye[0] - ye[1]).max() > 1e-3


def test_window_layer_equals_full_when_window_covers_all(tiny):
    m, W = tiny
    mw = dict(m, sliding_window=64 + 16, layer_sliding=[True, True])
    a = _engine_with_ctx(m, W).block_forward([0], [5], gamma=16)
    b = _engine_with_ctx(mw, W).block_forward([0], [5], gamma=16)
    assert np.allclose(a["logits"], b["logits"], atol=1e-12)
    mw2 = dict(m, sliding_window=20, layer_sliding=[True, True])
    c = _engine_with_ctx(mw2, W).block_forward([0], [5], gamma=16)
    assert np.abs(a["logits"] - c["logits"]).max() > 1e-4


def test_chunked_append_equals_one_shot(tiny):
    m, W = tiny
    H = synth.gen_hidden(m, 1001, 64)
    e1 = O.Engine(m, W, 128, 1)
    e1.ctx_kv_append(0, H)
    e2 = O.Engine(m, W, 128, 1)
    e2.ctx_kv_append(0, H[:23])
    e2.ctx_kv_append(0, H[23:])
    for l in range(m["num_layers"]):
        assert np.allclose(e1.seqs[0]["k"][l], e2.seqs[0]["k"][l], atol=1e-13)
        assert np.allclose(e1.seqs[0]["v"][l], e2.seqs[0]["v"][l], atol=1e-13)
    assert e1.block_table(0) == e2.block_table(0)


def test_bands_are_independent(tiny):
    m, W = tiny
    e = O.Engine(m, W, 128, 3, page_order=synth.gen_page_order(O.pool_pages(128, 16, 3)[1] - 1, 4))
    for s, n in [(0, 40), (1, 17), (2, 64)]:
        e.ctx_kv_append(s, synth.gen_hidden(m, 1001 + s, n))
    both = e.block_forward([2, 0, 1], [7, 8, 9], gamma=12)
    for i, (s, b) in enumerate([(2, 7), (0, 8), (1, 9)]):
        one = e.block_forward([s], [b], gamma=12)
        assert np.array_equal(one["logits"][0], both["logits"][i])


def test_lm_head_planted_argmax(tiny):
    m, W = tiny
    e = _engine_with_ctx(m, W)
    res = e.block_forward([0], [11], gamma=16, want_hidden=True)
    y = res["hidden"][0]
    W2 = dict(W)
    lm = O.widen(W["lm_head"]).copy()
    planted = {1: 901, 5: 3, 15: 1023}
    for row, tok in planted.items():
        lm[tok] = y[row] * 4.0
    W2["lm_head"] = synth.f32_to_bf16_bits(lm.astype(np.float32))
    e2 = _engine_with_ctx(m, W2)
    r2 = e2.block_forward([0], [11], gamma=16)
    for row, tok in planted.items():
        assert r2["tokens"][0][row - 1] == tok   # drafts come from rows 1..gamma-1


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_chunked_lm_head_equals_cached_and_scalar_dots(tiny, fmt):
    """The lm_head without cached weights takes the vocabulary in chunks (the branch the
    large-vocabulary parity tests run): equal to the cached product, chunk edges and a ragged
    last chunk included, and (bf16) to scalar dot products on sampled entries; the whole
    forward without cached weights equals the cached one."""
    m, W = tiny
    if fmt == "fp8":
        m = dict(m, weight_format="fp8")
    g = np.random.default_rng(7)
    y = g.standard_normal((15, m["hidden"]))
    a = O.Drafter(m, W).lm_head(y)
    b = O.Drafter(m, W, cache_weights=False).lm_head(y, chunk=100)   # 10 chunks of 100 and one of 24
    assert a.shape == b.shape == (15, m["vocab"])
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13 * np.abs(a).max())
    if fmt == "bf16":
        lm = W["lm_head"]
        for r, v in [(0, 0), (3, 99), (3, 100), (14, 1023), (7, 1000), (9, 512)]:
            w = [float(x) for x in O.widen(lm[v])]
            assert math.isclose(b[r, v], math.fsum(yi * wi for yi, wi in zip(y[r], w)), rel_tol=1e-12, abs_tol=1e-12)
    e1 = _engine_with_ctx(m, W)
    e2 = _engine_with_ctx(m, W, cache_weights=False)
    r1 = e1.block_forward([0], [11], gamma=16)
    r2 = e2.block_forward([0], [11], gamma=16)
    assert np.allclose(r1["logits"], r2["logits"], rtol=1e-12, atol=1e-12 * np.abs(r1["logits"]).max())
    assert np.array_equal(r1["tokens"], r2["tokens"])


def test_layer_capture_records_the_forward_and_changes_nothing(tiny):
    """The opt-in per-layer capture (the parity seam's dumps) leaves the forward unchanged,
    and what it records fits together: x1 = previous layer output + attn o_proj^T, the last
    layer's output through the final norm and lm_head gives the logits, and the captured
    block K/V are what the forward left as the block's keys."""
    m, W = tiny
    e = _engine_with_ctx(m, W)
    plain = e.block_forward([0], [11], gamma=16)
    r = e.block_forward([0], [11], gamma=16, capture=True, want_hidden=True)
    assert np.array_equal(plain["logits"], r["logits"]) and np.array_equal(plain["tokens"], r["tokens"])
    layers = r["layers"][0]
    assert len(layers) == m["num_layers"]
    x_prev = O.widen(W["embed_tokens"][[11] + [m["mask_token_id"]] * 15])
    for l, c in enumerate(layers):
        assert c["q"].shape == (16, m["num_q_heads"], m["head_dim"])
        assert c["k"].shape == c["v"].shape == (16, m["num_kv_heads"], m["head_dim"])
        o = c["attn"] @ O.widen(W[f"layers.{l}.o_proj"]).T
        assert np.allclose(c["x1"], x_prev + o, rtol=1e-12, atol=1e-12)
        assert np.array_equal(c["k"], O.round_bf16(c["k"]))     # cached K/V are bf16 values
        x_prev = c["x"]
    y = O.rms_norm(layers[-1]["x"], O.widen(W["norm"]), m["rms_eps"])
    assert np.allclose(y, r["hidden"][0], rtol=1e-12, atol=1e-12)
    assert np.allclose(y[1:] @ O.widen(W["lm_head"]).T, r["logits"][0], rtol=1e-10, atol=1e-10)


def test_engine_errors_leave_state_unchanged(tiny):
    m, W = tiny
    e = O.Engine(m, W, 40, 2)
    e.ctx_kv_append(0, synth.gen_hidden(m, 1, 30))
    bt, free = e.block_table(0), list(e.pool.free)
    with pytest.raises(O.PoolError) as ei:
        e.ctx_kv_append(0, synth.gen_hidden(m, 1, 11))
    assert ei.value.code == "ERANGE"
    with pytest.raises(O.PoolError):
        e.ctx_kv_append(0, synth.gen_hidden(m, 1, 2), positions=[5, 6])   # not increasing
    with pytest.raises(O.PoolError):
        e.block_forward([0, 0], [1, 2])
    with pytest.raises(O.PoolError):
        e.block_forward([0], [1], gamma=17)
    with pytest.raises(O.PoolError):
        e.block_forward([0], [1], gamma=1)
    assert e.block_table(0) == bt and e.pool.free == free and e.kv_len(0) == 30


def test_pool_exhaustion_is_all_or_nothing(tiny):
    m, W = tiny
    # an explicit 6-page pool (5 usable) shared by two sequences
    e = O.Engine(m, W, 64, 2, num_pages=6)
    e.ctx_kv_append(0, synth.gen_hidden(m, 1, 32))      # pages 1, 2
    e.ctx_kv_append(1, synth.gen_hidden(m, 2, 20))      # pages 3, 4
    assert e.pool.free == [5]
    before = (e.block_table(0), e.block_table(1), list(e.pool.free))
    # seq 0 needs 1 page (positions 32..47), seq 1 needs 1 (36 > 32): 2 > 1 free
    with pytest.raises(O.PoolError) as ei:
        e.block_forward([0, 1], [1, 2], gamma=16)
    assert ei.value.code == "EPOOL"
    assert (e.block_table(0), e.block_table(1), list(e.pool.free)) == before
    with pytest.raises(O.PoolError) as ei:
        e.ctx_kv_append(1, synth.gen_hidden(m, 3, 29))  # needs 2 pages
    assert ei.value.code == "EPOOL" and e.kv_len(1) == 20
    e.block_forward([0], [1], gamma=16)                # takes page 5
    assert e.block_table(0) == [1, 2, 5] and e.pool.free == []
    e.seq_reset(1)
    assert e.pool.free == [3, 4] and e.kv_len(1) == 0
    e.block_forward([1], [2], gamma=16)
    assert e.block_table(1) == [3]


def test_yarn_mscale_scales_cached_keys(tiny):
    """With unit k_norm weights a normed head has norm sqrt(hd * ms / (ms + eps)); RoPE
    preserves it, and YaRN's mscale multiplies it (memra page, rope_rows)."""
    m, W = tiny
    my = dict(m, rope_type="yarn", yarn_factor=8.0, yarn_orig_max_pos=64.0, yarn_beta_fast=32.0,
              yarn_beta_slow=1.0)
    W1 = dict(W)
    for l in range(m["num_layers"]):
        W1[f"layers.{l}.k_norm"] = np.full(m["head_dim"], 0x3F80, dtype=np.uint16)
    for mm, scale in [(m, 1.0), (my, 0.1 * math.log(8.0) + 1.0)]:
        e = _engine_with_ctx(mm, W1, n=9, kv_bf16=False)
        k = e.seqs[0]["k"][1]                       # [9, nkv, hd]
        n = np.linalg.norm(k, axis=-1)
        assert np.allclose(n, scale * math.sqrt(m["head_dim"]), rtol=1e-4)


# ---------------------------------------------------------------- the bf16 cache

def test_round_bf16_hand_values():
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -30, -(1 + 2 ** -8 + 2 ** -40),
                  3.140625, 1e-3, -0.0])
    want = [1.0, 1 + 2 ** -6, 1 + 2 ** -7, -(1 + 2 ** -7), 3.140625, 131 / 128 * 2 ** -10, -0.0]
    assert O.round_bf16(x).tolist() == want


def test_round_bf16_is_nearest_bf16():
    """Brute force against the two bf16 neighbours of every value."""
    g = np.random.default_rng(11)
    x = np.concatenate([g.standard_normal(20000), g.standard_normal(2000) * 1e-3, g.standard_normal(2000) * 300])
    r = O.round_bf16(x)
    bits = r.astype(np.float32).view(np.uint32)
    assert not (bits & 0xFFFF).any()                                    # representable in bf16
    lo = (x.astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32).astype(np.float64)
    _, e = np.frexp(lo)                       # |lo| = f 2^e, 0.5 <= f < 1: bf16 spacing 2^(e-8)
    hi = lo + np.sign(x) * np.ldexp(1.0, e - 8)
    # r is one of the neighbours, and no farther from x than the other one
    assert np.all((r == lo) | (r == hi))
    assert np.all(np.abs(r - x) <= np.minimum(np.abs(lo - x), np.abs(hi - x)))


def test_cache_holds_bf16_rounded_kv(tiny):
    m, W = tiny
    e1 = _engine_with_ctx(m, W, n=40)
    e0 = _engine_with_ctx(m, W, n=40, kv_bf16=False)
    for l in range(m["num_layers"]):
        for kv in ("k", "v"):
            a, b = e1.seqs[0][kv][l], e0.seqs[0][kv][l]
            assert np.array_equal(a, O.round_bf16(b))
            assert np.abs(a - b).max() <= 2 ** -8 * np.abs(b).max()
    # the block's own K/V enter attention through the cache as well: with kv_bf16 off the
    # logits move by a small, nonzero amount
    a = e1.block_forward([0], [3], gamma=16)["logits"]
    b = _engine_with_ctx(m, W, n=40, kv_bf16=False)
    b.seqs[0]["k"] = [O.round_bf16(k) for k in b.seqs[0]["k"]]
    b.seqs[0]["v"] = [O.round_bf16(v) for v in b.seqs[0]["v"]]
    bl = b.block_forward([0], [3], gamma=16)["logits"]
    assert 0 < np.abs(a - bl).max() < 0.05 * np.abs(a).max()


def test_batched_append_is_one_pass_over_all_rows(tiny):
    """The batched context precompute: one fc + hidden_norm + K/V pass over the rows of every
    sequence at once gives, row for row, what each sequence's own pass gives (the step is
    row-wise), and the engine's batched append equals the per-sequence appends in call order:
    same cached K/V, same block tables, pages taken in call order."""
    m, W = tiny
    order = synth.gen_page_order(O.pool_pages(200, 16, 3)[1] - 1, 9)
    e1 = O.Engine(m, W, 200, 3, page_order=order)
    e2 = O.Engine(m, W, 200, 3, page_order=order)
    for e in (e1, e2):
        e.ctx_kv_append(0, synth.gen_hidden(m, 5, 21))
    counts = {2: 17, 0: 9, 1: 0}
    H = {s: synth.gen_hidden(m, 30 + s, n) for s, n in counts.items()}
    Hall = np.concatenate([H[s] for s in (2, 0, 1)])
    pos_all = np.concatenate([np.arange(17), np.arange(21, 30), np.zeros(0, dtype=np.int64)])
    # the one-pass features and K/V, split back per sequence
    F_all = e1.d.ctx_features(Hall)
    kv_all = e1.d.ctx_kv(F_all, pos_all)
    F2 = e1.d.ctx_features(H[2])
    kv2 = e1.d.ctx_kv(F2, np.arange(17))
    assert np.allclose(F_all[:17], F2, rtol=0, atol=1e-12)
    for (ka, va), (kb, vb) in zip(kv_all, kv2):
        assert np.allclose(ka[:17], kb, rtol=0, atol=1e-12) and np.allclose(va[:17], vb, rtol=0, atol=1e-12)
    e1.ctx_kv_append_batch([2, 0, 1], [17, 9, 0], Hall)
    e2.ctx_kv_append(2, H[2])
    e2.ctx_kv_append(0, H[0])
    for s in range(3):
        assert e1.kv_len(s) == e2.kv_len(s) and e1.block_table(s) == e2.block_table(s)
        for l in range(m["num_layers"]):
            assert np.array_equal(e1.seqs[s]["k"][l], e2.seqs[s]["k"][l])
            assert np.array_equal(e1.seqs[s]["v"][l], e2.seqs[s]["v"][l])
    assert e1.pool.free == e2.pool.free
    # slots of the call, in row order
    assert np.array_equal(e1.last_slots, np.concatenate([e1.pool.slots(2, range(17)), e1.pool.slots(0, range(21, 30))]))


def test_batched_append_refusals_change_nothing(tiny):
    m, W = tiny
    e = O.Engine(m, W, 300, 3, num_pages=9)              # 8 usable pages
    e.ctx_kv_append(0, synth.gen_hidden(m, 1, 30))
    e.ctx_kv_append(1, synth.gen_hidden(m, 2, 10))
    state = lambda: ([e.block_table(s) for s in range(3)], list(e.pool.free), [e.kv_len(s) for s in range(3)])
    before = state()
    H = synth.gen_hidden(m, 3, 257)
    for seqs, counts, code in [([0, 0], [1, 1], "ERANGE"), ([3], [1], "ERANGE"), ([1, 0], [1, 271], "ERANGE"),
                               ([1, 2], [-1, 2], "EINVAL"), ([1, 2], [0, 0], "EINVAL"),
                               ([1, 2], [200, 57], "EINVAL"), ([1, 2], [40, 40], "EPOOL")]:
        with pytest.raises(O.PoolError) as ei:
            e.ctx_kv_append_batch(seqs, counts, H[:max(0, sum(counts))])
        assert ei.value.code == code, (seqs, counts)
    with pytest.raises(O.PoolError) as ei:
        e.ctx_kv_append_batch([1, 2], [2, 1], H[:3], positions=[40, 39, 0])
    assert ei.value.code == "EINVAL"
    assert state() == before


# ---- FP8 E4M3 weights ([metrale-fw] from_weights, the FP8 weights phase) -------------------

def test_e4m3_decode_table():
    """OCP E4M3: bias 7, 3 mantissa bits, subnormals m * 2^-9, largest finite 448, 0x7F/0xFF
    NaN, no infinities."""
    v = O.e4m3_decode(np.arange(256))
    hand = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0, 0x3C: 1.5,
            0x40: 2.0, 0x7E: 448.0, 0x81: -(2.0 ** -9), 0xB8: -1.0, 0xFE: -448.0}
    for c, want in hand.items():
        assert v[c] == want, hex(c)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.signbit(v[0x80]) and v[0x80] == 0.0
    # every code from the closed form, written out separately
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        mag = m / 8.0 * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        assert v[c] == (-mag if s else mag)
    fin = v[np.isfinite(v)]
    assert fin.max() == 448.0 and np.all(np.diff(O.e4m3_decode(np.arange(0x7F))) > 0)


def test_e4m3_encode_is_nearest_ties_to_even():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (2.0 ** -9, 0.02, 1.0, 100.0)])
    pos = O.e4m3_decode(np.arange(0x7F))
    got = O.e4m3_encode(x)
    # brute force: the nearest of all 127 magnitudes (ties: the even code), signs kept
    a = np.minimum(np.abs(x), 448.0)
    d = np.abs(a[:, None] - pos[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    want = np.where(cand[:, ::2].any(axis=1) & (cand.sum(axis=1) > 1),
                    np.argmax(cand & (np.arange(0x7F) % 2 == 0), axis=1), np.argmax(cand, axis=1))
    want = (want | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)
    assert np.array_equal(got, want)
    # midpoints go to the even code; beyond 448 saturates; signed zero
    mid = (pos[:-1] + pos[1:]) / 2
    code = O.e4m3_encode(mid)
    assert np.all(code % 2 == 0)
    assert list(O.e4m3_encode(np.array([449.0, 1e30, -1e30, 0.0, -0.0]))) == [0x7E, 0x7E, 0xFE, 0x00, 0x80]
    fin = [c for c in range(256) if (c & 0x7F) != 0x7F]
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(np.array(fin))), np.array(fin, dtype=np.uint8))


def test_e4m3_encode_f32_matches_reference():
    """The engine's float32 encoder equals the nearest-value encoder at every rounding
    boundary (each midpoint and its float32 neighbours, each value and its neighbours) and on
    a dense random sample."""
    pos = O.e4m3_decode(np.arange(0x7F)).astype(np.float32)
    mid = ((pos[:-1].astype(np.float64) + pos[1:]) / 2).astype(np.float32)
    pts = np.concatenate([pos, mid, np.array([448.0 * 1.0001], np.float32), np.array([2.0 ** -6, 2.0 ** -10], np.float32)])
    nb = np.concatenate([pts, np.nextafter(pts, np.float32(0)), np.nextafter(pts, np.float32(1e9))])
    nb = np.concatenate([nb, -nb])
    rng = np.random.default_rng(4)
    dense = np.concatenate([(rng.standard_normal(400000) * s).astype(np.float32) for s in (1e-4, 3e-3, 0.1, 4.0, 200.0)])
    for x in (nb, dense):
        assert np.array_equal(O.e4m3_encode_f32(x), O.e4m3_encode(x))


def test_fp8_row_quantization_properties():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((40, 512)) * 0.02).astype(np.float32)
    w[3] = 0.0
    w[7, 11] = -0.5                                  # a row whose maximum is negative
    bits = synth.f32_to_bf16_bits(w)
    codes, scale = O.quantize_rows_fp8(bits)
    wb = O.widen(bits)
    assert scale.dtype == np.float32 and scale[3] == 1.0 and not codes[3].any()
    amax_code = codes[np.arange(40), np.abs(wb).argmax(axis=1)]
    assert np.all((amax_code[np.arange(40) != 3] & 0x7F) == 0x7E) and codes[7, 11] == 0xFE
    deq = O.dequant_fp8(codes, scale)
    # error bound: half an E4M3 step: |w| * 2^-4 in the normal range, scale * 2^-10 below it
    bound = np.maximum(np.abs(wb) * 2.0 ** -4, scale[:, None].astype(np.float64) * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(np.abs(deq - wb) <= bound)


def test_fp8_forward_equals_bf16_on_lossless_weights_and_leaves_the_append(tiny):
    """FP8 quantizes exactly the forward's seven GEMM weights and the lm_head: on weights that
    FP8 represents exactly (rows of E4M3 values times a power of two, the row maximum 448
    times it) the FP8 forward is the bf16 forward; on random weights the forward changes and
    the context K/V (the append keeps bf16) do not."""
    m, W = tiny
    rng = np.random.default_rng(6)
    Wx = dict(W)
    for name in list(W):
        if name == "lm_head" or name.split(".")[-1] in O.Drafter.FP8_NAMES:
            n, k = W[name].shape
            codes = rng.integers(0, 0x7E, size=(n, k)) | (rng.integers(0, 2, size=(n, k)) << 7)
            codes[:, 0] = 0x7E                       # the row maximum: 448
            vals = O.e4m3_decode(codes) * 2.0 ** -14
            Wx[name] = synth.f32_to_bf16_bits(vals.astype(np.float32))
    H = synth.gen_hidden(m, 1001, 40)
    out = {}
    for fmt in ("bf16", "fp8"):
        for tag, weights in (("exact", Wx), ("random", W)):
            e = O.Engine(dict(m, weight_format=fmt), weights, 64, 1)
            e.ctx_kv_append(0, H)
            out[fmt, tag] = (e.block_forward([0], [5], gamma=16)["logits"], e.seqs[0]["k"][1], e.seqs[0]["v"][1])
    assert np.array_equal(out["fp8", "exact"][0], out["bf16", "exact"][0])
    assert np.array_equal(out["fp8", "random"][1], out["bf16", "random"][1])
    assert np.array_equal(out["fp8", "random"][2], out["bf16", "random"][2])
    assert np.abs(out["fp8", "random"][0] - out["bf16", "random"][0]).max() > 1e-4


# ---- DSpark Markov head ([memra] DflashDraft's markov head and generate_spec_dflash's chain) ----

@pytest.fixture(scope="module")
def dspark():
    m = synth.model("tiny-L2-h256-dspark")
    return m, synth.gen_weights(m, 1201)


def _dspark_engine(m, W, n_ctx=24, seed=1201):
    e = O.Engine(m, W, 64, 2)
    e.ctx_kv_append(0, synth.gen_hidden(m, seed, n_ctx, 3))
    e.ctx_kv_append(1, synth.gen_hidden(m, seed, n_ctx + 9, 4))
    return e


def test_markov_chain_by_the_full_bias_table(dspark):
    """Brute force: Bias[t, v] = <W1[t], W2[v]> for every previous token t at once (one
    [V, V] product), then the greedy walk t_{k+1} = argmax_v(L_k[v] + Bias[t_k, v]) from
    the bonus token over the head-less logits L."""
    m, W = dspark
    plain = dict(m, markov_rank=0)
    Wp = {k: v for k, v in W.items() if not k.startswith("markov")}
    bonus = [17, 900]
    got = _dspark_engine(m, W).block_forward([0, 1], bonus, gamma=16)
    base = _dspark_engine(plain, Wp).block_forward([0, 1], bonus, gamma=16)
    table = O.widen(W["markov_w1"]) @ O.widen(W["markov_w2"]).T        # [V prev, V next]
    for b in range(2):
        t = bonus[b]
        for k in range(15):
            row = base["logits"][b, k] + table[t]
            want = int(np.argmax(row))
            assert got["tokens"][b, k] == want
            np.testing.assert_allclose(got["logits"][b, k], row, rtol=0, atol=1e-12)
            t = want
    # the head changes the drafts (the bias is of the logits' size)
    assert (got["tokens"] != base["tokens"]).mean() > 0.3


def test_markov_planted_walk(dspark):
    """W1[t] = 64 e_(t mod R) and W2[v, j] = 1 iff v = j + 1: the bias is 64 on token t + 1
    and 0 elsewhere, far above the logits' spread, so the drafts walk bonus+1, bonus+2, ...
    This fixes which table the previous token indexes, which one the vocabulary indexes,
    and that row k takes the token drafted at row k-1."""
    m, W = dspark
    V, R = m["vocab"], m["markov_rank"]
    w1 = np.zeros((V, R), np.float32)
    w1[np.arange(V), np.arange(V) % R] = 64.0
    w2 = np.zeros((V, R), np.float32)
    w2[np.arange(1, R + 1), np.arange(R)] = 1.0
    Wx = dict(W, markov_w1=synth.f32_to_bf16_bits(w1), markov_w2=synth.f32_to_bf16_bits(w2))
    e = _dspark_engine(m, Wx)
    res = e.block_forward([0, 1], [40, 200], gamma=16)
    assert np.abs(res["logits"]).max() > 60
    assert res["tokens"].tolist() == [list(range(41, 56)), list(range(201, 216))]
    # transposed roles (W2 gathered by the previous token) would not walk
    assert not np.array_equal(O.widen(Wx["markov_w1"]), O.widen(Wx["markov_w2"]))


def test_markov_zero_head_is_plain_dflash_and_teacher_forcing_is_consistent(dspark):
    m, W = dspark
    V, R = m["vocab"], m["markov_rank"]
    zero = dict(W, markov_w2=np.zeros((V, R), np.uint16))
    plain = dict(m, markov_rank=0)
    Wp = {k: v for k, v in W.items() if not k.startswith("markov")}
    a = _dspark_engine(m, zero).block_forward([1, 0], [5, 6], gamma=9)
    b = _dspark_engine(plain, Wp).block_forward([1, 0], [5, 6], gamma=9)
    assert np.array_equal(a["tokens"], b["tokens"]) and np.array_equal(a["logits"], b["logits"])
    # forcing the chain onto its own tokens changes nothing; forcing other tokens changes
    # the rows after the first, and row 0 (the bonus's row) never
    e = _dspark_engine(m, W)
    free = e.block_forward([0, 1], [5, 6], gamma=9)
    prev = np.concatenate([[[5], [6]], free["tokens"][:, :-1]], axis=1)
    forced = e.block_forward([0, 1], [5, 6], gamma=9, markov_prev=prev)
    assert np.array_equal(forced["tokens"], free["tokens"]) and np.array_equal(forced["logits"], free["logits"])
    other = prev.copy()
    other[:, 1:] = (other[:, 1:] + 1) % V
    f2 = e.block_forward([0, 1], [5, 6], gamma=9, markov_prev=other)
    assert np.array_equal(f2["logits"][:, 0], free["logits"][:, 0])
    assert not np.allclose(f2["logits"][:, 1:], free["logits"][:, 1:])


# ---- DFlash2 ([atlas-head] the DFlash2 fields, scratch and kernel names; READINGS c21-c23) ----

@pytest.fixture(scope="module")
def dflash2():
    m = synth.model("tiny-L2-h256-dflash2")
    return m, synth.gen_weights(m, 1401)


def _plain_weights(W):
    return {k: v for k, v in W.items() if "_conv_" not in k and not k.startswith("selector")}


def test_top_k_is_destructive_argmax(dflash2):
    """The k candidates equal taking the argmax k times, removing it each time (ties to the
    lower index), on rows with planted exact ties."""
    rng = np.random.default_rng(7)
    x = np.round(rng.standard_normal((12, 300)) * 4) / 4          # many exact ties
    x[3, [5, 9, 200]] = 10.0
    idx, val = O.Drafter.top_k_candidates(x, 16)
    for r in range(x.shape[0]):
        row = x[r].copy()
        want = []
        for _ in range(16):
            j = int(np.argmax(row))
            want.append(j)
            row[j] = -np.inf
        assert idx[r].tolist() == want and np.array_equal(val[r], x[r, want])
    assert idx[3, :3].tolist() == [5, 9, 200]


def test_dconv_site_by_scalar_loops(dflash2):
    """The prepare and finish applications written as scalar loops over rows, taps and
    channels, with the dynamic tap of channel c taken from group c // group_size."""
    m, W = dflash2
    d = O.Drafter(m, W)
    rng = np.random.default_rng(8)
    T, h, k, gs = 5, m["hidden"], m["conv_kernel_size"], m["conv_group_size"]
    hn = rng.standard_normal((T, h))
    u, kern = d.dconv_prepare(1, "mlp", hn)
    base = O.widen(W["layers.1.mlp_conv_base"])
    proj = O.widen(W["layers.1.mlp_conv_proj"])
    sub = rng.standard_normal((T, h))
    v = d.dconv_finish(sub, kern)
    for t in range(T):
        for c in range(0, h, 37):
            g = c // gs
            ku = [base[0, j, c] + float(proj[(0 * k + j) * (h // gs) + g] @ hn[t]) for j in range(k)]
            kf = [base[1, j, c] + float(proj[(1 * k + j) * (h // gs) + g] @ hn[t]) for j in range(k)]
            want_u = sum(ku[j] * hn[t - j, c] for j in range(k) if t - j >= 0)
            want_v = sum(kf[j] * sub[t - j, c] for j in range(k) if t - j >= 0)
            assert abs(u[t, c] - want_u) < 1e-12 and abs(v[t, c] - want_v) < 1e-12
    # causal: row t depends on rows t and t-1 only
    hn2 = hn.copy()
    hn2[3] += 1.0
    u2, _ = d.dconv_prepare(1, "mlp", hn2)
    assert np.array_equal(u2[:3], u[:3]) and not np.allclose(u2[3:5], u[3:5])


def test_dflash2_with_identity_convs_and_zero_codebooks_is_plain_dflash(dflash2):
    """Base kernels [1, 0] for both applications, zero kernel projections and zero
    codebooks: the convs are the identity and the walk picks each row's top candidate, so
    the DFlash2 forward is the plain forward bit for bit (tokens and logits)."""
    m, W = dflash2
    Wx = dict(W)
    h, L = m["hidden"], m["num_layers"]
    ident = np.zeros((2, 2, h), np.float32)
    ident[:, 0, :] = 1.0
    for l in range(L):
        for site in ("attention", "mlp"):
            Wx[f"layers.{l}.{site}_conv_base"] = synth.f32_to_bf16_bits(ident)
            Wx[f"layers.{l}.{site}_conv_proj"] = np.zeros_like(W[f"layers.{l}.{site}_conv_proj"])
    for name in ("selector_pred", "selector_succ"):
        Wx[name] = np.zeros_like(W[name])
    plain = {k: v for k, v in m.items() if k not in ("conv_kernel_size", "conv_group_size", "selector_rank",
                                                     "selector_top_k")}
    outs = []
    for mm, ww in ((m, Wx), (plain, _plain_weights(W))):
        e = O.Engine(mm, ww, 64, 2)
        e.ctx_kv_append(0, synth.gen_hidden(m, 1401, 21, 0))
        e.ctx_kv_append(1, synth.gen_hidden(m, 1401, 40, 1))
        outs.append(e.block_forward([1, 0], [33, 600], gamma=16))
    assert np.array_equal(outs[0]["tokens"], outs[1]["tokens"])
    assert np.array_equal(outs[0]["logits"], outs[1]["logits"])
    # and the real DFlash2 weights do change the forward
    e = O.Engine(m, W, 64, 2)
    e.ctx_kv_append(0, synth.gen_hidden(m, 1401, 21, 0))
    e.ctx_kv_append(1, synth.gen_hidden(m, 1401, 40, 1))
    r = e.block_forward([1, 0], [33, 600], gamma=16)
    assert np.abs(r["logits"] - outs[1]["logits"]).max() > 1e-2


def test_selector_walk_planted_chain(dflash2):
    """H = ones (rows y = e_0, hidden_projection column 0 = 1), pred[t] = 10 e_(t mod R),
    succ[c] = e_((c - 1) mod R): a candidate scores +10 iff it is the previous pick + 1.
    Row r's candidates hold bonus + r + 1 at the lowest logit of the 16: the walk must
    still draft bonus+1, bonus+2, ... (unary scores alone would pick other tokens)."""
    m, W = dflash2
    V, R, h = m["vocab"], m["selector_rank"], m["hidden"]
    pred = np.zeros((V, R), np.float32)
    pred[np.arange(V), np.arange(V) % R] = 10.0
    succ = np.zeros((V, R), np.float32)
    succ[np.arange(V), (np.arange(V) - 1) % R] = 1.0
    hp = np.zeros((R, h), np.float32)
    hp[:, 0] = 1.0
    Wx = dict(W, selector_pred=synth.f32_to_bf16_bits(pred), selector_succ=synth.f32_to_bf16_bits(succ),
              selector_hidden_proj=synth.f32_to_bf16_bits(hp))
    d = O.Drafter(m, Wx)
    g, bonus = 6, 50
    y = np.zeros((g, h))
    y[:, 0] = 1.0
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((g, V))
    for r in range(g):
        others = rng.choice(np.setdiff1d(np.arange(300, V), [bonus + r + 1]), 15, replace=False)
        logits[r, others] = 10.0 + rng.random(15)
        logits[r, bonus + r + 1] = 9.5
    drafts, ex = d.selector_walk(y, logits, bonus)
    assert drafts.tolist() == list(range(bonus + 1, bonus + 1 + g))
    assert np.allclose(ex["sel_h"], 1.0)
    assert all(bonus + r + 1 in ex["cand"][r] for r in range(g))
    # teacher forcing on other previous tokens breaks the chain
    d2, _ = d.selector_walk(y, logits, bonus, prev=[0] * g)
    assert not any(d2[r] == bonus + r + 1 for r in range(g))

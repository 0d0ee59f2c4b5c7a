"""CPU-side checks of the boundary: the library loads, exports every entry point the
header declares, and rejects bad configurations before touching the GPU."""
import ctypes as C
import os
import re

import pytest

import synth
from block_diffusion_draft_02_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = []
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", f)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(dflash_\w+)\s*\(", txt, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_entry_point():
    L = B.lib()
    decl = _declared()
    assert {"dflash_create", "dflash_ctx_kv_append", "dflash_block_forward", "dflash_destroy"} <= set(decl)
    for n in decl:
        assert hasattr(L, n), n
    assert set(B.EXPORTED) == set(decl)


def test_strerror_names():
    L = B.lib()
    assert L.dflash_strerror(-3) == b"KV pool exhausted"
    assert L.dflash_strerror(0) == b"ok"


def _null_weights(m):
    lay = (B.dflash_layer_weights * m["num_layers"])()
    for l in range(m["num_layers"]):
        for f, _ in B.dflash_layer_weights._fields_:
            setattr(lay[l], f, 0x1000)
    w = B.dflash_weights(fc=0x1000, hidden_norm=0x1000, norm=0x1000, embed_tokens=0x1000,
                         lm_head=0x1000, layers=lay)
    return w, lay


@pytest.mark.parametrize("change", [
    dict(head_dim=48), dict(num_kv_heads=3), dict(gamma_max=17), dict(gamma_max=1),
    dict(hidden=200), dict(intermediate=640), dict(hidden=384), dict(mask_token_id=5000), dict(num_q_heads=32, num_kv_heads=2),
    dict(hidden=8448, target_hidden=8448, intermediate=8448),
])
def test_create_rejects_unsupported_shapes_before_any_gpu_call(change):
    m = dict(synth.model("tiny-L2-h256"), **change)
    cfg, keep = B.make_config(m, 128, 1)
    w, lay = _null_weights(synth.model("tiny-L2-h256"))
    ctx = C.c_void_p()
    rc = B.lib().dflash_create(C.byref(cfg), C.byref(w), None, C.byref(ctx))
    assert rc == B.DFLASH_EINVAL and not ctx.value


def test_create_rejects_bad_pool_arguments():
    m = synth.model("tiny-L2-h256")
    w, lay = _null_weights(m)
    # (max_seq_len + gamma_max + 1 must stay within 262144: an attention chunk's page ids
    # fit the kernel's table)
    for kw in [dict(max_batch=0), dict(max_batch=33), dict(num_pages=1), dict(max_seq=262144 - 16),
               dict(max_seq=0)]:
        cfg, keep = B.make_config(m, kw.get("max_seq", 128), kw.get("max_batch", 1), num_pages=kw.get("num_pages", 0))
        ctx = C.c_void_p()
        assert B.lib().dflash_create(C.byref(cfg), C.byref(w), None, C.byref(ctx)) == B.DFLASH_EINVAL
    # a weight format other than bf16 (0) and FP8 E4M3 (1)
    for fmt in (2, 7, -1):
        cfg, keep = B.make_config(m, 128, 1)
        cfg.weight_format = fmt
        ctx = C.c_void_p()
        assert B.lib().dflash_create(C.byref(cfg), C.byref(w), None, C.byref(ctx)) == B.DFLASH_EINVAL and not ctx.value
    # a page order that is not a permutation of 1..P-1 (P = 11 here)
    for order in ([1, 2, 3], list(range(0, 10)), [1] * 10):
        cfg, keep = B.make_config(m, 128, 1, page_order=order)
        ctx = C.c_void_p()
        assert B.lib().dflash_create(C.byref(cfg), C.byref(w), None, C.byref(ctx)) == B.DFLASH_EINVAL


def test_null_arguments():
    L = B.lib()
    m = synth.model("tiny-L2-h256")
    cfg, keep = B.make_config(m, 128, 1)
    ctx = C.c_void_p()
    assert L.dflash_create(C.byref(cfg), None, None, C.byref(ctx)) == B.DFLASH_EINVAL
    assert L.dflash_create(None, None, None, C.byref(ctx)) == B.DFLASH_EINVAL
    w, lay = _null_weights(m)
    lay[1].down_proj = None
    assert L.dflash_create(C.byref(cfg), C.byref(w), None, C.byref(ctx)) == B.DFLASH_EINVAL
    assert L.dflash_ctx_kv_append(None, 0, None, None, 1, None) == B.DFLASH_EINVAL
    assert L.dflash_ctx_kv_append_batch(None, 1, None, None, None, None, None) == B.DFLASH_EINVAL
    assert L.dflash_block_forward(None, 1, None, None, None, 16, None, None, None) == B.DFLASH_EINVAL
    L.dflash_destroy(None)


def test_create_rejects_misaligned_matrices():
    # matrices are streamed with 16-byte loads; the check comes before any GPU call
    L = B.lib()
    m = synth.model("tiny-L2-h256")
    cfg, keep = B.make_config(m, 128, 1)
    ctx = C.c_void_p()
    w, lay = _null_weights(m)
    lay[1].o_proj = 0x1002
    assert L.dflash_create(C.byref(cfg), C.byref(w), None, C.byref(ctx)) == B.DFLASH_EINVAL
    w, lay = _null_weights(m)
    w.lm_head = 0x1008
    assert L.dflash_create(C.byref(cfg), C.byref(w), None, C.byref(ctx)) == B.DFLASH_EINVAL
    assert not ctx.value


def test_config_struct_layout_matches_header():
    # offsets of the C struct on x86-64 (natural alignment)
    assert B.dflash_config.rope_theta.offset == 48
    assert B.dflash_config.yarn_factor.offset == 64
    assert B.dflash_config.layer_sliding.offset == 104
    assert B.dflash_config.page_order.offset == 128
    assert B.dflash_config.weight_format.offset == 136
    assert B.dflash_config.markov_rank.offset == 140
    assert B.dflash_config.selector_top_k.offset == 156
    assert C.sizeof(B.dflash_config) == 160
    assert C.sizeof(B.dflash_layer_weights) == 120 and C.sizeof(B.dflash_weights) == 88


def test_struct_layouts_match_the_c_compiler(tmp_path):
    """Every field offset and struct size of the ctypes mirrors equals what a C compiler
    makes of include/dflash.h."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = {"dflash_config": B.dflash_config, "dflash_layer_weights": B.dflash_layer_weights,
               "dflash_weights": B.dflash_weights}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "dflash.h"', "int main(void) {"]
    for name, st in structs.items():
        lines.append(f'  printf("{name} size %zu\\n", sizeof({name}));')
        for f, _ in st._fields_:
            lines.append(f'  printf("{name} {f} %zu\\n", offsetof({name}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    subprocess.run([cc, "-std=c99", "-I", inc, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for name, st in structs.items():
        assert got[(name, "size")] == C.sizeof(st), name
        for f, _ in st._fields_:
            assert got[(name, f)] == getattr(st, f).offset, (name, f)


def test_create_rejects_bad_markov_heads():
    m = synth.model("tiny-L2-h256-dspark")
    w, lay = _null_weights(m)
    ctx = C.c_void_p()
    for rank in (128, 300, 1024, -1):
        cfg, keep = B.make_config(dict(m, markov_rank=rank), 128, 1)
        w.markov_w1 = w.markov_w2 = 0x1000
        assert B.lib().dflash_create(C.byref(cfg), C.byref(w), None, C.byref(ctx)) == B.DFLASH_EINVAL
    cfg, keep = B.make_config(m, 128, 1)
    for w1, w2 in ((None, 0x1000), (0x1000, None), (0x1008, 0x1000), (0x1000, 0x1004)):
        w.markov_w1, w.markov_w2 = w1, w2
        assert B.lib().dflash_create(C.byref(cfg), C.byref(w), None, C.byref(ctx)) == B.DFLASH_EINVAL
    assert not ctx.value


def test_create_rejects_bad_dflash2_heads():
    m = synth.model("tiny-L2-h256-dflash2")
    w, lay = _null_weights(m)
    w.selector_pred = w.selector_succ = w.selector_hidden_proj = 0x1000
    ctx = C.c_void_p()
    # unsupported sizes, a partial configuration, and a Markov head beside DFlash2
    for change in (dict(conv_kernel_size=3), dict(conv_group_size=8), dict(selector_top_k=8), dict(selector_rank=128),
                   dict(selector_rank=0), dict(conv_kernel_size=0), dict(markov_rank=256)):
        cfg, keep = B.make_config(dict(m, **change), 128, 1)
        assert B.lib().dflash_create(C.byref(cfg), C.byref(w), None, C.byref(ctx)) == B.DFLASH_EINVAL, change
    # missing or misaligned DFlash2 weights (the layers' conv pointers are 0x1000 from _null_weights)
    cfg, keep = B.make_config(m, 128, 1)
    for field, val in (("selector_pred", None), ("selector_hidden_proj", 0x1008)):
        setattr(w, field, val)
        assert B.lib().dflash_create(C.byref(cfg), C.byref(w), None, C.byref(ctx)) == B.DFLASH_EINVAL
        setattr(w, field, 0x1000)
    lay[1].mlp_conv_base = None
    assert B.lib().dflash_create(C.byref(cfg), C.byref(w), None, C.byref(ctx)) == B.DFLASH_EINVAL
    assert not ctx.value


# ---- the binding checks every argument before it reaches the library ------------------


class _NoLib:
    """Stands in for the loaded library: any call into it fails the test."""

    def __getattr__(self, name):
        raise AssertionError(f"the binding called {name} with a bad argument")


def _unbound_drafter(m):
    d = B.Drafter.__new__(B.Drafter)
    d.m, d.L, d.ctx = m, _NoLib(), None
    return d


def test_binding_rejects_bad_tensors_and_lists_before_calling_the_library():
    import torch
    m = synth.model("tiny-L2-h256")
    d = _unbound_drafter(m)
    width = m["num_taps"] * m["target_hidden"]
    H = torch.zeros((8, width), dtype=torch.bfloat16)
    bad_hidden = [
        (torch.zeros((8, width), dtype=torch.float32), "bfloat16"),
        (torch.zeros((8, width + 1), dtype=torch.bfloat16), "num_taps"),
        (torch.zeros((width, 8), dtype=torch.bfloat16).t(), "contiguous"),
        (torch.zeros((8 * width,), dtype=torch.bfloat16), "num_taps"),
        (H, "GPU tensor"),   # every check passes but the device (this host has no GPU tensors)
    ]
    for t, why in bad_hidden:
        with pytest.raises(ValueError, match=why):
            d.dflash_ctx_kv_append(0, t)
    with pytest.raises(ValueError, match="positions must have 8"):
        d.dflash_ctx_kv_append(0, H, positions=[1, 2, 3])
    with pytest.raises(ValueError, match="counts must have 2"):
        d.dflash_ctx_kv_append_batch([0, 1], [8], H)
    with pytest.raises(ValueError, match="hold 9 rows"):
        d.dflash_ctx_kv_append_batch([0, 1], [4, 5], H)
    with pytest.raises(ValueError, match="positions must have 8"):
        d.dflash_ctx_kv_append_batch([0, 1], [4, 4], H, positions=list(range(7)))
    V = m["vocab"]
    toks = torch.zeros((2, 15), dtype=torch.int32)
    lg = torch.zeros((30, V), dtype=torch.float32)
    bad_forward = [
        (dict(seqs=[], bonus=[], draft_tokens=toks), "at least one"),
        (dict(seqs=[0, 1], bonus=[3], draft_tokens=toks), "bonus must have 2"),
        (dict(seqs=[0, 1], bonus=[3, 4], q_rope_pos=[9], draft_tokens=toks), "q_rope_pos must have 2"),
        (dict(seqs=[0, 1], bonus=[3, 4], draft_tokens=toks.to(torch.int64)), "int32"),
        (dict(seqs=[0, 1], bonus=[3, 4], draft_tokens=toks[:, :14].contiguous()), "28 elements, 30 needed"),
        (dict(seqs=[0, 1], bonus=[3, 4], draft_tokens=toks[:, ::2]), "contiguous"),
        (dict(seqs=[0, 1], bonus=[3, 4], draft_tokens=toks, logits=lg[:29]), "elements"),
        (dict(seqs=[0, 1], bonus=[3, 4], draft_tokens=toks, logits=lg.to(torch.float64)), "float32"),
        (dict(seqs=[0, 1], bonus=[3, 4], draft_tokens=toks, gamma=1), "gamma"),
        (dict(seqs=[0, 1], bonus=[3, 4], draft_tokens=toks, logits=lg), "GPU tensor"),
    ]
    for kw, why in bad_forward:
        for f in (d.dflash_block_forward, d.dflash_block_forward_noalloc):
            with pytest.raises(ValueError, match=why):
                f(**kw)
    with pytest.raises(ValueError, match="bytes"):
        d.dflash_debug_copy(B.DFLASH_BUF_POOL, torch.zeros(4, dtype=torch.int32), nbytes=17)


def test_binding_rejects_bad_weights_before_calling_the_library():
    import torch
    m = synth.model("tiny-L2-h256")
    shapes = B.weight_shapes(m)
    W = {k: torch.zeros(v, dtype=torch.bfloat16) for k, v in shapes.items()}
    for name, change, why in [("fc", lambda t: t[:, :-1].contiguous(), "shape"),
                              ("layers.1.k_norm", lambda t: t.float(), "bfloat16"),
                              ("lm_head", lambda t: t.t(), "contiguous|shape"),
                              ("norm", None, "missing"),
                              ("embed_tokens", lambda t: t, "GPU tensor")]:
        bad = dict(W)
        if change is None:
            del bad[name]
        else:
            bad[name] = change(W[name])
        with pytest.raises(ValueError, match=why):
            B.Drafter(m, bad, 128, 1)

"""ctypes binding of libdflash.so: the C ABI's structs and calls under the same names, plus
a small `Drafter` wrapper that turns a config dict and torch tensors into those structs.
Argument marshalling only: every step of the drafter runs in the HIP library. There is no
fallback; if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes as C
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdflash.so")

DFLASH_OK, DFLASH_EINVAL, DFLASH_ENOMEM, DFLASH_EPOOL, DFLASH_ERANGE, DFLASH_EHIP = 0, -1, -2, -3, -4, -5
DFLASH_WEIGHTS_BF16, DFLASH_WEIGHTS_FP8_E4M3 = 0, 1
CODE_NAMES = {0: "OK", -1: "EINVAL", -2: "ENOMEM", -3: "EPOOL", -4: "ERANGE", -5: "EHIP"}
DFLASH_BUF_POOL, DFLASH_BUF_KPOS, DFLASH_BUF_SLOTS, DFLASH_BUF_BLOCKTAB, DFLASH_BUF_HIDDEN = 0, 1, 2, 3, 4
DFLASH_BUF_HIDDEN_LO, DFLASH_BUF_FP8_LMHEAD, DFLASH_BUF_FP8_LMHEAD_SCALE = 5, 6, 7
DFLASH_BUF_SEL_IDX, DFLASH_BUF_SEL_VALS = 8, 9
DFLASH_BUF_CTX_FEAT, DFLASH_BUF_CTX_FEAT_LO = 10, 11
DFLASH_BUF_LAYER_Q, DFLASH_BUF_LAYER_Q_LO, DFLASH_BUF_LAYER_ATTN, DFLASH_BUF_LAYER_ATTN_LO = 12, 13, 14, 15
DFLASH_BUF_LAYER_X1, DFLASH_BUF_LAYER_X = 16, 17


class dflash_config(C.Structure):
    _fields_ = [
        ("num_layers", C.c_int32), ("hidden", C.c_int32), ("num_q_heads", C.c_int32),
        ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("intermediate", C.c_int32),
        ("vocab", C.c_int32), ("num_taps", C.c_int32), ("target_hidden", C.c_int32),
        ("gamma_max", C.c_int32), ("mask_token_id", C.c_int32), ("rms_eps", C.c_float),
        ("rope_theta", C.c_double), ("rope_type", C.c_int32),
        ("yarn_factor", C.c_double), ("yarn_orig_max_pos", C.c_double),
        ("yarn_beta_fast", C.c_double), ("yarn_beta_slow", C.c_double),
        ("sliding_window", C.c_int32), ("layer_sliding", C.POINTER(C.c_uint8)),
        ("max_seq_len", C.c_int32), ("max_batch", C.c_int32), ("num_pages", C.c_int32),
        ("page_order", C.POINTER(C.c_int32)), ("weight_format", C.c_int32),
        ("markov_rank", C.c_int32), ("conv_kernel_size", C.c_int32), ("conv_group_size", C.c_int32),
        ("selector_rank", C.c_int32), ("selector_top_k", C.c_int32),
    ]


class dflash_layer_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "q_proj", "k_proj", "v_proj", "o_proj", "q_norm", "k_norm", "input_layernorm",
        "post_attention_layernorm", "gate_proj", "up_proj", "down_proj",
        "attention_conv_base", "attention_conv_proj", "mlp_conv_base", "mlp_conv_proj")]


class dflash_weights(C.Structure):
    _fields_ = [("fc", C.c_void_p), ("hidden_norm", C.c_void_p), ("norm", C.c_void_p),
                ("embed_tokens", C.c_void_p), ("lm_head", C.c_void_p),
                ("layers", C.POINTER(dflash_layer_weights)),
                ("markov_w1", C.c_void_p), ("markov_w2", C.c_void_p),
                ("selector_pred", C.c_void_p), ("selector_succ", C.c_void_p),
                ("selector_hidden_proj", C.c_void_p)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m block_diffusion_draft_02_amd.build` (no fallback path exists)")
        L = C.CDLL(_LIB_PATH)
        vp, i32, i64p, i32p = C.c_void_p, C.c_int32, C.POINTER(C.c_int64), C.POINTER(C.c_int32)
        L.dflash_create.argtypes = [C.POINTER(dflash_config), C.POINTER(dflash_weights), vp, C.POINTER(vp)]
        L.dflash_ctx_kv_append.argtypes = [vp, i32, vp, i32p, i32, vp]
        L.dflash_ctx_kv_append_batch.argtypes = [vp, i32, i32p, i32p, vp, i32p, vp]
        L.dflash_block_forward.argtypes = [vp, i32, i32p, i32p, i32p, i32, vp, vp, vp]
        L.dflash_block_forward_noalloc.argtypes = [vp, i32, i32p, i32p, i32p, i32, vp, vp, vp]
        L.dflash_destroy.argtypes = [vp]
        L.dflash_destroy.restype = None
        L.dflash_seq_reset.argtypes = [vp, i32]
        L.dflash_seq_info.argtypes = [vp, i32, i32p, i32p, i32p, i32]
        L.dflash_pool_geometry.argtypes = [vp, i64p, i64p, i64p, i64p, i64p]
        L.dflash_debug_copy.argtypes = [vp, i32, vp, C.c_size_t, C.c_size_t, vp]
        L.dflash_debug_capture.argtypes = [vp, i32]
        L.dflash_last_error.argtypes = [vp]
        L.dflash_last_error.restype = C.c_char_p
        L.dflash_timing.argtypes = [vp, C.c_uint32]
        L.dflash_timing_read.argtypes = [vp, C.POINTER(C.c_double), i64p, i32]
        L.dflash_strerror.argtypes = [C.c_int]
        L.dflash_strerror.restype = C.c_char_p
        for f in ("dflash_create", "dflash_ctx_kv_append", "dflash_ctx_kv_append_batch", "dflash_block_forward",
                  "dflash_block_forward_noalloc", "dflash_seq_reset",
                  "dflash_seq_info", "dflash_pool_geometry", "dflash_debug_copy", "dflash_debug_capture",
                  "dflash_timing", "dflash_timing_read"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


EXPORTED = ("dflash_create", "dflash_ctx_kv_append", "dflash_ctx_kv_append_batch", "dflash_block_forward",
            "dflash_block_forward_noalloc", "dflash_destroy",
            "dflash_seq_reset", "dflash_seq_info", "dflash_pool_geometry", "dflash_debug_copy",
            "dflash_debug_capture", "dflash_last_error", "dflash_strerror", "dflash_timing", "dflash_timing_read")

K_CLASSES = ("prologue", "gemm", "qkv_post", "attn", "attn_combine", "resid_norm", "silu",
             "lmhead", "argmax", "append_gemm", "append_misc", "markov", "dconv", "selector")


class DflashError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{CODE_NAMES.get(code, code)}: {msg}")
        self.code = code
        self.name = CODE_NAMES.get(code, str(code))


def _i32_array(vals):
    if vals is None:
        return None
    vals = [int(v) for v in vals]
    return (C.c_int32 * max(1, len(vals)))(*vals)


def make_config(m: dict, max_seq_len: int, max_batch: int, num_pages: int = 0, page_order=None):
    """dflash_config from a model dict (the keys of synth.MODELS). Returns (struct, keepalive)."""
    ls = m.get("layer_sliding")
    ls_arr = (C.c_uint8 * m["num_layers"])(*[1 if x else 0 for x in ls]) if ls else None
    po = _i32_array(page_order)
    cfg = dflash_config(
        num_layers=m["num_layers"], hidden=m["hidden"], num_q_heads=m["num_q_heads"],
        num_kv_heads=m["num_kv_heads"], head_dim=m["head_dim"], intermediate=m["intermediate"],
        vocab=m["vocab"], num_taps=m["num_taps"], target_hidden=m["target_hidden"],
        gamma_max=m["gamma_max"], mask_token_id=m["mask_token_id"], rms_eps=m["rms_eps"],
        rope_theta=m["rope_theta"], rope_type=1 if m.get("rope_type") == "yarn" else 0,
        yarn_factor=m.get("yarn_factor", 0.0), yarn_orig_max_pos=m.get("yarn_orig_max_pos", 0.0),
        yarn_beta_fast=m.get("yarn_beta_fast", 0.0), yarn_beta_slow=m.get("yarn_beta_slow", 0.0),
        sliding_window=int(m.get("sliding_window") or 0),
        layer_sliding=C.cast(ls_arr, C.POINTER(C.c_uint8)) if ls_arr is not None else None,
        max_seq_len=max_seq_len, max_batch=max_batch, num_pages=num_pages,
        page_order=C.cast(po, C.POINTER(C.c_int32)) if po is not None else None,
        weight_format=DFLASH_WEIGHTS_FP8_E4M3 if m.get("weight_format") == "fp8" else DFLASH_WEIGHTS_BF16,
        markov_rank=int(m.get("markov_rank", 0)),
        conv_kernel_size=int(m.get("conv_kernel_size", 0)), conv_group_size=int(m.get("conv_group_size", 0)),
        selector_rank=int(m.get("selector_rank", 0)), selector_top_k=int(m.get("selector_top_k", 0)))
    return cfg, (ls_arr, po)


def _ptr(t):
    return C.c_void_p(t.data_ptr())


def _check_tensor(t, name, dtype, numel=None, device=True, shape=None):
    """Raise ValueError unless `t` is a contiguous torch tensor of `dtype` with at least `numel`
    elements (or exactly `shape`), on a GPU when `device`: the library reads and writes through
    the raw pointer, so anything else would read or write outside the tensor."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, {numel} needed")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got one on {t.device}")


def _check_len(vals, name, n):
    if vals is not None and len(vals) != n:
        raise ValueError(f"{name} must have {n} entries, got {len(vals)}")


def weight_shapes(m: dict) -> dict:
    """Shape of every weight the drafter reads, by the names Drafter takes."""
    h, hd = m["hidden"], m["head_dim"]
    qd, kvd, ff, V = m["num_q_heads"] * hd, m["num_kv_heads"] * hd, m["intermediate"], m["vocab"]
    out = {"fc": (h, m["num_taps"] * m["target_hidden"]), "hidden_norm": (h,), "norm": (h,),
           "embed_tokens": (V, h), "lm_head": (V, h)}
    for l in range(m["num_layers"]):
        p = f"layers.{l}."
        out.update({p + "q_proj": (qd, h), p + "k_proj": (kvd, h), p + "v_proj": (kvd, h), p + "o_proj": (h, qd),
                    p + "q_norm": (hd,), p + "k_norm": (hd,), p + "input_layernorm": (h,),
                    p + "post_attention_layernorm": (h,), p + "gate_proj": (ff, h), p + "up_proj": (ff, h),
                    p + "down_proj": (h, ff)})
        if m.get("selector_rank", 0):
            k, ng = m["conv_kernel_size"], 2 * m["conv_kernel_size"] * h // m["conv_group_size"]
            for site in ("attention", "mlp"):
                out.update({f"{p}{site}_conv_base": (2, k, h), f"{p}{site}_conv_proj": (ng, h)})
    if m.get("markov_rank", 0):
        out.update({"markov_w1": (V, m["markov_rank"]), "markov_w2": (V, m["markov_rank"])})
    if m.get("selector_rank", 0):
        r = m["selector_rank"]
        out.update({"selector_pred": (V, r), "selector_succ": (V, r), "selector_hidden_proj": (r, h)})
    return out


def _stream(stream):
    if stream is not None:
        return C.c_void_p(stream)
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


class Drafter:
    """One dflash_ctx. `weights` maps the synth weight names to device bf16 torch tensors,
    which must outlive the object."""

    def __init__(self, m: dict, weights: dict, max_seq_len: int, max_batch: int,
                 num_pages: int = 0, page_order=None, stream=None):
        import torch
        self.ctx = None
        self.m = m
        shapes = weight_shapes(m)
        for dev in (False, True):   # every property but the device first, then the devices
            for name, shape in shapes.items():
                if name not in weights:
                    raise ValueError(f"weight {name} is missing")
                _check_tensor(weights[name], name, torch.bfloat16, shape=shape, device=dev)
        self.L = lib()
        self.weights = weights
        cfg, self._keep = make_config(m, max_seq_len, max_batch, num_pages, page_order)
        nl = m["num_layers"]
        lay = (dflash_layer_weights * nl)()
        for l in range(nl):
            p = f"layers.{l}."
            for f in dflash_layer_weights._fields_:
                if p + f[0] in weights:
                    setattr(lay[l], f[0], weights[p + f[0]].data_ptr())
        w = dflash_weights(fc=weights["fc"].data_ptr(), hidden_norm=weights["hidden_norm"].data_ptr(),
                           norm=weights["norm"].data_ptr(), embed_tokens=weights["embed_tokens"].data_ptr(),
                           lm_head=weights["lm_head"].data_ptr(), layers=lay)
        if m.get("markov_rank", 0):
            w.markov_w1 = weights["markov_w1"].data_ptr()
            w.markov_w2 = weights["markov_w2"].data_ptr()
        if m.get("selector_rank", 0):
            w.selector_pred = weights["selector_pred"].data_ptr()
            w.selector_succ = weights["selector_succ"].data_ptr()
            w.selector_hidden_proj = weights["selector_hidden_proj"].data_ptr()
        ctx = C.c_void_p()
        rc = self.L.dflash_create(C.byref(cfg), C.byref(w), _stream(stream), C.byref(ctx))
        if rc != DFLASH_OK:
            raise DflashError(rc, "dflash_create failed")
        self.ctx = ctx

    def _check(self, rc):
        if rc != DFLASH_OK:
            raise DflashError(rc, self.L.dflash_last_error(self.ctx).decode())

    def close(self):
        if getattr(self, "ctx", None):
            self.L.dflash_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- the calls -------------------------------------------------------------------------
    def _check_hidden(self, target_hidden, rows=None):
        import torch
        width = self.m["num_taps"] * self.m["target_hidden"]
        if getattr(target_hidden, "ndim", 0) != 2 or int(target_hidden.shape[1]) != width:
            raise ValueError(f"target_hidden must be [rows, {width}] (num_taps * target_hidden)")
        if rows is not None and int(target_hidden.shape[0]) != rows:
            raise ValueError(f"target_hidden must hold {rows} rows, got {int(target_hidden.shape[0])}")
        _check_tensor(target_hidden, "target_hidden", torch.bfloat16)

    def _check_forward(self, seqs, bonus, q_rope_pos, gamma, draft_tokens, logits):
        import torch
        n = len(seqs)
        if n < 1:
            raise ValueError("seqs must name at least one sequence")
        _check_len(bonus, "bonus", n)
        _check_len(q_rope_pos, "q_rope_pos", n)
        if not isinstance(gamma, int) or gamma < 2:
            raise ValueError("gamma must be an int >= 2")
        # every property but the device first, then the devices
        for dev in (False, True):
            _check_tensor(draft_tokens, "draft_tokens", torch.int32, numel=n * (gamma - 1), device=dev)
            if logits is not None:
                _check_tensor(logits, "logits", torch.float32, numel=n * (gamma - 1) * self.m["vocab"], device=dev)

    def dflash_ctx_kv_append(self, seq, target_hidden, positions=None, stream=None):
        if getattr(target_hidden, "ndim", 0) != 2:
            raise ValueError("target_hidden must be [rows, num_taps * target_hidden]")
        n = int(target_hidden.shape[0])
        _check_len(positions, "positions", n)
        self._check_hidden(target_hidden)
        pos = _i32_array(positions)
        self._check(self.L.dflash_ctx_kv_append(self.ctx, seq, _ptr(target_hidden), pos, n, _stream(stream)))

    def dflash_ctx_kv_append_batch(self, seqs, counts, target_hidden, positions=None, stream=None):
        """New rows of several sequences in one pass: target_hidden holds sum(counts) rows,
        the sequences' rows one after another in the order of seqs."""
        _check_len(counts, "counts", len(seqs))
        _check_len(positions, "positions", int(sum(counts)))
        self._check_hidden(target_hidden, rows=int(sum(counts)))
        s, n, pos = _i32_array(seqs), _i32_array(counts), _i32_array(positions)
        self._check(self.L.dflash_ctx_kv_append_batch(self.ctx, len(seqs), s, n, _ptr(target_hidden), pos,
                                                      _stream(stream)))

    def dflash_block_forward(self, seqs, bonus, draft_tokens, logits=None, q_rope_pos=None,
                             gamma=None, stream=None):
        gamma = self.m["gamma_max"] if gamma is None else gamma
        self._check_forward(seqs, bonus, q_rope_pos, gamma, draft_tokens, logits)
        s, b, q = _i32_array(seqs), _i32_array(bonus), _i32_array(q_rope_pos)
        self._check(self.L.dflash_block_forward(
            self.ctx, len(seqs), s, b, q, gamma, _ptr(draft_tokens),
            _ptr(logits) if logits is not None else None, _stream(stream)))

    def dflash_block_forward_noalloc(self, seqs, bonus, draft_tokens, logits=None, q_rope_pos=None,
                                     gamma=None, stream=None):
        """dflash_block_forward with its partials in the library's static per-device scratch."""
        gamma = self.m["gamma_max"] if gamma is None else gamma
        self._check_forward(seqs, bonus, q_rope_pos, gamma, draft_tokens, logits)
        s, b, q = _i32_array(seqs), _i32_array(bonus), _i32_array(q_rope_pos)
        self._check(self.L.dflash_block_forward_noalloc(
            self.ctx, len(seqs), s, b, q, gamma, _ptr(draft_tokens),
            _ptr(logits) if logits is not None else None, _stream(stream)))

    def dflash_seq_reset(self, seq):
        self._check(self.L.dflash_seq_reset(self.ctx, seq))

    def dflash_seq_info(self, seq, cap=1 << 16):
        kv, npg = C.c_int32(), C.c_int32()
        bt = (C.c_int32 * cap)()
        self._check(self.L.dflash_seq_info(self.ctx, seq, C.byref(kv), C.byref(npg), bt, cap))
        return kv.value, list(bt[: npg.value])

    def dflash_pool_geometry(self):
        vals = [C.c_int64() for _ in range(5)]
        self._check(self.L.dflash_pool_geometry(self.ctx, *[C.byref(v) for v in vals]))
        keys = ("num_pages", "pages_per_seq", "page_layer_bytes", "pool_bytes", "fused_kv_weight_bytes")
        return dict(zip(keys, [v.value for v in vals]))

    def dflash_timing(self, classes):
        """Time the launches of the named classes (see K_CLASSES); [] turns timing off."""
        mask = 0
        for c in classes:
            mask |= 1 << K_CLASSES.index(c)
        self._check(self.L.dflash_timing(self.ctx, mask))

    def dflash_timing_read(self):
        """{class: (milliseconds, launches)} since the last read."""
        n = len(K_CLASSES)
        ms, cnt = (C.c_double * n)(), (C.c_int64 * n)()
        self._check(self.L.dflash_timing_read(self.ctx, ms, cnt, n))
        return {K_CLASSES[i]: (ms[i], cnt[i]) for i in range(n)}

    def dflash_debug_capture(self, on=True):
        """Capture each layer's intermediates of the following forwards (see dflash.h)."""
        self._check(self.L.dflash_debug_capture(self.ctx, 1 if on else 0))

    def dflash_debug_copy(self, buffer, dst, offset=0, nbytes=None, stream=None):
        """Copy into a torch tensor (host or device) `dst`; nbytes defaults to dst's size."""
        if not dst.is_contiguous():
            raise ValueError("dst must be contiguous")
        cap = dst.numel() * dst.element_size()
        nbytes = cap if nbytes is None else nbytes
        if nbytes > cap:
            raise ValueError(f"dst holds {cap} bytes, {nbytes} requested")
        self._check(self.L.dflash_debug_copy(self.ctx, buffer, C.c_void_p(dst.data_ptr()), offset, nbytes,
                                             _stream(stream)))

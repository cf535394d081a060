"""ctypes binding of libspecverify: the C ABI's calls under the same names.

Argument marshalling only -- every computation runs in the library's HIP
kernels.  Device buffers are torch tensors (PyTorch supplies device memory and
streams); the binding passes their addresses.  Importing this module does not
touch the GPU; loading fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspecverify.so")

SPEC_F32, SPEC_BF16 = 0, 1
STATUS = {0: "SPEC_OK", -1: "SPEC_EINVAL", -2: "SPEC_ENOMEM", -3: "SPEC_EHIP", -4: "SPEC_EUNSUPPORTED",
          -5: "SPEC_EDEVICE"}

# Every symbol the C header declares.
EXPORTS = ("spec_model_create", "spec_model_destroy", "spec_workspace_bytes", "spec_sampler_workspace_bytes",
           "spec_verify_forward", "spec_verify_forward_trace", "spec_softmax_pq", "spec_reject_sample",
           "spec_draft_sample",
           "spec_decode_step", "spec_decode_step_static", "spec_linear",
           "spec_kv_set_len", "spec_last_error", "spec_commit_round", "spec_ngram_propose")


class SpecError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class spec_model_cfg(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("dtype", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("rms_eps", ctypes.c_float)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class spec_weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("lm_head", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("attn_norm", _PP), ("wqkv", _PP), ("wo", _PP), ("mlp_norm", _PP), ("wgu", _PP), ("wd", _PP)]


class spec_kv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("len", ctypes.c_void_p), ("B", ctypes.c_int32),
                ("max_ctx", ctypes.c_int32)]


class spec_trace(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("q", ctypes.c_void_p), ("attn", ctypes.c_void_p), ("h_mid", ctypes.c_void_p),
                ("mlp", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libspecverify and declare its signatures (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -m draft_then_verify_amd.build); "
                           "there is no fallback path")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "spec_model_create": (i32, [ctypes.POINTER(spec_model_cfg), ctypes.POINTER(spec_weights), ctypes.POINTER(vp)]),
        "spec_model_destroy": (None, [vp]),
        "spec_workspace_bytes": (sz, [vp, i32, i32, i32]),
        "spec_sampler_workspace_bytes": (sz, [i64, i32, i32]),
        "spec_verify_forward": (i32, [vp, ctypes.POINTER(spec_kv), i32, i32, vp, vp, vp, sz, vp]),
        "spec_verify_forward_trace": (i32, [vp, ctypes.POINTER(spec_kv), i32, i32, vp, vp, ctypes.POINTER(spec_trace),
                                            vp, sz, vp]),
        "spec_softmax_pq": (i32, [vp, i64, i32, f32, vp, vp, sz, vp]),
        "spec_reject_sample": (i32, [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "spec_draft_sample": (i32, [vp, i64, i32, i32, f32, vp, vp, i64, vp, i32, vp, sz, vp]),
        "spec_decode_step": (i32, [vp, ctypes.POINTER(spec_kv), i32, i32, f32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   sz, vp]),
        "spec_decode_step_static": (i32, [vp, ctypes.POINTER(spec_kv), i32, i32, f32, vp, vp, vp, vp, vp, vp, vp, vp,
                                          vp, vp]),
        "spec_linear": (i32, [i32, i32, vp, vp, i32, i32, i32, vp, vp, vp, vp, f32, vp]),
        "spec_kv_set_len": (i32, [ctypes.POINTER(spec_kv), i32, vp, i32, vp]),
        "spec_commit_round": (i32, [i32, i32, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, i32, vp]),
        "spec_ngram_propose": (i32, [i32, i32, i32, i32, vp, vp, i32, vp, vp, i32, vp, vp, vp, vp, vp]),
        "spec_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def spec_last_error() -> str:
    return load_library().spec_last_error().decode()


def _check(status: int):
    if status != 0:
        raise SpecError(status, spec_last_error())


def _ptr(t) -> int | None:
    """Device address of a tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor or None")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


# --- model / KV handles ----------------------------------------------------------

class SpecModel:
    """spec_model handle over device weights (a dict as produced by
    synth.make_weights, moved to the GPU).  ``n_layers`` < the shape's count
    builds a self-speculative drafter over the same tensors."""

    def __init__(self, shape, weights: dict, n_layers: int | None = None):
        lib = load_library()
        L = shape.n_layers if n_layers is None else n_layers
        self.shape, self.n_layers, self.weights = shape, L, weights
        self.dtype = SPEC_BF16 if shape.dtype == "bf16" else SPEC_F32
        self.cfg = spec_model_cfg(shape.d_model, L, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.d_ff,
                                  shape.vocab, self.dtype, shape.rope_theta, shape.rms_eps)

        def arr(name):
            t = weights[name]
            return (ctypes.c_void_p * L)(*[t[i].data_ptr() for i in range(L)])

        self._arrays = {n: arr(n) for n in ("attn_norm", "wqkv", "wo", "mlp_norm", "wgu", "wd")}
        a = self._arrays
        self._w = spec_weights(weights["embed"].data_ptr(), weights["lm_head"].data_ptr(),
                               weights["final_norm"].data_ptr(),
                               ctypes.cast(a["attn_norm"], _PP), ctypes.cast(a["wqkv"], _PP),
                               ctypes.cast(a["wo"], _PP), ctypes.cast(a["mlp_norm"], _PP),
                               ctypes.cast(a["wgu"], _PP), ctypes.cast(a["wd"], _PP))
        h = ctypes.c_void_p()
        _check(lib.spec_model_create(ctypes.byref(self.cfg), ctypes.byref(self._w), ctypes.byref(h)))
        self.handle = h

    def workspace_bytes(self, B: int, m: int, max_ctx: int) -> int:
        return int(load_library().spec_workspace_bytes(self.handle, B, m, max_ctx))

    def close(self):
        if getattr(self, "handle", None):
            load_library().spec_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class KVCache:
    """Contiguous per-sequence KV cache on the device: k, v
    [L, B, Hkv, max_ctx, hd] in the model dtype; len [B] int32."""

    def __init__(self, shape, n_layers: int, B: int, max_ctx: int, device="cuda"):
        dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
        dims = (n_layers, B, shape.n_kv_heads, max_ctx, shape.head_dim)
        self.k = torch.zeros(dims, dtype=dt, device=device)
        self.v = torch.zeros(dims, dtype=dt, device=device)
        self.len = torch.zeros(B, dtype=torch.int32, device=device)
        self.B, self.max_ctx = B, max_ctx
        self.struct = spec_kv(self.k.data_ptr(), self.v.data_ptr(), self.len.data_ptr(), B, max_ctx)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# --- the C ABI calls ---------------------------------------------------------------

def spec_workspace_bytes(model: SpecModel, B: int, m: int, max_ctx: int) -> int:
    return int(load_library().spec_workspace_bytes(model.handle, B, m, max_ctx))


def spec_sampler_workspace_bytes(rows: int, B: int, vocab: int) -> int:
    return int(load_library().spec_sampler_workspace_bytes(rows, B, vocab))


def spec_verify_forward(model: SpecModel, kv: KVCache, B: int, m: int, tokens, logits, ws, stream=None):
    _check(load_library().spec_verify_forward(model.handle, ctypes.byref(kv.struct), B, m, _ptr(tokens),
                                              _ptr(logits), _ptr(ws), _nbytes(ws), _stream(stream)))


def spec_verify_forward_trace(model: SpecModel, kv: KVCache, B: int, m: int, tokens, logits, trace: dict, ws,
                              stream=None):
    """trace: dict of device tensors by member name (h, q, attn, h_mid, mlp);
    missing members are not captured."""
    t = spec_trace(*[_ptr(trace.get(k)) for k in ("h", "q", "attn", "h_mid", "mlp")])
    _check(load_library().spec_verify_forward_trace(model.handle, ctypes.byref(kv.struct), B, m, _ptr(tokens),
                                                    _ptr(logits), ctypes.byref(t), _ptr(ws), _nbytes(ws),
                                                    _stream(stream)))


def spec_softmax_pq(logits, rows: int, vocab: int, temperature: float, probs, ws, stream=None):
    _check(load_library().spec_softmax_pq(_ptr(logits), rows, vocab, temperature, _ptr(probs), _ptr(ws),
                                          _nbytes(ws), _stream(stream)))


def spec_reject_sample(B: int, gamma: int, vocab: int, p, q, draft, n_draft, u_acc, u_res, n_accepted, emitted, ws,
                       stream=None):
    _check(load_library().spec_reject_sample(B, gamma, vocab, _ptr(p), _ptr(q), _ptr(draft), _ptr(n_draft),
                                             _ptr(u_acc), _ptr(u_res), _ptr(n_accepted), _ptr(emitted), _ptr(ws),
                                             _nbytes(ws), _stream(stream)))


def _strided_ptr(t, off: int, rows: int, ld: int, width: int) -> int:
    """Address of element `off` of a contiguous tensor whose rows
    off + r * ld .. + width - 1 (r < rows) the call will touch."""
    if not isinstance(t, torch.Tensor) or not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    if off < 0 or ld < width or off + (rows - 1) * ld + width > t.numel():
        raise ValueError(f"strided rows (offset {off}, {rows} x {ld}, width {width}) outside {t.numel()} elements")
    return t.data_ptr() + off * t.element_size()


def spec_draft_sample(logits, ld_logits: int, B: int, vocab: int, temperature: float, u, q, ld_q: int, tokens,
                      ld_tokens: int, ws, stream=None, logits_off: int = 0, q_off: int = 0, tokens_off: int = 0):
    """The drafter's sampling step over B rows strided through larger buffers:
    row b of the logits at logits_off + b * ld_logits, of q at
    q_off + b * ld_q, its token at tokens_off + b * ld_tokens (elements)."""
    _check(load_library().spec_draft_sample(_strided_ptr(logits, logits_off, B, ld_logits, vocab), ld_logits, B, vocab,
                                            temperature, _ptr(u), _strided_ptr(q, q_off, B, ld_q, vocab), ld_q,
                                            _strided_ptr(tokens, tokens_off, B, ld_tokens, 1), ld_tokens, _ptr(ws),
                                            _nbytes(ws), _stream(stream)))


def spec_decode_step(target: SpecModel, kv: KVCache, B: int, gamma: int, temperature: float, last_tok, draft, n_draft,
                     q, u_acc, u_res, n_accepted, emitted, logits_out, ws, stream=None):
    _check(load_library().spec_decode_step(target.handle, ctypes.byref(kv.struct), B, gamma, temperature,
                                           _ptr(last_tok), _ptr(draft), _ptr(n_draft), _ptr(q), _ptr(u_acc),
                                           _ptr(u_res), _ptr(n_accepted), _ptr(emitted), _ptr(logits_out), _ptr(ws),
                                           _nbytes(ws), _stream(stream)))


def spec_decode_step_static(target: SpecModel, kv: KVCache, B: int, gamma: int, temperature: float, last_tok, draft,
                            n_draft, q, u_acc, u_res, n_accepted, emitted, logits_out, stream=None):
    _check(load_library().spec_decode_step_static(target.handle, ctypes.byref(kv.struct), B, gamma, temperature,
                                                  _ptr(last_tok), _ptr(draft), _ptr(n_draft), _ptr(q), _ptr(u_acc),
                                                  _ptr(u_res), _ptr(n_accepted), _ptr(emitted), _ptr(logits_out),
                                                  _stream(stream)))


def spec_linear(W, x, M: int, N: int, K: int, epilogue: int = 0, y=None, z=None, hn=None, gain=None, eps: float = 1e-6,
                stream=None):
    """y / z from x, or (hn given) from RMSNorm(hn) * gain made while staging."""
    dt = SPEC_BF16 if W.dtype == torch.bfloat16 else SPEC_F32
    _check(load_library().spec_linear(dt, epilogue, _ptr(W), _ptr(x), M, N, K, _ptr(y), _ptr(z), _ptr(hn), _ptr(gain),
                                      eps, _stream(stream)))


def spec_commit_round(B: int, gamma: int, n_accepted, emitted, tok2, last, out_tokens, out_len, cap: int,
                      n_stop: int = 0, kv_len=None, n_rounds=None, n_log=None, log_cap: int = 0, stream=None):
    _check(load_library().spec_commit_round(B, gamma, _ptr(n_accepted), _ptr(emitted), _ptr(tok2), _ptr(last),
                                            _ptr(out_tokens), _ptr(out_len), cap, n_stop, _ptr(kv_len),
                                            _ptr(n_rounds), _ptr(n_log), log_cap, _stream(stream)))


def spec_ngram_propose(B: int, n_min: int, n_max: int, gamma: int, prefix, prefix_len, P: int, out, out_len,
                       cap: int, fill_off, drafts, n_draft, n_found=None, stream=None):
    _check(load_library().spec_ngram_propose(B, n_min, n_max, gamma, _ptr(prefix), _ptr(prefix_len), P, _ptr(out),
                                             _ptr(out_len), cap, _ptr(fill_off), _ptr(drafts), _ptr(n_draft),
                                             _ptr(n_found), _stream(stream)))


def spec_kv_set_len(kv: KVCache, B: int, src, add: int, stream=None):
    _check(load_library().spec_kv_set_len(ctypes.byref(kv.struct), B, _ptr(src), add, _stream(stream)))

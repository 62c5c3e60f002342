"""ctypes binding of libcpspec.so (include/cp_spec.h).

Argument marshalling only: torch supplies device memory and the HIP stream,
every step of the round runs in the library's HIP kernels.  Functions keep
the C names without the ``cp_spec_`` prefix.  If the library is not built the
first use raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcpspec.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "cp_spec.h")

OK, WARN_AR_FALLBACK = 0, 1
EINVAL, EUNSUPPORTED, EHIP, EWORKSPACE = -1, -2, -3, -4
F32, BF16 = 0, 1
FLAG_TOPK, FLAG_ARGMAX, FLAG_CDF, FLAG_ACCEPT = 1, 2, 4, 8
MAX_OFFSETS = 8
MAX_TREE = 63


class Cfg(C.Structure):
    _fields_ = [("layers", C.c_int32), ("hidden", C.c_int32),
                ("q_heads", C.c_int32), ("kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("code_groups", C.c_int32), ("vocab", C.c_int32),
                ("weight_dtype", C.c_int32), ("rope_theta", C.c_float),
                ("rms_eps", C.c_float), ("verify_size", C.c_int32),
                ("greedy", C.c_int32), ("temperature", C.c_float),
                ("top_k", C.c_int32), ("max_streams", C.c_int32),
                ("draft_offsets", C.c_int32), ("fused_draft", C.c_int32),
                ("tree_nodes", C.c_int32),
                ("tree_parent", C.c_int32 * MAX_TREE)]


class Weights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("heads", C.c_void_p),
                ("final_norm", C.c_void_p), ("layer", C.POINTER(C.c_void_p)),
                ("draft_offsets", C.c_void_p)]


class Stats(C.Structure):
    _fields_ = [("frames", C.c_int64), ("codes", C.c_int64),
                ("prefill_passes", C.c_int64), ("rounds", C.c_int64),
                ("proposed", C.c_int64 * MAX_OFFSETS),
                ("accepted", C.c_int64 * MAX_OFFSETS),
                ("bonus", C.c_int64), ("near_tie_accept", C.c_int64),
                ("near_tie_argmax", C.c_int64), ("near_tie_cdf", C.c_int64),
                ("near_tie_topk", C.c_int64)]

    def as_dict(self) -> dict:
        d = {}
        for name, _ in self._fields_:
            v = getattr(self, name)
            d[name] = list(v) if name in ("proposed", "accepted") else int(v)
        return d


STATS_WORDS = C.sizeof(Stats) // 8

KERNEL_KINDS = ("draft_heads", "qkv", "attention", "o_proj", "gate_up",
                "down", "target_heads")


class KernelTiming(C.Structure):
    _fields_ = [("avg_us", C.c_double), ("bytes_per_launch", C.c_double),
                ("flops_per_launch", C.c_double), ("launches", C.c_int32),
                ("rows", C.c_int32), ("matrix_cores", C.c_int32),
                ("reserved", C.c_int32)]

_P = C.c_void_p
_SIGS = {
    "cp_spec_workspace_bytes": (C.c_size_t, [C.POINTER(Cfg)]),
    "cp_spec_create": (C.c_int, [C.POINTER(Weights), C.POINTER(Cfg), _P,
                                 C.c_size_t, C.POINTER(_P)]),
    "cp_spec_destroy": (None, [_P]),
    "cp_spec_last_error": (C.c_char_p, []),
    "cp_spec_decode_frames": (C.c_int, [_P, _P, C.c_int32, C.c_int32, _P, _P,
                                        _P, _P, _P, _P]),
    "cp_spec_get_stats": (C.c_int, [_P, _P, C.POINTER(Stats)]),
    "cp_spec_head_logits": (C.c_int, [_P, _P, C.c_int32, _P, _P, C.c_int32,
                                      _P]),
    "cp_spec_topk_sample": (C.c_int, [_P, _P, C.c_int32, _P, _P, _P, _P, _P]),
    "cp_spec_talker_feedback": (C.c_int, [_P, _P, C.c_int32, _P, _P]),
    "cp_spec_accept": (C.c_int, [_P, _P, C.c_int32, C.c_int32, _P, _P, _P, _P,
                                 _P, _P, _P, _P, _P]),
    "cp_spec_accept_noalloc": (C.c_int, [_P, C.c_int32, C.c_int32, C.c_int32,
                                         C.c_int32, _P, _P, _P, _P, _P, _P,
                                         _P, _P, _P]),
    "cp_spec_walk_step": (C.c_int, [_P, _P, C.c_int32, C.c_int32, _P, _P,
                                    _P, _P, _P, _P, _P, _P, _P]),
    "cp_spec_decoder_forward": (C.c_int, [_P, _P, C.c_int32, C.c_int32, _P,
                                          _P, _P]),
    "cp_spec_time_kernel": (C.c_int, [_P, _P, C.c_int32, C.c_int32,
                                      C.c_int32, C.POINTER(KernelTiming)]),
}

_lib = None


def header_symbols() -> list[str]:
    """Every function the C header declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cp_spec_\w+)\s*\(", text)))


def lib():
    """Load libcpspec.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} missing: build it with "
                               "__graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class CpSpecError(RuntimeError):
    def __init__(self, rc, msg):
        super().__init__(f"cp_spec error {rc}: {msg}")
        self.rc = rc


def _check(rc):
    if rc < 0:
        raise CpSpecError(rc, lib().cp_spec_last_error().decode())
    return rc


def make_cfg(c: dict, max_streams: int | None = None) -> Cfg:
    """Cfg struct from a workload dictionary (see synth.config)."""
    return Cfg(layers=c["layers"], hidden=c["hidden"], q_heads=c["q_heads"],
               kv_heads=c["kv_heads"], head_dim=c["head_dim"], ffn=c["ffn"],
               code_groups=c["groups"], vocab=c["vocab"],
               weight_dtype=BF16 if c["dtype"] == "bf16" else F32,
               rope_theta=c["rope_theta"], rms_eps=c["rms_eps"],
               verify_size=c["verify_size"], greedy=int(bool(c["greedy"])),
               temperature=c["temperature"], top_k=c["top_k"],
               max_streams=max_streams or c["streams"],
               draft_offsets=int(c.get("draft_offsets", 0)),
               fused_draft=int(c.get("fused_draft", 0)),
               tree_nodes=len(c.get("tree") or ()),
               tree_parent=(C.c_int32 * MAX_TREE)(
                   *(list(c.get("tree") or ()) + [0] * MAX_TREE)[:MAX_TREE]))


def workspace_bytes(cfg: Cfg) -> int:
    return int(lib().cp_spec_workspace_bytes(C.byref(cfg)))


def last_error() -> str:
    return lib().cp_spec_last_error().decode()


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def weights_to_device(w: dict, device="cuda") -> dict:
    """Copy synth.make_weights() arrays to device tensors (bf16 bit patterns
    travel as int16)."""
    import torch

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(device)

    out = {"embed": dev(w["embed"]), "heads": dev(w["heads"]),
           "final_norm": dev(w["final_norm"]),
           "layers": [{k: dev(v) for k, v in lw.items()} for lw in w["layers"]]}
    if w.get("draft_offsets") is not None:
        out["draft_offsets"] = dev(np.asarray(w["draft_offsets"], np.float32))
    return out


LAYER_ORDER = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate",
               "w_up", "w_down")


class Handle:
    """cp_spec handle: device weights (borrowed) + a torch-allocated workspace."""

    def __init__(self, c: dict, wdev: dict, max_streams: int | None = None,
                 cfg_overrides: dict | None = None):
        import torch
        self.cfg = make_cfg(c, max_streams)
        for k, v in (cfg_overrides or {}).items():
            setattr(self.cfg, k, v)
        n = workspace_bytes(self.cfg)
        if n == 0:
            raise CpSpecError(-1, last_error())
        self.workspace = torch.empty(n, dtype=torch.uint8, device="cuda")
        self.wdev = wdev
        ptrs = []
        for lw in wdev["layers"]:
            ptrs += [lw[k].data_ptr() for k in LAYER_ORDER]
        self._layer_ptrs = (C.c_void_p * len(ptrs))(*ptrs)
        self.weights = Weights(wdev["embed"].data_ptr(),
                               wdev["heads"].data_ptr(),
                               wdev["final_norm"].data_ptr(),
                               C.cast(self._layer_ptrs, C.POINTER(C.c_void_p)),
                               wdev["draft_offsets"].data_ptr()
                               if wdev.get("draft_offsets") is not None else None)
        h = C.c_void_p()
        self.status = _check(lib().cp_spec_create(
            C.byref(self.weights), C.byref(self.cfg),
            C.c_void_p(self.workspace.data_ptr()), n, C.byref(h)))
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            lib().cp_spec_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def decode_frames(self, h_frame, c0, seeds, out_codes, out_flags=None,
                      stats=None, stream=None):
        F, B = int(c0.shape[0]), int(c0.shape[1])
        return _check(lib().cp_spec_decode_frames(
            self.h, _stream(stream), B, F, _ptr(h_frame), _ptr(c0),
            _ptr(seeds), _ptr(out_codes), _ptr(out_flags), _ptr(stats)))

    def head_logits(self, x, head, apply_final_norm, logits, stream=None):
        return _check(lib().cp_spec_head_logits(
            self.h, _stream(stream), int(x.shape[0]), _ptr(x), _ptr(head),
            int(apply_final_norm), _ptr(logits)))

    def topk_sample(self, logits, u=None, probs=None, codes=None, flags=None,
                    stream=None):
        return _check(lib().cp_spec_topk_sample(
            self.h, _stream(stream), int(logits.shape[0]), _ptr(logits),
            _ptr(u), _ptr(probs), _ptr(codes), _ptr(flags)))

    def talker_feedback(self, codes, out, stream=None):
        """codes [n][G] int32 -> out [n][H] float32 (sum of E_g[c_g])."""
        return _check(lib().cp_spec_talker_feedback(
            self.h, _stream(stream), int(codes.shape[0]), _ptr(codes), _ptr(out)))

    def accept(self, gamma, draft, q, p, u_accept, u_target, n_out, codes_out,
               flags_out=None, stream=None):
        B, W = int(draft.shape[0]), int(draft.shape[1])
        return _check(lib().cp_spec_accept(
            self.h, _stream(stream), B, W, _ptr(gamma), _ptr(draft), _ptr(q),
            _ptr(p), _ptr(u_accept), _ptr(u_target), _ptr(n_out),
            _ptr(codes_out), _ptr(flags_out)))

    def walk_step(self, p, q, n_children, children, u_accept, u_target,
                  accepted, codes, flags=None, stream=None):
        n, maxc = int(children.shape[0]), int(children.shape[1])
        return _check(lib().cp_spec_walk_step(
            self.h, _stream(stream), n, maxc, _ptr(p), _ptr(q),
            _ptr(n_children), _ptr(children), _ptr(u_accept), _ptr(u_target),
            _ptr(accepted), _ptr(codes), _ptr(flags)))

    def time_kernel(self, kind: str, n_streams: int, iters: int,
                    stream=None) -> dict:
        out = KernelTiming()
        _check(lib().cp_spec_time_kernel(
            self.h, _stream(stream), n_streams, KERNEL_KINDS.index(kind),
            iters, C.byref(out)))
        return {"kind": kind, "avg_us": out.avg_us,
                "bytes_per_launch": out.bytes_per_launch,
                "flops_per_launch": out.flops_per_launch,
                "launches": out.launches, "rows": out.rows,
                "matrix_cores": bool(out.matrix_cores)}

    def decoder_forward(self, x, pos, kv, stream=None):
        B, R = int(pos.shape[0]), int(pos.shape[1])
        return _check(lib().cp_spec_decoder_forward(
            self.h, _stream(stream), B, R, _ptr(x), _ptr(pos), _ptr(kv)))


def accept_noalloc(vocab, greedy, gamma, draft, q, p, u_accept, u_target,
                   n_out, codes_out, flags_out=None, stream=None):
    """cp_spec_accept_noalloc: the accept step without a handle, its scratch
    in the library's static per-GPU array."""
    B, W = int(draft.shape[0]), int(draft.shape[1])
    return _check(lib().cp_spec_accept_noalloc(
        _stream(stream), int(vocab), int(bool(greedy)), B, W, _ptr(gamma),
        _ptr(draft), _ptr(q), _ptr(p), _ptr(u_accept), _ptr(u_target),
        _ptr(n_out), _ptr(codes_out), _ptr(flags_out)))


def get_stats(stats_tensor, stream=None) -> dict:
    out = Stats()
    _check(lib().cp_spec_get_stats(_ptr(stats_tensor), _stream(stream),
                                   C.byref(out)))
    return out.as_dict()


def new_stats_tensor():
    import torch
    return torch.zeros(STATS_WORDS, dtype=torch.int64, device="cuda")

"""Python binding of ``libsk.so`` (include/sk.h), argument marshalling only.

Every function takes torch tensors that live on the GPU, checks dtype,
device, contiguity and size, and calls the C entry point of the same name on
torch's current stream.  All computation happens in the HIP kernels; nothing
here falls back to the CPU.  A non-OK status raises :class:`SkError` with the
library's message.
"""

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsk.so")

SK_OK, SK_E_ARG, SK_E_UNSUPPORTED, SK_E_BUDGET, SK_E_WORKSPACE, SK_E_DEVICE = range(6)
TIER_FP16, TIER_INT8, TIER_INT4, TIER_DROP = 0, 1, 2, 3
OVERFLOW_REJECT, OVERFLOW_DROP, OVERFLOW_FALLBACK = 0, 1, 2

EXPORTS = [
    "sk_plan_make", "sk_score_workspace_bytes", "sk_score", "sk_score_rowlse",
    "sk_score_colsum_workspace_bytes", "sk_score_colsum", "sk_assign_workspace_bytes",
    "sk_assign_tiers", "sk_pack", "sk_unpack", "sk_status_string", "sk_last_error",
    "sk_layout_version", "sk_recency_weight", "sk_score_kvnorm", "sk_upgrade_bytes",
    "sk_upgrade_pack", "sk_upgrade_unpack", "sk_balanced_keys", "sk_decode_workspace_bytes",
    "sk_decode_attention", "sk_score_noalloc", "sk_score_layers_workspace_bytes",
    "sk_score_layers", "sk_score_rowlse_layers", "sk_score_colsum_layers_workspace_bytes",
    "sk_score_colsum_layers",
]

SCORE_SCRATCH_BYTES = 32 << 20   # SK_SCORE_SCRATCH_BYTES


class SkError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} [status {status}]")
        self.status = status


class _Shape(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class _Policy(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("n_sink", ctypes.c_int32),
                ("three_tier", ctypes.c_int32), ("budget", ctypes.c_double),
                ("overflow", ctypes.c_int32)]


class _Plan(ctypes.Structure):
    _fields_ = [("n16", ctypes.c_int64), ("n8", ctypes.c_int64), ("n4", ctypes.c_int64),
                ("n_drop", ctypes.c_int64), ("n_sink", ctypes.c_int64), ("budget_units", ctypes.c_int64),
                ("used_units", ctypes.c_int64), ("payload_bytes", ctypes.c_int64),
                ("off_c16", ctypes.c_int64), ("off_c8", ctypes.c_int64),
                ("off_c4", ctypes.c_int64), ("off_s8", ctypes.c_int64),
                ("off_s4", ctypes.c_int64), ("n_tokens", ctypes.c_int64),
                ("n_layers", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("layout_version", ctypes.c_int32),
                ("check", ctypes.c_uint64)]


class _Paged(ctypes.Structure):
    _fields_ = [("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("block_size", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64)]


@dataclass(frozen=True)
class Shape:
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int

    def c(self):
        return _Shape(self.n_layers, self.n_q_heads, self.n_kv_heads, self.head_dim)


@dataclass(frozen=True)
class Policy:
    n_tokens: int
    n_sink: int
    three_tier: int
    budget: float
    overflow: int = OVERFLOW_REJECT

    def c(self):
        return _Policy(self.n_tokens, self.n_sink, self.three_tier, float(self.budget),
                       self.overflow)


_lib = None


def lib():
    """Load libsk.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m serving_sk_score_amd.build`")
        _lib = bind(LIB_PATH)
    return _lib


def bind(path):
    """Load a build of the C ABI at `path` and declare the signatures of its
    entry points (lib() binds the in-tree libsk.so this way)."""
    L = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "sk_plan_make": (i32, [P(_Shape), P(_Policy), P(_Plan)]),
        "sk_score_workspace_bytes": (sz, [P(_Shape), i64]),
        "sk_score": (i32, [P(_Shape), i64, vp, vp, vp, i32, vp, sz, vp]),
        "sk_score_noalloc": (i32, [P(_Shape), i64, vp, vp, vp, i32, vp]),
        "sk_score_rowlse": (i32, [P(_Shape), i64, vp, vp, vp, vp]),
        "sk_score_colsum_workspace_bytes": (sz, [P(_Shape), i64]),
        "sk_score_colsum": (i32, [P(_Shape), i64, vp, vp, vp, vp, i32, vp, sz, vp]),
        "sk_score_layers_workspace_bytes": (sz, [P(_Shape), i64]),
        "sk_score_layers": (i32, [P(_Shape), i64, vp, vp, vp, i32, vp, sz, vp]),
        "sk_score_rowlse_layers": (i32, [P(_Shape), i64, vp, vp, vp, vp]),
        "sk_score_colsum_layers_workspace_bytes": (sz, [P(_Shape), i64]),
        "sk_score_colsum_layers": (i32, [P(_Shape), i64, vp, vp, vp, vp, i32, vp, sz, vp]),
        "sk_assign_workspace_bytes": (sz, [i64]),
        "sk_assign_tiers": (i32, [P(_Policy), P(_Plan), vp, vp, vp, vp, sz, vp]),
        "sk_pack": (i32, [P(_Shape), P(_Plan), vp, vp, vp, vp, vp, vp]),
        "sk_unpack": (i32, [P(_Shape), P(_Plan), vp, vp, vp, vp, P(_Paged), vp]),
        "sk_status_string": (ctypes.c_char_p, [i32]),
        "sk_last_error": (ctypes.c_char_p, []),
        "sk_layout_version": (i32, []),
        "sk_recency_weight": (i32, [i64, ctypes.c_double, vp, vp, vp]),
        "sk_score_kvnorm": (i32, [P(_Shape), i64, vp, vp, i32, vp]),
        "sk_upgrade_bytes": (sz, [P(_Shape), i64]),
        "sk_balanced_keys": (i32, [i64, i32, vp, vp]),
        "sk_decode_workspace_bytes": (sz, [P(_Shape), P(_Plan), i32]),
        "sk_decode_attention": (i32, [P(_Shape), P(_Plan), vp, i32, i32, vp, vp, vp, vp, sz,
                                      vp]),
        "sk_upgrade_pack": (i32, [P(_Shape), i64, vp, vp, vp, i64, vp, vp]),
        "sk_upgrade_unpack": (i32, [P(_Shape), i64, vp, vp, i64, vp, vp, P(_Paged), vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


def _check(status):
    if status != SK_OK:
        msg = lib().sk_last_error().decode() or lib().sk_status_string(status).decode()
        raise SkError(status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, dtype, numel=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} needs at least {numel} elements (got {t.numel()})")


class Plan:
    """Tier counts and payload layout (see sk_plan in include/sk.h)."""

    def __init__(self, c_plan):
        self._c = c_plan
        for f, _ in _Plan._fields_:
            setattr(self, f, getattr(c_plan, f))

    @property
    def c(self):
        return self._c

    def counts(self):
        return self.n16, self.n8, self.n4


def plan_make(shape: Shape, policy: Policy) -> Plan:
    out = _Plan()
    _check(lib().sk_plan_make(ctypes.byref(shape.c()), ctypes.byref(policy.c()),
                              ctypes.byref(out)))
    return Plan(out)


def score_workspace_bytes(shape: Shape, n: int) -> int:
    return int(lib().sk_score_workspace_bytes(ctypes.byref(shape.c()), n))


def colsum_workspace_bytes(shape: Shape, n: int) -> int:
    return int(lib().sk_score_colsum_workspace_bytes(ctypes.byref(shape.c()), n))


def _qk(shape, q, k):
    n = q.shape[0] if q.dim() == 3 else -1
    _need(q, "q", torch.float16, shape=(n, shape.n_q_heads, shape.head_dim))
    _need(k, "k", torch.float16, shape=(n, shape.n_kv_heads, shape.head_dim))
    return n


def score(shape: Shape, q, k, out, accumulate=False, ws=None):
    """One layer's column sums into out (fp32 [n]); ws: uint8 workspace."""
    n = _qk(shape, q, k)
    _need(out, "score", torch.float32, shape=(n,))
    need = score_workspace_bytes(shape, n)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    _need(ws, "ws", torch.uint8, numel=need)
    _check(lib().sk_score(ctypes.byref(shape.c()), n, _ptr(q), _ptr(k), _ptr(out),
                          int(bool(accumulate)), _ptr(ws), ws.numel(), _stream(q)))
    return out


def score_noalloc(shape: Shape, q, k, out, accumulate=False):
    """sk_score without a workspace (the library's static scratch is used)."""
    n = _qk(shape, q, k)
    _need(out, "score", torch.float32, shape=(n,))
    _check(lib().sk_score_noalloc(ctypes.byref(shape.c()), n, _ptr(q), _ptr(k), _ptr(out),
                                  int(bool(accumulate)), _stream(q)))
    return out


def score_rowlse(shape: Shape, q, k, lse):
    n = _qk(shape, q, k)
    _need(lse, "lse", torch.float32, shape=(shape.n_q_heads, n))
    _check(lib().sk_score_rowlse(ctypes.byref(shape.c()), n, _ptr(q), _ptr(k), _ptr(lse),
                                 _stream(q)))
    return lse


def score_colsum(shape: Shape, q, k, lse, out, accumulate=False, ws=None):
    n = _qk(shape, q, k)
    _need(lse, "lse", torch.float32, shape=(shape.n_q_heads, n))
    _need(out, "score", torch.float32, shape=(n,))
    need = colsum_workspace_bytes(shape, n)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(ws, "ws", torch.uint8, numel=need)
    _check(lib().sk_score_colsum(ctypes.byref(shape.c()), n, _ptr(q), _ptr(k), _ptr(lse),
                                 _ptr(out), int(bool(accumulate)), _ptr(ws), ws.numel(),
                                 _stream(q)))
    return out


def score_layers_workspace_bytes(shape: Shape, n: int) -> int:
    return int(lib().sk_score_layers_workspace_bytes(ctypes.byref(shape.c()), n))


def colsum_layers_workspace_bytes(shape: Shape, n: int) -> int:
    return int(lib().sk_score_colsum_layers_workspace_bytes(ctypes.byref(shape.c()), n))


def _qk_layers(shape, q, k):
    n = q.shape[1] if q.dim() == 4 else -1
    L = shape.n_layers
    _need(q, "q", torch.float16, shape=(L, n, shape.n_q_heads, shape.head_dim))
    _need(k, "k", torch.float16, shape=(L, n, shape.n_kv_heads, shape.head_dim))
    return n


def score_layers(shape: Shape, q, k, out, accumulate=False, ws=None):
    """Every layer's column sums into out (fp32 [n]) with one launch per pass;
    q fp16 [L][n][Hq][d], k fp16 [L][n][Hkv][d]."""
    n = _qk_layers(shape, q, k)
    _need(out, "score", torch.float32, shape=(n,))
    need = score_layers_workspace_bytes(shape, n)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(ws, "ws", torch.uint8, numel=need)
    _check(lib().sk_score_layers(ctypes.byref(shape.c()), n, _ptr(q), _ptr(k), _ptr(out),
                                 int(bool(accumulate)), _ptr(ws), ws.numel(), _stream(q)))
    return out


def score_rowlse_layers(shape: Shape, q, k, lse):
    """lse fp32 [L][Hq][n] of every layer, one launch."""
    n = _qk_layers(shape, q, k)
    _need(lse, "lse", torch.float32, shape=(shape.n_layers, shape.n_q_heads, n))
    _check(lib().sk_score_rowlse_layers(ctypes.byref(shape.c()), n, _ptr(q), _ptr(k),
                                        _ptr(lse), _stream(q)))
    return lse


def score_colsum_layers(shape: Shape, q, k, lse, out, accumulate=False, ws=None):
    n = _qk_layers(shape, q, k)
    _need(lse, "lse", torch.float32, shape=(shape.n_layers, shape.n_q_heads, n))
    _need(out, "score", torch.float32, shape=(n,))
    need = colsum_layers_workspace_bytes(shape, n)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(ws, "ws", torch.uint8, numel=need)
    _check(lib().sk_score_colsum_layers(ctypes.byref(shape.c()), n, _ptr(q), _ptr(k),
                                        _ptr(lse), _ptr(out), int(bool(accumulate)), _ptr(ws),
                                        ws.numel(), _stream(q)))
    return out


def recency_weight(score_in, lam, out=None):
    """out[j] = score_in[j] * exp(-lam * (n - 1 - j)); out may be score_in."""
    n = score_in.shape[0] if score_in.dim() == 1 else -1
    _need(score_in, "score_in", torch.float32, shape=(n,))
    if out is None:
        out = torch.empty_like(score_in)
    _need(out, "score_out", torch.float32, shape=(n,))
    _check(lib().sk_recency_weight(n, float(lam), _ptr(score_in), _ptr(out), _stream(score_in)))
    return out


def score_kvnorm(shape: Shape, k, out, accumulate=False):
    """KV-norm fallback score of k (fp16 [L][n][H_kv][d]) into out (fp32 [n])."""
    n = k.shape[1] if k.dim() == 4 else -1
    _need(k, "k", torch.float16, shape=_kv_shape(shape, n))
    _need(out, "score", torch.float32, shape=(n,))
    _check(lib().sk_score_kvnorm(ctypes.byref(shape.c()), n, _ptr(k), _ptr(out),
                                 int(bool(accumulate)), _stream(k)))
    return out


def balanced_keys(n: int, n_sink: int, keys):
    """Ranking keys of the Balanced variant into keys (fp32 [n])."""
    _need(keys, "keys", torch.float32, shape=(n,))
    _check(lib().sk_balanced_keys(n, n_sink, _ptr(keys), _stream(keys)))
    return keys


def assign_tiers(policy: Policy, plan: Plan, score_t, amap, order, ws=None):
    n = policy.n_tokens
    _need(score_t, "score", torch.float32, shape=(n,))
    _need(amap, "map", torch.int32, shape=(n,))
    _need(order, "order", torch.int32, shape=(n,))
    need = int(lib().sk_assign_workspace_bytes(n))
    if ws is None and need:
        ws = torch.empty(need, dtype=torch.uint8, device=score_t.device)
    _check(lib().sk_assign_tiers(ctypes.byref(policy.c()), ctypes.byref(plan.c),
                                 _ptr(score_t), _ptr(amap), _ptr(order), _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream(score_t)))
    return amap, order


def _kv_shape(shape, n):
    return (shape.n_layers, n, shape.n_kv_heads, shape.head_dim)


def pack(shape: Shape, plan: Plan, k, v, amap, order, payload):
    n = plan.n_tokens
    _need(k, "k", torch.float16, shape=_kv_shape(shape, n))
    _need(v, "v", torch.float16, shape=_kv_shape(shape, n))
    _need(amap, "map", torch.int32, shape=(n,))
    if order is not None:
        _need(order, "order", torch.int32, shape=(n,))
    _need(payload, "payload", torch.uint8, numel=plan.payload_bytes)
    _check(lib().sk_pack(ctypes.byref(shape.c()), ctypes.byref(plan.c), _ptr(k), _ptr(v),
                         _ptr(amap), _ptr(order), _ptr(payload), _stream(k)))
    return payload


def unpack(shape: Shape, plan: Plan, payload, amap, k_out, v_out):
    n = plan.n_tokens
    _need(payload, "payload", torch.uint8, numel=plan.payload_bytes)
    _need(amap, "map", torch.int32, shape=(n,))
    _need(k_out, "k_out", torch.float16, shape=_kv_shape(shape, n))
    _need(v_out, "v_out", torch.float16, shape=_kv_shape(shape, n))
    _check(lib().sk_unpack(ctypes.byref(shape.c()), ctypes.byref(plan.c), _ptr(payload),
                           _ptr(amap), _ptr(k_out), _ptr(v_out), None, _stream(payload)))
    return k_out, v_out


def unpack_paged(shape: Shape, plan: Plan, payload, amap, k_cache, v_cache, block_table,
                 block_size=16):
    n = plan.n_tokens
    _need(payload, "payload", torch.uint8, numel=plan.payload_bytes)
    _need(amap, "map", torch.int32, shape=(n,))
    nb = k_cache.shape[1] if k_cache.dim() == 5 else -1
    cshape = (shape.n_layers, nb, block_size, shape.n_kv_heads, shape.head_dim)
    _need(k_cache, "k_cache", torch.float16, shape=cshape)
    _need(v_cache, "v_cache", torch.float16, shape=cshape)
    _need(block_table, "block_table", torch.int32, numel=(n + block_size - 1) // block_size)
    pg = _Paged(k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(), block_size, nb)
    _check(lib().sk_unpack(ctypes.byref(shape.c()), ctypes.byref(plan.c), _ptr(payload),
                           _ptr(amap), None, None, ctypes.byref(pg), _stream(payload)))
    return k_cache, v_cache


def upgrade_bytes(shape: Shape, n_up: int) -> int:
    return int(lib().sk_upgrade_bytes(ctypes.byref(shape.c()), n_up))


def _tokens(tokens):
    m = tokens.shape[0] if tokens.dim() == 1 else -1
    _need(tokens, "tokens", torch.int32, shape=(m,))
    return m


def upgrade_pack(shape: Shape, k, v, tokens, payload):
    """fp16 rows of the listed tokens (int32 [m], u32 bit patterns) into payload."""
    n = k.shape[1] if k.dim() == 4 else -1
    _need(k, "k", torch.float16, shape=_kv_shape(shape, n))
    _need(v, "v", torch.float16, shape=_kv_shape(shape, n))
    m = _tokens(tokens)
    _need(payload, "payload", torch.uint8, numel=upgrade_bytes(shape, m))
    _check(lib().sk_upgrade_pack(ctypes.byref(shape.c()), n, _ptr(k), _ptr(v), _ptr(tokens), m,
                                 _ptr(payload), _stream(k)))
    return payload


def upgrade_unpack(shape: Shape, n: int, payload, tokens, k_out, v_out):
    m = _tokens(tokens)
    _need(payload, "payload", torch.uint8, numel=upgrade_bytes(shape, m))
    _need(k_out, "k_out", torch.float16, shape=_kv_shape(shape, n))
    _need(v_out, "v_out", torch.float16, shape=_kv_shape(shape, n))
    _check(lib().sk_upgrade_unpack(ctypes.byref(shape.c()), n, _ptr(payload), _ptr(tokens), m,
                                   _ptr(k_out), _ptr(v_out), None, _stream(payload)))
    return k_out, v_out


def upgrade_unpack_paged(shape: Shape, n: int, payload, tokens, k_cache, v_cache, block_table,
                         block_size=16):
    m = _tokens(tokens)
    _need(payload, "payload", torch.uint8, numel=upgrade_bytes(shape, m))
    nb = k_cache.shape[1] if k_cache.dim() == 5 else -1
    cshape = (shape.n_layers, nb, block_size, shape.n_kv_heads, shape.head_dim)
    _need(k_cache, "k_cache", torch.float16, shape=cshape)
    _need(v_cache, "v_cache", torch.float16, shape=cshape)
    _need(block_table, "block_table", torch.int32, numel=(n + block_size - 1) // block_size)
    pg = _Paged(k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(), block_size, nb)
    _check(lib().sk_upgrade_unpack(ctypes.byref(shape.c()), n, _ptr(payload), _ptr(tokens), m,
                                   None, None, ctypes.byref(pg), _stream(payload)))
    return k_cache, v_cache


def decode_workspace_bytes(shape: Shape, plan: Plan, n_layers_q: int) -> int:
    return int(lib().sk_decode_workspace_bytes(ctypes.byref(shape.c()), ctypes.byref(plan.c),
                                               n_layers_q))


def decode_attention(shape: Shape, plan: Plan, payload, q, out, lse=None, layer0=0, ws=None):
    """Attention of q (fp16 [nl][H_q][d], layers layer0..layer0+nl-1) over the
    sent tokens, read straight from the payload; out fp32 [nl][H_q][d], lse
    fp32 [nl][H_q] (natural log) or None."""
    nl = q.shape[0] if q.dim() == 3 else -1
    _need(q, "q", torch.float16, shape=(nl, shape.n_q_heads, shape.head_dim))
    _need(out, "out", torch.float32, shape=(nl, shape.n_q_heads, shape.head_dim))
    if lse is not None:
        _need(lse, "lse", torch.float32, shape=(nl, shape.n_q_heads))
    _need(payload, "payload", torch.uint8, numel=plan.payload_bytes)
    need = decode_workspace_bytes(shape, plan, nl)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(ws, "ws", torch.uint8, numel=need)
    _check(lib().sk_decode_attention(ctypes.byref(shape.c()), ctypes.byref(plan.c), _ptr(payload),
                                     layer0, nl, _ptr(q), _ptr(out), _ptr(lse), _ptr(ws),
                                     ws.numel(), _stream(q)))
    return out

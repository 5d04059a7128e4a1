"""Python binding of libw4v (W4A16 speculative-verify kernels for gfx950).

Argument marshalling only: every step of the path runs in the HIP library.
PyTorch supplies device memory and the current stream.  The binding raises
``W4VError`` on a non-zero status and ``RuntimeError`` when the library has
not been built -- there is no fallback implementation.

The calls follow the organisers' page "Efficient LLM Challenge Results",
section 3 (W4A16 group-128 target, 8-bit lm_head, greedy verification of K
drafts padded with -1 sentinels); the C declarations are in include/w4v.h.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4v.so")

_lib = None

W4V_OK = 0
W4V_ERR_INVALID_ARG = -1
W4V_ERR_UNSUPPORTED = -2
W4V_ERR_ALIGNMENT = -3
W4V_ERR_WORKSPACE = -4
W4V_ERR_HIP = -5

GROUP_SIZE = 128

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/w4v.h
SIGNATURES = {
    "w4v_status_string": (ctypes.c_char_p, [_int]),
    "w4v_abi_version": (_int, []),
    "w4v_read_probe_blocks": (_int, []),
    "w4v_read_probe": (_int, [_vp, _sz, _vp, _vp]),
    "w4a16_gemm_workspace_size": (_sz, [_int, _int, _int, _int]),
    "w4a16_gemm": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _i64, _int, _int, _int, _int,
                          ctypes.c_float, _vp, _sz, _vp]),
    "w4a16_gemm_noalloc": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _i64, _int, _int, _int, _int,
                                  ctypes.c_float, _vp]),
    "w8a16_lmhead_argmax_workspace_size": (_sz, [_int, _int, _int]),
    "w8a16_lmhead_argmax": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _int, _int, _int, _vp, _sz,
                                   _vp]),
    "greedy_verify": (_int, [_vp, _vp, _int, _int, _int, _vp, _vp, _vp]),
    "ngram_draft": (_int, [_vp, _i64, _vp, _int, _int, _int, _int, _vp, _vp]),
    "append_accepted": (_int, [_vp, _i64, _vp, _int, _int, _vp, _vp, _vp]),
    "w8a16_lmhead_argmax_verify": (_int, [_vp, _i64, _vp, _vp, _vp, _vp, _int, _int, _vp, _int,
                                          _int, _vp, _vp, _vp, _sz, _vp]),
    "f16_lmhead_argmax_workspace_size": (_sz, [_int, _int, _int]),
    "f16_lmhead_argmax_verify": (_int, [_vp, _i64, _vp, _vp, _vp, _int, _int, _int, _vp, _int,
                                        _int, _vp, _vp, _vp, _sz, _vp]),
    "gdn_state_commit": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _vp]),
    "f16_gemm_workspace_size": (_sz, [_int, _int, _int]),
    "f16_gemm": (_int, [_vp, _i64, _vp, _i64, _vp, _i64, _int, _int, _int, ctypes.c_float, _vp,
                        _sz, _vp]),
}


class ChainLinearDesc(ctypes.Structure):
    """Mirror of w4v_chain_linear (include/w4v.h)."""
    _fields_ = [("qweight", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("qzeros", ctypes.c_void_p), ("K", ctypes.c_int), ("N", ctypes.c_int),
                ("alpha", ctypes.c_float)]


SIGNATURES.update({
    "w4a16_chain_workspace_size": (_sz, [_vp, _int, _int]),
    "w4a16_chain_prepare": (_int, [_vp, _int, _int, _vp, _sz]),
    "w4a16_chain": (_int, [_vp, _i64, _vp, _i64, _int, _int, _int, _vp, _vp]),
})

CHAIN_ERROR_OFFSET = 28      # byte offset of the chain workspace's error word


class W4VError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load(path: str | None = None):
    """Load libw4v.so (once).  Raises RuntimeError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(hipcc, gfx950); there is no fallback path")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().w4v_status_string(status).decode()


def abi_version() -> int:
    return load().w4v_abi_version()


def _check(status: int, where: str):
    if status != W4V_OK:
        raise W4VError(status, where)


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _require(t, dtype, name):
    import torch
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() >= 1 and t.numel() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride in its last dimension")
    return torch


# ------------------------------------------------------------------- workspaces
def gemm_workspace_size(m: int, n: int, k: int, group_size: int = GROUP_SIZE) -> int:
    return int(load().w4a16_gemm_workspace_size(m, n, k, group_size))


def lmhead_workspace_size(m: int, h: int, v: int) -> int:
    return int(load().w8a16_lmhead_argmax_workspace_size(m, h, v))


def new_workspace(nbytes: int, device="cuda"):
    """Zeroed device workspace (uint8) of at least ``nbytes`` bytes, 256-byte aligned."""
    import torch
    t = torch.zeros(max(int(nbytes), 1) + 256, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % 256
    return t[off:off + max(int(nbytes), 1)]


# ------------------------------------------------------------------- calls
def w4a16_gemm(x, qweight, scales, qzeros, alpha: float = 1.0, out=None, workspace=None,
               group_size: int = GROUP_SIZE, stream=None, no_workspace: bool = False):
    """y[M, N] = fp16(alpha * x[:, :K] @ dequant(qweight, scales, qzeros)).

    x: fp16 [M, >=K] (a column slice of a wider tensor is fine: its row stride
    is passed as ldx); qweight: int32 [K/8, N]; scales: fp16 [K/g, N];
    qzeros: int32 [K/g, N/8] with g = group_size (128 or 32).  ``out`` may be a
    row-strided fp16 [M, N] view.  ``no_workspace`` passes none at all (a shape
    whose plan needs a workspace then fails with W4V_ERR_WORKSPACE).
    """
    torch = _require(x, __import__("torch").float16, "x")
    _require(qweight, torch.int32, "qweight")
    _require(scales, torch.float16, "scales")
    _require(qzeros, torch.int32, "qzeros")
    k = qweight.shape[0] * 8
    n = qweight.shape[1]
    m = x.shape[0]
    if x.shape[1] < k:
        raise ValueError(f"x has {x.shape[1]} columns, the weights need {k}")
    if group_size > 0 and k % group_size == 0 and (
            tuple(scales.shape) != (k // group_size, n) or tuple(qzeros.shape) != (k // group_size, n // 8)):
        raise ValueError(f"scales {tuple(scales.shape)} / qzeros {tuple(qzeros.shape)} do not fit "
                         f"K={k}, N={n} at group size {group_size}")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float16, device=x.device)
    _require(out, torch.float16, "out")
    need = gemm_workspace_size(m, n, k, group_size)
    if no_workspace:
        workspace = None
    elif workspace is None and need > 0:
        workspace = new_workspace(need, x.device)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().w4a16_gemm(_ptr(x), x.stride(0), _ptr(qweight), _ptr(scales), _ptr(qzeros),
                           _ptr(out), out.stride(0), m, n, k, group_size, ctypes.c_float(alpha),
                           _ptr(workspace), wbytes, _stream(stream))
    _check(st, "w4a16_gemm")
    return out


STATIC_SCRATCH_BYTES = 32 << 20     # W4V_STATIC_SCRATCH_BYTES


def w4a16_gemm_noalloc(x, qweight, scales, qzeros, alpha: float = 1.0, out=None,
                       group_size: int = GROUP_SIZE, stream=None):
    """w4a16_gemm without a workspace: the library's per-GPU static scratch
    holds the plan's split-K state.  ``out`` must be given when the caller
    cannot allocate (otherwise one fp16 [M, N] tensor is allocated here).
    Shapes needing more than STATIC_SCRATCH_BYTES raise W4VError."""
    torch = _require(x, __import__("torch").float16, "x")
    _require(qweight, torch.int32, "qweight")
    _require(scales, torch.float16, "scales")
    _require(qzeros, torch.int32, "qzeros")
    k = qweight.shape[0] * 8
    n = qweight.shape[1]
    m = x.shape[0]
    if x.shape[1] < k:
        raise ValueError(f"x has {x.shape[1]} columns, the weights need {k}")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float16, device=x.device)
    _require(out, torch.float16, "out")
    st = load().w4a16_gemm_noalloc(_ptr(x), x.stride(0), _ptr(qweight), _ptr(scales),
                                   _ptr(qzeros), _ptr(out), out.stride(0), m, n, k, group_size,
                                   ctypes.c_float(alpha), _stream(stream))
    _check(st, "w4a16_gemm_noalloc")
    return out


def w8a16_lmhead_argmax(h, w, scales, target_ids=None, max_logits=None, want_max=True,
                        workspace=None, stream=None):
    """(target_ids int32 [M], max_logits fp32 [M] or None) for h fp16 [M, H], w int8 [V, H]."""
    torch = _require(h, __import__("torch").float16, "h")
    _require(w, torch.int8, "w")
    _require(scales, torch.float16, "scales")
    m, hdim = h.shape[0], w.shape[1]
    v = w.shape[0]
    if target_ids is None:
        target_ids = torch.empty(m, dtype=torch.int32, device=h.device)
    if want_max and max_logits is None:
        max_logits = torch.empty(m, dtype=torch.float32, device=h.device)
    need = lmhead_workspace_size(m, hdim, v)
    if workspace is None and need > 0:
        workspace = new_workspace(need, h.device)
    wbytes = workspace.numel() if workspace is not None else 0
    st = load().w8a16_lmhead_argmax(_ptr(h), h.stride(0), _ptr(w), _ptr(scales),
                                    _ptr(target_ids), _ptr(max_logits), m, hdim, v,
                                    _ptr(workspace), wbytes, _stream(stream))
    _check(st, "w8a16_lmhead_argmax")
    return target_ids, max_logits


def read_probe(src, out=None, stream=None):
    """Read every byte of the device tensor src once (the HBM read-bandwidth probe);
    returns out, int32 [w4v_read_probe_blocks()], one XOR word per block."""
    import torch
    if src.device.type != "cuda" or not src.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    nb = load().w4v_read_probe_blocks()
    if out is None:
        out = torch.empty(nb, dtype=torch.int32, device=src.device)
    st = load().w4v_read_probe(_ptr(src), src.numel() * src.element_size(), _ptr(out),
                               _stream(stream))
    _check(st, "w4v_read_probe")
    return out


def greedy_verify(target_ids, draft_ids, vocab: int, accepted_len=None, out_tokens=None,
                  stream=None):
    """(accepted_len int32 [B], out_tokens int32 [B, K+1]) from target_ids [B, K+1], drafts [B, K]."""
    torch = _require(target_ids, __import__("torch").int32, "target_ids")
    b, k1 = target_ids.shape
    k = k1 - 1
    _require(draft_ids, torch.int32, "draft_ids")
    if tuple(draft_ids.shape) != (b, k):
        raise ValueError(f"draft_ids must be [{b}, {k}], got {tuple(draft_ids.shape)}")
    if not (target_ids.is_contiguous() and draft_ids.is_contiguous()):
        raise ValueError("target_ids and draft_ids must be contiguous")
    if accepted_len is None:
        accepted_len = torch.empty(b, dtype=torch.int32, device=target_ids.device)
    if out_tokens is None:
        out_tokens = torch.empty((b, k1), dtype=torch.int32, device=target_ids.device)
    st = load().greedy_verify(_ptr(target_ids), _ptr(draft_ids) if k > 0 else None, b, k, vocab,
                              _ptr(accepted_len), _ptr(out_tokens), _stream(stream))
    _check(st, "greedy_verify")
    return accepted_len, out_tokens


def w8a16_lmhead_argmax_verify(h, w, scales, draft_ids, target_ids=None, max_logits=None,
                               accepted_len=None, out_tokens=None, want_max=True,
                               workspace=None, stream=None):
    """lm_head + argmax + greedy verify in one launch; h has B*(K+1) rows.

    Returns (target_ids [B*(K+1)], max_logits or None, accepted_len [B], out_tokens [B, K+1]).
    """
    torch = _require(h, __import__("torch").float16, "h")
    _require(w, torch.int8, "w")
    _require(scales, torch.float16, "scales")
    _require(draft_ids, torch.int32, "draft_ids")
    b, k = draft_ids.shape
    m = b * (k + 1)
    if h.shape[0] != m:
        raise ValueError(f"h has {h.shape[0]} rows, B*(K+1) = {m}")
    if not draft_ids.is_contiguous():
        raise ValueError("draft_ids must be contiguous")
    hdim, v = w.shape[1], w.shape[0]
    dev = h.device
    if target_ids is None:
        target_ids = torch.empty(m, dtype=torch.int32, device=dev)
    if want_max and max_logits is None:
        max_logits = torch.empty(m, dtype=torch.float32, device=dev)
    if accepted_len is None:
        accepted_len = torch.empty(b, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((b, k + 1), dtype=torch.int32, device=dev)
    need = lmhead_workspace_size(m, hdim, v)
    if workspace is None and need > 0:
        workspace = new_workspace(need, dev)
    wbytes = workspace.numel() if workspace is not None else 0
    st = load().w8a16_lmhead_argmax_verify(
        _ptr(h), h.stride(0), _ptr(w), _ptr(scales), _ptr(target_ids), _ptr(max_logits), hdim, v,
        _ptr(draft_ids) if k > 0 else None, b, k, _ptr(accepted_len), _ptr(out_tokens),
        _ptr(workspace), wbytes, _stream(stream))
    _check(st, "w8a16_lmhead_argmax_verify")
    return target_ids, max_logits, accepted_len, out_tokens


def f16_lmhead_argmax_verify(h, w, draft_ids=None, target_ids=None, max_logits=None,
                             accepted_len=None, out_tokens=None, want_max=True, workspace=None,
                             stream=None):
    """fp16 lm_head (w fp16 [V, H]) + argmax, and the greedy verify when ``draft_ids``
    (int32 [B, K]) is given (then h has B*(K+1) rows).

    Returns (target_ids [M], max_logits or None, accepted_len [B] or None, out_tokens or None).
    """
    torch = _require(h, __import__("torch").float16, "h")
    _require(w, torch.float16, "w")
    m, hdim, v = h.shape[0], w.shape[1], w.shape[0]
    dev = h.device
    b = k = 0
    if draft_ids is not None:
        _require(draft_ids, torch.int32, "draft_ids")
        b, k = draft_ids.shape
        if m != b * (k + 1):
            raise ValueError(f"h has {m} rows, B*(K+1) = {b * (k + 1)}")
        if not draft_ids.is_contiguous():
            raise ValueError("draft_ids must be contiguous")
        if accepted_len is None:
            accepted_len = torch.empty(b, dtype=torch.int32, device=dev)
        if out_tokens is None:
            out_tokens = torch.empty((b, k + 1), dtype=torch.int32, device=dev)
    if target_ids is None:
        target_ids = torch.empty(m, dtype=torch.int32, device=dev)
    if want_max and max_logits is None:
        max_logits = torch.empty(m, dtype=torch.float32, device=dev)
    need = int(load().f16_lmhead_argmax_workspace_size(m, hdim, v))
    if workspace is None and need > 0:
        workspace = new_workspace(need, dev)
    wbytes = workspace.numel() if workspace is not None else 0
    st = load().f16_lmhead_argmax_verify(
        _ptr(h), h.stride(0), _ptr(w), _ptr(target_ids), _ptr(max_logits), m, hdim, v,
        _ptr(draft_ids) if k > 0 else None, b, k, _ptr(accepted_len), _ptr(out_tokens),
        _ptr(workspace), wbytes, _stream(stream))
    _check(st, "f16_lmhead_argmax_verify")
    return target_ids, max_logits, accepted_len, out_tokens


def gdn_state_commit(state, k, v, alpha, beta, accepted_len, stream=None):
    """Advance state fp32 [B, H, D, D] (in place) by the accepted positions 0 .. a_b of the
    block: k, v fp32 [B, T, H, D], alpha, beta fp32 [B, T, H], accepted_len int32 [B]."""
    torch = _require(state, __import__("torch").float32, "state")
    for t, name in ((k, "k"), (v, "v"), (alpha, "alpha"), (beta, "beta")):
        _require(t, torch.float32, name)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _require(accepted_len, torch.int32, "accepted_len")
    if not state.is_contiguous():
        raise ValueError("state must be contiguous")
    b, h, d, d2 = state.shape
    t = k.shape[1]
    if d != d2 or tuple(k.shape) != (b, t, h, d) or tuple(v.shape) != (b, t, h, d) or \
            tuple(alpha.shape) != (b, t, h) or tuple(beta.shape) != (b, t, h) or \
            tuple(accepted_len.shape) != (b,):
        raise ValueError("gdn_state_commit: shapes do not match state [B, H, D, D]")
    st = load().gdn_state_commit(_ptr(state), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                 _ptr(accepted_len), b, t, h, d, _stream(stream))
    _check(st, "gdn_state_commit")
    return state


def f16_gemm_workspace_size(m: int, n: int, k: int) -> int:
    return int(load().f16_gemm_workspace_size(m, n, k))


def f16_gemm(x, w, alpha: float = 1.0, out=None, workspace=None, stream=None):
    """y[M, N] = fp16(alpha * x[:, :K] @ w.T) for fp16 w [N, K] (vendor library GEMM)."""
    torch = _require(x, __import__("torch").float16, "x")
    _require(w, torch.float16, "w")
    n, k = w.shape
    m = x.shape[0]
    if x.shape[1] < k:
        raise ValueError(f"x has {x.shape[1]} columns, the weights need {k}")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float16, device=x.device)
    _require(out, torch.float16, "out")
    need = f16_gemm_workspace_size(m, n, k)
    if workspace is None and need > 0:
        workspace = new_workspace(need, x.device)
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load().f16_gemm(_ptr(x), x.stride(0), _ptr(w), w.stride(0), _ptr(out), out.stride(0), m,
                         n, k, ctypes.c_float(alpha), _ptr(workspace), wbytes, _stream(stream))
    _check(st, "f16_gemm")
    return out


# ------------------------------------------------------------------- chain of linears
class Chain:
    """A prepared chain of W4A16 linears run in one launch (w4a16_chain).

    ``linears``: sequence of (qweight, scales, qzeros, alpha) GPU tensors in
    the w4a16_gemm layouts; linear l reads the leading K_l columns of linear
    l-1's output.  The workspace is allocated and prepared here, once.
    """

    def __init__(self, linears, m: int, device="cuda"):
        import torch
        self.m = int(m)
        self._keep = list(linears)
        descs = (ChainLinearDesc * len(self._keep))()
        for d, (qw, sc, qz, alpha) in zip(descs, self._keep):
            _require(qw, torch.int32, "qweight")
            _require(sc, torch.float16, "scales")
            _require(qz, torch.int32, "qzeros")
            d.qweight, d.scales, d.qzeros = qw.data_ptr(), sc.data_ptr(), qz.data_ptr()
            d.K, d.N, d.alpha = qw.shape[0] * 8, qw.shape[1], float(alpha)
        self._descs = descs
        self.k0 = descs[0].K
        self.n_last = descs[len(descs) - 1].N
        lib = load()
        need = int(lib.w4a16_chain_workspace_size(ctypes.cast(descs, ctypes.c_void_p),
                                                  len(descs), self.m))
        if need == 0:
            # re-run the checks through prepare to get the status
            _check(lib.w4a16_chain_prepare(ctypes.cast(descs, ctypes.c_void_p), len(descs),
                                           self.m, None, 0), "w4a16_chain_prepare")
        self.workspace = new_workspace(need, device)
        _check(lib.w4a16_chain_prepare(ctypes.cast(descs, ctypes.c_void_p), len(descs), self.m,
                                       _ptr(self.workspace), need), "w4a16_chain_prepare")

    def __call__(self, x, out=None, stream=None):
        import torch
        _require(x, torch.float16, "x")
        if x.shape[0] != self.m or x.shape[1] < self.k0:
            raise ValueError(f"x must be [{self.m}, >={self.k0}]")
        if out is None:
            out = torch.empty((self.m, self.n_last), dtype=torch.float16, device=x.device)
        _require(out, torch.float16, "out")
        st = load().w4a16_chain(_ptr(x), x.stride(0), _ptr(out), out.stride(0), self.m, self.k0,
                                self.n_last, _ptr(self.workspace), _stream(stream))
        _check(st, "w4a16_chain")
        return out

    def error(self) -> int:
        """The kernel's error word (synchronises): 0 ok, 1 wait timed out, 2 not prepared."""
        w = self.workspace[CHAIN_ERROR_OFFSET:CHAIN_ERROR_OFFSET + 4]
        return int(w.cpu().view(__import__("torch").int32).item())


# ------------------------------------------------------------------- drafting
def ngram_draft(history, lengths, n_max: int, n_min: int, k: int, drafts=None, stream=None):
    """Prompt-lookup drafts int32 [B, k] (-1 padded) for histories int32 [B, ld] with
    lengths int32 [B]."""
    torch = _require(history, __import__("torch").int32, "history")
    _require(lengths, torch.int32, "lengths")
    b = history.shape[0]
    if lengths.shape[0] != b:
        raise ValueError("lengths must have one entry per history row")
    if drafts is None:
        drafts = torch.empty((b, k), dtype=torch.int32, device=history.device)
    _require(drafts, torch.int32, "drafts")
    if b > 0 and (drafts.shape[0] != b or drafts.shape[1] != k or drafts.stride(0) != k):
        raise ValueError("drafts must be a contiguous int32 [B, k] tensor")
    st = load().ngram_draft(_ptr(history), history.stride(0) if b > 0 else max(1, history.shape[1]),
                            _ptr(lengths), b, n_max, n_min, k, _ptr(drafts), _stream(stream))
    _check(st, "ngram_draft")
    return drafts


def append_accepted(history, lengths, out_tokens, accepted_len, stream=None):
    """Append out_tokens[b][0 .. accepted_len[b]] to history row b (in place, up to the row's
    capacity history.shape[1]); lengths grows in place."""
    torch = _require(history, __import__("torch").int32, "history")
    _require(lengths, torch.int32, "lengths")
    _require(out_tokens, torch.int32, "out_tokens")
    _require(accepted_len, torch.int32, "accepted_len")
    b = history.shape[0]
    if b > 0 and history.stride(0) != history.shape[1]:
        raise ValueError("history rows must be contiguous: the row capacity is its width")
    k = out_tokens.shape[1] - 1
    if b > 0 and (out_tokens.shape[0] != b or out_tokens.stride(0) != k + 1):
        raise ValueError("out_tokens must be a contiguous int32 [B, K+1] tensor")
    st = load().append_accepted(_ptr(history), history.shape[1], _ptr(lengths), b, k,
                                _ptr(out_tokens), _ptr(accepted_len), _stream(stream))
    _check(st, "append_accepted")
    return history, lengths

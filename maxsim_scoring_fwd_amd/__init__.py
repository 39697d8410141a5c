"""MI355X-native late-interaction MaxSim scoring.

Thin Python front end of libmaxsim.so (the C-ABI in include/maxsim.h). The
functions here only marshal arguments: torch tensors supply device memory and
the current HIP stream, and every step of the computation runs in the HIP
kernels of libmaxsim. There is no CPU fallback: if the library is missing or no
gfx950 device is present, the calls raise.

    score(q_i, d_j) summed:  out[b] = sum_i max_j <q_i, d_j>
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmaxsim.so")

MAXSIM_BF16, MAXSIM_FP16, MAXSIM_FP32 = 0, 1, 2
_TORCH_DTYPE = {torch.bfloat16: MAXSIM_BF16, torch.float16: MAXSIM_FP16,
                torch.float32: MAXSIM_FP32}

STATUS = {0: "MAXSIM_OK", -1: "MAXSIM_ERR_NULL", -2: "MAXSIM_ERR_SHAPE", -3: "MAXSIM_ERR_DTYPE",
          -4: "MAXSIM_ERR_ALIGN", -5: "MAXSIM_ERR_UNSUPPORTED", -6: "MAXSIM_ERR_LAUNCH",
          -7: "MAXSIM_ERR_DEVICE", -8: "MAXSIM_ERR_SCRATCH"}


class MaxSimError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: {STATUS.get(status, status)} ({msg})")
        self.status = status


_lib_handle = None


def lib() -> ctypes.CDLL:
    """The loaded libmaxsim.so with argument types declared."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                              "python -m maxsim_scoring_fwd_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.maxsim_score.argtypes = [vp, i32, vp, vp, i64, i32, i32, vp, vp]
        L.maxsim_score_fixed.argtypes = [vp, i32, vp, i64, i32, vp, i32, i32, vp, vp]
        L.maxsim_score_i8.argtypes = [vp, vp, i32, vp, vp, vp, i64, i32, i32, vp, vp, vp, vp]
        L.maxsim_pq_tables.argtypes = [vp, i32, i32, vp, i32, i32, i32, vp, vp]
        L.maxsim_score_pq.argtypes = [vp, i32, i32, i32, vp, vp, i64, i32, vp, vp]
        L.maxsim_score_argmax.argtypes = [vp, i32, vp, vp, i64, i32, i32, i32, vp, vp, vp, vp]
        L.maxsim_score_batch.argtypes = [vp, i32, i32, vp, vp, i64, i32, i32, i32, vp, vp]
        L.maxsim_backward.argtypes = [vp, i32, vp, vp, i64, i32, i32, i32, vp, vp, vp, vp, i32,
                                      vp, ctypes.c_size_t, vp]
        L.maxsim_backward_workspace_size.argtypes = [i32, i32, i64]
        L.maxsim_backward_workspace_size.restype = ctypes.c_size_t
        L.maxsim_topk.argtypes = [vp, i64, i32, i32, vp, vp, vp, ctypes.c_size_t, vp]
        L.maxsim_topk_workspace_size.argtypes = [i64, i32, i32]
        L.maxsim_topk_workspace_size.restype = ctypes.c_size_t
        L.maxsim_topk_no_alloc.argtypes = [vp, i64, i32, i32, vp, vp, vp]
        L.maxsim_topk_scratch_bytes.argtypes = []
        L.maxsim_topk_scratch_bytes.restype = ctypes.c_size_t
        L.maxsim_status_string.argtypes = [i32]
        L.maxsim_status_string.restype = ctypes.c_char_p
        L.maxsim_version.argtypes = []
        for f in ("maxsim_score", "maxsim_score_fixed", "maxsim_score_i8", "maxsim_pq_tables",
                  "maxsim_score_pq", "maxsim_version", "maxsim_score_argmax", "maxsim_backward",
                  "maxsim_score_batch", "maxsim_topk", "maxsim_topk_no_alloc"):
            getattr(L, f).restype = ctypes.c_int
        _lib_handle = L
    return _lib_handle


def _check(rc: int, func: str):
    if rc != 0:
        raise MaxSimError(rc, func, lib().maxsim_status_string(rc).decode())


def _dev(t: torch.Tensor | None, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _TORCH_DTYPE:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return _TORCH_DTYPE[t.dtype]


def _out(out, n, device, dtype=torch.float32):
    if out is None:
        return torch.empty(n, dtype=dtype, device=device)
    _need(out, "out", dtype, numel=n)
    return out


# Host-side checks of dtypes and shapes. The library takes every type from its arguments
# (the storage dtype from Q, offsets as int64, argmax as int32 ...) and cannot see a
# tensor's dtype, so a mismatch here would make the kernels read past the end of a buffer.
def _need(t, name: str, dtypes, shape=None, numel=None, dim=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if not isinstance(dtypes, (tuple, list)):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(x) for x in dtypes)}, "
                         f"got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dimensions, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")


_FLOAT_STORAGE = tuple(_TORCH_DTYPE)


def _query(Q: torch.Tensor, dim: int = 2) -> None:
    _need(Q, "Q", _FLOAT_STORAGE, dim=dim)


def _docs_like(Q: torch.Tensor, D: torch.Tensor, doc_offsets) -> None:
    """D shares Q's dtype and embedding dimension; [n_docs, nd, d] without offsets, else
    [n_tokens, d] with int64 offsets [n_docs + 1]."""
    _need(D, "D", Q.dtype, dim=2 if doc_offsets is not None else 3)
    if D.shape[-1] != Q.shape[-1]:
        raise ValueError(f"D has d = {D.shape[-1]}, Q has d = {Q.shape[-1]}")
    if doc_offsets is not None:
        _need(doc_offsets, "doc_offsets", torch.int64, dim=1)
        if doc_offsets.numel() < 1:
            raise ValueError("doc_offsets needs n_docs + 1 >= 1 entries")


def maxsim_score(Q: torch.Tensor, D: torch.Tensor, doc_offsets: torch.Tensor,
                 out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """CSR documents. Q [q_len, d], D [n_tokens, d] (same dtype), doc_offsets int64
    [n_docs+1]; returns fp32 scores [n_docs]."""
    _query(Q)
    if doc_offsets is None:
        raise ValueError("maxsim_score needs doc_offsets (use maxsim_score_fixed without)")
    _docs_like(Q, D, doc_offsets)
    n_docs = doc_offsets.numel() - 1
    out = _out(out, n_docs, Q.device)
    _check(lib().maxsim_score(_dev(Q, "Q"), Q.shape[0], _dev(D, "D"),
                              _dev(doc_offsets, "doc_offsets"), n_docs, Q.shape[1],
                              _dtype_code(Q), _dev(out, "out"), _stream(stream)), "maxsim_score")
    return out


def maxsim_score_fixed(Q: torch.Tensor, D: torch.Tensor, doc_lens: torch.Tensor | None = None,
                       out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Fixed-length documents. Q [q_len, d], D [n_docs, nd, d]; doc_lens int32 [n_docs]
    (optional) masks trailing padding tokens. Returns fp32 scores [n_docs]."""
    _query(Q)
    _docs_like(Q, D, None)
    n_docs, nd = D.shape[0], D.shape[1]
    _need(doc_lens, "doc_lens", torch.int32, numel=n_docs)
    out = _out(out, n_docs, Q.device)
    _check(lib().maxsim_score_fixed(_dev(Q, "Q"), Q.shape[0], _dev(D, "D"), n_docs, nd,
                                    _dev(doc_lens, "doc_lens"), Q.shape[1], _dtype_code(Q),
                                    _dev(out, "out"), _stream(stream)), "maxsim_score_fixed")
    return out


def maxsim_score_i8(Q: torch.Tensor, q_scale: torch.Tensor, D: torch.Tensor,
                    d_scale: torch.Tensor, doc_offsets: torch.Tensor | None = None,
                    out: torch.Tensor | None = None, with_token_max: bool = False, stream=None):
    """INT8 x INT8 with per-token fp32 scales. Fixed layout (D [n_docs, nd, d]) when
    doc_offsets is None, else CSR (D [n_tokens, d]). Returns scores, or (scores, tok_max,
    tok_arg) with with_token_max."""
    _need(Q, "Q", torch.int8, dim=2)
    q_len, d = Q.shape
    _need(q_scale, "q_scale", torch.float32, numel=q_len)
    _need(D, "D", torch.int8, dim=2 if doc_offsets is not None else 3)
    if D.shape[-1] != d:
        raise ValueError(f"D has d = {D.shape[-1]}, Q has d = {d}")
    if doc_offsets is None:
        n_docs, nd = D.shape[0], D.shape[1]
    else:
        _need(doc_offsets, "doc_offsets", torch.int64, dim=1)
        n_docs, nd = doc_offsets.numel() - 1, 0
    _need(d_scale, "d_scale", torch.float32, numel=D.numel() // max(d, 1))
    out = _out(out, n_docs, Q.device)
    tm = ta = None
    if with_token_max:
        tm = torch.empty((n_docs, q_len), dtype=torch.float32, device=Q.device)
        ta = torch.empty((n_docs, q_len), dtype=torch.int32, device=Q.device)
    _check(lib().maxsim_score_i8(_dev(Q, "Q"), _dev(q_scale, "q_scale"), q_len, _dev(D, "D"),
                                 _dev(d_scale, "d_scale"), _dev(doc_offsets, "doc_offsets"),
                                 n_docs, nd, d, _dev(out, "out"), _dev(tm, "tok_max"),
                                 _dev(ta, "tok_arg"), _stream(stream)), "maxsim_score_i8")
    return (out, tm, ta) if with_token_max else out


def _docs(D: torch.Tensor, doc_offsets):
    """(n_docs, nd) of fixed documents D [n_docs, nd, d] or CSR tokens D [n_tokens, d]."""
    if doc_offsets is None:
        return D.shape[0], D.shape[1]
    return doc_offsets.numel() - 1, 0


def maxsim_score_argmax(Q: torch.Tensor, D: torch.Tensor, doc_offsets: torch.Tensor | None = None,
                        out=None, tok_max=None, tok_arg=None, stream=None):
    """Scores with per-token maxima and argmax (lowest index on ties). Fixed layout
    (D [n_docs, nd, d]) when doc_offsets is None, else CSR (D [n_tokens, d]). Returns
    (scores fp32 [n_docs], tok_max fp32 [n_docs, q_len], tok_arg int32 [n_docs, q_len])."""
    _query(Q)
    _docs_like(Q, D, doc_offsets)
    q_len, d = Q.shape
    n_docs, nd = _docs(D, doc_offsets)
    out = _out(out, n_docs, Q.device)
    _need(tok_max, "tok_max", torch.float32, shape=(n_docs, q_len))
    _need(tok_arg, "tok_arg", torch.int32, shape=(n_docs, q_len))
    if tok_max is None:
        tok_max = torch.empty((n_docs, q_len), dtype=torch.float32, device=Q.device)
    if tok_arg is None:
        tok_arg = torch.empty((n_docs, q_len), dtype=torch.int32, device=Q.device)
    _check(lib().maxsim_score_argmax(_dev(Q, "Q"), q_len, _dev(D, "D"),
                                     _dev(doc_offsets, "doc_offsets"), n_docs, nd, d,
                                     _dtype_code(Q), _dev(out, "out"), _dev(tok_max, "tok_max"),
                                     _dev(tok_arg, "tok_arg"), _stream(stream)),
           "maxsim_score_argmax")
    return out, tok_max, tok_arg


def maxsim_score_batch(Q: torch.Tensor, D: torch.Tensor, doc_offsets: torch.Tensor | None = None,
                       out=None, stream=None) -> torch.Tensor:
    """Several queries in one pass over the documents. Q [n_q, q_len, d]; fixed documents
    D [n_docs, nd, d] when doc_offsets is None, else CSR D [n_tokens, d]. Returns fp32 scores
    [n_q, n_docs]."""
    _query(Q, dim=3)
    _docs_like(Q, D, doc_offsets)
    n_q, q_len, d = Q.shape
    n_docs, nd = _docs(D, doc_offsets)
    if out is None:
        out = torch.empty((n_q, n_docs), dtype=torch.float32, device=Q.device)
    _need(out, "out", torch.float32, numel=n_q * n_docs)
    _check(lib().maxsim_score_batch(_dev(Q, "Q"), n_q, q_len, _dev(D, "D"),
                                    _dev(doc_offsets, "doc_offsets"), n_docs, nd, d,
                                    _dtype_code(Q), _dev(out, "out"), _stream(stream)),
           "maxsim_score_batch")
    return out


def topk_workspace_size(n: int, rows: int, k: int) -> int:
    """Bytes of workspace maxsim_topk needs."""
    return int(lib().maxsim_topk_workspace_size(n, rows, k))


def maxsim_topk(scores: torch.Tensor, k: int, out_scores=None, out_index=None, workspace=None,
                stream=None):
    """The k best entries of each row of scores ([n] or [rows, n] fp32) by (score
    descending, index ascending). Returns (values, indices) shaped [k] or [rows, k]."""
    _need(scores, "scores", torch.float32)
    if scores.dim() not in (1, 2):
        raise ValueError("scores must be [n] or [rows, n]")
    rows, n = (1, scores.shape[0]) if scores.dim() == 1 else scores.shape
    shape = (k,) if scores.dim() == 1 else (rows, k)
    _need(out_scores, "out_scores", torch.float32, numel=rows * k)
    _need(out_index, "out_index", torch.int32, numel=rows * k)
    _need(workspace, "workspace", torch.uint8)
    if out_scores is None:
        out_scores = torch.empty(shape, dtype=torch.float32, device=scores.device)
    if out_index is None:
        out_index = torch.empty(shape, dtype=torch.int32, device=scores.device)
    need = topk_workspace_size(n, rows, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().maxsim_topk(_dev(scores, "scores"), n, rows, k, _dev(out_scores, "out_scores"),
                             _dev(out_index, "out_index"), _dev(workspace, "workspace"), ws_bytes,
                             _stream(stream)), "maxsim_topk")
    return out_scores, out_index


def maxsim_topk_no_alloc(scores: torch.Tensor, k: int, out_scores: torch.Tensor,
                         out_index: torch.Tensor, stream=None):
    """maxsim_topk with the library's static scratch memory instead of a workspace: the
    library allocates nothing (outputs are the caller's). Calls overlapping on one GPU race."""
    _need(scores, "scores", torch.float32)
    if scores.dim() not in (1, 2):
        raise ValueError("scores must be [n] or [rows, n]")
    rows, n = (1, scores.shape[0]) if scores.dim() == 1 else scores.shape
    _need(out_scores, "out_scores", torch.float32, numel=rows * k)
    _need(out_index, "out_index", torch.int32, numel=rows * k)
    _check(lib().maxsim_topk_no_alloc(_dev(scores, "scores"), n, rows, k,
                                      _dev(out_scores, "out_scores"), _dev(out_index, "out_index"),
                                      _stream(stream)), "maxsim_topk_no_alloc")
    return out_scores, out_index


def topk_scratch_bytes() -> int:
    """Bytes of the static scratch array maxsim_topk_no_alloc uses on each GPU."""
    return int(lib().maxsim_topk_scratch_bytes())


def backward_workspace_size(q_len: int, d: int, n_docs: int) -> int:
    """Bytes of workspace maxsim_backward needs to produce dQ."""
    return int(lib().maxsim_backward_workspace_size(q_len, d, n_docs))


def maxsim_backward(Q: torch.Tensor, D: torch.Tensor, tok_arg: torch.Tensor,
                    grad_out: torch.Tensor, doc_offsets: torch.Tensor | None = None,
                    want_dQ: bool = True, want_dD: bool = True, grad_dtype=torch.float32,
                    dQ=None, dD=None, workspace=None, stream=None):
    """Gradients of sum_b grad_out[b] * score_b from the forward argmax tok_arg. Returns
    (dQ [q_len, d], dD shaped like D), each None when not asked for; grad_dtype is float32
    or the dtype of Q and D."""
    _query(Q)
    _docs_like(Q, D, doc_offsets)
    if grad_dtype not in (torch.float32, Q.dtype):
        raise ValueError("grad_dtype must be float32 or the dtype of Q")
    q_len, d = Q.shape
    n_docs, nd = _docs(D, doc_offsets)
    _need(tok_arg, "tok_arg", torch.int32, shape=(n_docs, q_len))
    _need(grad_out, "grad_out", torch.float32, numel=n_docs)
    _need(dQ, "dQ", grad_dtype, shape=(q_len, d))
    _need(dD, "dD", grad_dtype, shape=tuple(D.shape))
    _need(workspace, "workspace", torch.uint8)
    if want_dQ and dQ is None:
        dQ = torch.empty((q_len, d), dtype=grad_dtype, device=Q.device)
    if want_dD and dD is None:
        dD = torch.empty(D.shape, dtype=grad_dtype, device=Q.device)
    if not want_dQ:
        dQ = None
    if not want_dD:
        dD = None
    ws_bytes = 0
    if dQ is not None:
        ws_bytes = backward_workspace_size(q_len, d, n_docs)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=Q.device)
        ws_bytes = workspace.numel() * workspace.element_size()
    else:
        workspace = None
    _check(lib().maxsim_backward(_dev(Q, "Q"), q_len, _dev(D, "D"), _dev(doc_offsets, "doc_offsets"),
                                 n_docs, nd, d, _dtype_code(Q), _dev(tok_arg, "tok_arg"),
                                 _dev(grad_out, "grad_out"), _dev(dQ, "dQ"), _dev(dD, "dD"),
                                 _TORCH_DTYPE[grad_dtype], _dev(workspace, "workspace"), ws_bytes,
                                 _stream(stream)), "maxsim_backward")
    return dQ, dD


class MaxSimFunction(torch.autograd.Function):
    """Differentiable MaxSim scores: the forward keeps the argmax, the backward turns it
    into dQ and dD with the library's kernels (gradients in the input dtype)."""

    @staticmethod
    def forward(ctx, Q, D, doc_offsets):
        scores, _, tok_arg = maxsim_score_argmax(Q, D, doc_offsets)
        ctx.save_for_backward(Q, D, doc_offsets, tok_arg)
        return scores

    @staticmethod
    def backward(ctx, grad_scores):
        Q, D, doc_offsets, tok_arg = ctx.saved_tensors
        dQ, dD = maxsim_backward(Q, D, tok_arg, grad_scores.float().contiguous(), doc_offsets,
                                 want_dQ=ctx.needs_input_grad[0], want_dD=ctx.needs_input_grad[1],
                                 grad_dtype=Q.dtype)
        return dQ, dD, None


def maxsim(Q: torch.Tensor, D: torch.Tensor, doc_offsets: torch.Tensor | None = None):
    """Scores [n_docs] that autograd can differentiate with respect to Q and D."""
    return MaxSimFunction.apply(Q, D, doc_offsets)


def maxsim_pq_tables(Q: torch.Tensor, C: torch.Tensor, T: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    """PQ distance tables T [q_len, M, K] fp32 from Q [q_len, M*dsub] and C [M, K, dsub] fp32."""
    _query(Q)
    _need(C, "C", torch.float32, dim=3)
    M, K, dsub = C.shape
    if Q.shape[1] != M * dsub:
        raise ValueError(f"Q has d = {Q.shape[1]}, the codebook M * dsub = {M * dsub}")
    if T is None:
        T = torch.empty((Q.shape[0], M, K), dtype=torch.float32, device=Q.device)
    _need(T, "T", torch.float32, shape=(Q.shape[0], M, K))
    _check(lib().maxsim_pq_tables(_dev(Q, "Q"), Q.shape[0], _dtype_code(Q), _dev(C, "C"), M, K,
                                  dsub, _dev(T, "T"), _stream(stream)), "maxsim_pq_tables")
    return T


def maxsim_score_pq(T: torch.Tensor, codes: torch.Tensor, doc_offsets: torch.Tensor | None = None,
                    nd: int = 0, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Fused PQ lookup scoring. T [q_len, M, K] fp32, codes uint8 [n_tokens, M]; CSR when
    doc_offsets is given, else fixed documents of nd tokens."""
    _need(T, "T", torch.float32, dim=3)
    q_len, M, K = T.shape
    _need(codes, "codes", torch.uint8, dim=2)
    if codes.shape[1] != M:
        raise ValueError(f"codes have {codes.shape[1]} subspaces, T has M = {M}")
    if doc_offsets is not None:
        _need(doc_offsets, "doc_offsets", torch.int64, dim=1)
    elif nd < 1:
        raise ValueError("fixed documents need nd >= 1")
    n_docs = doc_offsets.numel() - 1 if doc_offsets is not None else codes.shape[0] // max(nd, 1)
    out = _out(out, n_docs, T.device)
    _check(lib().maxsim_score_pq(_dev(T, "T"), q_len, M, K, _dev(codes, "codes"),
                                 _dev(doc_offsets, "doc_offsets"), n_docs, nd, _dev(out, "out"),
                                 _stream(stream)), "maxsim_score_pq")
    return out


def version() -> int:
    return lib().maxsim_version()


# ---- measurement helpers (include/maxsim_calib.h) ----

def _calib_lib():
    L = lib()
    if not getattr(L, "_calib_bound", False):
        vp = ctypes.c_void_p
        L.maxsim_calib_read.argtypes = [vp, ctypes.c_size_t, ctypes.c_int, vp, vp]
        L.maxsim_calib_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
        L.maxsim_calib_write.argtypes = [vp, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, vp]
        L.maxsim_calib_write.restype = ctypes.c_int
        L.maxsim_calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]
        L.maxsim_calib_read.restype = ctypes.c_int
        L.maxsim_calib_copy.restype = ctypes.c_int
        L.maxsim_calib_mfma.restype = ctypes.c_int
        L.maxsim_calib_valu.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp]
        L.maxsim_calib_valu.restype = ctypes.c_int
        L.maxsim_calib_mix.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]
        L.maxsim_calib_mix.restype = ctypes.c_int
        L.maxsim_calib_lds.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp]
        L.maxsim_calib_lds.restype = ctypes.c_int
        L._calib_bound = True
    return L


def calib_read(src: torch.Tensor, sink: torch.Tensor, stream=None, wgs_per_cu: int = 1):
    """Stream-read every byte of src (achievable read bandwidth) with wgs_per_cu workgroups
    of 4 waves per CU (0: as many as fit); sink: >= 65536 words."""
    _check(_calib_lib().maxsim_calib_read(_dev(src, "src"), src.numel() * src.element_size(),
                                          int(wgs_per_cu), _dev(sink, "sink"), _stream(stream)),
           "maxsim_calib_read")


def calib_write(dst: torch.Tensor, stream=None, wgs_per_cu: int = 2, contig: bool = True):
    """Stream a fixed pattern into every byte of dst (achievable write bandwidth) with
    wgs_per_cu workgroups of 4 waves per CU (0: as many as fit), each wave writing one
    contiguous range (contig) or blocks dealt in turn."""
    _check(_calib_lib().maxsim_calib_write(_dev(dst, "dst"), dst.numel() * dst.element_size(),
                                           int(wgs_per_cu), int(bool(contig)), _stream(stream)),
           "maxsim_calib_write")


def calib_copy(src: torch.Tensor, dst: torch.Tensor, stream=None):
    """Plain 128-bit copy of src into dst (known traffic for counter scaling)."""
    _check(_calib_lib().maxsim_calib_copy(_dev(src, "src"), _dev(dst, "dst"),
                                          src.numel() * src.element_size(), _stream(stream)),
           "maxsim_calib_copy")


def calib_mfma(kind: int, iters: int, waves_per_simd: int, sink: torch.Tensor, stream=None) -> float:
    """Launch independent MFMA chains (kind 0: 16x16x32 bf16, 1: 32x32x16 bf16, 2: 16x16x64
    int8, 3: 32x32x32 int8); returns the FLOP / integer-op count of the launch."""
    ops = ctypes.c_double(0.0)
    _check(_calib_lib().maxsim_calib_mfma(kind, iters, waves_per_simd, _dev(sink, "sink"),
                                          ctypes.addressof(ops), _stream(stream)),
           "maxsim_calib_mfma")
    return ops.value


def calib_valu(iters: int, waves_per_simd: int, sink: torch.Tensor, stream=None) -> float:
    """Launch independent fp32 FMA chains; returns the FLOP count of the launch."""
    ops = ctypes.c_double(0.0)
    _check(_calib_lib().maxsim_calib_valu(iters, waves_per_simd, _dev(sink, "sink"),
                                          ctypes.addressof(ops), _stream(stream)), "maxsim_calib_valu")
    return ops.value


def calib_mix(valu_per_mfma: int, iters: int, waves_per_simd: int, sink: torch.Tensor,
              stream=None) -> float:
    """Launch int8 MFMA chains with valu_per_mfma independent FMAs per MFMA; returns the
    int8 integer-op count of the launch."""
    ops = ctypes.c_double(0.0)
    _check(_calib_lib().maxsim_calib_mix(valu_per_mfma, iters, waves_per_simd, _dev(sink, "sink"),
                                         ctypes.addressof(ops), _stream(stream)), "maxsim_calib_mix")
    return ops.value


def calib_lds(pattern: int, iters: int, sink: torch.Tensor, stream=None) -> float:
    """Launch the LDS read-rate kernel (0: contiguous, 1: PQ lookups); returns LDS bytes read."""
    b = ctypes.c_double(0.0)
    _check(_calib_lib().maxsim_calib_lds(pattern, iters, _dev(sink, "sink"), ctypes.addressof(b),
                                         _stream(stream)), "maxsim_calib_lds")
    return b.value

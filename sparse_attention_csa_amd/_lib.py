"""ctypes binding of libcsa.so (include/csa.h).  Argument marshalling only:
torch tensors are passed as device pointers, the stream is torch's current
HIP stream, and every step of the computation runs in the library's kernels.
There is no fallback: if the library is missing, loading fails loudly.
"""

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcsa.so")

CSA_OK, CSA_ERR_ARG, CSA_ERR_UNSUPPORTED, CSA_ERR_WORKSPACE, CSA_ERR_DEVICE = range(5)
CSA_F32, CSA_BF16, CSA_E4M3, CSA_MXFP4, CSA_FP8BF16 = 0, 1, 2, 3, 4
CSA_VIS_PRIOR_BLOCKS, CSA_VIS_COMPLETED = 0, 1
CSA_LAYER_CSA, CSA_LAYER_HCA = 1, 2

STATUS_NAMES = {0: "CSA_OK", 1: "CSA_ERR_ARG", 2: "CSA_ERR_UNSUPPORTED", 3: "CSA_ERR_WORKSPACE",
                4: "CSA_ERR_DEVICE"}

# exported entry points, as declared in include/csa.h
EXPORTS = [
    "csa_last_error", "csa_abi_version", "csa_compress", "csa_index_topk_workspace",
    "csa_index_topk", "csa_attend_workspace", "csa_attend", "hca_attend",
    "hybrid_layer_workspace", "hybrid_layer_decode", "hybrid_layer_prefill",
    "csa_profile_enable", "csa_profile_collect", "csa_test_set_fused_wait_polls",
    "csa_test_set_fold_fusion",
    "hybrid_layer_noalloc_scratch_bytes", "hybrid_layer_decode_noalloc",
]


class CsaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class LayerDesc(C.Structure):
    _fields_ = [("kind", C.c_int), ("H", C.c_int), ("c", C.c_int), ("H_I", C.c_int),
                ("d_I", C.c_int), ("m", C.c_int), ("overlap", C.c_int), ("k", C.c_int),
                ("n_win", C.c_int), ("vis", C.c_int), ("kv_dtype", C.c_int),
                ("idx_dtype", C.c_int), ("scale", C.c_float), ("split_rows", C.c_int),
                ("score_bf16", C.c_int), ("norm_rope", C.c_int), ("rope_dims", C.c_int),
                ("norm_eps", C.c_float)]


class LayerState(C.Structure):
    _fields_ = [("B", C.c_int), ("E_cap", C.c_int), ("kv_cache", C.c_void_p),
                ("idx_cache", C.c_void_p), ("idx_scale", C.c_void_p), ("n_entries", C.c_void_p),
                ("win_ring", C.c_void_p), ("tail", C.c_void_p), ("idx_tail", C.c_void_p),
                ("bias_a", C.c_void_p), ("bias_b", C.c_void_p), ("ibias_a", C.c_void_p),
                ("ibias_b", C.c_void_p), ("sink", C.c_void_p), ("q_norm_w", C.c_void_p),
                ("kv_norm_w", C.c_void_p), ("rope_inv_freq", C.c_void_p), ("kv_scale", C.c_void_p),
                ("block_table", C.c_void_p), ("page_entries", C.c_int)]


class DecodeIO(C.Structure):
    _fields_ = [("pos", C.c_void_p), ("q", C.c_void_p), ("q_idx", C.c_void_p),
                ("q_scale", C.c_void_p), ("w_idx", C.c_void_p), ("x_new", C.c_void_p),
                ("streams", C.c_void_p), ("idx_streams", C.c_void_p), ("out", C.c_void_p),
                ("lse", C.c_void_p), ("topk_idx", C.c_void_p), ("topk_cnt", C.c_void_p)]


class PrefillIO(C.Structure):
    _fields_ = [("pos0", C.c_int64), ("T", C.c_int), ("q", C.c_void_p), ("q_idx", C.c_void_p),
                ("q_scale", C.c_void_p), ("w_idx", C.c_void_p), ("win", C.c_void_p),
                ("streams", C.c_void_p), ("idx_streams", C.c_void_p), ("out", C.c_void_p),
                ("lse", C.c_void_p), ("topk_idx", C.c_void_p), ("topk_cnt", C.c_void_p),
                ("seq_pos0", C.c_void_p), ("seq_len", C.c_void_p)]


class KernelTime(C.Structure):
    _fields_ = [("name", C.c_char * 48), ("launches", C.c_int64), ("total_ms", C.c_double)]


_LIB = None

P = C.c_void_p
I = C.c_int
I64 = C.c_int64
SZ = C.c_size_t
F = C.c_float


def _declare(lib):
    sig = {
        "csa_last_error": (C.c_char_p, []),
        "csa_abi_version": (I, []),
        "csa_compress": (I, [I, P, P, I, P, P, P, P, P, P, P, I, I, I, I, P, I, P, I, I64, P]),
        "csa_index_topk_workspace": (SZ, [I, I, I, I]),
        "csa_index_topk": (I, [I, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, P, P, P, P, SZ, P]),
        "csa_attend_workspace": (SZ, [I, I, I, I, I]),
        "csa_attend": (I, [I, P, P, I, P, P, I, P, I, P, I, P, P, F, I, I, I, I, P, P, P, SZ, P]),
        "hca_attend": (I, [I, P, P, I, P, I, I, P, I, P, I, P, P, F, I, I, I, I, P, P, P, SZ, P]),
        "hybrid_layer_workspace": (SZ, [C.POINTER(LayerDesc), I, I, I]),
        "hybrid_layer_decode": (I, [C.POINTER(LayerDesc), C.POINTER(LayerState),
                                    C.POINTER(DecodeIO), P, SZ, P]),
        "hybrid_layer_prefill": (I, [C.POINTER(LayerDesc), C.POINTER(LayerState),
                                     C.POINTER(PrefillIO), P, SZ, P]),
        "csa_profile_enable": (I, [I]),
        "csa_profile_collect": (I, [C.POINTER(KernelTime), I]),
        "csa_test_set_fused_wait_polls": (I, [I]),
        "csa_test_set_fold_fusion": (I, [I]),
        "hybrid_layer_noalloc_scratch_bytes": (SZ, []),
        "hybrid_layer_decode_noalloc": (I, [C.POINTER(LayerDesc), C.POINTER(LayerState),
                                            C.POINTER(DecodeIO), P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def lib():
    """The loaded library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m sparse_attention_csa_amd.build` "
                "(there is no fallback implementation)")
        lb = C.CDLL(LIB_PATH)
        _declare(lb)
        _LIB = lb
    return _LIB


def last_error():
    return lib().csa_last_error().decode()


def check(status):
    if status != CSA_OK:
        raise CsaError(status, last_error())
    return status


# ---------------------------------------------------------------- marshalling
def ptr(t):
    """Device (or host) address of a tensor, or None."""
    if t is None:
        return None
    return t.data_ptr()


def stream_handle(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return CSA_E4M3
    raise ValueError(f"unsupported dtype {t.dtype}")


def _ws(nbytes, device):
    import torch
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- entry points
def csa_compress(content_a, logits_a, m, bias_a=None, content_b=None, logits_b=None, bias_b=None,
                 prev_content_b=None, prev_logits_b=None, score_w=None, out=None, out_scale=None,
                 out_dtype=None, out_first_entry=0, out_code=None, stream=None):
    """Compress a block-aligned chunk.  content_a [B][T][c]; logits [B][T][c|1]
    (or score_w [c]); out [B][E_cap][c] (allocated [B][T/m][c] when None).
    out_code overrides the storage format taken from out's dtype (CSA_MXFP4:
    out is uint8 [B][E_cap][c/2], out_scale uint8 [B][E_cap][c/32])."""
    import torch
    B, T, c = content_a.shape
    lw = logits_a.shape[-1] if logits_a is not None else 1
    if out is None:
        od = out_dtype if out_dtype is not None else content_a.dtype
        out = torch.empty((B, T // m, c), dtype=od, device=content_a.device)
    E_cap = out.shape[1]
    code = dtype_code(out) if out_code is None else out_code
    check(lib().csa_compress(dtype_code(content_a), ptr(content_a), ptr(logits_a), lw, ptr(score_w),
                             ptr(bias_a), ptr(content_b), ptr(logits_b), ptr(bias_b),
                             ptr(prev_content_b), ptr(prev_logits_b), B, T, c, m, ptr(out), code,
                             ptr(out_scale), E_cap, out_first_entry, stream_handle(stream)))
    return out


def csa_index_topk(q_idx, w_idx, k_idx, q_pos, n_entries, m, k, vis=CSA_VIS_PRIOR_BLOCKS,
                   q_scale=None, k_scale=None, scores=None, ws=None, idx_dtype=None, score_bf16=False,
                   stream=None):
    """Indexer scores + top-k.  Returns (topk_idx [B][Tq][k], topk_cnt [B][Tq]).
    idx_dtype (a CSA_* code) overrides the format taken from q_idx's dtype;
    CSA_MXFP4 vectors are uint8 [..][d_I/2] with uint8 scales [..][d_I/32]."""
    import torch
    code = dtype_code(q_idx) if idx_dtype is None else idx_dtype
    B, Tq, H_I, d_I = q_idx.shape
    if code == CSA_MXFP4:
        d_I *= 2
    E_cap = k_idx.shape[1]
    dev = q_idx.device
    topk_idx = torch.empty((B, Tq, k), dtype=torch.int32, device=dev)
    topk_cnt = torch.empty((B, Tq), dtype=torch.int32, device=dev)
    need = lib().csa_index_topk_workspace(B, Tq, E_cap, k)
    if ws is None:
        ws = _ws(need, dev)
    check(lib().csa_index_topk(code, ptr(q_idx), ptr(q_scale), ptr(w_idx), ptr(k_idx),
                               ptr(k_scale), ptr(q_pos), ptr(n_entries), B, Tq, H_I, d_I, E_cap, m,
                               k, vis, int(bool(score_bf16)), ptr(topk_idx), ptr(topk_cnt), ptr(scores), ptr(ws),
                               ws.numel(), stream_handle(stream)))
    return topk_idx, topk_cnt


def csa_attend(q, kv, topk_idx, topk_cnt, win, win_pos0, n_win, q_pos, scale, sink=None,
               out=None, lse=None, ws=None, stream=None):
    """Sparse attention.  q [B][Tq][H][c]; kv [B][E_cap][c]; win [B][W_cap][c]."""
    import torch
    B, Tq, H, c = q.shape
    k = topk_idx.shape[-1]
    if out is None:
        out = torch.empty_like(q)
    need = lib().csa_attend_workspace(B, Tq, H, c, k + n_win)
    if ws is None:
        ws = _ws(need, q.device)
    check(lib().csa_attend(dtype_code(q), ptr(q), ptr(kv), kv.shape[1], ptr(topk_idx),
                           ptr(topk_cnt), k, ptr(win), win.shape[1], ptr(win_pos0), n_win,
                           ptr(sink), ptr(q_pos), float(scale), B, Tq, H, c, ptr(out), ptr(lse),
                           ptr(ws), ws.numel(), stream_handle(stream)))
    return out


def hca_attend(q, kv, n_entries, m, win, win_pos0, n_win, q_pos, scale, sink=None,
               vis=CSA_VIS_PRIOR_BLOCKS, out=None, lse=None, ws=None, stream=None):
    """Dense attention over every visible entry + window + sink."""
    import torch
    B, Tq, H, c = q.shape
    if out is None:
        out = torch.empty_like(q)
    need = lib().csa_attend_workspace(B, Tq, H, c, kv.shape[1] + n_win)
    if ws is None:
        ws = _ws(need, q.device)
    check(lib().hca_attend(dtype_code(q), ptr(q), ptr(kv), kv.shape[1], ptr(n_entries), m, vis,
                           ptr(win), win.shape[1], ptr(win_pos0), n_win, ptr(sink), ptr(q_pos),
                           float(scale), B, Tq, H, c, ptr(out), ptr(lse), ptr(ws), ws.numel(),
                           stream_handle(stream)))
    return out


def hybrid_layer_workspace(desc, B, T, E_cap):
    return lib().hybrid_layer_workspace(C.byref(desc), B, T, E_cap)


def hybrid_layer_decode(desc, state, io, ws, stream=None):
    check(lib().hybrid_layer_decode(C.byref(desc), C.byref(state), C.byref(io), ptr(ws), ws.numel(),
                                    stream_handle(stream)))


def hybrid_layer_decode_noalloc(desc, state, io, stream=None):
    check(lib().hybrid_layer_decode_noalloc(C.byref(desc), C.byref(state), C.byref(io),
                                            stream_handle(stream)))


def hybrid_layer_prefill(desc, state, io, ws, stream=None):
    check(lib().hybrid_layer_prefill(C.byref(desc), C.byref(state), C.byref(io), ptr(ws),
                                     ws.numel(), stream_handle(stream)))


def set_fused_wait_polls(polls):
    """Test hook: the fused top-k's poll budget (negative = default); returns
    the previous value."""
    return lib().csa_test_set_fused_wait_polls(int(polls))


def set_fold_fusion(on):
    """Test hook: whether decode steps may fold inside the scoring kernel or
    the dense attention; returns the previous setting."""
    return lib().csa_test_set_fold_fusion(1 if on else 0)


def profile_enable(on=True):
    check(lib().csa_profile_enable(1 if on else 0))


def profile_collect():
    """{kernel name: (launches, total_ms)} since the previous collect."""
    buf = (KernelTime * 64)()
    n = lib().csa_profile_collect(buf, 64)
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(min(n, 64))}

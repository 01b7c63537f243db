"""ctypes binding of libpeagle.so: the C ABI of include/peagle.h, one Python
function per entry point with the same name.  Argument marshalling only --
every step of the drafter runs in the library's HIP kernels.

Device pointers are passed as integers (e.g. ``tensor.data_ptr()``); streams
as the integer HIP stream handle (``torch.cuda.current_stream().cuda_stream``).
A missing or unloadable library raises immediately: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpeagle.so")

PE_OK = 0
PE_ERR_INVALID_ARGUMENT = -1
PE_ERR_UNSUPPORTED = -2
PE_ERR_WORKSPACE = -3
PE_ERR_HIP = -4
PE_F32 = 0
PE_BF16 = 1
PE_K_MAX = 16
PE_DECODE_ROWS_MAX = 64
PE_NOALLOC_SCRATCH_BYTES = 32 << 20
PE_INPUT_TARGET = 0
PE_INPUT_DRAFTER = 1

EXPORTS = (
    "pe_model_create", "pe_model_destroy", "pe_draft_workspace_size", "pe_workspace_init",
    "pe_draft_forward", "pe_accept", "pe_last_error", "pe_version", "pe_profile_enable",
    "pe_profile_read", "pe_mask_create", "pe_mask_destroy", "pe_mask_materialize",
    "pe_train_workspace_size", "pe_train_forward", "pe_cod_rows", "pe_partition",
    "pe_draft_extend", "pe_partition_chunk", "pe_train_forward_chunk", "pe_model_prepare_backward",
    "pe_train_step_workspace_size", "pe_train_step", "pe_draft_shape_check", "pe_draft_forward_noalloc",
)


class PeConfig(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("intermediate", ctypes.c_int32), ("vocab", ctypes.c_int32),
        ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int32),
    ]


class PeLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")]


class PeWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("fc", ctypes.c_void_p),
                ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("layers", ctypes.POINTER(PeLayerWeights))]


class PeLayerGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")]


class PeGrads(ctypes.Structure):
    _fields_ = [("fc", ctypes.c_void_p), ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("mask_emb", ctypes.c_void_p), ("h_shared", ctypes.c_void_p), ("embed_rows", ctypes.c_void_p),
                ("layers", ctypes.POINTER(PeLayerGrads))]


class PeagleError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} returned {status}: {message}")
        self.status = status
        self.message = message


_lib = None


def load(path: str = LIB_PATH):
    """Load libpeagle.so once and declare the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m drafting_eagle_draft_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "pe_model_create": [ctypes.POINTER(PeConfig), ctypes.POINTER(PeWeights), vp,
                            ctypes.POINTER(vp)],
        "pe_model_destroy": [vp],
        "pe_draft_workspace_size": [vp, i32, i32, i64, ctypes.POINTER(sz)],
        "pe_draft_shape_check": [ctypes.POINTER(PeConfig), i32, i32, i64, i32],
        "pe_workspace_init": [vp, sz, vp],
        "pe_draft_forward": [vp, i32, i32, i32, vp, vp, vp, vp, vp, i64, ctypes.POINTER(vp),
                             ctypes.POINTER(vp), vp, vp, vp, sz, vp],
        "pe_draft_forward_noalloc": [vp, i32, i32, i32, vp, vp, vp, vp, vp, i64, ctypes.POINTER(vp),
                                     ctypes.POINTER(vp), vp, vp, vp],
        "pe_accept": [i32, i32, vp, vp, vp, vp, vp],
        "pe_profile_enable": [vp, i32],
        "pe_profile_read": [vp, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double)],
        "pe_mask_create": [i32, i32, vp, ctypes.POINTER(vp)],
        "pe_mask_destroy": [vp],
        "pe_mask_materialize": [vp, i32, vp, i32, vp, vp],
        "pe_train_workspace_size": [vp, i32, i32, i32, ctypes.POINTER(sz)],
        "pe_train_forward": [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp],
        "pe_cod_rows": [i32, i32, ctypes.c_double, ctypes.c_double, vp, vp, ctypes.POINTER(i32)],
        "pe_partition": [i32, i32, i32, vp, i32, vp],
        "pe_draft_extend": [vp, i32, i32, i32, vp, i32, vp, vp, i32, i64, ctypes.POINTER(vp),
                            ctypes.POINTER(vp), vp, vp, vp, vp, sz, vp],
        "pe_partition_chunk": [i32, i32, i32, i32, vp, i32, vp, vp, ctypes.POINTER(i32),
                               ctypes.POINTER(i32), ctypes.POINTER(i32)],
        "pe_train_forward_chunk": [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, i32, i32, vp, i32, vp, vp,
                                   vp, sz, vp],
        "pe_model_prepare_backward": [vp, ctypes.POINTER(PeWeights), vp],
        "pe_train_step_workspace_size": [vp, i32, i32, i32, i32, ctypes.POINTER(sz)],
        "pe_train_step": [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, i32, i32, vp, ctypes.c_float, vp,
                          ctypes.POINTER(PeGrads), vp, sz, vp],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.pe_last_error.argtypes = []
    L.pe_last_error.restype = ctypes.c_char_p
    L.pe_version.argtypes = []
    L.pe_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(fn: str, status: int):
    if status != PE_OK:
        raise PeagleError(fn, status, pe_last_error())


def pe_last_error() -> str:
    return load().pe_last_error().decode()


def pe_version() -> str:
    return load().pe_version().decode()


def pe_model_create(cfg: PeConfig, weights: PeWeights, stream: int = 0) -> int:
    out = ctypes.c_void_p()
    _check("pe_model_create",
           load().pe_model_create(ctypes.byref(cfg), ctypes.byref(weights), stream, ctypes.byref(out)))
    return out.value


def pe_model_destroy(model: int) -> None:
    _check("pe_model_destroy", load().pe_model_destroy(model))


def pe_draft_workspace_size(model: int, B: int, K: int, ctx_stride: int) -> int:
    n = ctypes.c_size_t()
    _check("pe_draft_workspace_size",
           load().pe_draft_workspace_size(model, B, K, ctx_stride, ctypes.byref(n)))
    return n.value


def pe_draft_shape_check(cfg: PeConfig, B: int, K: int, ctx_stride: int, num_cus: int) -> None:
    """Host-only: raises PeagleError when the draft forward cannot run this shape."""
    _check("pe_draft_shape_check", load().pe_draft_shape_check(ctypes.byref(cfg), B, K, ctx_stride, num_cus))


def pe_workspace_init(workspace: int, ws_bytes: int, stream: int = 0) -> None:
    _check("pe_workspace_init", load().pe_workspace_init(workspace, ws_bytes, stream))


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * max(1, len(ptrs)))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr


def pe_draft_forward(model: int, N: int, B: int, K: int, hidden3: int, token_ids: int,
                     mask_emb: int, h_shared: int, ctx_lens: int, ctx_stride: int,
                     k_cache, v_cache, draft_out: int, logits_out: int | None,
                     workspace: int, ws_bytes: int, stream: int = 0) -> None:
    """k_cache / v_cache: sequences of N device pointers (one per layer)."""
    kc = _ptr_array(list(k_cache)) if k_cache is not None else None
    vc = _ptr_array(list(v_cache)) if v_cache is not None else None
    _check("pe_draft_forward", load().pe_draft_forward(
        model, N, B, K, hidden3, token_ids, mask_emb, h_shared, ctx_lens, ctx_stride,
        ctypes.cast(kc, ctypes.POINTER(ctypes.c_void_p)) if kc is not None else None,
        ctypes.cast(vc, ctypes.POINTER(ctypes.c_void_p)) if vc is not None else None,
        draft_out, logits_out, workspace, ws_bytes, stream))


def pe_draft_forward_noalloc(model: int, N: int, B: int, K: int, hidden3: int, token_ids: int,
                             mask_emb: int, h_shared: int, ctx_lens: int, ctx_stride: int,
                             k_cache, v_cache, draft_out: int, logits_out: int | None,
                             stream: int = 0) -> None:
    """pe_draft_forward on the library's per-device scratch (no workspace)."""
    kc = _ptr_array(list(k_cache)) if k_cache is not None else None
    vc = _ptr_array(list(v_cache)) if v_cache is not None else None
    _check("pe_draft_forward_noalloc", load().pe_draft_forward_noalloc(
        model, N, B, K, hidden3, token_ids, mask_emb, h_shared, ctx_lens, ctx_stride,
        ctypes.cast(kc, ctypes.POINTER(ctypes.c_void_p)) if kc is not None else None,
        ctypes.cast(vc, ctypes.POINTER(ctypes.c_void_p)) if vc is not None else None,
        draft_out, logits_out, stream))


def pe_draft_extend(model: int, N: int, B: int, T: int, inputs: int, input_kind: int, token_ids: int,
                    ctx_lens: int, pos_offset: int, ctx_stride: int, k_cache, v_cache,
                    draft_out: int | None, logits_out: int | None, z_out: int | None,
                    workspace: int, ws_bytes: int, stream: int = 0) -> None:
    """k_cache / v_cache: sequences of N device pointers; the block's keys and
    values are appended at positions ctx_lens[b] + pos_offset + t."""
    kc = _ptr_array(list(k_cache)) if k_cache is not None else None
    vc = _ptr_array(list(v_cache)) if v_cache is not None else None
    _check("pe_draft_extend", load().pe_draft_extend(
        model, N, B, T, inputs, input_kind, token_ids, ctx_lens, pos_offset, ctx_stride,
        ctypes.cast(kc, ctypes.POINTER(ctypes.c_void_p)) if kc is not None else None,
        ctypes.cast(vc, ctypes.POINTER(ctypes.c_void_p)) if vc is not None else None,
        draft_out, logits_out, z_out, workspace, ws_bytes, stream))


def pe_accept(B: int, K: int, draft: int, target: int, accept_len: int,
              out_tokens: int | None = None, stream: int = 0) -> None:
    _check("pe_accept", load().pe_accept(B, K, draft, target, accept_len, out_tokens, stream))


def pe_profile_enable(model: int, enable: bool) -> None:
    _check("pe_profile_enable", load().pe_profile_enable(model, 1 if enable else 0))


def pe_profile_read(model: int):
    """(launch count, mean LM-head launch duration in ms) since enable/last read."""
    n = ctypes.c_int32()
    ms = ctypes.c_double()
    _check("pe_profile_read", load().pe_profile_read(model, ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def pe_mask_create(n_max: int, K: int, stream: int = 0) -> int:
    out = ctypes.c_void_p()
    _check("pe_mask_create", load().pe_mask_create(n_max, K, stream, ctypes.byref(out)))
    return out.value


def pe_mask_destroy(mask: int) -> None:
    _check("pe_mask_destroy", load().pe_mask_destroy(mask))


def pe_mask_materialize(mask: int, n: int, rows: int, L: int, out: int, stream: int = 0) -> None:
    _check("pe_mask_materialize", load().pe_mask_materialize(mask, n, rows, L, out, stream))


def pe_train_workspace_size(model: int, n: int, K: int, L: int) -> int:
    b = ctypes.c_size_t()
    _check("pe_train_workspace_size", load().pe_train_workspace_size(model, n, K, L, ctypes.byref(b)))
    return b.value


def pe_train_forward(model: int, mask: int, N: int, n: int, K: int, hidden3: int, token_ids: int,
                     mask_emb: int, h_shared: int, rows: int, L: int, logits_out: int | None,
                     argmax_out: int | None, workspace: int, ws_bytes: int, stream: int = 0) -> None:
    _check("pe_train_forward", load().pe_train_forward(
        model, mask, N, n, K, hidden3, token_ids, mask_emb, h_shared, rows, L, logits_out,
        argmax_out, workspace, ws_bytes, stream))


def pe_train_forward_chunk(model: int, mask: int, N: int, n: int, K: int, hidden3: int, token_ids: int,
                           mask_emb: int, h_shared: int, cells: int, L: int, n_lead: int, out_rows: int | None,
                           L_out: int, logits_out: int | None, argmax_out: int | None, workspace: int,
                           ws_bytes: int, stream: int = 0) -> None:
    _check("pe_train_forward_chunk", load().pe_train_forward_chunk(
        model, mask, N, n, K, hidden3, token_ids, mask_emb, h_shared, cells, L, n_lead, out_rows, L_out,
        logits_out, argmax_out, workspace, ws_bytes, stream))


def pe_model_prepare_backward(model: int, weights: PeWeights, stream: int = 0) -> None:
    _check("pe_model_prepare_backward", load().pe_model_prepare_backward(model, ctypes.byref(weights), stream))


def pe_train_step_workspace_size(model: int, N: int, n: int, K: int, L: int) -> int:
    out = ctypes.c_size_t()
    _check("pe_train_step_workspace_size", load().pe_train_step_workspace_size(model, N, n, K, L, ctypes.byref(out)))
    return out.value


def pe_train_step(model: int, mask: int, N: int, n: int, K: int, hidden3: int, token_ids: int, mask_emb: int,
                  h_shared: int, cells: int, L: int, n_lead: int, labels: int, loss_scale: float,
                  loss_out: int | None, grads: PeGrads, workspace: int, ws_bytes: int, stream: int = 0) -> None:
    _check("pe_train_step", load().pe_train_step(
        model, mask, N, n, K, hidden3, token_ids, mask_emb, h_shared, cells, L, n_lead, labels, loss_scale,
        loss_out, ctypes.byref(grads), workspace, ws_bytes, stream))


def pe_cod_rows(n: int, K: int, r: float, floor_rate: float, U):
    """Host COD sampling: U float64 array [n*K] -> int32 array of kept grid indices."""
    import numpy as np
    U = np.ascontiguousarray(U, dtype=np.float64)
    if U.size != n * K:
        raise ValueError(f"U has {U.size} entries, n*K = {n * K}")
    rows = np.empty(max(1, n * K), dtype=np.int32)
    L = ctypes.c_int32()
    _check("pe_cod_rows", load().pe_cod_rows(n, K, r, floor_rate, U.ctypes.data, rows.ctypes.data,
                                             ctypes.byref(L)))
    return rows[:L.value].copy()


def pe_partition(n: int, K: int, S: int, rows):
    """Host partition of kept rows into S chunks -> int32 chunk index per row."""
    import numpy as np
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    out = np.empty(max(1, rows.size), dtype=np.int32)
    _check("pe_partition", load().pe_partition(n, K, S, rows.ctypes.data, rows.size, out.ctypes.data))
    return out[:rows.size].copy()


def pe_partition_chunk(n: int, K: int, S: int, s: int, rows):
    """Cells of chunk s -> (cells int32 [Lc], n_lead, out_rows int32 [Lc - n_lead], n_chunk)."""
    import numpy as np
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    cells = np.empty(max(1, rows.size), dtype=np.int32)
    out_rows = np.empty(max(1, rows.size), dtype=np.int32)
    Lc, lead, nc = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check("pe_partition_chunk", load().pe_partition_chunk(
        n, K, S, s, rows.ctypes.data, rows.size, cells.ctypes.data, out_rows.ctypes.data, ctypes.byref(Lc),
        ctypes.byref(lead), ctypes.byref(nc)))
    return cells[:Lc.value].copy(), lead.value, out_rows[:Lc.value - lead.value].copy(), nc.value

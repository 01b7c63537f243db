"""Device-side helpers around the C ABI for tests, the smoke check and the
benchmark.  PyTorch is used only to hold device memory and to supply the
HIP stream; all drafter arithmetic runs in libpeagle.so.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as pe


def _dtype(cfg) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def to_device(a, cfg, device) -> torch.Tensor:
    """float32 host array holding dtype-exact values -> device tensor of the dtype."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    return t.to(_dtype(cfg)) if cfg.dtype == "bf16" else t


def stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream


class Drafter:
    """A pe_model built from host weights (dict from synth.drafter_weights)."""

    def __init__(self, cfg, weights, device="cuda:0", backward=False):
        self.cfg = cfg
        self.device = torch.device(device)
        torch.cuda.set_device(self.device)
        self.embed = to_device(weights["embed"], cfg, self.device)  # kept: read by reference
        keep = []

        def dev(a):
            t = to_device(a, cfg, self.device)
            keep.append(t)
            return t.data_ptr()

        layers = (pe.PeLayerWeights * max(1, cfg.n_layers))()
        for l, lw in enumerate(weights["layers"]):
            layers[l] = pe.PeLayerWeights(*[dev(lw[k]) for k in (
                "attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")])
        w = pe.PeWeights(self.embed.data_ptr(), dev(weights["fc"]), dev(weights["final_norm"]),
                         dev(weights["lm_head"]), layers)
        c = pe.PeConfig(cfg.hidden, cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                        cfg.intermediate, cfg.vocab, cfg.rope_theta, cfg.rms_eps,
                        pe.PE_BF16 if cfg.dtype == "bf16" else pe.PE_F32)
        self.handle = pe.pe_model_create(c, w, stream_handle())
        if backward:
            pe.pe_model_prepare_backward(self.handle, w, stream_handle())
        del keep  # the model holds its own tiled copies of every weight but the embedding

    def close(self):
        if self.handle:
            pe.pe_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace(self, B, K, ctx_stride):
        n = pe.pe_draft_workspace_size(self.handle, B, K, ctx_stride)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        pe.pe_workspace_init(ws.data_ptr(), ws.numel(), stream_handle())
        return ws


class DecodeBuffers:
    """Device copies of one decode call's inputs plus its outputs."""

    def __init__(self, drafter: Drafter, inp, N=None, want_logits=False):
        cfg, dev = drafter.cfg, drafter.device
        self.N = cfg.n_layers if N is None else N
        self.K = int(inp["K"])
        self.B = int(len(inp["token_ids"]))
        self.ctx_stride = int(inp["ctx_stride"])
        self.hidden3 = to_device(inp["hidden3"], cfg, dev)
        self.token_ids = torch.from_numpy(np.asarray(inp["token_ids"], np.int32)).to(dev)
        self.mask_emb = to_device(inp["mask_emb"], cfg, dev)
        self.h_shared = to_device(inp["h_shared"], cfg, dev)
        self.ctx_lens = torch.from_numpy(np.asarray(inp["ctx_lens"], np.int32)).to(dev)
        self.k_cache = [to_device(k, cfg, dev) for k in inp["k_cache"][:self.N]]
        self.v_cache = [to_device(v, cfg, dev) for v in inp["v_cache"][:self.N]]
        self.draft = torch.full((self.B, self.K), -1, dtype=torch.int32, device=dev)
        self.logits = (torch.empty((self.B, self.K, cfg.vocab), dtype=torch.float32, device=dev)
                       if want_logits else None)
        self.ws = drafter.workspace(self.B, self.K, self.ctx_stride)

    def launch(self, drafter: Drafter, stream: int | None = None):
        pe.pe_draft_forward(
            drafter.handle, self.N, self.B, self.K, self.hidden3.data_ptr(),
            self.token_ids.data_ptr(), self.mask_emb.data_ptr(), self.h_shared.data_ptr(),
            self.ctx_lens.data_ptr(), self.ctx_stride,
            [t.data_ptr() for t in self.k_cache], [t.data_ptr() for t in self.v_cache],
            self.draft.data_ptr(), self.logits.data_ptr() if self.logits is not None else None,
            self.ws.data_ptr(), self.ws.numel(), stream_handle() if stream is None else stream)


def cache_with_room(cache, extra):
    """Device copy of one layer's cache [B, nkv, C, hd] with `extra` more positions."""
    B, nkv, C, hd = cache.shape
    out = torch.zeros((B, nkv, C + extra, hd), dtype=cache.dtype, device=cache.device)
    out[:, :, :C] = cache
    return out


class ExtendBuffers:
    """One drafter-cache extension call (pe_draft_extend) on device buffers.

    inputs: host array [B, T, 3H] (kind PE_INPUT_TARGET, dtype data) or
    [B, T, H] fp32 (PE_INPUT_DRAFTER).  The caches (lists of device tensors
    [B, nkv, C, hd]) are extended in place.
    """

    def __init__(self, drafter: Drafter, inputs, kind, token_ids, ctx_lens, k_cache, v_cache, N=None,
                 pos_offset=0, want_draft=True, want_logits=True, want_z=True):
        cfg, dev = drafter.cfg, drafter.device
        self.N = cfg.n_layers if N is None else N
        inputs = np.asarray(inputs)
        self.B, self.T = inputs.shape[0], inputs.shape[1]
        self.kind = kind
        self.pos_offset = pos_offset
        if kind == pe.PE_INPUT_TARGET:
            self.inputs = to_device(inputs, cfg, dev)
        else:
            self.inputs = torch.from_numpy(np.ascontiguousarray(inputs, np.float32)).to(dev)
        self.tok = torch.from_numpy(np.ascontiguousarray(token_ids, np.int32)).to(dev)
        self.ctx_lens = torch.from_numpy(np.asarray(ctx_lens, np.int32)).to(dev)
        self.k_cache, self.v_cache = list(k_cache)[:self.N], list(v_cache)[:self.N]
        self.ctx_stride = int(self.k_cache[0].shape[2]) if self.N > 0 else 1
        B, T = self.B, self.T
        self.draft = torch.full((B, T), -1, dtype=torch.int32, device=dev) if want_draft else None
        self.logits = (torch.empty((B, T, cfg.vocab), dtype=torch.float32, device=dev)
                       if want_logits else None)
        self.z = torch.empty((B, T, cfg.hidden), dtype=torch.float32, device=dev) if want_z else None
        self.ws = drafter.workspace(B, T, self.ctx_stride)

    def launch(self, drafter: Drafter, stream: int | None = None):
        pe.pe_draft_extend(
            drafter.handle, self.N, self.B, self.T, self.inputs.data_ptr(), self.kind, self.tok.data_ptr(),
            self.ctx_lens.data_ptr(), self.pos_offset, self.ctx_stride,
            [t.data_ptr() for t in self.k_cache], [t.data_ptr() for t in self.v_cache],
            self.draft.data_ptr() if self.draft is not None else None,
            self.logits.data_ptr() if self.logits is not None else None,
            self.z.data_ptr() if self.z is not None else None,
            self.ws.data_ptr(), self.ws.numel(), stream_handle() if stream is None else stream)


class Eagle3Chain:
    """The autoregressive EAGLE-3 drafter on the library's kernels: K
    sequential one-row cache extensions per sequence.  Step 0 takes the new
    token and the target hidden state; step j > 0 takes step j-1's draft
    token and its final-norm output, at pos_offset j.  All steps are enqueued
    on the device with no host synchronisation; caches get K spare positions."""

    def __init__(self, drafter: Drafter, inp, K, N=None, want_logits=False):
        cfg, dev = drafter.cfg, drafter.device
        self.N = cfg.n_layers if N is None else N
        self.K = K
        self.B = B = int(len(inp["token_ids"]))
        self.hidden3 = to_device(inp["hidden3"], cfg, dev)
        self.tok0 = torch.from_numpy(np.asarray(inp["token_ids"], np.int32)).to(dev)
        self.ctx_lens = torch.from_numpy(np.asarray(inp["ctx_lens"], np.int32)).to(dev)
        C = int(inp["ctx_stride"])
        self.k_cache = [cache_with_room(to_device(k, cfg, dev), K) for k in inp["k_cache"][:self.N]]
        self.v_cache = [cache_with_room(to_device(v, cfg, dev), K) for v in inp["v_cache"][:self.N]]
        self.ctx_stride = C + K
        self.drafts = torch.full((K, B), -1, dtype=torch.int32, device=dev)
        self.logits = (torch.empty((K, B, cfg.vocab), dtype=torch.float32, device=dev)
                       if want_logits else None)
        self.z = torch.empty((2, B, cfg.hidden), dtype=torch.float32, device=dev)
        self.ws = drafter.workspace(B, 1, self.ctx_stride)

    def launch(self, drafter: Drafter, stream: int | None = None):
        s = stream_handle() if stream is None else stream
        kc = [t.data_ptr() for t in self.k_cache]
        vc = [t.data_ptr() for t in self.v_cache]
        for j in range(self.K):
            if j == 0:
                inputs, kind, tok = self.hidden3.data_ptr(), pe.PE_INPUT_TARGET, self.tok0.data_ptr()
            else:
                inputs, kind = self.z[(j - 1) % 2].data_ptr(), pe.PE_INPUT_DRAFTER
                tok = self.drafts[j - 1].data_ptr()
            pe.pe_draft_extend(drafter.handle, self.N, self.B, 1, inputs, kind, tok, self.ctx_lens.data_ptr(), j,
                               self.ctx_stride, kc, vc, self.drafts[j].data_ptr(),
                               self.logits[j].data_ptr() if self.logits is not None else None,
                               self.z[j % 2].data_ptr(), self.ws.data_ptr(), self.ws.numel(), s)

    def result(self):
        """(drafts [B, K], logits [B, K, V] or None) on host."""
        torch.cuda.synchronize()
        d = self.drafts.cpu().numpy().T.copy()
        lg = self.logits.cpu().numpy().transpose(1, 0, 2).copy() if self.logits is not None else None
        return d, lg


def draft_forward(drafter: Drafter, inp, N=None, want_logits=False):
    """Run one forward; returns (draft [B,K] int32, logits [B,K,V] float32 or None) on host."""
    buf = DecodeBuffers(drafter, inp, N=N, want_logits=want_logits)
    buf.launch(drafter)
    torch.cuda.synchronize()
    return (buf.draft.cpu().numpy(),
            buf.logits.cpu().numpy() if buf.logits is not None else None)


def accept(draft: np.ndarray, target: np.ndarray, device="cuda:0", with_tokens=True):
    """Greedy acceptance on the GPU; returns (accept_len [B], out_tokens [B,K+1] or None)."""
    draft = np.ascontiguousarray(draft, np.int32)
    target = np.ascontiguousarray(target, np.int32)
    B, K = draft.shape
    d = torch.from_numpy(draft).to(device)
    t = torch.from_numpy(target).to(device)
    a = torch.full((max(B, 1),), -7, dtype=torch.int32, device=device)
    o = torch.full((max(B, 1), K + 1), -7, dtype=torch.int32, device=device) if with_tokens else None
    pe.pe_accept(B, K, d.data_ptr(), t.data_ptr(), a.data_ptr(),
                 o.data_ptr() if o is not None else None, stream_handle())
    torch.cuda.synchronize()
    return a.cpu().numpy()[:B], (o.cpu().numpy()[:B] if o is not None else None)


class TrainMask:
    """The amortized mask handle, built once for sequences of up to n_max positions."""

    def __init__(self, n_max: int, K: int):
        self.n_max, self.K = n_max, K
        self.handle = pe.pe_mask_create(n_max, K, stream_handle())

    def close(self):
        if self.handle:
            pe.pe_mask_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def materialize(self, n: int, rows, device="cuda:0") -> np.ndarray:
        """Dense boolean mask [L, L] of kept rows ``rows`` (tiny sizes only)."""
        r = torch.from_numpy(np.ascontiguousarray(rows, np.int32)).to(device)
        L = r.numel()
        out = torch.full((L, L), 7, dtype=torch.uint8, device=device)
        pe.pe_mask_materialize(self.handle, n, r.data_ptr(), L, out.data_ptr(), stream_handle())
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def materialize_device(self, n: int, rows_dev: torch.Tensor) -> torch.Tensor:
        L = rows_dev.numel()
        out = torch.empty((L, L), dtype=torch.uint8, device=rows_dev.device)
        pe.pe_mask_materialize(self.handle, n, rows_dev.data_ptr(), L, out.data_ptr(), stream_handle())
        return out


class TrainBuffers:
    """Device copies of one training-shape call's inputs plus its outputs."""

    def __init__(self, drafter: Drafter, mask: TrainMask, inp, rows, N=None, want_logits=True,
                 want_argmax=True):
        cfg, dev = drafter.cfg, drafter.device
        self.N = cfg.n_layers if N is None else N
        self.n = int(len(inp["token_ids"]))
        self.K = mask.K
        self.hidden3 = to_device(inp["hidden3"], cfg, dev)
        self.token_ids = torch.from_numpy(np.asarray(inp["token_ids"], np.int32)).to(dev)
        self.mask_emb = to_device(inp["mask_emb"], cfg, dev)
        self.h_shared = to_device(inp["h_shared"], cfg, dev)
        self.rows = torch.from_numpy(np.ascontiguousarray(rows, np.int32)).to(dev)
        self.L = int(self.rows.numel())
        self.logits = (torch.empty((self.L, cfg.vocab), dtype=_dtype(cfg), device=dev)
                       if want_logits else None)
        self.argmax = (torch.full((self.L,), -1, dtype=torch.int32, device=dev)
                       if want_argmax else None)
        nbytes = pe.pe_train_workspace_size(drafter.handle, self.n, self.K, self.L)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        pe.pe_workspace_init(self.ws.data_ptr(), self.ws.numel(), stream_handle())

    def launch(self, drafter: Drafter, mask: TrainMask, stream: int | None = None):
        pe.pe_train_forward(
            drafter.handle, mask.handle, self.N, self.n, self.K, self.hidden3.data_ptr(),
            self.token_ids.data_ptr(), self.mask_emb.data_ptr(), self.h_shared.data_ptr(),
            self.rows.data_ptr(), self.L,
            self.logits.data_ptr() if self.logits is not None else None,
            self.argmax.data_ptr() if self.argmax is not None else None,
            self.ws.data_ptr(), self.ws.numel(), stream_handle() if stream is None else stream)


def train_forward(drafter: Drafter, mask: TrainMask, inp, rows, N=None, want_logits=True):
    """Run one training-shape forward; returns (argmax [L] int32, logits [L,V] float32 or None) on host."""
    buf = TrainBuffers(drafter, mask, inp, rows, N=N, want_logits=want_logits)
    buf.launch(drafter, mask)
    torch.cuda.synchronize()
    return (buf.argmax.cpu().numpy(),
            buf.logits.float().cpu().numpy() if buf.logits is not None else None)


class PartitionedTrain:
    """The training-shape forward as S independent chunk forwards (sequence
    partition: each chunk runs its own cells plus its depth-0 completion and
    writes its own rows of the whole sequence's outputs).  Chunk layouts
    come from the library's host partition; one workspace serves the
    largest chunk, and the chunks run one after another on one stream."""

    def __init__(self, drafter: Drafter, mask: TrainMask, inp, rows, S, N=None, want_logits=True):
        cfg, dev = drafter.cfg, drafter.device
        self.N = cfg.n_layers if N is None else N
        self.n = n = int(len(inp["token_ids"]))
        self.K = K = mask.K
        self.S = S
        rows = np.ascontiguousarray(rows, np.int32)
        self.L = int(rows.size)
        self.hidden3 = to_device(inp["hidden3"], cfg, dev)
        self.token_ids = torch.from_numpy(np.asarray(inp["token_ids"], np.int32)).to(dev)
        self.mask_emb = to_device(inp["mask_emb"], cfg, dev)
        self.h_shared = to_device(inp["h_shared"], cfg, dev)
        self.chunks = []
        ws_bytes = 256
        for s in range(S):
            cells, lead, out_rows, nc = pe.pe_partition_chunk(n, K, S, s, rows)
            self.chunks.append((torch.from_numpy(cells).to(dev), lead,
                                torch.from_numpy(out_rows).to(dev) if out_rows.size else None, nc))
            ws_bytes = max(ws_bytes, pe.pe_train_workspace_size(drafter.handle, nc, K, int(cells.size)))
        self.cells_total = sum(int(c[0].numel()) for c in self.chunks)
        self.logits = (torch.empty((self.L, cfg.vocab), dtype=_dtype(cfg), device=dev)
                       if want_logits else None)
        self.argmax = torch.full((self.L,), -1, dtype=torch.int32, device=dev)
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        pe.pe_workspace_init(self.ws.data_ptr(), self.ws.numel(), stream_handle())

    def launch(self, drafter: Drafter, mask: TrainMask, stream: int | None = None):
        st = stream_handle() if stream is None else stream
        for cells, lead, out_rows, nc in self.chunks:
            pe.pe_train_forward_chunk(
                drafter.handle, mask.handle, self.N, nc, self.K, self.hidden3.data_ptr(),
                self.token_ids.data_ptr(), self.mask_emb.data_ptr(), self.h_shared.data_ptr(),
                cells.data_ptr(), int(cells.numel()), lead,
                out_rows.data_ptr() if out_rows is not None else None, self.L,
                self.logits.data_ptr() if self.logits is not None else None, self.argmax.data_ptr(),
                self.ws.data_ptr(), self.ws.numel(), st)

    def result(self):
        torch.cuda.synchronize()
        return (self.argmax.cpu().numpy(),
                self.logits.float().cpu().numpy() if self.logits is not None else None)


LAYER_GRADS = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


class Grads:
    """Zeroed fp32 gradient buffers on the device in the weights' layouts,
    accumulated by pe_train_step calls."""

    def __init__(self, cfg, n, N=None, device="cuda:0"):
        N = cfg.n_layers if N is None else N
        H, I, hd = cfg.hidden, cfg.intermediate, cfg.head_dim
        nq, nkv, V = cfg.n_q_heads, cfg.n_kv_heads, cfg.vocab
        z = lambda *shape: torch.zeros(shape, dtype=torch.float32, device=device)
        self.t = {"fc": z(H, 3 * H), "final_norm": z(H), "lm_head": z(V, H), "mask_emb": z(H),
                  "h_shared": z(3 * H), "embed_rows": z(n, H)}
        shapes = {"attn_norm": (H,), "wq": (nq * hd, H), "wk": (nkv * hd, H), "wv": (nkv * hd, H),
                  "wo": (H, nq * hd), "mlp_norm": (H,), "w_gate": (I, H), "w_up": (I, H), "w_down": (H, I)}
        self.layers = [{k: z(*shapes[k]) for k in LAYER_GRADS} for _ in range(N)]
        self._lg = (pe.PeLayerGrads * max(1, N))()
        for l, g in enumerate(self.layers):
            self._lg[l] = pe.PeLayerGrads(*[g[k].data_ptr() for k in LAYER_GRADS])
        self.c = pe.PeGrads(*[self.t[k].data_ptr() for k in ("fc", "final_norm", "lm_head", "mask_emb",
                                                               "h_shared", "embed_rows")], self._lg)

    def numpy(self):
        torch.cuda.synchronize()
        out = {k: v.cpu().numpy() for k, v in self.t.items()}
        out["layers"] = [{k: v.cpu().numpy() for k, v in g.items()} for g in self.layers]
        return out


class TrainStep:
    """One pe_train_step call (forward, loss, backward) on device buffers.

    cells: kept cells (whole sequence, or one chunk's cells with n_lead);
    labels: host int [n] (label of position p; negative: not scored);
    loss_scale defaults to 1 / (number of scored cells)."""

    def __init__(self, drafter: Drafter, mask: TrainMask, inp, cells, labels, N=None, n_lead=0, n=None,
                 loss_scale=None, grads: Grads | None = None):
        cfg, dev = drafter.cfg, drafter.device
        self.N = cfg.n_layers if N is None else N
        self.n = int(len(inp["token_ids"])) if n is None else n
        self.K = mask.K
        self.hidden3 = to_device(inp["hidden3"], cfg, dev)
        self.token_ids = torch.from_numpy(np.asarray(inp["token_ids"], np.int32)).to(dev)
        self.mask_emb = to_device(inp["mask_emb"], cfg, dev)
        self.h_shared = to_device(inp["h_shared"], cfg, dev)
        cells = np.ascontiguousarray(cells, np.int32)
        self.cells = torch.from_numpy(cells).to(dev)
        self.L = int(cells.size)
        self.n_lead = n_lead
        labels = np.asarray(labels, np.int32)
        self.labels = torch.from_numpy(labels).to(dev)
        if loss_scale is None:
            pos = cells[n_lead:] // self.K
            loss_scale = 1.0 / max(1, int(np.sum(labels[pos] >= 0)))
        self.loss_scale = float(loss_scale)
        self.loss = torch.zeros(1, dtype=torch.float32, device=dev)
        self.grads = grads if grads is not None else Grads(cfg, int(len(inp["token_ids"])), self.N, dev)
        nbytes = pe.pe_train_step_workspace_size(drafter.handle, self.N, self.n, self.K, self.L)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        pe.pe_workspace_init(self.ws.data_ptr(), self.ws.numel(), stream_handle())

    def launch(self, drafter: Drafter, mask: TrainMask, stream: int | None = None):
        pe.pe_train_step(drafter.handle, mask.handle, self.N, self.n, self.K, self.hidden3.data_ptr(),
                         self.token_ids.data_ptr(), self.mask_emb.data_ptr(), self.h_shared.data_ptr(),
                         self.cells.data_ptr(), self.L, self.n_lead, self.labels.data_ptr(), self.loss_scale,
                         self.loss.data_ptr(), self.grads.c, self.ws.data_ptr(), self.ws.numel(),
                         stream_handle() if stream is None else stream)

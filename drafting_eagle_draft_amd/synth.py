"""Seeded synthetic inputs shaped like the P-EAGLE drafter workloads.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the drafter's arithmetic, so both the CPU oracle tests and
the GPU path can take their inputs from it without sharing any computation.

Every tensor is drawn from NumPy's PCG64 in row chunks, each chunk seeded by
(config seed, crc32(tensor name), chunk index).  Any row range can therefore
be regenerated on its own, and large tensors are drawn by several threads.

Recipe (the same for every workload):
  * projection matrices, embedding table, fc, LM head, mask embedding:
    N(0, 0.02);
  * RMSNorm gains: 1.0 (``gain_jitter`` > 0 gives 1 + N(0, jitter), used to
    catch gain-indexing mistakes);
  * target hidden states (3H wide) and the shared hidden state: N(0, 1);
  * token ids: uniform on [0, V);
  * cached keys and values (already rotated): N(0, 1);
  * ragged context lengths: uniform on [lo, hi];
  * COD uniforms: U[0, 1) per (position, depth) grid cell.

Values are returned as float32 arrays that hold the exact value of the
storage dtype (bf16-rounded with round-to-nearest-even for bf16 configs).
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

__all__ = [
    "DrafterShape", "CONFIGS", "config", "tensor", "drafter_weights",
    "decode_inputs", "train_inputs", "cod_uniforms", "planted_targets",
    "ACCEPT_TABLE_AVERAGE",
]

_CHUNK_ELEMS = 1 << 22  # elements per seeded chunk (rows are grouped to about this many)


@dataclass(frozen=True)
class DrafterShape:
    """Shape of one synthetic workload."""
    name: str
    seed: int
    hidden: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    vocab: int
    K: int
    dtype: str  # "f32" or "bf16"
    rope_theta: float = 500000.0
    rms_eps: float = 1e-5
    # decode workloads
    batch: int = 0
    ctx: int = 0                 # fixed context length (0 when ragged)
    ctx_range: tuple = ()        # (lo, hi) inclusive for ragged contexts
    # training-shape workload
    seq_len: int = 0
    n_max: int = 0
    cod_rate: float = 0.8
    cod_floor: float = 0.2
    extra: dict = field(default_factory=dict)

    @property
    def ctx_stride(self) -> int:
        return self.ctx if self.ctx else (self.ctx_range[1] if self.ctx_range else 0)


CONFIGS = {
    "tiny_f32": DrafterShape(
        name="tiny_f32", seed=1001, hidden=256, n_layers=1, n_q_heads=4, n_kv_heads=2,
        head_dim=64, intermediate=1024, vocab=4096, K=4, dtype="f32", batch=1, ctx=64),
    "gptoss20b_k8_ctx4k": DrafterShape(
        name="gptoss20b_k8_ctx4k", seed=1002, hidden=2880, n_layers=4, n_q_heads=64,
        n_kv_heads=8, head_dim=64, intermediate=8192, vocab=201088, K=8, dtype="bf16",
        batch=2, ctx=4096),
    "gptoss20b_k8_ctx16k": DrafterShape(
        name="gptoss20b_k8_ctx16k", seed=1003, hidden=2880, n_layers=4, n_q_heads=64,
        n_kv_heads=8, head_dim=64, intermediate=8192, vocab=201088, K=8, dtype="bf16",
        batch=2, ctx=16384),
    "qwen3coder30b_k8_ragged": DrafterShape(
        name="qwen3coder30b_k8_ragged", seed=1004, hidden=2048, n_layers=4, n_q_heads=32,
        n_kv_heads=4, head_dim=128, intermediate=6144, vocab=151936, K=8, dtype="bf16",
        batch=4, ctx_range=(1024, 8192)),
    "train_gptoss20b_n8192_k8": DrafterShape(
        name="train_gptoss20b_n8192_k8", seed=1005, hidden=2880, n_layers=1, n_q_heads=64,
        n_kv_heads=8, head_dim=64, intermediate=8192, vocab=201088, K=8, dtype="bf16",
        seq_len=8192, n_max=20480, cod_rate=0.8, cod_floor=0.2),
}


def config(name: str, **overrides) -> DrafterShape:
    """Return a named workload shape, optionally with fields replaced."""
    cfg = CONFIGS[name]
    return replace(cfg, **overrides) if overrides else cfg


def _round_bf16_inplace(x: np.ndarray) -> None:
    """Round float32 values in place to the nearest bf16 (ties to even)."""
    u = x.view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def tensor(seed: int, name: str, shape, std: float = 1.0, mean: float = 0.0,
           dtype: str = "bf16", rows: tuple | None = None) -> np.ndarray:
    """Draw N(mean, std) of ``shape`` (rows = shape[0]) rounded to ``dtype``.

    ``rows=(r0, r1)`` returns only that row range, bit-identical to the same
    rows of the full tensor.
    """
    shape = tuple(int(s) for s in shape)
    nrows = shape[0]
    row_elems = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    rows_per_chunk = max(1, _CHUNK_ELEMS // max(1, row_elems))
    r0, r1 = rows if rows is not None else (0, nrows)
    tid = zlib.crc32(name.encode())
    out = np.empty((r1 - r0,) + shape[1:], dtype=np.float32)
    flat = out.reshape(r1 - r0, row_elems)
    c0, c1 = r0 // rows_per_chunk, (r1 - 1) // rows_per_chunk if r1 > r0 else -1

    def work(c):
        cr0 = c * rows_per_chunk
        cr1 = min(nrows, cr0 + rows_per_chunk)
        rng = np.random.Generator(np.random.PCG64([seed, tid, c]))
        blk = rng.standard_normal((cr1 - cr0) * row_elems, dtype=np.float32)
        blk = blk.reshape(cr1 - cr0, row_elems)
        lo, hi = max(cr0, r0), min(cr1, r1)
        sub = blk[lo - cr0:hi - cr0]
        sub *= np.float32(std)
        if mean:
            sub += np.float32(mean)
        if dtype == "bf16":
            sub = np.ascontiguousarray(sub)
            _round_bf16_inplace(sub)
        flat[lo - r0:hi - r0] = sub

    chunks = list(range(c0, c1 + 1))
    if len(chunks) > 1:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, chunks))
    else:
        for c in chunks:
            work(c)
    return out


def _gain(cfg: DrafterShape, name: str, n: int, jitter: float) -> np.ndarray:
    if jitter <= 0:
        return np.ones(n, dtype=np.float32)
    return tensor(cfg.seed, name, (n,), std=jitter, mean=1.0, dtype=cfg.dtype)


def drafter_weights(cfg: DrafterShape, gain_jitter: float = 0.0, with_embed: bool = True):
    """All drafter parameters as a dict of float32 arrays in [out, in] layout."""
    H, I, V = cfg.hidden, cfg.intermediate, cfg.vocab
    qd, kd = cfg.n_q_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
    s, dt = cfg.seed, cfg.dtype
    w = {
        "fc": tensor(s, "fc", (H, 3 * H), 0.02, dtype=dt),
        "final_norm": _gain(cfg, "final_norm", H, gain_jitter),
        "lm_head": tensor(s, "lm_head", (V, H), 0.02, dtype=dt),
        "layers": [],
    }
    if with_embed:
        w["embed"] = tensor(s, "embed", (V, H), 0.02, dtype=dt)
    for l in range(cfg.n_layers):
        p = f"layer{l}."
        w["layers"].append({
            "attn_norm": _gain(cfg, p + "attn_norm", H, gain_jitter),
            "wq": tensor(s, p + "wq", (qd, H), 0.02, dtype=dt),
            "wk": tensor(s, p + "wk", (kd, H), 0.02, dtype=dt),
            "wv": tensor(s, p + "wv", (kd, H), 0.02, dtype=dt),
            "wo": tensor(s, p + "wo", (H, qd), 0.02, dtype=dt),
            "mlp_norm": _gain(cfg, p + "mlp_norm", H, gain_jitter),
            "w_gate": tensor(s, p + "w_gate", (I, H), 0.02, dtype=dt),
            "w_up": tensor(s, p + "w_up", (I, H), 0.02, dtype=dt),
            "w_down": tensor(s, p + "w_down", (H, I), 0.02, dtype=dt),
        })
    return w


def embed_rows(cfg: DrafterShape, ids) -> np.ndarray:
    """Rows ``ids`` of the embedding table without drawing the whole table."""
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    out = np.empty((len(ids), cfg.hidden), dtype=np.float32)
    for i, t in enumerate(ids):
        out[i] = tensor(cfg.seed, "embed", (cfg.vocab, cfg.hidden), 0.02, dtype=cfg.dtype,
                        rows=(int(t), int(t) + 1))[0]
    return out


def decode_inputs(cfg: DrafterShape, batch: int | None = None, ctx_lens=None,
                  ctx_stride: int | None = None, K: int | None = None, tag: str = ""):
    """Per-call inputs of one parallel-drafting step.

    Cache layout is [n_layers][B, n_kv_heads, ctx_stride, head_dim]; positions
    at or beyond a sequence's context length hold draws too but are never read.
    """
    B = cfg.batch if batch is None else batch
    K = cfg.K if K is None else K
    s, dt, H, V = cfg.seed, cfg.dtype, cfg.hidden, cfg.vocab
    rng = np.random.Generator(np.random.PCG64([s, zlib.crc32(("ids" + tag).encode())]))
    token_ids = rng.integers(0, V, size=B, dtype=np.int64).astype(np.int32)
    if ctx_lens is None:
        if cfg.ctx:
            ctx_lens = np.full(B, cfg.ctx, dtype=np.int32)
        else:
            lo, hi = cfg.ctx_range
            ctx_lens = rng.integers(lo, hi + 1, size=B, dtype=np.int64).astype(np.int32)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    C = int(ctx_stride if ctx_stride is not None else max(int(ctx_lens.max()), 1))
    if cfg.ctx_stride and ctx_stride is None:
        C = max(C, cfg.ctx_stride)
    kv_shape = (B, cfg.n_kv_heads, C, cfg.head_dim)
    k_cache = [tensor(s, f"kcache{l}{tag}", kv_shape, 1.0, dtype=dt) for l in range(cfg.n_layers)]
    v_cache = [tensor(s, f"vcache{l}{tag}", kv_shape, 1.0, dtype=dt) for l in range(cfg.n_layers)]
    return {
        "K": K,
        "hidden3": tensor(s, "hidden3" + tag, (B, 3 * H), 1.0, dtype=dt),
        "token_ids": token_ids,
        "mask_emb": tensor(s, "mask_emb", (H,), 0.02, dtype=dt),
        "h_shared": tensor(s, "h_shared", (3 * H,), 1.0, dtype=dt),
        "ctx_lens": ctx_lens,
        "ctx_stride": C,
        "k_cache": k_cache,
        "v_cache": v_cache,
    }


def cod_uniforms(cfg: DrafterShape, n: int, K: int, tag: str = "") -> np.ndarray:
    """U[0,1) per (position, depth) cell; the COD keep test consumes these."""
    rng = np.random.Generator(np.random.PCG64([cfg.seed, zlib.crc32(("cod" + tag).encode())]))
    return rng.random((n, K))


def train_inputs(cfg: DrafterShape, n: int | None = None, tag: str = ""):
    """Per-sequence inputs of the training-shape forward."""
    n = cfg.seq_len if n is None else n
    s, dt, H, V = cfg.seed, cfg.dtype, cfg.hidden, cfg.vocab
    rng = np.random.Generator(np.random.PCG64([s, zlib.crc32(("tids" + tag).encode())]))
    return {
        "hidden3": tensor(s, "train_hidden3" + tag, (n, 3 * H), 1.0, dtype=dt),
        "token_ids": rng.integers(0, V, size=n, dtype=np.int64).astype(np.int32),
        "mask_emb": tensor(s, "mask_emb", (H,), 0.02, dtype=dt),
        "h_shared": tensor(s, "h_shared", (3 * H,), 1.0, dtype=dt),
    }


# Per-position acceptance rates (fraction of rounds in which draft position k
# was accepted), Average row of the acceptance table in "Speeding LLM
# inference with P-EAGLE in vLLM Speculators", section "Example model".
# Position 8 extends the table geometrically (ratio of the last two entries).
ACCEPT_TABLE_AVERAGE = (0.749, 0.499, 0.319, 0.204, 0.131, 0.085, 0.055)


def planted_targets(drafts: np.ndarray, V: int, seed: int, rates=ACCEPT_TABLE_AVERAGE):
    """Target tokens that agree with ``drafts`` on a random prefix.

    For each sequence a break point a is drawn so that P(a >= k) follows
    ``rates`` (extended geometrically to K); target[:a] = drafts[:a],
    target[a] differs from drafts[a] (when a < K), the rest is uniform.
    """
    drafts = np.asarray(drafts, dtype=np.int64)
    B, K = drafts.shape
    surv = list(rates)
    while len(surv) < K:
        surv.append(surv[-1] * (surv[-1] / surv[-2]))
    surv = np.array([1.0] + surv[:K])  # P(a >= k) for k = 0..K
    rng = np.random.Generator(np.random.PCG64([seed, zlib.crc32(b"planted")]))
    u = rng.random(B)
    a = np.array([int(np.sum(surv[1:] > ui)) for ui in u])  # a >= k iff u < surv[k]
    tgt = rng.integers(0, V, size=(B, K + 1), dtype=np.int64)
    for b in range(B):
        tgt[b, :a[b]] = drafts[b, :a[b]]
        if a[b] < K and tgt[b, a[b]] == drafts[b, a[b]]:
            tgt[b, a[b]] = (drafts[b, a[b]] + 1) % V
    return tgt.astype(np.int32), a

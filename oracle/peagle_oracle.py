"""CPU oracle for the P-EAGLE parallel-drafter hot path (NumPy, float64).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP
library and imports nothing from it; it is slow and plain on purpose, so that
each step can be checked against the pages by eye.

Sources (cited by page title and section):
  [RH] "Speeding LLM inference with P-EAGLE in vLLM Speculators"
       (Red Hat Developer): sections "COD sampling", "A learnable mask
       parameter", "Flex-attention mask", "Example model".
  [TD] "P-EAGLE: A Technical Deep Dive into Parallel Speculative Decoding":
       section "2. The P-EAGLE Parallel Drafter", "Memory and Training
       Complexity".
  [PN] "P-EAGLE: Parallel-Drafting EAGLE with Scalable Training" (notes on
       arXiv:2602.01469): section 2 (architecture), 3.1 (amortized mask
       construction), 3.2 (sequence partitioning), appendix B (RoPE).
  [E4] "EAGLE-4" (lightseek.org): "EAGLE-4 overview" (accepted prefix plus one
       bonus token).

Readings where the pages leave a step open (each is listed with its reason in
the design notes): fusion of token embedding and projected hidden state is an
addition; h_shared is 3H wide and goes through the same fc; RMSNorm eps 1e-5;
rotate-half RoPE with frequencies theta^(-2i/hd); a final RMSNorm before an
untied LM head; ties in argmax go to the lowest index; COD keeps a child with
conditional probability r given its parent (marginal r^d, floored at 0.2).

Every function here is pinned by tests in tests/ against closed forms,
invariants, brute force or values the pages print; see each docstring.
"""
from __future__ import annotations

import math
import numpy as np

F64 = np.float64

# ---------------------------------------------------------------------------
# Elementary pieces of a LLaMA-3 style decoder layer ([PN] section 2 names the
# layer family; the formulas are the standard ones).
# ---------------------------------------------------------------------------


def rmsnorm(x, gain, eps):
    """x / sqrt(mean(x^2) + eps) * gain over the last axis."""
    x = np.asarray(x, dtype=F64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=F64)


def rope_inv_freq(head_dim, theta):
    """Angular frequency of each rotated pair: theta^(-2i/head_dim)."""
    i = np.arange(head_dim // 2, dtype=F64)
    return np.power(F64(theta), -2.0 * i / head_dim)


def rope(a, pos, theta):
    """Rotate-half RoPE of vectors ``a`` [..., hd] at position(s) ``pos``.

    Pair (i, i + hd/2) is rotated by angle pos * theta^(-2i/hd).  ``pos`` may
    be a scalar or broadcast against a[..., 0].
    """
    a = np.asarray(a, dtype=F64)
    hd = a.shape[-1]
    half = hd // 2
    phi = np.asarray(pos, dtype=F64)[..., None] * rope_inv_freq(hd, theta)
    c, s = np.cos(phi), np.sin(phi)
    lo, hi = a[..., :half], a[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def silu(z):
    """z * sigmoid(z)."""
    z = np.asarray(z, dtype=F64)
    return z / (1.0 + np.exp(-z))


def softmax(s):
    """Max-subtracted softmax over the last axis."""
    s = np.asarray(s, dtype=F64)
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def linear(x, w, chunk_rows=16384):
    """x @ w.T in float64 for w in [out, in] layout.

    The weight is upcast a block of output rows at a time so that very large
    matrices (the 201088-row LM head) never need a full float64 copy; every
    output element is still one dot product over the full input width.
    """
    x = np.asarray(x, dtype=F64)
    out_dim = w.shape[0]
    y = np.empty(x.shape[:-1] + (out_dim,), dtype=F64)
    for r0 in range(0, out_dim, chunk_rows):
        r1 = min(out_dim, r0 + chunk_rows)
        y[..., r0:r1] = x @ np.asarray(w[r0:r1], dtype=F64).T
    return y


def argmax_lowest(logits):
    """Index of the largest logit, the lowest index among equal maxima."""
    return np.argmax(np.asarray(logits), axis=-1)  # NumPy returns the first maximum


def top2_margin(logits):
    """Largest minus second-largest logit along the last axis."""
    part = np.partition(np.asarray(logits, dtype=F64), -2, axis=-1)
    return part[..., -1] - part[..., -2]


# ---------------------------------------------------------------------------
# Input fusion ([TD] "2. The P-EAGLE Parallel Drafter"; [PN] section 2;
# [RH] "A learnable mask parameter").
# ---------------------------------------------------------------------------


def fuse_inputs(w, hidden3, token_ids, mask_emb, h_shared, K):
    """Layer-0 inputs of the K-position block, shape [B, K, H].

    The next-token position uses the new token's embedding plus the
    fc-projected concatenation of three target hidden states.  Every later
    position uses the shared mask-token embedding plus the fc projection of
    the shared hidden state h_shared (3H wide, as the learnable mask_hidden).
    """
    hidden3 = np.asarray(hidden3, dtype=F64)
    B = hidden3.shape[0]
    H = w["fc"].shape[0]
    x = np.empty((B, K, H), dtype=F64)
    ntp = linear(hidden3, w["fc"])                      # [B, H]
    mtp = linear(np.asarray(h_shared, F64)[None], w["fc"])[0]  # [H]
    for b in range(B):
        x[b, 0] = np.asarray(w["embed_rows"][b], dtype=F64) + ntp[b]
        for k in range(1, K):
            x[b, k] = np.asarray(mask_emb, dtype=F64) + mtp
    return x


# ---------------------------------------------------------------------------
# Decode forward ([TD] "2. The P-EAGLE Parallel Drafter"; [PN] section 2;
# attention visibility from [RH] "Flex-attention mask" restricted to one
# rollout: the block's query k sees the whole cached context and block rows
# 0..k).
# ---------------------------------------------------------------------------


def _layer_qkv(x, lw, cfg):
    u = rmsnorm(x, lw["attn_norm"], cfg.rms_eps)
    hd = cfg.head_dim
    q = linear(u, lw["wq"]).reshape(x.shape[:-1] + (cfg.n_q_heads, hd))
    k = linear(u, lw["wk"]).reshape(x.shape[:-1] + (cfg.n_kv_heads, hd))
    v = linear(u, lw["wv"]).reshape(x.shape[:-1] + (cfg.n_kv_heads, hd))
    return q, k, v


def _layer_finish(x, attn, lw, cfg):
    """O projection with residual, then the SwiGLU MLP with residual."""
    x = x + linear(attn, lw["wo"])
    u = rmsnorm(x, lw["mlp_norm"], cfg.rms_eps)
    return x + linear(silu(linear(u, lw["w_gate"])) * linear(u, lw["w_up"]), lw["w_down"])


def attend(q, keys, vals, scale):
    """softmax(q . keys^T * scale) @ vals for q [G, hd], keys/vals [n, hd]."""
    p = softmax((np.asarray(q, F64) @ np.asarray(keys, F64).T) * scale)
    return p @ np.asarray(vals, F64)


def draft_forward(w, cfg, hidden3, token_ids, mask_emb, h_shared, ctx_lens,
                  k_cache, v_cache, K, N=None, return_hidden=False):
    """Logits [B, K, V] of one parallel-drafting forward.

    ``w["embed_rows"]`` holds E[token_ids[b]] (the only embedding rows read).
    k_cache[l] / v_cache[l]: [B, n_kv, C, hd], keys already rotated.
    N layers are run (default: all of them).
    """
    N = cfg.n_layers if N is None else N
    B = len(token_ids)
    nq, nkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    G = nq // nkv
    scale = 1.0 / math.sqrt(hd)
    x = fuse_inputs(w, hidden3, token_ids, mask_emb, h_shared, K)
    pos = np.asarray(ctx_lens, dtype=F64)[:, None] + np.arange(K)[None, :]  # [B, K]
    for l in range(N):
        lw = w["layers"][l]
        q, k, v = _layer_qkv(x, lw, cfg)
        q = rope(q, pos[:, :, None], cfg.rope_theta)
        k = rope(k, pos[:, :, None], cfg.rope_theta)
        attn = np.empty((B, K, nq, hd), dtype=F64)
        for b in range(B):
            C = int(ctx_lens[b])
            for g in range(nkv):
                ck = np.asarray(k_cache[l][b, g, :C], dtype=F64)
                cv = np.asarray(v_cache[l][b, g, :C], dtype=F64)
                for kp in range(K):
                    keys = np.concatenate([ck, k[b, :kp + 1, g]], axis=0)
                    vals = np.concatenate([cv, v[b, :kp + 1, g]], axis=0)
                    attn[b, kp, g * G:(g + 1) * G] = attend(q[b, kp, g * G:(g + 1) * G],
                                                            keys, vals, scale)
        x = _layer_finish(x, attn.reshape(B, K, nq * hd), lw, cfg)
    z = rmsnorm(x, w["final_norm"], cfg.rms_eps)
    logits = linear(z, w["lm_head"])
    if return_hidden:
        return logits, z
    return logits


def eagle3_step(w, cfg, hidden3_b, token_id, ctx_len, k_cache_b, v_cache_b, N=None):
    """One autoregressive EAGLE-3 drafter step for a single sequence.

    Written separately from ``draft_forward`` (explicit per-head loops) so
    that the K = 1 case of the parallel drafter, which the pages describe as
    plain EAGLE-3 next-token prediction, can be checked against it.
    k_cache_b[l]: [n_kv, C, hd].  Returns the logits [V].
    """
    N = cfg.n_layers if N is None else N
    nq, nkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    x = (np.asarray(w["embed_rows"][0], F64)
         + np.asarray(w["fc"], F64) @ np.asarray(hidden3_b, F64))
    for l in range(N):
        lw = w["layers"][l]
        ms = float(np.dot(x, x)) / x.shape[0]
        u = x * (1.0 / math.sqrt(ms + cfg.rms_eps)) * np.asarray(lw["attn_norm"], F64)
        q = (np.asarray(lw["wq"], F64) @ u).reshape(nq, hd)
        kk = (np.asarray(lw["wk"], F64) @ u).reshape(nkv, hd)
        vv = (np.asarray(lw["wv"], F64) @ u).reshape(nkv, hd)
        half = hd // 2
        for h in range(nq):
            q[h] = _rotate_once(q[h], ctx_len, cfg.rope_theta, half)
        for g in range(nkv):
            kk[g] = _rotate_once(kk[g], ctx_len, cfg.rope_theta, half)
        out = np.zeros(nq * hd)
        for h in range(nq):
            g = h // (nq // nkv)
            keys = list(np.asarray(k_cache_b[l][g, :ctx_len], F64)) + [kk[g]]
            vals = list(np.asarray(v_cache_b[l][g, :ctx_len], F64)) + [vv[g]]
            sc = np.array([np.dot(q[h], kv) / math.sqrt(hd) for kv in keys])
            e = np.exp(sc - sc.max())
            e /= e.sum()
            out[h * hd:(h + 1) * hd] = sum(ei * vi for ei, vi in zip(e, vals))
        x = x + np.asarray(lw["wo"], F64) @ out
        ms = float(np.dot(x, x)) / x.shape[0]
        u = x * (1.0 / math.sqrt(ms + cfg.rms_eps)) * np.asarray(lw["mlp_norm"], F64)
        gt = np.asarray(lw["w_gate"], F64) @ u
        up = np.asarray(lw["w_up"], F64) @ u
        x = x + np.asarray(lw["w_down"], F64) @ (gt / (1.0 + np.exp(-gt)) * up)
    ms = float(np.dot(x, x)) / x.shape[0]
    z = x * (1.0 / math.sqrt(ms + cfg.rms_eps)) * np.asarray(w["final_norm"], F64)
    return linear(z[None], w["lm_head"])[0]


def _rotate_once(a, pos, theta, half):
    out = np.array(a, dtype=F64)
    for i in range(half):
        ang = pos * theta ** (-2.0 * i / (2 * half))
        c, s = math.cos(ang), math.sin(ang)
        out[i] = a[i] * c - a[i + half] * s
        out[i + half] = a[i + half] * c + a[i] * s
    return out


# ---------------------------------------------------------------------------
# Depth-0 rows appended to the drafter's cache, and the autoregressive EAGLE-3
# baseline built from them.
#   [RH] "Flex-attention mask": depth-0 positions carry real tokens and real
#   hidden states and attend causally to each other (the base context).
#   [TD] "Technical Architecture: From Sequential to Parallel": EAGLE needs K
#   sequential forward passes for K draft tokens.  [PN] section 2: each step
#   depends on the previous step's token and hidden state.  [E4] "EAGLE-4":
#   each drafting step takes the previous step's final-norm state as its input.
# ---------------------------------------------------------------------------


def draft_extend(w, cfg, inputs, input_kind, embed_rows, ctx_lens, k_cache, v_cache, N=None):
    """Forward of T real (depth-0) rows per sequence, whose keys and values
    then extend the drafter's cache.

    inputs: [B, T, 3H] target hidden states (input_kind "target": the row's
    layer-0 input is E[token] + fc(h)) or [B, T, H] drafter output states
    (input_kind "drafter": E[token] + z, the fed-back state taking the place
    of the projected target state).  embed_rows: [B, T, H] = E[token].
    Row t of sequence b sits at position ctx_lens[b] + t and attends to cache
    rows [0, ctx_lens[b]) and to rows 0..t of the block.

    Returns (logits [B, T, V], z [B, T, H] the final-norm output,
    k_new, v_new: per layer [B, n_kv, T, hd], keys rotated) -- k_new/v_new are
    what a cache append writes at positions ctx_lens[b] .. ctx_lens[b] + T - 1.
    """
    N = cfg.n_layers if N is None else N
    inputs = np.asarray(inputs, dtype=F64)
    B, T = inputs.shape[0], inputs.shape[1]
    nq, nkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    G = nq // nkv
    scale = 1.0 / math.sqrt(hd)
    if input_kind == "target":
        x = np.asarray(embed_rows, F64) + linear(inputs.reshape(B * T, -1), w["fc"]).reshape(B, T, -1)
    elif input_kind == "drafter":
        x = np.asarray(embed_rows, F64) + inputs
    else:
        raise ValueError(input_kind)
    pos = np.asarray(ctx_lens, dtype=F64)[:, None] + np.arange(T)[None, :]
    k_new, v_new = [], []
    for l in range(N):
        lw = w["layers"][l]
        q, k, v = _layer_qkv(x, lw, cfg)
        q = rope(q, pos[:, :, None], cfg.rope_theta)
        k = rope(k, pos[:, :, None], cfg.rope_theta)
        k_new.append(np.transpose(k, (0, 2, 1, 3)).copy())
        v_new.append(np.transpose(v, (0, 2, 1, 3)).copy())
        attn = np.empty((B, T, nq, hd), dtype=F64)
        for b in range(B):
            C = int(ctx_lens[b])
            for g in range(nkv):
                ck = np.asarray(k_cache[l][b, g, :C], dtype=F64)
                cv = np.asarray(v_cache[l][b, g, :C], dtype=F64)
                for t in range(T):
                    keys = np.concatenate([ck, k[b, :t + 1, g]], axis=0)
                    vals = np.concatenate([cv, v[b, :t + 1, g]], axis=0)
                    attn[b, t, g * G:(g + 1) * G] = attend(q[b, t, g * G:(g + 1) * G], keys, vals, scale)
        x = _layer_finish(x, attn.reshape(B, T, nq * hd), lw, cfg)
    z = rmsnorm(x, w["final_norm"], cfg.rms_eps)
    return linear(z.reshape(B * T, -1), w["lm_head"]).reshape(B, T, -1), z, k_new, v_new


def eagle3_chain(w, cfg, hidden3, token_ids, ctx_lens, k_cache, v_cache, K, embed_lookup, N=None,
                 feed_tokens=None):
    """K autoregressive EAGLE-3 drafter steps per sequence (the sequential
    baseline P-EAGLE replaces).

    Step 0 takes the new token and the target's hidden state (3H, through
    fc) at position ctx_lens[b]; step j > 0 takes step j-1's draft token and
    its final-norm output state z at position ctx_lens[b] + j.  Each step's
    keys and values join the cache before the next step.  embed_lookup(ids)
    returns the embedding rows of int ids.  The caller's caches are not
    modified.  Returns (drafts [B, K] int32, logits [B, K, V]).

    feed_tokens: optional [B, K]; step j + 1 then takes feed_tokens[:, j]
    instead of step j's own argmax (drafts still hold the argmaxes).  This
    follows another chain whose near-tied argmax went the other way.
    """
    N = cfg.n_layers if N is None else N
    B = len(token_ids)
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    kc, vc = [], []
    for l in range(N):
        shp = np.asarray(k_cache[l]).shape
        cap = max(shp[2], int(ctx.max()) + K)
        a = np.zeros(shp[:2] + (cap, shp[3]), dtype=F64)
        c = np.zeros_like(a)
        a[:, :, :shp[2]] = k_cache[l]
        c[:, :, :shp[2]] = v_cache[l]
        kc.append(a)
        vc.append(c)
    drafts = np.zeros((B, K), dtype=np.int32)
    logits = None
    tok = np.asarray(token_ids, dtype=np.int64)
    inputs, kind = np.asarray(hidden3, F64)[:, None, :], "target"
    for j in range(K):
        lg, z, kn, vn = draft_extend(w, cfg, inputs, kind, np.asarray(embed_lookup(tok), F64)[:, None, :],
                                     ctx + j, kc, vc, N)
        for l in range(N):
            for b in range(B):
                kc[l][b, :, ctx[b] + j] = kn[l][b, :, 0]
                vc[l][b, :, ctx[b] + j] = vn[l][b, :, 0]
        if logits is None:
            logits = np.zeros((B, K, lg.shape[-1]), dtype=F64)
        logits[:, j] = lg[:, 0]
        drafts[:, j] = argmax_lowest(lg[:, 0])
        tok = (drafts[:, j] if feed_tokens is None else np.asarray(feed_tokens)[:, j]).astype(np.int64)
        inputs, kind = z, "drafter"
    return drafts, logits


# ---------------------------------------------------------------------------
# Greedy acceptance ([RH] introduction: the verifier accepts the correct
# prefix; [E4] "EAGLE-4 overview": longest agreeing path plus one bonus token).
# ---------------------------------------------------------------------------


def accept(draft, target):
    """accept_len [B] and emitted tokens [B, K+1] (entries past a+1 are -1).

    accept_len = the number of leading draft tokens equal to the target's;
    the round emits target[0..accept_len] (the accepted prefix plus the
    target's own next token).
    """
    draft = np.asarray(draft)
    target = np.asarray(target)
    B, K = draft.shape
    alen = np.zeros(B, dtype=np.int32)
    out = np.full((B, K + 1), -1, dtype=np.int32)
    for b in range(B):
        a = 0
        while a < K and draft[b, a] == target[b, a]:
            a += 1
        alen[b] = a
        out[b, :a + 1] = target[b, :a + 1]
    return alen, out


# ---------------------------------------------------------------------------
# COD sampling ([RH] "COD sampling"; [PN] section 3 challenge analysis and
# 3.2: geometric decay rate r = 0.8 in the paper's setup).
# ---------------------------------------------------------------------------


def cod_keep(n, K, U, r=0.8, floor=0.2):
    """Boolean keep grid [n, K] over (position p, depth d).

    Depth 0 keeps every position.  A depth-d cell (p, d), d >= 1, needs its
    parent (p-1, d-1) kept and is then kept when U[p, d] < r_d, where
    r_d = max(r^d, floor) / max(r^(d-1), floor), so that the marginal keep
    rate of depth d is max(r^d, floor).  Cells with p < d have no anchor.
    """
    keep = np.zeros((n, K), dtype=bool)
    keep[:, 0] = True

    def marginal(d):
        return max(r ** d, floor)

    for d in range(1, K):
        rate = marginal(d) / marginal(d - 1)
        for p in range(d, n):
            keep[p, d] = keep[p - 1, d - 1] and U[p, d] < rate
    return keep


def cod_rows(keep):
    """Retained grid indices p*K + d in ascending (position-major) order."""
    n, K = keep.shape
    return np.array([p * K + d for p in range(n) for d in range(K) if keep[p, d]],
                    dtype=np.int64)


# ---------------------------------------------------------------------------
# Attention visibility ([RH] "Flex-attention mask"; chain structure of
# [PN] 3.2).  A cell (p, d) belongs to the rollout anchored at a = p - d.
# ---------------------------------------------------------------------------


def mask_allowed(p, d, pk, dk):
    """May query cell (p, d) attend to key cell (pk, dk)?

    Depth-0 keys are visible up to and including the query's anchor; a
    deeper key is visible when it lies on the query's own rollout chain at a
    depth not beyond the query's.
    """
    a = p - d
    if dk == 0:
        return pk <= a
    return (pk - dk == a) and dk <= d


def mask_fresh(rows, K):
    """Mask over retained grid rows built cell by cell from the predicate."""
    rows = np.asarray(rows)
    L = len(rows)
    m = np.zeros((L, L), dtype=bool)
    for i in range(L):
        p, d = divmod(int(rows[i]), K)
        for j in range(L):
            pk, dk = divmod(int(rows[j]), K)
            m[i, j] = mask_allowed(p, d, pk, dk)
    return m


def mask_precompute(n_max, K):
    """Full position-major grid mask for the longest sequence, built once
    ([PN] 3.1: precompute at the maximum length, then slice)."""
    return mask_fresh(np.arange(n_max * K), K)


def mask_slice(m_pre, n, K, rows):
    """Top-left [nK, nK] slice of the precomputed mask, then the retained
    rows and columns of one COD sample ([PN] 3.1)."""
    s = m_pre[:n * K, :n * K]
    rows = np.asarray(rows)
    return s[np.ix_(rows, rows)]


# ---------------------------------------------------------------------------
# Sequence partitioning ([PN] 3.2 and its invariant
# Chunk(p, d) = Chunk(p-1, d-1) for d >= 2).
# ---------------------------------------------------------------------------


def partition(n, K, S, rows):
    """Chunk of every retained row and the depth-0 completion of each chunk.

    Segments are equal-width index ranges b_s = floor(s n / S).  Depth-0 and
    depth-1 cells go to the segment of their position; a deeper cell goes to
    the chunk of its parent (p-1, d-1).  Chunk s is completed with every
    depth-0 row whose position lies before the end of segment s.
    Returns (chunk_of_row [L], bounds [S+1], completion list of position
    arrays).
    """
    bounds = [(s * n) // S for s in range(S + 1)]

    def seg(p):
        for s in range(S):
            if bounds[s] <= p < bounds[s + 1]:
                return s
        raise ValueError(p)

    chunk = {}
    for r in sorted(int(x) for x in rows):   # position-major: parents come first
        p, d = divmod(r, K)
        if d <= 1:
            chunk[(p, d)] = seg(p)
        else:
            chunk[(p, d)] = chunk[(p - 1, d - 1)]
    chunk_of_row = np.array([chunk[divmod(int(r), K)] for r in rows], dtype=np.int64)
    completion = [np.arange(0, bounds[s + 1]) for s in range(S)]
    return chunk_of_row, np.array(bounds), completion


# ---------------------------------------------------------------------------
# Training-shape forward over a COD layout ([TD] "Memory and Training
# Complexity"; [PN] 3 and 3.2; visibility from [RH] "Flex-attention mask").
# ---------------------------------------------------------------------------


def train_forward(w, cfg, hidden3, token_ids, mask_emb, h_shared, rows, K, N=None,
                  lm_rows=None, return_kv=False):
    """Logits of retained grid rows of one sequence.

    Row (p, d) takes E[x_p] + fc(h_p) at depth 0 and mask_emb + fc(h_shared)
    deeper, sits at RoPE position p, and attends to the retained rows the
    predicate allows (its anchor's depth-0 prefix and its own chain).
    ``w["embed_rows"]`` holds E[token_ids[p]] for every position p.
    ``lm_rows`` optionally restricts the LM head to those indices into
    ``rows`` (the layers always run on every row).  Returns logits
    [len(lm_rows) or L, V]; with ``return_kv`` also the per-layer rotated
    keys and values [L, n_kv, hd].
    """
    N = cfg.n_layers if N is None else N
    rows = np.asarray(rows, dtype=np.int64)
    L = len(rows)
    P, D = rows // K, rows % K
    nq, nkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    G = nq // nkv
    scale = 1.0 / math.sqrt(hd)
    hid = np.asarray(hidden3, F64)
    ntp = linear(hid, w["fc"])
    mtp = linear(np.asarray(h_shared, F64)[None], w["fc"])[0]
    x = np.empty((L, cfg.hidden), dtype=F64)
    for i in range(L):
        if D[i] == 0:
            x[i] = np.asarray(w["embed_rows"][P[i]], F64) + ntp[P[i]]
        else:
            x[i] = np.asarray(mask_emb, F64) + mtp
    # Keys each row may see: depth-0 rows of positions <= anchor, then the
    # row's own chain (depths 1..d at the same anchor).
    # The depth-0 cells of positions up to the largest anchor must be present
    # (a chunk of a sequence partition holds no depth-0 cells beyond it).
    index = {(int(P[i]), int(D[i])): i for i in range(L)}
    depth0 = np.array([index[(p, 0)] for p in range(int((P - D).max()) + 1)]) if L else np.zeros(0, int)
    kv_out = []
    for l in range(N):
        lw = w["layers"][l]
        q, k, v = _layer_qkv(x, lw, cfg)
        q = rope(q, P[:, None].astype(F64), cfg.rope_theta)
        k = rope(k, P[:, None].astype(F64), cfg.rope_theta)
        kv_out.append((k.copy(), v.copy()))
        attn = np.zeros((L, nq, hd), dtype=F64)
        # With one layer and a restricted LM head, rows outside lm_rows feed
        # nothing but their keys and values, so their attention is skipped.
        need = range(L) if (lm_rows is None or l + 1 < N) else [int(t) for t in lm_rows]
        for i in need:
            a = int(P[i] - D[i])
            keys_idx = list(depth0[:a + 1]) + [index[(a + dd, dd)] for dd in range(1, int(D[i]) + 1)]
            for g in range(nkv):
                attn[i, g * G:(g + 1) * G] = attend(q[i, g * G:(g + 1) * G],
                                                    k[keys_idx, g], v[keys_idx, g], scale)
        if l + 1 == N and lm_rows is not None:
            sel = np.asarray(lm_rows)
            x = x[sel]
            attn = attn[sel]
        x = _layer_finish(x, attn.reshape(len(x), nq * hd), lw, cfg)
    z = rmsnorm(x, w["final_norm"], cfg.rms_eps)
    sel = np.arange(len(z)) if (lm_rows is None or N > 0) else np.asarray(lm_rows)
    logits = linear(z[sel], w["lm_head"])
    if return_kv:
        return logits, kv_out
    return logits


# ---------------------------------------------------------------------------
# Training loss and gradients over a COD layout ([TD] "Memory and Training
# Complexity": training runs the K-depth layout in one forward and backward,
# with gradients accumulated over the chunks of a sequence partition; [PN] 3
# and 3.2).  Each cell (p, d) predicts the token after position p (reading:
# anchor a = p - d, depth d drafts the token at a + d + 1); the loss is the
# cross-entropy of the cell's logits against labels[p], summed over cells
# with a label and multiplied by loss_scale.  The backward is written out
# step by step (reverse order of the forward), not derived automatically.
# ---------------------------------------------------------------------------


def silu_grad(z):
    """d silu / dz = s (1 + z (1 - s)), s = sigmoid(z)."""
    z = np.asarray(z, dtype=F64)
    sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


def rmsnorm_backward(x, gain, eps, dy):
    """Gradients of y = x r g, r = (mean(x^2) + eps)^(-1/2), over the last
    axis: returns (dx, dgain summed over rows)."""
    x = np.asarray(x, F64)
    g = np.asarray(gain, F64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    gdy = dy * g
    dx = r * gdy - x * r ** 3 * np.mean(gdy * x, axis=-1, keepdims=True)
    return dx, np.sum(dy * x * r, axis=0)


def train_loss_grads(w, cfg, hidden3, token_ids, mask_emb, h_shared, rows, K, labels,
                     loss_scale=None, loss_rows=None, N=None):
    """Loss and parameter gradients of the training-shape forward.

    labels: int [n]; cell (p, d) is scored against labels[p] (negative: not
    scored).  loss_rows: optional indices into ``rows`` of the cells whose
    loss counts (a chunk scores only its own cells); default all.
    loss_scale: multiplies the summed cross-entropy; default 1 / (number of
    scored cells).  ``w["embed_rows"]`` holds E[token_ids[p]].

    Returns (loss, grads) with grads keys fc, final_norm, lm_head, mask_emb,
    h_shared, embed_rows ([n, H], the gradient of E[token_ids[p]] as used at
    position p), and layers[l] with attn_norm, wq, wk, wv, wo, mlp_norm,
    w_gate, w_up, w_down.
    """
    N = cfg.n_layers if N is None else N
    rows = np.asarray(rows, dtype=np.int64)
    L = len(rows)
    P, D = rows // K, rows % K
    n = len(np.asarray(token_ids))
    H, nq, nkv, hd = cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    G = nq // nkv
    scale = 1.0 / math.sqrt(hd)
    eps = cfg.rms_eps
    hid = np.asarray(hidden3, F64)
    hs = np.asarray(h_shared, F64)
    Wf = lambda a: np.asarray(a, F64)

    # ---- forward, keeping what the backward needs
    ntp = hid @ Wf(w["fc"]).T
    mtp = Wf(w["fc"]) @ hs
    deep = D > 0
    x = np.where(deep[:, None], Wf(mask_emb)[None] + mtp[None], 0.0)
    x[~deep] = Wf(w["embed_rows"])[P[~deep]] + ntp[P[~deep]]
    index = {(int(P[i]), int(D[i])): i for i in range(L)}
    depth0 = [index[(p, 0)] for p in range(int((P - D).max()) + 1)] if L else []
    keys_of = [depth0[:int(P[i] - D[i]) + 1] + [index[(int(P[i] - D[i]) + j, j)] for j in range(1, int(D[i]) + 1)]
               for i in range(L)]
    saved = []
    for l in range(N):
        lw = w["layers"][l]
        u1 = rmsnorm(x, lw["attn_norm"], eps)
        q = rope((u1 @ Wf(lw["wq"]).T).reshape(L, nq, hd), P[:, None].astype(F64), cfg.rope_theta)
        k = rope((u1 @ Wf(lw["wk"]).T).reshape(L, nkv, hd), P[:, None].astype(F64), cfg.rope_theta)
        v = (u1 @ Wf(lw["wv"]).T).reshape(L, nkv, hd)
        probs = []
        a = np.zeros((L, nq, hd))
        for i in range(L):
            ki = keys_of[i]
            pr = np.empty((nq, len(ki)))
            for h in range(nq):
                g = h // G
                pr[h] = softmax(q[i, h] @ k[ki, g].T * scale)
                a[i, h] = pr[h] @ v[ki, g]
            probs.append(pr)
        a = a.reshape(L, nq * hd)
        xm = x + a @ Wf(lw["wo"]).T
        u2 = rmsnorm(xm, lw["mlp_norm"], eps)
        ga = u2 @ Wf(lw["w_gate"]).T
        ub = u2 @ Wf(lw["w_up"]).T
        hh = silu(ga) * ub
        saved.append((x, u1, q, k, v, probs, a, xm, u2, ga, ub, hh))
        x = xm + hh @ Wf(lw["w_down"]).T
    z = rmsnorm(x, w["final_norm"], eps)
    logits = z @ Wf(w["lm_head"]).T

    # ---- loss: cross-entropy of each scored cell against labels[p]
    lab = np.asarray(labels, dtype=np.int64)[P]
    scored = lab >= 0
    if loss_rows is not None:
        keep = np.zeros(L, dtype=bool)
        keep[np.asarray(loss_rows, dtype=np.int64)] = True
        scored &= keep
    if loss_scale is None:
        loss_scale = 1.0 / max(int(scored.sum()), 1)
    mx = logits.max(axis=1, keepdims=True)
    lse = mx[:, 0] + np.log(np.sum(np.exp(logits - mx), axis=1))
    idx = np.flatnonzero(scored)
    loss = loss_scale * float(np.sum(lse[idx] - logits[idx, lab[idx]]))
    dlogits = np.zeros_like(logits)
    dlogits[idx] = np.exp(logits[idx] - lse[idx, None])
    dlogits[idx, lab[idx]] -= 1.0
    dlogits *= loss_scale

    # ---- backward
    grads = {"layers": [None] * N}
    grads["lm_head"] = dlogits.T @ z
    dz = dlogits @ Wf(w["lm_head"])
    dx, grads["final_norm"] = rmsnorm_backward(x, w["final_norm"], eps, dz)
    for l in reversed(range(N)):
        lw = w["layers"][l]
        x_in, u1, q, k, v, probs, a, xm, u2, ga, ub, hh = saved[l]
        gl = {}
        # MLP: x = xm + (silu(ga) * ub) @ w_down^T
        gl["w_down"] = dx.T @ hh
        dh = dx @ Wf(lw["w_down"])
        dga = dh * ub * silu_grad(ga)
        dub = dh * silu(ga)
        gl["w_gate"] = dga.T @ u2
        gl["w_up"] = dub.T @ u2
        du2 = dga @ Wf(lw["w_gate"]) + dub @ Wf(lw["w_up"])
        dxm_n, gl["mlp_norm"] = rmsnorm_backward(xm, lw["mlp_norm"], eps, du2)
        dxm = dx + dxm_n
        # O projection: xm = x_in + a @ wo^T
        gl["wo"] = dxm.T @ a
        da = (dxm @ Wf(lw["wo"])).reshape(L, nq, hd)
        # attention, row by row over each row's visible keys
        dq = np.zeros((L, nq, hd))
        dk = np.zeros((L, nkv, hd))
        dv = np.zeros((L, nkv, hd))
        for i in range(L):
            ki = keys_of[i]
            for h in range(nq):
                g = h // G
                pr = probs[i][h]
                dv[ki, g] += pr[:, None] * da[i, h][None, :]
                dp = v[ki, g] @ da[i, h]
                ds = pr * (dp - np.dot(pr, dp))
                dq[i, h] = scale * (ds @ k[ki, g])
                dk[ki, g] += scale * ds[:, None] * q[i, h][None, :]
        # RoPE is a rotation: its transpose rotates by the opposite angle
        dq = rope(dq, -P[:, None].astype(F64), cfg.rope_theta).reshape(L, nq * hd)
        dk = rope(dk, -P[:, None].astype(F64), cfg.rope_theta).reshape(L, nkv * hd)
        dv = dv.reshape(L, nkv * hd)
        gl["wq"] = dq.T @ u1
        gl["wk"] = dk.T @ u1
        gl["wv"] = dv.T @ u1
        du1 = dq @ Wf(lw["wq"]) + dk @ Wf(lw["wk"]) + dv @ Wf(lw["wv"])
        dx_n, gl["attn_norm"] = rmsnorm_backward(x_in, lw["attn_norm"], eps, du1)
        dx = dxm + dx_n
        grads["layers"][l] = gl
    # fusion: depth-0 cells E[x_p] + fc(h_p), deeper cells mask_emb + fc(h_shared)
    d_shared = dx[deep].sum(axis=0)
    grads["mask_emb"] = d_shared.copy()
    grads["h_shared"] = d_shared @ Wf(w["fc"])
    d_ntp = np.zeros((n, H))
    d_ntp[P[~deep]] = dx[~deep]
    grads["embed_rows"] = d_ntp.copy()
    grads["fc"] = d_ntp.T @ hid + np.outer(d_shared, hs)
    return loss, grads


def chunk_cells(n, K, S, rows, s):
    """Cells the forward of chunk s of a sequence partition runs on ([PN]
    3.2): the depth-0 completion (every depth-0 cell of a position before
    the end of segment s) joined with the chunk's own cells, ascending.
    Returns (cells, own) with own the indices into ``rows`` of the chunk's
    own cells, in the order they appear in ``cells``."""
    rows = np.asarray(rows, dtype=np.int64)
    chunk_of_row, _, completion = partition(n, K, S, rows)
    own = np.nonzero(chunk_of_row == s)[0]
    cells = np.union1d(np.asarray(completion[s], dtype=np.int64) * K, rows[own])
    return cells, own


def train_forward_partitioned(w, cfg, hidden3, token_ids, mask_emb, h_shared, rows, K, S, N=None):
    """The training-shape forward run chunk by chunk ([PN] 3.2): each chunk
    is a forward over its own cells plus its depth-0 completion, with no
    state shared between chunks; the logits of each chunk's own cells are
    placed at their rows.  Every cell belongs to exactly one chunk, so the
    result has the shape of train_forward's."""
    rows = np.asarray(rows, dtype=np.int64)
    n = len(np.asarray(token_ids))
    out = None
    for s in range(S):
        cells, own = chunk_cells(n, K, S, rows, s)
        if len(own) == 0:
            continue
        lg = train_forward(w, cfg, hidden3, token_ids, mask_emb, h_shared, cells, K, N,
                           lm_rows=np.searchsorted(cells, rows[own]))
        if out is None:
            out = np.zeros((len(rows), lg.shape[-1]), dtype=F64)
        out[own] = lg
    return out

"""GPU parity of the training-shape forward and the amortized mask against
the CPU oracle, through the C ABI.

Layouts come from COD sampling of the n x K cell grid; small shapes span
several 128-row GEMM blocks with a ragged tail, several 64-key attention
tiles, GQA group sizes that do and do not divide the 64-row query tile,
K = 1 (plain causal prefill), N = 0, and the training size itself on a
seeded stratified sample of rows.
"""
import time

import numpy as np
import pytest
import torch

from drafting_eagle_draft_amd import runner, synth
from oracle import peagle_oracle as po
from tests.gpu_util import MARGIN, TOL, log
from tests.layout_util import key_closure

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from drafting_eagle_draft_amd import binding
    binding.load()


def train_small(name="train_small", **kw):
    base = dict(name=name, seed=3001, hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2,
                head_dim=64, intermediate=768, vocab=8192 + 48, K=8, dtype="bf16", seq_len=300,
                n_max=512)
    base.update(kw)
    return synth.DrafterShape(**base)


def cod_layout(cfg, n, K, r=None, tag=""):
    U = synth.cod_uniforms(cfg, n, K, tag=tag)
    return po.cod_rows(po.cod_keep(n, K, U, r=cfg.cod_rate if r is None else r, floor=cfg.cod_floor))


def oracle_train(cfg, w, inp, rows, K, N=None, lm_rows=None):
    wr = dict(w, embed_rows=w["embed"][inp["token_ids"]])
    return po.train_forward(wr, cfg, inp["hidden3"], inp["token_ids"], inp["mask_emb"],
                            inp["h_shared"], rows, K, N=N, lm_rows=lm_rows)


def compare(cfg, ref, argmax, logits, tol=None):
    """Parity rule on rows: logits within tol; argmax equal where the margin is decided."""
    tol = TOL[cfg.dtype] if tol is None else tol
    margin = po.top2_margin(ref)
    ok = margin > MARGIN
    ref_tok = po.argmax_lowest(ref)
    stats = {"rows": int(ref.shape[0]), "decided": int(ok.sum()),
             "mismatch_decided": int(np.sum(argmax[ok] != ref_tok[ok])),
             "mismatch_all": int(np.sum(argmax != ref_tok))}
    if logits is not None:
        stats["max_abs"] = float(np.max(np.abs(logits.astype(np.float64) - ref)))
        assert stats["max_abs"] <= tol, stats
    assert stats["mismatch_decided"] == 0, stats
    assert np.all((argmax >= 0) & (argmax < cfg.vocab))
    return stats


def run_train_case(cfg, w, inp, rows, K, N=None, n_max=None):
    t0 = time.time()
    d = runner.Drafter(cfg, w)
    mask = runner.TrainMask(n_max or max(len(inp["token_ids"]), 1), K)
    argmax, logits = runner.train_forward(d, mask, inp, rows, N=N)
    t1 = time.time()
    ref = oracle_train(cfg, w, inp, rows, K, N=N)
    t2 = time.time()
    stats = compare(cfg, ref, argmax, logits)
    log(f"  {cfg.name} n={len(inp['token_ids'])} K={K} L={len(rows)} N={N}: "
        f"gpu {t1 - t0:.1f}s oracle {t2 - t1:.1f}s {stats}")
    mask.close()
    d.close()
    return stats


# ---------------------------------------------------------------- amortized mask


@pytest.mark.parametrize("n_max,K,ns", [(48, 8, [1, 17, 48]), (40, 4, [40, 3]), (20, 1, [20])])
def test_mask_slice_matches_fresh_and_oracle(n_max, K, ns):
    cfg = synth.config("tiny_f32")
    m_pre = po.mask_precompute(n_max, K)
    mask = runner.TrainMask(n_max, K)
    for n in ns:
        rows = cod_layout(cfg, n, K, r=0.7, tag=f"mask{n}")
        got = mask.materialize(n, rows).astype(bool)
        np.testing.assert_array_equal(got, po.mask_slice(m_pre, n, K, rows))
        np.testing.assert_array_equal(got, po.mask_fresh(rows, K))
    mask.close()


def test_mask_at_training_size_sampled():
    """n_max 20480, K 8, one n = 8192 COD sample (L ~ 34K): 10^6 seeded
    entries against the predicate, and every row sums to p + 1."""
    cfg = synth.config("train_gptoss20b_n8192_k8")
    n, K = cfg.seq_len, cfg.K
    rows = cod_layout(cfg, n, K)
    L = len(rows)
    mask = runner.TrainMask(cfg.n_max, K)
    rows_dev = torch.from_numpy(rows.astype(np.int32)).cuda()
    m = mask.materialize_device(n, rows_dev)
    sums = m.sum(dim=1, dtype=torch.int64).cpu().numpy()
    np.testing.assert_array_equal(sums, rows // K + 1)
    rng = np.random.default_rng(5)
    ii = rng.integers(0, L, 1_000_000)
    jj = rng.integers(0, L, 1_000_000)
    # Half of the sample inside the diagonal band, where the chain keys sit.
    jj[::2] = np.clip(ii[::2] + rng.integers(-40, 41, ii[::2].size), 0, L - 1)
    got = m[torch.from_numpy(ii).cuda(), torch.from_numpy(jj).cuda()].cpu().numpy().astype(bool)
    P, D = rows // K, rows % K
    want = np.array([po.mask_allowed(int(P[i]), int(D[i]), int(P[j]), int(D[j]))
                     for i, j in zip(ii, jj)])
    np.testing.assert_array_equal(got, want)
    del m
    mask.close()


# ---------------------------------------------------------------- tiny fp32


@pytest.mark.parametrize("n,K,N,r", [
    (40, 4, 1, 0.8),     # default tiny shape
    (70, 8, 1, 0.8),     # 2 key tiles, ragged rows
    (33, 1, 1, 0.8),     # K = 1: causal prefill only
    (1, 4, 1, 0.8),      # a single cell
    (50, 16, 1, 0.9),    # K = 16
    (45, 6, 0, 0.7),     # N = 0: fusion, final norm, LM head
])
def test_train_tiny_f32(n, K, N, r):
    cfg = synth.config("tiny_f32")
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.train_inputs(cfg, n=n, tag=f"t{n}_{K}")
    rows = cod_layout(cfg, n, K, r=r, tag=f"t{n}_{K}")
    run_train_case(cfg, w, inp, rows, K, N=N, n_max=n + 13)


# ---------------------------------------------------------------- bf16 small


@pytest.mark.parametrize("kw", [
    dict(),                                                                   # hd 64, G 4
    dict(name="train_small_hd128", head_dim=128, seed=3002),                  # hd 128
    dict(name="train_small_g8", n_q_heads=16, n_kv_heads=2, seed=3003),       # G 8
    dict(name="train_small_g3", n_q_heads=6, n_kv_heads=2, seed=3004),        # G 3 (64 % G != 0)
])
def test_train_bf16_small(kw):
    cfg = train_small(**kw)
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.train_inputs(cfg)
    rows = cod_layout(cfg, cfg.seq_len, cfg.K)
    run_train_case(cfg, w, inp, rows, cfg.K, n_max=cfg.n_max)


def test_train_repeat_is_identical_and_argmax_only():
    cfg = train_small(name="train_small_rep", seed=3005, seq_len=150)
    w = synth.drafter_weights(cfg)
    inp = synth.train_inputs(cfg)
    rows = cod_layout(cfg, cfg.seq_len, cfg.K)
    d = runner.Drafter(cfg, w)
    mask = runner.TrainMask(cfg.n_max, cfg.K)
    buf = runner.TrainBuffers(d, mask, inp, rows)
    outs = []
    for _ in range(20):  # repeat-run bit identity over 20 runs
        buf.launch(d, mask)
        torch.cuda.synchronize()
        outs.append((buf.argmax.cpu().numpy().copy(), buf.logits.float().cpu().numpy().copy()))
    for a, lg in outs[1:]:
        np.testing.assert_array_equal(a, outs[0][0])
        np.testing.assert_array_equal(lg, outs[0][1])
    nolog = runner.TrainBuffers(d, mask, inp, rows, want_logits=False)
    nolog.launch(d, mask)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(nolog.argmax.cpu().numpy(), outs[0][0])
    mask.close()
    d.close()


# ---------------------------------------------------------------- sequence partition


def run_partitioned(cfg, w, inp, rows, K, S, n_max, N=None):
    """Chunked forward (each chunk with its depth-0 completion) against the
    whole forward on the GPU (identical: every row's arithmetic is the same)
    and against the oracle's partitioned forward (parity rule)."""
    d = runner.Drafter(cfg, w)
    mask = runner.TrainMask(n_max, K)
    whole_arg, whole_lg = runner.train_forward(d, mask, inp, rows, N=N)
    part = runner.PartitionedTrain(d, mask, inp, rows, S, N=N)
    part.launch(d, mask)
    arg, lg = part.result()
    cells = part.cells_total
    del part
    mask.close()
    d.close()
    np.testing.assert_array_equal(arg, whole_arg)
    np.testing.assert_array_equal(lg, whole_lg)
    wr = dict(w, embed_rows=w["embed"][inp["token_ids"]])
    ref = po.train_forward_partitioned(wr, cfg, inp["hidden3"], inp["token_ids"], inp["mask_emb"],
                                       inp["h_shared"], rows, K, S, N=N)
    stats = compare(cfg, ref, arg, lg)
    log(f"  {cfg.name} n={len(inp['token_ids'])} K={K} S={S} L={len(rows)} chunk cells={cells}: {stats}")


@pytest.mark.parametrize("n,K,S", [(70, 8, 2), (70, 8, 7), (33, 4, 3), (5, 4, 5)])
def test_train_partitioned_tiny_f32(n, K, S):
    cfg = synth.config("tiny_f32")
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.train_inputs(cfg, n=n, tag=f"part{n}_{K}")
    rows = cod_layout(cfg, n, K, r=0.8, tag=f"part{n}_{K}")
    run_partitioned(cfg, w, inp, rows, K, S, n_max=n + 5)


@pytest.mark.parametrize("S", [2, 4])
def test_train_partitioned_bf16_small(S):
    cfg = train_small(name="train_small_part", seed=3006)
    w = synth.drafter_weights(cfg, gain_jitter=0.1)
    inp = synth.train_inputs(cfg)
    rows = cod_layout(cfg, cfg.seq_len, cfg.K)
    run_partitioned(cfg, w, inp, rows, cfg.K, S, n_max=cfg.n_max)


def test_train_chunk_rejects_bad_lead_and_missing_rows():
    from drafting_eagle_draft_amd import binding as pe
    cfg = synth.config("tiny_f32")
    w = synth.drafter_weights(cfg)
    d = runner.Drafter(cfg, w)
    mask = runner.TrainMask(16, 4)
    cells = torch.arange(0, 16, 4, dtype=torch.int32, device="cuda")
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    out = torch.empty(4, dtype=torch.int32, device="cuda")
    h = torch.zeros((4, 3 * cfg.hidden), dtype=torch.float32, device="cuda")
    t = torch.zeros(4, dtype=torch.int32, device="cuda")
    for lead, rows_ptr in [(5, out.data_ptr()), (-1, out.data_ptr()), (1, None)]:
        with pytest.raises(pe.PeagleError):
            pe.pe_train_forward_chunk(d.handle, mask.handle, 1, 4, 4, h.data_ptr(), t.data_ptr(), h.data_ptr(),
                                      h.data_ptr(), cells.data_ptr(), 4, lead, rows_ptr, 4, None,
                                      out.data_ptr(), ws.data_ptr(), ws.numel(), 0)
    mask.close()
    d.close()


# ---------------------------------------------------------------- training size


@pytest.mark.timeout(400)
def test_train_full_size_sampled_rows():
    """GPT-OSS-20B-shaped drafter layer, n = 8192, K = 8, COD r = 0.8: every
    row runs on the GPU; a seeded sample of 256 rows per depth (2048 rows)
    is checked against the oracle, run on the rows those depend on."""
    cfg = synth.config("train_gptoss20b_n8192_k8")
    n, K = cfg.seq_len, cfg.K
    t0 = time.time()
    w = synth.drafter_weights(cfg)
    inp = synth.train_inputs(cfg)
    rows = cod_layout(cfg, n, K)
    L = len(rows)
    log(f"  inputs {time.time() - t0:.1f}s, L = {L}")
    d = runner.Drafter(cfg, w)
    mask = runner.TrainMask(cfg.n_max, K)
    buf = runner.TrainBuffers(d, mask, inp, rows)
    buf.launch(d, mask)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    D = rows % K
    sample = np.sort(np.concatenate([rng.choice(np.flatnonzero(D == dd), 256, replace=False)
                                     for dd in range(K)]))
    idx = torch.from_numpy(sample).cuda()
    logits = buf.logits[idx].float().cpu().numpy()
    argmax = buf.argmax[idx].cpu().numpy()
    all_arg = buf.argmax.cpu().numpy()
    assert np.all((all_arg >= 0) & (all_arg < cfg.vocab))
    del buf
    mask.close()
    d.close()
    torch.cuda.empty_cache()
    t1 = time.time()
    sub, lm = key_closure(rows, K, sample)
    ref = oracle_train(cfg, w, inp, sub, K, lm_rows=lm)
    log(f"  oracle {time.time() - t1:.1f}s")
    stats = compare(cfg, ref, argmax, logits)
    log(f"  {cfg.name} L={L} sample={len(sample)} {stats}")


@pytest.mark.timeout(400)
def test_train_full_size_partitioned_equals_whole():
    """The training size (n = 8192, K = 8, COD r = 0.8) in S = 4 chunks:
    every row's logits and argmax equal the whole forward's."""
    cfg = synth.config("train_gptoss20b_n8192_k8")
    n, K = cfg.seq_len, cfg.K
    w = synth.drafter_weights(cfg)
    inp = synth.train_inputs(cfg)
    rows = cod_layout(cfg, n, K)
    d = runner.Drafter(cfg, w)
    mask = runner.TrainMask(cfg.n_max, K)
    whole = runner.TrainBuffers(d, mask, inp, rows)
    whole.launch(d, mask)
    part = runner.PartitionedTrain(d, mask, inp, rows, 4)
    part.launch(d, mask)
    torch.cuda.synchronize()
    same_arg = bool(torch.equal(part.argmax, whole.argmax))
    same_lg = bool(torch.equal(part.logits, whole.logits))
    log(f"  {cfg.name} L={len(rows)} S=4 chunk cells={part.cells_total}: argmax equal {same_arg}, "
        f"logits equal {same_lg}")
    del part, whole
    mask.close()
    d.close()
    torch.cuda.empty_cache()
    assert same_arg and same_lg

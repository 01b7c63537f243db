"""C ABI checks that need no GPU: the library loads, exports every entry
point its header declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

from drafting_eagle_draft_amd import binding as pe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "peagle.h")

pytestmark = pytest.mark.skipif(not os.path.exists(pe.LIB_PATH),
                                reason="libpeagle.so not built (run __graft_entry__.build())")


def declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:pe_status|const char \*)\s*(pe_\w+)\s*\(", txt, re.M)))


def test_header_declares_the_abi():
    names = declared()
    for n in ("pe_draft_forward", "pe_accept", "pe_model_create", "pe_last_error"):
        assert n in names
    assert set(names) == set(pe.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(pe.LIB_PATH)
    for n in declared():
        assert hasattr(lib, n), n


def _cfg(**kw):
    base = dict(hidden=256, n_layers=1, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=1024,
                vocab=4096, rope_theta=5e5, rms_eps=1e-5, dtype=pe.PE_F32)
    base.update(kw)
    return pe.PeConfig(**base)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(n_q_heads=6, n_kv_heads=4), pe.PE_ERR_INVALID_ARGUMENT, "multiple"),
    (dict(head_dim=96), pe.PE_ERR_UNSUPPORTED, "head_dim"),
    (dict(dtype=7), pe.PE_ERR_INVALID_ARGUMENT, "dtype"),
    (dict(vocab=4095), pe.PE_ERR_UNSUPPORTED, "multiples"),
    (dict(hidden=64), pe.PE_ERR_UNSUPPORTED, ">="),
    (dict(head_dim=128), pe.PE_ERR_UNSUPPORTED, "fp32"),
    (dict(rope_theta=0.0), pe.PE_ERR_INVALID_ARGUMENT, "rope_theta"),
])
def test_model_create_rejects_bad_config(kw, code, needle):
    layers = (pe.PeLayerWeights * 1)(pe.PeLayerWeights(*([16] * 9)))
    w = pe.PeWeights(16, 16, 16, 16, layers)
    with pytest.raises(pe.PeagleError) as ei:
        pe.pe_model_create(_cfg(**kw), w, 0)
    assert ei.value.status == code
    assert needle in ei.value.message


def test_model_create_rejects_null_weights():
    layers = (pe.PeLayerWeights * 1)(pe.PeLayerWeights(*([16] * 8 + [0])))
    with pytest.raises(pe.PeagleError) as ei:
        pe.pe_model_create(_cfg(), pe.PeWeights(16, 16, 16, 16, layers), 0)
    assert ei.value.status == pe.PE_ERR_INVALID_ARGUMENT and "layer 0" in ei.value.message
    with pytest.raises(pe.PeagleError):
        pe.pe_model_create(_cfg(), pe.PeWeights(0, 16, 16, 16, layers), 0)


@pytest.mark.parametrize("B,K,code", [(-1, 4, pe.PE_ERR_INVALID_ARGUMENT),
                                      (2, 0, pe.PE_ERR_INVALID_ARGUMENT),
                                      (2, 17, pe.PE_ERR_INVALID_ARGUMENT)])
def test_accept_rejects_bad_sizes(B, K, code):
    with pytest.raises(pe.PeagleError) as ei:
        pe.pe_accept(B, K, 16, 16, 16, None, 0)
    assert ei.value.status == code


def test_accept_rejects_null_and_allows_empty():
    with pytest.raises(pe.PeagleError):
        pe.pe_accept(3, 4, 0, 16, 16, None, 0)
    pe.pe_accept(0, 4, 0, 0, 0, None, 0)  # nothing to do, nothing enqueued


def test_forward_and_workspace_reject_null_model():
    with pytest.raises(pe.PeagleError) as ei:
        pe.pe_draft_forward(None, 0, 1, 4, 16, 16, 16, 16, 16, 0, None, None, 16, None, 16, 1 << 20, 0)
    assert ei.value.status == pe.PE_ERR_INVALID_ARGUMENT
    with pytest.raises(pe.PeagleError):
        pe.pe_draft_workspace_size(None, 1, 4, 0)
    with pytest.raises(pe.PeagleError):
        pe.pe_workspace_init(None, 16, 0)


def test_mask_create_rejects_bad_sizes():
    for n_max, K in [(0, 8), (16, 0), (16, 17), (1 << 22, 8)]:
        with pytest.raises(pe.PeagleError) as ei:
            pe.pe_mask_create(n_max, K, 0)
        assert ei.value.status == pe.PE_ERR_INVALID_ARGUMENT


def test_train_entry_points_reject_null_handles():
    with pytest.raises(pe.PeagleError):
        pe.pe_train_forward(None, None, 0, 8, 8, 16, 16, 16, 16, 16, 8, None, None, 16, 1 << 20, 0)
    with pytest.raises(pe.PeagleError):
        pe.pe_mask_materialize(None, 8, 16, 8, 16, 0)
    with pytest.raises(pe.PeagleError):
        pe.pe_train_workspace_size(None, 8, 8, 8)
    with pytest.raises(pe.PeagleError):
        pe.pe_mask_destroy(None)


def _llama8b(**kw):
    """A LLaMA-3-8B-shaped drafter layer (H 4096, I 14336, 32 q / 8 kv heads of 128)."""
    base = dict(hidden=4096, n_layers=1, n_q_heads=32, n_kv_heads=8, head_dim=128, intermediate=14336,
                vocab=128256, rope_theta=5e5, rms_eps=1e-5, dtype=pe.PE_BF16)
    base.update(kw)
    return pe.PeConfig(**base)


@pytest.mark.parametrize("B,K", [(1, 1), (2, 8), (4, 8), (8, 8), (4, 16), (63, 1)])
def test_shape_check_plans_long_contractions(B, K):
    """Every projection of a LLaMA-3-8B-shaped drafter has a K split whose
    activation fragments fit in registers, up to 64 activation rows (the
    14336-wide down projection at B*K = 64 needs more than 16 splits)."""
    pe.pe_draft_shape_check(_llama8b(), B, K, 8192, 256)
    pe.pe_draft_shape_check(_llama8b(), B, K, 8192, 80)


def test_shape_check_rejects_infeasible_contraction():
    # 64 activation rows leave 2 tile slots per wave: chunks of 16 k-tiles, at
    # most 64 of them, so a 65536-wide contraction cannot be planned.
    with pytest.raises(pe.PeagleError) as ei:
        pe.pe_draft_shape_check(_llama8b(intermediate=65536), 8, 8, 4096, 256)
    assert ei.value.status == pe.PE_ERR_UNSUPPORTED and "contraction" in ei.value.message
    pe.pe_draft_shape_check(_llama8b(intermediate=65536), 1, 8, 4096, 256)  # 8 rows: more slots


def test_shape_check_bounds_the_cache_slice():
    # One (sequence, kv head) slice of ctx_stride * 128 bf16 elements must
    # stay below 2 GiB.
    pe.pe_draft_shape_check(_llama8b(), 2, 8, 1 << 22, 256)
    with pytest.raises(pe.PeagleError) as ei:
        pe.pe_draft_shape_check(_llama8b(), 2, 8, 1 << 23, 256)
    assert ei.value.status == pe.PE_ERR_UNSUPPORTED and "cache slice" in ei.value.message


def test_shape_check_rejects_bad_arguments():
    with pytest.raises(pe.PeagleError) as ei:
        pe.pe_draft_shape_check(_llama8b(), 8, 9, 4096, 256)
    assert ei.value.status == pe.PE_ERR_UNSUPPORTED
    with pytest.raises(pe.PeagleError) as ei:
        pe.pe_draft_shape_check(_llama8b(head_dim=96), 2, 8, 4096, 256)
    assert ei.value.status == pe.PE_ERR_UNSUPPORTED
    with pytest.raises(pe.PeagleError) as ei:
        pe.pe_draft_shape_check(_llama8b(), 2, 8, -1, 256)
    assert ei.value.status == pe.PE_ERR_INVALID_ARGUMENT

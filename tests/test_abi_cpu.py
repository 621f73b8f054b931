"""The C-ABI library on the host (no GPU): it loads, exports every symbol that
include/sf.h declares, its host-only entry point (the n-gram proposer) agrees
with the oracle, and arguments are rejected before any device work."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sfb = pytest.importorskip("speculative_decoding_verification_decode_amd")


def _lib():
    try:
        return sfb.lib()
    except ImportError as e:
        pytest.fail(f"libsf.so must be built before the tests run: {e}")


def test_every_declared_symbol_is_exported():
    hdr = open(os.path.join(ROOT, "include", "sf.h")).read()
    declared = set(re.findall(r"^(?:sf_status|int32_t|const char\*)\s+(sf_\w+)\s*\(", hdr, re.M))
    assert len(declared) >= 18
    L = _lib()
    missing = [n for n in sorted(declared) if not hasattr(L, n)]
    assert not missing, missing


def test_binding_declares_every_header_function():
    hdr = open(os.path.join(ROOT, "include", "sf.h")).read()
    declared = set(re.findall(r"^(?:sf_status|int32_t|const char\*)\s+(sf_\w+)\s*\(", hdr, re.M))
    for n in declared:
        assert callable(getattr(sfb, n, None)), n


def test_ngram_propose_matches_oracle():
    _lib()
    rng = np.random.default_rng(0)
    for _ in range(400):
        n = int(rng.integers(0, 60))
        h = rng.integers(0, 5, size=n).astype(np.int32)
        for (mn, mx, k) in [(2, 4, 8), (2, 2, 3), (1, 3, 5), (3, 4, 1)]:
            got = sfb.sf_ngram_propose(h, mn, mx, k).tolist()
            assert got == oracle.propose(h.tolist(), mn, mx, k)


def test_ngram_propose_on_lookup_history():
    h = synth.lookup_history(152064, 4096, 4002)
    for cut in range(8, 4096, 61):
        assert sfb.sf_ngram_propose(h[:cut], 2, 4, 8).tolist() == oracle.propose(h[:cut].tolist(), 2, 4, 8)


def test_ngram_propose_rejects_bad_arguments():
    with pytest.raises(sfb.SFError) as e:
        sfb.sf_ngram_propose([1, 2, 3], 3, 2, 8)
    assert e.value.code == sfb.SF_E_ARG
    with pytest.raises(sfb.SFError):
        sfb.sf_ngram_propose([1, 2, 3], 0, 2, 8)
    assert sfb.sf_ngram_propose([], 2, 4, 8).tolist() == []
    assert sfb.sf_ngram_propose([7, 7, 7, 7], 2, 4, 0).tolist() == []


@pytest.mark.parametrize("field,value", [("hidden", 100), ("head_dim", 96), ("n_kv_heads", 3), ("vocab", 4095),
                                         ("ffn", 0), ("n_layers", 0), ("rope_base", 0.5), ("hidden", 8192)])
def test_model_create_rejects_bad_shapes_on_host(field, value):
    d = sfb.desc_from_shape(synth.TINY)
    setattr(d, field, value)
    ptrs = [1] * len(sfb.weight_order(d))   # never dereferenced: the shape check comes first
    with pytest.raises(sfb.SFError) as e:
        sfb.sf_model_create(d, ptrs, None)
    assert e.value.code == sfb.SF_E_ARG


@pytest.mark.parametrize("field,value", [("hidden", 288), ("ffn", 1056)])
def test_nf4_model_create_rejects_shapes_off_the_64_input_blocks(field, value):
    """NF4 scales cover 64 consecutive inputs, so hidden and ffn must be multiples of 64
    (multiples of 32 suffice for bf16 stacks); refused before any device work."""
    d = sfb.desc_from_shape(synth.TINY)
    setattr(d, field, value)
    ptrs = [1] * len(sfb.weight_order(d, nf4=True))
    with pytest.raises(sfb.SFError) as e:
        sfb.sf_model_create_nf4(d, ptrs, None)
    assert e.value.code == sfb.SF_E_ARG


def test_model_create_rejects_null_weight_on_host():
    d = sfb.desc_from_shape(synth.TINY)
    ptrs = [1] * len(sfb.weight_order(d))
    ptrs[5] = 0
    with pytest.raises(sfb.SFError) as e:
        sfb.sf_model_create(d, ptrs, None)
    assert e.value.code == sfb.SF_E_ARG and "5" in str(e.value)


def test_null_handles_are_rejected():
    L = _lib()
    null = ctypes.c_void_p()
    assert L.sf_verify(null, None, None, 0, None, None, None) == sfb.SF_E_ARG
    assert L.sf_verify_device(null, None, None, 0) == sfb.SF_E_ARG
    assert L.sf_rollback(null, 0, 0) == sfb.SF_E_ARG
    assert L.sf_set_next(null, 0, 0) == sfb.SF_E_ARG
    assert L.sf_draft_step(null, 1, None) == sfb.SF_E_ARG
    assert L.sf_prefill(null, 0, None, 1, None) == sfb.SF_E_ARG
    assert L.sf_cache_alloc(null, 1, 16, 4, ctypes.byref(ctypes.c_void_p())) == sfb.SF_E_ARG
    assert L.sf_cache_free(null) == sfb.SF_E_ARG
    assert L.sf_model_free(null) == sfb.SF_E_ARG
    assert L.sf_sync(null) == sfb.SF_E_ARG
    assert L.sf_round_create(null, null, 1, ctypes.byref(ctypes.c_void_p())) == sfb.SF_E_ARG
    assert L.sf_round_run(null, 1) == sfb.SF_E_ARG
    assert L.sf_round_free(null) == sfb.SF_E_ARG
    assert L.sf_snapshot_save(null) == sfb.SF_E_ARG
    assert L.sf_snapshot_restore(null) == sfb.SF_E_ARG
    assert "NULL" in sfb.sf_last_error()


def test_weight_order_matches_generator_names():
    for shape in (synth.TINY, synth.QWEN05B, synth.QWEN7B, synth.QWEN7B_HALF):
        assert sfb.weight_order(sfb.desc_from_shape(shape)) == synth.tensor_names(shape)


def test_nf4_table_matches_oracle():
    """The library's NF4 level table (what the GEMM decodes codes to) equals the oracle's
    table built from the format's definition."""
    from oracle import nf4
    assert np.array_equal(sfb.sf_nf4_levels().astype(np.float64), nf4.table().numpy())


def test_nf4_weight_order_pairs_projections():
    d = sfb.desc_from_shape(synth.TINY)
    names = sfb.weight_order(d, nf4=True)
    assert len(names) == len(sfb.weight_order(d)) + 7 * d.n_layers
    assert names[2:4] == ["l0.wq", "l0.wq"]


@pytest.mark.parametrize("nf4", [False, True])
def test_injected_allocation_failure_is_reported_and_leaves_nothing(monkeypatch, nf4):
    """SF_FAULT=alloc: the first device allocation of sf_model_create fails as an out-of-memory
    hipMalloc would; the call returns SF_E_NOMEM with a message, hands out no model, and the
    next call (fault off) is checked afresh.  The weights and stream are stand-ins that the
    library never touches before its first allocation."""
    d = sfb.desc_from_shape(synth.TINY)
    ptrs = [1] * len(sfb.weight_order(d, nf4=nf4))
    create = sfb.sf_model_create_nf4 if nf4 else sfb.sf_model_create
    monkeypatch.setenv("SF_FAULT", "alloc")
    with pytest.raises(sfb.SFError) as e:
        create(d, ptrs, 0x1000)
    assert e.value.code == sfb.SF_E_NOMEM and "hipMalloc" in str(e.value)
    L = _lib()
    out = ctypes.c_void_p()
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    fn = L.sf_model_create_nf4 if nf4 else L.sf_model_create
    assert fn(ctypes.byref(d), arr, ctypes.c_void_p(0x1000), ctypes.byref(out)) == sfb.SF_E_NOMEM
    assert not out.value
    monkeypatch.delenv("SF_FAULT")
    ptrs[3] = 0
    with pytest.raises(sfb.SFError) as e:
        create(d, ptrs, 0x1000)
    assert e.value.code == sfb.SF_E_ARG


def test_debug_checks_on_the_regular_build_report_state():
    """The regular library compiles the device checks away: sf_debug_checks says so
    (SF_E_STATE, bits 0) without touching a device, and rejects a NULL pointer."""
    L = _lib()
    bits = ctypes.c_uint32(7)
    assert L.sf_debug_checks(ctypes.byref(bits), 0) == sfb.SF_E_STATE
    assert bits.value == 0 and "without device checks" in sfb.sf_last_error()
    assert L.sf_debug_checks(None, 0) == sfb.SF_E_ARG


def test_checking_library_builds_and_exports_every_symbol():
    """The checking build (SF_CHECKS=1) compiles for gfx950 and exports the same C ABI."""
    from speculative_decoding_verification_decode_amd import build as b
    path = b.CHECKS_LIB if os.path.exists(b.CHECKS_LIB) else b.build_checks()
    hdr = open(os.path.join(ROOT, "include", "sf.h")).read()
    declared = set(re.findall(r"^(?:sf_status|int32_t|const char\*)\s+(sf_\w+)\s*\(", hdr, re.M))
    L = ctypes.CDLL(path)
    missing = [n for n in sorted(declared) if not hasattr(L, n)]
    assert not missing, missing


def test_binding_sizes_outputs_from_the_cache_and_rejects_unknown_handles():
    """The library writes [n_seqs] and [n_seqs][...] host outputs, so the binding takes their
    sizes from the cache it allocated, never from the caller; a handle it did not allocate is
    refused before any call into the library."""
    bogus = ctypes.c_void_p(0x1000)
    with pytest.raises(ValueError):
        sfb.sf_draft_step(bogus, 2)
    with pytest.raises(ValueError):
        sfb.sf_verify(bogus, np.zeros((1, 4), np.int32))

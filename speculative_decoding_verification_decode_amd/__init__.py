"""Python binding of libsf, the MI355X speculative-decoding verify library.

Argument marshalling only: every step of the verify pass runs in the HIP
kernels behind the C ABI declared in include/sf.h; this module turns numpy
arrays and torch tensors into pointers and status codes into exceptions.
PyTorch is used for device memory (weights, caller buffers) and streams.

The functions keep the C names (sf_model_create, sf_cache_alloc, sf_verify,
sf_rollback, sf_draft_step, sf_ngram_propose, ...).  There is no fallback: if
libsf.so has not been built, loading fails with an error.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SF_LIB names another build of the same library (the host-AddressSanitizer build that the CPU
# tests make); by default the in-tree libsf.so.
LIB_PATH = os.environ.get("SF_LIB") or os.path.join(_HERE, "libsf.so")

SF_OK = 0
SF_E_ARG = -1
SF_E_CAPACITY = -2
SF_E_STATE = -3
SF_E_HIP = -4
SF_E_NOMEM = -5

SF_NO_COMMIT = 1
SF_FORCE_ACCEPT = 2
SF_DEBUG_LOGITS = 4

SF_KERNEL_QKV = 0
SF_KERNEL_ATTENTION = 1
SF_KERNEL_OPROJ = 2
SF_KERNEL_GATEUP = 3
SF_KERNEL_DOWN = 4
SF_KERNEL_LMHEAD = 5
SF_KERNEL_VERIFY = 6

_NAMES = {SF_E_ARG: "SF_E_ARG", SF_E_CAPACITY: "SF_E_CAPACITY", SF_E_STATE: "SF_E_STATE",
          SF_E_HIP: "SF_E_HIP", SF_E_NOMEM: "SF_E_NOMEM"}


class SFError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code


class sf_model_desc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("rope_base", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("has_head", ctypes.c_int32), ("tied_head", ctypes.c_int32), ("qkv_bias", ctypes.c_int32)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_PI = ctypes.POINTER(ctypes.c_int32)
_lib = None


def lib():
    """Load libsf.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m "
                              "speculative_decoding_verification_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "sf_model_create": [ctypes.POINTER(sf_model_desc), ctypes.POINTER(_P), _P, ctypes.POINTER(_P)],
            "sf_model_free": [_P],
            "sf_cache_alloc": [_P, _I, _I, _I, ctypes.POINTER(_P)],
            "sf_cache_free": [_P],
            "sf_prefill": [_P, _I, _PI, _I, _PI],
            "sf_verify": [_P, _PI, _PI, ctypes.c_uint32, _PI, _PI, _P],
            "sf_verify_device": [_P, _P, _P, ctypes.c_uint32],
            "sf_results_device": [_P, ctypes.POINTER(_P), ctypes.POINTER(_P)],
            "sf_verify_device_static": [_P, _P, _P, ctypes.c_uint32, _P],
            "sf_rollback": [_P, _I, _I],
            "sf_set_next": [_P, _I, _I],
            "sf_snapshot_save": [_P],
            "sf_model_create_nf4": [ctypes.POINTER(sf_model_desc), ctypes.POINTER(_P), _P, ctypes.POINTER(_P)],
            "sf_nf4_levels": [ctypes.POINTER(ctypes.c_float)],
            "sf_snapshot_restore": [_P],
            "sf_cache_state": [_P, _I, _PI, _PI],
            "sf_draft_step": [_P, _I, _PI],
            "sf_round_create": [_P, _P, _I, ctypes.POINTER(_P)],
            "sf_round_run": [_P, _I],
            "sf_round_free": [_P],
            "sf_ngram_propose": [_PI, _I, _I, _I, _I, _PI],
            "sf_kv_write": [_P, _I, _P, _P, _I, _I],
            "sf_kv_read": [_P, _I, _P, _P, _I, _I],
            "sf_sync": [_P],
            "sf_time_kernel": [_P, _I, _I, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)],
            "sf_debug_counters": [_P, ctypes.POINTER(ctypes.c_int64), _PI],
            "sf_debug_checks": [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int32],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int32
        L.sf_last_error.argtypes = []
        L.sf_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def sf_last_error():
    return lib().sf_last_error().decode()


def _check(st):
    if st != SF_OK:
        raise SFError(st, sf_last_error())
    return st


def _i32(a):
    """int32 C-contiguous numpy array and a pointer to it (None stays NULL)."""
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(_PI)


def _ptr(x):
    """Device pointer of a torch tensor, an int address, or None."""
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


# ------------------------------------------------------------------ description and weights

def desc_from_shape(shape):
    """sf_model_desc from an object with the fields of a decoder shape."""
    return sf_model_desc(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                         shape.ffn, shape.vocab, float(shape.rope_base), float(shape.rms_eps),
                         int(shape.has_head), int(shape.tied_head), int(shape.qkv_bias))


def weight_order(desc, nf4=False):
    """Tensor names in the order sf_model_create expects them; with nf4, each projection
    appears twice (its codes, then its scales), as sf_model_create_nf4 expects."""
    def proj(n):
        return [n, n] if nf4 else [n]
    names = ["embed"]
    for i in range(desc.n_layers):
        p = f"l{i}."
        names += [p + "ln1"] + proj(p + "wq") + ([p + "bq"] if desc.qkv_bias else [])
        names += proj(p + "wk") + ([p + "bk"] if desc.qkv_bias else [])
        names += proj(p + "wv") + ([p + "bv"] if desc.qkv_bias else [])
        names += proj(p + "wo") + [p + "ln2"] + proj(p + "wg") + proj(p + "wu") + proj(p + "wd")
    if desc.has_head:
        names += ["final_norm"] + ([] if desc.tied_head else ["lm_head"])
    return names


# ------------------------------------------------------------------ C functions

def sf_model_create(desc, weight_ptrs, stream=None):
    """weight_ptrs: device addresses in weight_order(desc).  Returns the model handle."""
    arr = (_P * len(weight_ptrs))(*[int(p) for p in weight_ptrs])
    out = _P()
    _check(lib().sf_model_create(ctypes.byref(desc), arr, _ptr(stream), ctypes.byref(out)))
    return out


def sf_model_create_nf4(desc, weight_ptrs, stream=None):
    """weight_ptrs: device addresses in weight_order(desc, nf4=True).  Returns the model handle."""
    arr = (_P * len(weight_ptrs))(*[int(p) for p in weight_ptrs])
    out = _P()
    _check(lib().sf_model_create_nf4(ctypes.byref(desc), arr, _ptr(stream), ctypes.byref(out)))
    return out


def sf_nf4_levels():
    out = np.zeros(16, dtype=np.float32)
    _check(lib().sf_nf4_levels(out.ctypes.data_as(ctypes.POINTER(ctypes.c_float))))
    return out


def sf_model_free(model):
    _check(lib().sf_model_free(model))


# (n_seqs, k_max) of every cache this module allocated, by handle: the library writes
# [n_seqs] and [n_seqs][...] host outputs, so their buffers are sized from the cache itself.
_CACHE_SHAPES = {}


def _handle(cache):
    return cache.value if isinstance(cache, ctypes.c_void_p) else cache


def _cache_shape(cache):
    try:
        return _CACHE_SHAPES[_handle(cache)]
    except KeyError:
        raise ValueError("not a cache allocated through sf_cache_alloc") from None


def sf_cache_alloc(model, n_seqs, capacity, k_max):
    out = _P()
    _check(lib().sf_cache_alloc(model, n_seqs, capacity, k_max, ctypes.byref(out)))
    _CACHE_SHAPES[out.value] = (int(n_seqs), int(k_max))
    return out


def sf_cache_free(cache):
    _check(lib().sf_cache_free(cache))
    _CACHE_SHAPES.pop(_handle(cache), None)


def sf_prefill(cache, seq, tokens):
    arr, p = _i32(tokens)
    nxt = ctypes.c_int32(0)
    _check(lib().sf_prefill(cache, seq, p, len(arr), ctypes.byref(nxt)))
    return nxt.value


def sf_verify(cache, draft, k=None, flags=0, dev_out=None):
    """draft: int array [n_seqs][k_max] of the cache's shape (one sequence: a 1-D array of at
    most k_max drafts, zero-padded here); k: [n_seqs] or None.  Returns (accepted [n_seqs],
    target [n_seqs][k_max+1])."""
    n_seqs, k_max = _cache_shape(cache)
    if draft is not None:
        draft = np.asarray(draft, dtype=np.int32)
        if n_seqs == 1 and draft.ndim <= 1 and draft.size <= k_max:
            draft = np.concatenate([draft.reshape(-1), np.zeros(k_max - draft.size, np.int32)])
        if draft.size != n_seqs * k_max:
            raise ValueError(f"draft has {draft.size} ids; the cache takes [{n_seqs}][{k_max}]")
    d, dp = _i32(draft)
    if k is not None and np.asarray(k).size != n_seqs:
        raise ValueError(f"k has {np.asarray(k).size} entries; the cache has {n_seqs} sequences")
    kk, kp = _i32(k)
    acc = np.zeros(n_seqs, dtype=np.int32)
    tgt = np.zeros((n_seqs, k_max + 1), dtype=np.int32)
    _check(lib().sf_verify(cache, dp, kp, flags, acc.ctypes.data_as(_PI), tgt.ctypes.data_as(_PI),
                           _ptr(dev_out)))
    return acc, tgt


def sf_verify_device(cache, dev_draft, dev_k=None, flags=0):
    _check(lib().sf_verify_device(cache, _ptr(dev_draft), _ptr(dev_k), flags))


def sf_verify_device_static(cache, dev_draft, dev_k, flags, dev_result):
    """The no-allocation verify: results (accepted then targets, int32) go to dev_result."""
    _check(lib().sf_verify_device_static(cache, _ptr(dev_draft), _ptr(dev_k), flags, _ptr(dev_result)))


def sf_results_device(cache):
    a, t = _P(), _P()
    _check(lib().sf_results_device(cache, ctypes.byref(a), ctypes.byref(t)))
    return a.value, t.value


def sf_rollback(cache, seq, pos):
    _check(lib().sf_rollback(cache, seq, pos))


def sf_snapshot_save(cache):
    _check(lib().sf_snapshot_save(cache))


def sf_snapshot_restore(cache):
    _check(lib().sf_snapshot_restore(cache))


def sf_set_next(cache, seq, token):
    _check(lib().sf_set_next(cache, seq, token))


def sf_cache_state(cache, seq):
    ln, nx = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().sf_cache_state(cache, seq, ctypes.byref(ln), ctypes.byref(nx)))
    return ln.value, nx.value


def sf_draft_step(cache, n_steps):
    """Tokens [n_seqs][n_steps] of n_steps greedy steps of every sequence of the cache."""
    n_seqs, _ = _cache_shape(cache)
    out = np.zeros((n_seqs, n_steps), dtype=np.int32)
    _check(lib().sf_draft_step(cache, n_steps, out.ctypes.data_as(_PI)))
    return out


def sf_round_create(drafter_cache, verifier_cache, k):
    out = _P()
    _check(lib().sf_round_create(drafter_cache, verifier_cache, k, ctypes.byref(out)))
    return out


def sf_round_run(round_, n_rounds=1):
    _check(lib().sf_round_run(round_, n_rounds))


def sf_round_free(round_):
    _check(lib().sf_round_free(round_))


def sf_ngram_propose(hist, min_n=2, max_n=4, k_max=8):
    h, hp = _i32(hist)
    out = np.zeros(max(k_max, 1), dtype=np.int32)
    n = lib().sf_ngram_propose(hp, len(h), min_n, max_n, k_max, out.ctypes.data_as(_PI))
    if n < 0:
        raise SFError(n, sf_last_error())
    return out[:n].copy()


def sf_kv_write(cache, seq, dev_k, dev_v, n_pos, src_positions):
    _check(lib().sf_kv_write(cache, seq, _ptr(dev_k), _ptr(dev_v), n_pos, src_positions))


def sf_kv_read(cache, seq, dev_k, dev_v, n_pos, dst_positions):
    _check(lib().sf_kv_read(cache, seq, _ptr(dev_k), _ptr(dev_v), n_pos, dst_positions))


def sf_sync(cache):
    _check(lib().sf_sync(cache))


def sf_time_kernel(cache, kernel, iters):
    """Returns (mean microseconds per launch, algorithmic bytes per launch)."""
    us, by = ctypes.c_float(0), ctypes.c_double(0)
    _check(lib().sf_time_kernel(cache, kernel, iters, ctypes.byref(us), ctypes.byref(by)))
    return us.value, by.value


def sf_debug_counters(cache):
    """(sum, max) of the cache's k-split arrival counters; both 0 between passes."""
    sm, mx = ctypes.c_int64(0), ctypes.c_int32(0)
    _check(lib().sf_debug_counters(cache, ctypes.byref(sm), ctypes.byref(mx)))
    return sm.value, mx.value


SF_CHECK_TOKEN, SF_CHECK_K, SF_CHECK_POS, SF_CHECK_COMMIT, SF_CHECK_NAN = 1, 2, 4, 8, 16


def sf_debug_checks(clear=False):
    """Invariant bits (SF_CHECK_*) the checking build's kernels recorded on the current device,
    optionally cleared; raises SFError (SF_E_STATE) on the regular build."""
    bits = ctypes.c_uint32(0)
    _check(lib().sf_debug_checks(ctypes.byref(bits), 1 if clear else 0))
    return bits.value


# ------------------------------------------------------------------ torch conveniences

def is_nf4(weights):
    """True if the projections come as (codes, scales) pairs."""
    return isinstance(weights.get("l0.wq"), tuple)


def upload_weights(weights, desc, device="cuda"):
    """Copy bf16 bit arrays (numpy uint16, by name) and, for NF4 projections, their (codes
    uint8, scales uint16) pairs to the device; returns (tensors, pointers) in weight_order."""
    import torch
    nf4 = is_nf4(weights)
    tensors, seen = [], {}
    for name in weight_order(desc, nf4):
        w = weights[name]
        if isinstance(w, tuple):
            i = seen.get(name, 0)
            seen[name] = i + 1
            a = np.ascontiguousarray(w[i])
            a = a.view(np.int16) if a.dtype == np.uint16 else a
        else:
            a = np.ascontiguousarray(w).view(np.int16)
        tensors.append(torch.from_numpy(a).to(device))
    return tensors, [t.data_ptr() for t in tensors]


class Engine:
    """A model plus one cache on a torch stream (a new one unless `stream` is given: engines
    that take part in one speculative round share a stream)."""

    def __init__(self, shape, weights, n_seqs=1, capacity=128, k_max=4, keep_weights=False, stream=None):
        import torch
        self.stream = stream if stream is not None else torch.cuda.Stream()
        self.desc = desc_from_shape(shape)
        self.n_seqs, self.capacity, self.k_max = n_seqs, capacity, k_max
        tensors, ptrs = upload_weights(weights, self.desc)
        torch.cuda.synchronize()
        create = sf_model_create_nf4 if is_nf4(weights) else sf_model_create
        self.model = create(self.desc, ptrs, self.stream.cuda_stream)
        self._weights = tensors if keep_weights else None
        del tensors
        self.cache = sf_cache_alloc(self.model, n_seqs, capacity, k_max)

    def close(self):
        if self.cache is not None:
            sf_cache_free(self.cache)
            self.cache = None
        if self.model is not None:
            sf_model_free(self.model)
            self.model = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

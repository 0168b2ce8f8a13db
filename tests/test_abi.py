"""C-ABI checks that need no GPU: exports, workspace sizes, host-side validation.

The validation cases pass arguments that the host checks must reject before
any launch.  They run only where no GPU device node exists: there, even a
validation bug could only end in a failed launch (no device), never in a
kernel touching a bogus pointer.
"""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "engram.h")
NO_GPU = not os.path.exists("/dev/kfd")
# Set by tests/test_abi_sanitized.py: run the validation cases against the
# host-sanitized build of the library, without importing torch.
SANITIZED_LIB = os.environ.get("ENGRAM_ABI_SANITIZED_LIB")


class _Constants:
    """The binding's constants and workspace helper, for a process that
    loads only the sanitized library."""
    ENGRAM_OK, ENGRAM_ERR_ARG, ENGRAM_ERR_UNSUPPORTED, ENGRAM_ERR_HIP = 0, 1, 2, 3
    ENGRAM_ROWS_Q2K, ENGRAM_ROWS_FP8_E4M3_E8M0 = 0, 1

    def __init__(self, path):
        self.LIB_PATH = path
        self._lib = ctypes.CDLL(path)
        self._lib.engram_workspace_bytes.argtypes = [ctypes.c_int32] * 5
        self._lib.engram_workspace_bytes.restype = ctypes.c_size_t

    def engram_workspace_bytes(self, *a):
        return int(self._lib.engram_workspace_bytes(*a))


@pytest.fixture(scope="module")
def eg():
    if SANITIZED_LIB:
        return _Constants(SANITIZED_LIB)
    import __graft_entry__
    __graft_entry__._ensure_built()
    import gram_hash_memory_amd
    return gram_hash_memory_amd


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"ENGRAM_API\s+[\w\s\*]+?\b(engram_\w+)\s*\(", text)))


def test_header_declares_the_five_calls_and_helpers():
    names = declared_functions()
    for want in ("engram_hash", "engram_history_update", "engram_rows", "engram_project", "engram_project_q2k",
                 "engram_project_fp8", "engram_quantize_mxfp8", "engram_project_mxfp8",
                 "engram_stage_mxfp8", "engram_project_mxfp8_staged", "engram_gate",
                 "engram_gate_layers", "engram_forward", "engram_workspace_bytes", "engram_last_error"):
        assert want in names


def test_library_exports_every_declared_symbol(eg):
    lib = ctypes.CDLL(eg.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(eg.EXPORTS)


def test_library_exports_nothing_else(eg):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", eg.LIB_PATH], capture_output=True,
                         text=True).stdout
    ours = {line.split()[-1] for line in out.splitlines()
            if " T " in line and "engram" in line.lower()}
    assert ours == set(declared_functions())


def test_workspace_bytes(eg):
    def a256(x):
        return (x + 255) // 256 * 256
    T, L, cols, hc, dim = 8192, 1, 24, 4, 4096
    want = a256(T * L * cols * 4) + a256(T * cols * 256 * 2) + a256(T * (hc + 1) * dim * 2)
    assert eg.engram_workspace_bytes(T, L, cols, hc, dim) == want
    # several layers: every layer's kv (the gates run in one pass after the projections)
    L = 2
    want = a256(T * L * cols * 4) + a256(T * cols * 256 * 2) + L * a256(T * (hc + 1) * dim * 2)
    assert eg.engram_workspace_bytes(T, L, cols, hc, dim) == want
    assert eg.engram_workspace_bytes(0, 1, 24, 4, 4096) == 0
    assert eg.engram_workspace_bytes(-1, 1, 24, 4, 4096) == 0


# ------------------------------------------------------------ raw C validation

class _HP(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("max_ngram", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("pad_id", ctypes.c_int32),
                ("multipliers", ctypes.c_void_p), ("primes", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p)]


class _TK(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("n_seqs", ctypes.c_int32),
                ("lookback_depth", ctypes.c_int32), ("cids", ctypes.c_void_p),
                ("cu_seqlens", ctypes.c_void_p), ("doc_ids", ctypes.c_void_p),
                ("token_mask", ctypes.c_void_p), ("lookback", ctypes.c_void_p),
                ("lookback_live", ctypes.c_void_p)]


class _LY(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("num_rows", ctypes.c_int64), ("table", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("wkv", ctypes.c_void_p),
                ("q_weight", ctypes.c_void_p), ("k_weight", ctypes.c_void_p),
                ("wkv_mx", ctypes.c_void_p), ("wkv_mx_scales", ctypes.c_void_p)]


FAKE = 0x10000      # aligned, never dereferenced by the host checks


def _raw(eg):
    lib = ctypes.CDLL(SANITIZED_LIB or eg.LIB_PATH)
    lib.engram_last_error.restype = ctypes.c_char_p
    lib.engram_hash.argtypes = [ctypes.POINTER(_HP), ctypes.POINTER(_TK), ctypes.c_void_p,
                                ctypes.c_void_p]
    lib.engram_rows.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.engram_project.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int32] * 3 + [ctypes.c_void_p]
    lib.engram_project_q2k.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p]
    lib.engram_project_fp8.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.engram_gate_layers.argtypes = ([ctypes.c_void_p] * 4 + [ctypes.c_int32, ctypes.c_void_p] +
                                       [ctypes.c_int32] * 3 + [ctypes.c_float] * 3 +
                                       [ctypes.c_void_p])
    lib.engram_history_update.argtypes = [ctypes.POINTER(_TK), ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]
    lib.engram_quantize_mxfp8.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.engram_project_mxfp8.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_void_p]
    lib.engram_stage_mxfp8.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
    lib.engram_project_mxfp8_staged.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.engram_forward.argtypes = [ctypes.POINTER(_HP), ctypes.POINTER(_TK),
                                   ctypes.POINTER(_LY), ctypes.c_void_p, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_float, ctypes.c_float,
                                   ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_void_p, ctypes.c_void_p]
    lib.engram_gate.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int32] * 3 +
                                [ctypes.c_float] * 3 + [ctypes.c_void_p])
    return lib


def _tables(L=1, N=4, H=2):
    cols = (N - 1) * H
    m = np.ones((L, N), np.int64)
    p = np.full((L, cols), 7, np.int64)
    o = (np.arange(cols, dtype=np.int64) * 7)[None].repeat(L, 0)
    return m, p, o


def _hp(m, p, o, L=1, N=4, H=2, pad=0):
    return _HP(L, N, H, pad, m.ctypes.data, p.ctypes.data, o.ctypes.data)


@pytest.mark.skipif(not NO_GPU, reason="validation-rejection cases run only without a GPU")
class TestValidation:
    def test_hash_rejects(self, eg):
        lib = _raw(eg)
        m, p, o = _tables()
        tk = _TK(16, 1, 0, FAKE, FAKE, None, None, None, None)
        assert lib.engram_hash(None, ctypes.byref(tk), FAKE, None) == eg.ENGRAM_ERR_ARG
        cases = [
            (_hp(m, p, o, L=5), eg.ENGRAM_ERR_UNSUPPORTED, "n_layers"),
            (_hp(m, p, o, N=1), eg.ENGRAM_ERR_UNSUPPORTED, "max_ngram"),
            (_hp(m, p, o, N=9), eg.ENGRAM_ERR_UNSUPPORTED, "max_ngram"),
            (_hp(m, p, o, H=0), eg.ENGRAM_ERR_ARG, "n_heads"),
        ]
        for hp, st, msg in cases:
            assert lib.engram_hash(ctypes.byref(hp), ctypes.byref(tk), FAKE, None) == st
            assert msg in lib.engram_last_error().decode()
        bad_p = p.copy()
        bad_p[0, 3] = 0
        hp = _hp(m, bad_p, o)
        assert lib.engram_hash(ctypes.byref(hp), ctypes.byref(tk), FAKE, None) == eg.ENGRAM_ERR_ARG
        assert "primes" in lib.engram_last_error().decode()
        big_o = o.copy()
        big_o[0, 5] = 2**31 - 3
        hp = _hp(m, p, big_o)
        assert lib.engram_hash(ctypes.byref(hp), ctypes.byref(tk), FAKE, None) == eg.ENGRAM_ERR_ARG
        hp = _hp(m, p, o)
        for bad in (_TK(16, 0, 0, FAKE, FAKE, None, None, None, None),
                    _TK(16, 1, 4, FAKE, FAKE, None, None, FAKE, None),      # depth > N-1
                    _TK(16, 1, 0, None, FAKE, None, None, None, None),
                    _TK(16, 1, 0, FAKE + 2, FAKE, None, None, None, None),  # misaligned
                    _TK(16, 1, 2, FAKE, FAKE, None, None, None, FAKE),      # live w/o lookback
                    _TK(-1, 1, 0, FAKE, FAKE, None, None, None, None)):
            assert lib.engram_hash(ctypes.byref(hp), ctypes.byref(bad), FAKE, None) == eg.ENGRAM_ERR_ARG
        assert lib.engram_hash(ctypes.byref(hp), ctypes.byref(tk), None, None) == eg.ENGRAM_ERR_ARG
        empty = _TK(0, 0, 0, None, None, None, None, None, None)
        assert lib.engram_hash(ctypes.byref(hp), ctypes.byref(empty), None, None) == eg.ENGRAM_OK

    def test_rows_rejects(self, eg):
        lib = _raw(eg)
        Q, F = eg.ENGRAM_ROWS_Q2K, eg.ENGRAM_ROWS_FP8_E4M3_E8M0
        ok = dict(fmt=Q, table=FAKE, scales=None, nrows=100, ids=FAKE, stride=24, cols=24, T=8,
                  rows=FAKE, bad=None)

        def call(**kw):
            a = dict(ok, **kw)
            return lib.engram_rows(a["fmt"], a["table"], a["scales"], a["nrows"], a["ids"],
                                   a["stride"], a["cols"], a["T"], a["rows"], a["bad"], None)
        for kw in (dict(fmt=7), dict(nrows=0), dict(cols=0), dict(stride=23), dict(T=-1),
                   dict(table=None), dict(ids=None), dict(rows=None), dict(rows=FAKE + 8),
                   dict(table=FAKE + 2), dict(ids=FAKE + 1), dict(bad=FAKE + 2),
                   dict(fmt=F, scales=None), dict(fmt=F, scales=FAKE, table=FAKE + 4)):
            assert call(**kw) == eg.ENGRAM_ERR_ARG, kw
        assert call(T=0, table=None, ids=None, rows=None) == eg.ENGRAM_OK

    def test_project_rejects(self, eg):
        lib = _raw(eg)
        for args in ((FAKE, FAKE, FAKE, 8, 100, 64),       # K not a multiple of 64
                     (FAKE, FAKE, FAKE, 8, 0, 64),
                     (FAKE, FAKE, FAKE, 8, 64, 0),
                     (FAKE, FAKE, FAKE, -1, 64, 64),
                     (None, FAKE, FAKE, 8, 64, 64),
                     (FAKE, FAKE + 8, FAKE, 8, 64, 64)):
            assert lib.engram_project(*args, None) == eg.ENGRAM_ERR_ARG, args
        assert lib.engram_project(None, None, None, 0, 64, 64, None) == eg.ENGRAM_OK

    def test_project_q2k_rejects(self, eg):
        lib = _raw(eg)
        ok = dict(table=FAKE, nrows=100, ids=FAKE, stride=24, cols=24, wkv=FAKE, kv=FAKE, T=8,
                  N=512, bad=None)

        def call(**kw):
            a = dict(ok, **kw)
            return lib.engram_project_q2k(a["table"], a["nrows"], a["ids"], a["stride"],
                                          a["cols"], a["wkv"], a["kv"], a["T"], a["N"],
                                          a["bad"], None)
        for kw in (dict(nrows=0), dict(cols=0), dict(stride=23), dict(T=-1), dict(N=0),
                   dict(table=None), dict(table=FAKE + 2), dict(ids=None), dict(ids=FAKE + 1),
                   dict(wkv=None), dict(wkv=FAKE + 8), dict(kv=FAKE + 8), dict(bad=FAKE + 2)):
            assert call(**kw) == eg.ENGRAM_ERR_ARG, kw
        # 2^31 / 84 rows and more no longer fit the kernel's 32-bit block offsets.
        too_many = 2147483504 // 84 + 1
        assert call(nrows=too_many) == eg.ENGRAM_ERR_UNSUPPORTED
        assert "exceeds" in lib.engram_last_error().decode()
        assert call(nrows=too_many - 1, T=0, table=None, ids=None, wkv=None,
                    kv=None) == eg.ENGRAM_OK

    def test_history_update_rejects(self, eg):
        lib = _raw(eg)
        tk = _TK(16, 2, 0, FAKE, FAKE, None, None, None, None)
        for depth, hist, live in ((0, FAKE, FAKE), (8, FAKE, FAKE), (3, None, FAKE),
                                  (3, FAKE, None), (3, FAKE + 2, FAKE)):
            assert lib.engram_history_update(ctypes.byref(tk), depth, hist, live,
                                             None) == eg.ENGRAM_ERR_ARG, (depth, hist, live)
        bad = _TK(16, 0, 0, FAKE, FAKE, None, None, None, None)
        assert lib.engram_history_update(ctypes.byref(bad), 3, FAKE, FAKE,
                                         None) == eg.ENGRAM_ERR_ARG
        empty = _TK(0, 0, 0, None, None, None, None, None, None)
        assert lib.engram_history_update(ctypes.byref(empty), 3, None, None,
                                         None) == eg.ENGRAM_OK

    def test_gate_layers_rejects(self, eg):
        lib = _raw(eg)
        P = ctypes.c_void_p * 2
        good = P(FAKE, FAKE)
        bad1 = P(FAKE, FAKE + 4)                  # layer 1's kv misaligned

        def call(n=2, kv=good, q=good, k=good, T=8):
            return lib.engram_gate_layers(FAKE, kv, q, k, n, None, T, 4, 4096, 1e-6, 1e-6,
                                          1 / 64, None)
        assert call(n=0) == eg.ENGRAM_ERR_UNSUPPORTED
        assert call(n=5) == eg.ENGRAM_ERR_UNSUPPORTED
        assert call(kv=None) == eg.ENGRAM_ERR_ARG
        assert call(kv=bad1) == eg.ENGRAM_ERR_ARG
        assert lib.engram_last_error().decode().startswith("layer 1: ")
        assert call(T=0, kv=None, q=None, k=None) == eg.ENGRAM_OK

    def test_quantize_mxfp8_rejects(self, eg):
        lib = _raw(eg)
        for args in ((FAKE, 8, 0, FAKE, FAKE), (FAKE, 8, 48, FAKE, FAKE),
                     (FAKE, -1, 64, FAKE, FAKE), (None, 8, 64, FAKE, FAKE),
                     (FAKE, 8, 64, None, FAKE), (FAKE, 8, 64, FAKE, None),
                     (FAKE + 2, 8, 64, FAKE, FAKE), (FAKE, 8, 64, FAKE + 4, FAKE)):
            assert lib.engram_quantize_mxfp8(*args, None) == eg.ENGRAM_ERR_ARG, args
        assert lib.engram_quantize_mxfp8(None, 0, 64, None, None, None) == eg.ENGRAM_OK

    def test_project_mxfp8_rejects(self, eg):
        lib = _raw(eg)
        ok = dict(table=FAKE, scales=FAKE, nrows=100, ids=FAKE, stride=24, cols=24, wc=FAKE,
                  ws=FAKE, kv=FAKE, T=8, N=512, bad=None)

        def call(**kw):
            a = dict(ok, **kw)
            return lib.engram_project_mxfp8(a["table"], a["scales"], a["nrows"], a["ids"],
                                            a["stride"], a["cols"], a["wc"], a["ws"], a["kv"],
                                            a["T"], a["N"], a["bad"], None)
        for kw in (dict(nrows=0), dict(cols=0), dict(stride=23), dict(T=-1), dict(N=0),
                   dict(table=None), dict(table=FAKE + 4), dict(scales=None),
                   dict(scales=FAKE + 2), dict(ids=None), dict(ids=FAKE + 1), dict(wc=None),
                   dict(wc=FAKE + 8), dict(ws=None), dict(ws=FAKE + 1), dict(kv=None),
                   dict(kv=FAKE + 8), dict(bad=FAKE + 2)):
            assert call(**kw) == eg.ENGRAM_ERR_ARG, kw
        # the weight and the ids are read through 32-bit-offset buffer descriptors
        assert call(N=2147483632 // 6144 + 1) == eg.ENGRAM_ERR_UNSUPPORTED
        assert "exceeds" in lib.engram_last_error().decode()
        assert call(T=2147483632 // (24 * 4) + 1) == eg.ENGRAM_ERR_UNSUPPORTED
        # a table of 2^32 bytes and more is fine (64-bit row addresses)
        assert call(nrows=2**25, T=0, table=None, ids=None, wc=None, ws=None,
                    kv=None) == eg.ENGRAM_OK

    def test_stage_mxfp8_rejects(self, eg):
        lib = _raw(eg)
        ok = dict(table=FAKE, scales=FAKE, nrows=100, ids=FAKE, stride=24, cols=24, T=8,
                  ac=FAKE, asc=FAKE, bad=None)

        def call(**kw):
            a = dict(ok, **kw)
            return lib.engram_stage_mxfp8(a["table"], a["scales"], a["nrows"], a["ids"],
                                          a["stride"], a["cols"], a["T"], a["ac"], a["asc"],
                                          a["bad"], None)
        for kw in (dict(nrows=0), dict(cols=0), dict(stride=23), dict(T=-1), dict(table=None),
                   dict(table=FAKE + 4), dict(scales=None), dict(scales=FAKE + 2),
                   dict(ids=None), dict(ids=FAKE + 1), dict(ac=None), dict(ac=FAKE + 8),
                   dict(asc=None), dict(asc=FAKE + 2), dict(bad=FAKE + 2)):
            assert call(**kw) == eg.ENGRAM_ERR_ARG, kw
        assert call(T=0, table=None, ids=None, ac=None, asc=None) == eg.ENGRAM_OK

    def test_project_mxfp8_staged_rejects(self, eg):
        lib = _raw(eg)
        ok = dict(ac=FAKE, asc=FAKE, cols=24, wc=FAKE, ws=FAKE, kv=FAKE, T=300, N=512)

        def call(**kw):
            a = dict(ok, **kw)
            return lib.engram_project_mxfp8_staged(a["ac"], a["asc"], a["cols"], a["wc"],
                                                   a["ws"], a["kv"], a["T"], a["N"], None)
        for kw in (dict(cols=0), dict(T=-1), dict(N=0), dict(ac=None), dict(ac=FAKE + 8),
                   dict(asc=None), dict(asc=FAKE + 2), dict(wc=None), dict(wc=FAKE + 8),
                   dict(ws=None), dict(ws=FAKE + 1), dict(kv=None), dict(kv=FAKE + 8)):
            assert call(**kw) == eg.ENGRAM_ERR_ARG, kw
        # the weight and the activation are read through 32-bit-offset buffer descriptors
        assert call(N=2147483632 // 6144 + 1) == eg.ENGRAM_ERR_UNSUPPORTED
        assert "exceeds" in lib.engram_last_error().decode()
        assert call(T=2147483632 // 6144 + 1) == eg.ENGRAM_ERR_UNSUPPORTED
        assert "activation" in lib.engram_last_error().decode()
        assert call(T=0, ac=None, asc=None, wc=None, ws=None, kv=None) == eg.ENGRAM_OK

    def test_project_fp8_rejects(self, eg):
        lib = _raw(eg)
        ok = dict(table=FAKE, scales=FAKE, nrows=100, ids=FAKE, stride=24, cols=24, wkv=FAKE,
                  kv=FAKE, T=300, N=512, bad=None)

        def call(**kw):
            a = dict(ok, **kw)
            return lib.engram_project_fp8(a["table"], a["scales"], a["nrows"], a["ids"],
                                          a["stride"], a["cols"], a["wkv"], a["kv"], a["T"],
                                          a["N"], a["bad"], None)
        for kw in (dict(nrows=0), dict(cols=0), dict(stride=23), dict(T=-1), dict(N=0),
                   dict(table=None), dict(table=FAKE + 4), dict(scales=None),
                   dict(scales=FAKE + 2), dict(ids=None), dict(ids=FAKE + 1), dict(wkv=None),
                   dict(wkv=FAKE + 8), dict(kv=None), dict(kv=FAKE + 8), dict(bad=FAKE + 2)):
            assert call(**kw) == eg.ENGRAM_ERR_ARG, kw
        # the ids are read through a 32-bit-offset buffer descriptor
        assert call(T=2147483632 // (24 * 4) + 1) == eg.ENGRAM_ERR_UNSUPPORTED
        assert "exceeds" in lib.engram_last_error().decode()
        # a table of 2^32 bytes and more is fine (64-bit row addresses)
        assert call(nrows=2**25, T=0, table=None, ids=None, wkv=None, kv=None) == eg.ENGRAM_OK

    def test_forward_mx_layer_rejects(self, eg):
        lib = _raw(eg)
        m, p, o = _tables()
        hp = _hp(m, p, o)
        tk = _TK(16, 1, 0, FAKE, FAKE, None, None, None, None)
        F, Q = eg.ENGRAM_ROWS_FP8_E4M3_E8M0, eg.ENGRAM_ROWS_Q2K
        ws = eg.engram_workspace_bytes(16, 1, 6, 2, 64)

        def call(**kw):
            d = dict(fmt=F, num_rows=64, table=FAKE, scales=FAKE, wkv=None, q_weight=FAKE,
                     k_weight=FAKE, wkv_mx=FAKE, wkv_mx_scales=FAKE)
            d.update(kw)
            ly = _LY(d["fmt"], d["num_rows"], d["table"], d["scales"], d["wkv"],
                     d["q_weight"], d["k_weight"], d["wkv_mx"], d["wkv_mx_scales"])
            return lib.engram_forward(ctypes.byref(hp), ctypes.byref(tk), ctypes.byref(ly), FAKE,
                                      2, 64, 1e-6, 1e-6, 0.1, FAKE, ws, None, None)
        for kw, msg in ((dict(fmt=Q, scales=None), "FP8"), (dict(wkv_mx_scales=None), "scales"),
                        (dict(wkv_mx=None), "codes"), (dict(wkv_mx=FAKE + 8), "codes"),
                        (dict(scales=None), "scales"), (dict(table=FAKE + 4), "table")):
            assert call(**kw) == eg.ENGRAM_ERR_ARG, kw
            err = lib.engram_last_error().decode()
            assert err.startswith("layer 0: ") and msg in err, (kw, err)
        # without wkv_mx the layer needs the bf16 wkv
        assert call(wkv_mx=None, wkv_mx_scales=None) == eg.ENGRAM_ERR_ARG

    def test_forward_rejects(self, eg):
        lib = _raw(eg)
        m, p, o = _tables()                       # 6 columns of 7 rows: rows 0..41
        T, hc, dim = 16, 2, 64
        Q = eg.ENGRAM_ROWS_Q2K
        ws_need = eg.engram_workspace_bytes(T, 1, 6, hc, dim)

        def call(num_rows=42, ws=FAKE, ws_bytes=ws_need, n_layers=1, layers=None, **kw):
            hp = _hp(m, p, o)
            tk = _TK(T, 1, 0, FAKE, FAKE, None, None, None, None)
            d = dict(table=FAKE, wkv=FAKE, q_weight=FAKE, k_weight=FAKE)
            d.update(kw)
            ly = _LY(Q, num_rows, d["table"], None, d["wkv"], d["q_weight"], d["k_weight"],
                     None, None)
            return lib.engram_forward(ctypes.byref(hp), ctypes.byref(tk),
                                      None if layers == "null" else ctypes.byref(ly), FAKE, hc,
                                      dim, 1e-6, 1e-6, 0.125, ws, ws_bytes, None, None)
        # the hash's buckets must lie inside the table: offsets + primes <= num_rows
        assert call(num_rows=41) == eg.ENGRAM_ERR_ARG
        err = lib.engram_last_error().decode()
        assert "offsets + primes" in err and "42" in err and "41" in err, err
        # the workspace must hold ids, one layer's rows and every layer's kv
        assert call(ws_bytes=ws_need - 1) == eg.ENGRAM_ERR_ARG
        assert "workspace_bytes" in lib.engram_last_error().decode()
        assert call(ws=None) == eg.ENGRAM_ERR_ARG
        assert call(ws=FAKE + 128) == eg.ENGRAM_ERR_ARG       # not 256-byte aligned
        assert "256" in lib.engram_last_error().decode()
        assert call(layers="null") == eg.ENGRAM_ERR_ARG
        for kw in (dict(table=None), dict(table=FAKE + 2), dict(wkv=None), dict(wkv=FAKE + 8),
                   dict(q_weight=None), dict(k_weight=FAKE + 4)):
            assert call(**kw) == eg.ENGRAM_ERR_ARG, kw
            assert lib.engram_last_error().decode().startswith("layer 0: "), kw

    def test_forward_noalloc_rejects_shapes_beyond_the_static_array(self, eg):
        lib = _raw(eg)
        lib.engram_forward_noalloc.argtypes = [ctypes.POINTER(_HP), ctypes.POINTER(_TK),
                                               ctypes.POINTER(_LY), ctypes.c_void_p,
                                               ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                               ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                               ctypes.c_void_p]
        m, p, o = _tables()
        hp = _hp(m, p, o)
        hc, dim = 4, 4096
        ly = _LY(eg.ENGRAM_ROWS_Q2K, 42, FAKE, None, FAKE, FAKE, FAKE, None, None)
        limit = 32 << 20
        for T, st in ((512, None), (1024, eg.ENGRAM_ERR_UNSUPPORTED)):
            need = eg.engram_workspace_bytes(T, 1, 6, hc, dim)
            tk = _TK(T, 1, 0, FAKE, FAKE, None, None, None, None)
            if st is None:
                assert need <= limit                 # allowed: not called here (no GPU)
                continue
            assert need > limit
            assert lib.engram_forward_noalloc(ctypes.byref(hp), ctypes.byref(tk),
                                              ctypes.byref(ly), FAKE, hc, dim, 1e-6, 1e-6,
                                              0.0156, None, None) == st
            assert "static array" in lib.engram_last_error().decode()
        # the other checks are engram_forward's, before any workspace is looked up
        bad = _TK(16, 0, 0, FAKE, FAKE, None, None, None, None)
        assert lib.engram_forward_noalloc(ctypes.byref(hp), ctypes.byref(bad), ctypes.byref(ly),
                                          FAKE, hc, dim, 1e-6, 1e-6, 0.0156, None,
                                          None) == eg.ENGRAM_ERR_ARG
        empty = _TK(0, 0, 0, None, None, None, None, None, None)
        assert lib.engram_forward_noalloc(ctypes.byref(hp), ctypes.byref(empty),
                                          ctypes.byref(ly), None, hc, dim, 1e-6, 1e-6, 0.0156,
                                          None, None) == eg.ENGRAM_OK

    def test_gate_rejects(self, eg):
        lib = _raw(eg)
        ok = [FAKE, FAKE, FAKE, FAKE, None, 8, 4, 4096, 1e-6, 1e-6, 1 / 64]
        for i, v, st in ((6, 9, eg.ENGRAM_ERR_UNSUPPORTED), (6, 0, eg.ENGRAM_ERR_UNSUPPORTED),
                         (7, 100, eg.ENGRAM_ERR_UNSUPPORTED), (7, 16384, eg.ENGRAM_ERR_UNSUPPORTED),
                         (5, -1, eg.ENGRAM_ERR_ARG), (8, -1.0, eg.ENGRAM_ERR_ARG),
                         (0, None, eg.ENGRAM_ERR_ARG), (1, FAKE + 4, eg.ENGRAM_ERR_ARG)):
            a = list(ok)
            a[i] = v
            assert lib.engram_gate(*a, None) == st, (i, v)
        a = list(ok)
        a[5] = 0
        a[0] = None
        assert lib.engram_gate(*a, None) == eg.ENGRAM_OK


def test_binding_refuses_host_tensors(eg):
    import torch
    h = torch.zeros(4, 2, 8)
    with pytest.raises(TypeError):
        eg.engram_gate(h, h, h, h, None, 4, 2, 8, 1e-6, 1e-6, 0.3, stream=0)


def test_library_was_built_from_these_sources(eg):
    # The library records the sha256 of the sources it was built from; the
    # binding refuses to load a library whose record differs from the tree.
    import importlib.util
    path = os.path.join(ROOT, "gram_hash_memory_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_engram_build_test", path)
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    assert eg.engram_build_id() == b.build_id()
    assert eg.BUILD_ID.startswith("sha256:") and len(eg.BUILD_ID) == 7 + 64
    assert b.library_is_current()
    b.build_id = lambda: "sha256:" + "0" * 64           # as if a source had changed
    assert not b.library_is_current()

"""The C ABI without a GPU: the library loads, exports every symbol that
include/hata.h declares, and every argument check returns its status before
anything is launched."""
import ctypes
import os
import re

import pytest

from hash_top_sparse_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hata.h")

OK, ENULL, ESHAPE, EUNSUP, EALIGN, EWS, EHIP = range(7)
P = ctypes.c_void_p
F = ctypes.c_float
A = P(0x10000)        # aligned, never dereferenced: validation fails or the hook fires first
MIS = P(0x10008)      # 8-byte but not 16-byte aligned
MIS2 = P(0x10002)     # 2-byte but not 4-byte aligned


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from hash_top_sparse_amd import build
        build.build()
    return binding.load()


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(hata_[a-z_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(binding.exported_symbols()) == set(names)


def _hip_imports():
    import shutil
    import subprocess

    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", binding.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    return sorted({ln.split()[-1].split("@")[0] for ln in out.splitlines() if ln.strip()})


def test_library_never_allocates_or_creates_streams(lib):
    """The library imports no allocation, free or stream-creation routine of
    the HIP runtime, and synchronises only inside hata_workspace_check (the
    diagnostic that reads the workspace's error word)."""
    syms = [s for s in _hip_imports() if s.startswith("hip")]
    assert "hipLaunchKernel" in syms            # the import list was read
    banned = ("hipMalloc", "hipFree", "hipHostMalloc", "hipHostFree", "hipStreamCreate", "hipStreamDestroy",
              "hipEventCreate", "hipDeviceSynchronize", "hipEventSynchronize", "hipHostRegister",
              "hipExtMalloc", "hipMallocAsync", "hipMemAlloc")
    bad = [s for s in syms if s.startswith(banned)]
    assert not bad, bad
    waits = [s for s in syms if "Synchronize" in s or s in ("hipMemcpy", "hipMemset", "hipMemcpyDtoH")]
    assert set(waits) <= {"hipStreamSynchronize", "hipMemcpy"}, waits


def test_status_strings(lib):
    for s in range(7):
        assert binding.status_string(s).startswith("HATA_")
    assert "unknown" in binding.status_string(99)
    assert lib.hata_version() >= 100


def _enc(**kw):
    a = dict(x=A, x_rows=16, B=1, H=4, n_new=1, W=A, Hkv=1, d=128, r=128, codes=A, cap=16, pos=None)
    a.update(kw)
    return binding.raw_call("hata_encode_append", a["x"], a["x_rows"], a["B"], a["H"], a["n_new"],
                            a["W"], a["Hkv"], a["d"], a["r"], a["codes"], a["cap"], a["pos"], None)


def test_encode_append_validation():
    assert _enc(x=None) == ENULL
    assert _enc(codes=None) == ENULL
    assert _enc(d=64) == EUNSUP
    assert _enc(r=96) == EUNSUP
    assert _enc(r=512) == EUNSUP
    assert _enc(H=6, Hkv=4) == ESHAPE
    assert _enc(n_new=-1) == ESHAPE
    assert "n_new" in binding.last_error_message()
    assert _enc(n_new=17) == ESHAPE            # more rows than x_rows without pos
    assert _enc(codes=MIS) == EALIGN
    assert _enc(n_new=0) == OK                 # nothing to do, nothing launched


def _ham(**kw):
    a = dict(qc=A, kc=A, B=1, Hq=32, Hkv=8, r=128, cap=1024, seq=A, max_len=1024, sc=A)
    a.update(kw)
    return binding.raw_call("hata_hamming_scores", a["qc"], a["kc"], a["B"], a["Hq"], a["Hkv"],
                            a["r"], ctypes.c_int64(a["cap"]), a["seq"], ctypes.c_int64(a["max_len"]),
                            a["sc"], None)


def test_hamming_validation():
    assert _ham(kc=None) == ENULL
    assert _ham(Hq=12, Hkv=4) == EUNSUP        # G = 3
    assert _ham(Hq=30, Hkv=8) == ESHAPE        # not a multiple
    assert _ham(max_len=2048) == ESHAPE        # max_len > cap
    assert _ham(max_len=0) == ESHAPE
    assert _ham(kc=MIS) == EALIGN
    assert _ham(r=96) == EUNSUP
    assert _ham(r=16) == EUNSUP


def _topk(**kw):
    a = dict(sc=A, B=1, Hkv=8, cap=1024, seq=A, max_len=1024, k=512, max_score=512, idx=A)
    a.update(kw)
    return binding.raw_call("hata_topk", a["sc"], a["B"], a["Hkv"], ctypes.c_int64(a["cap"]), a["seq"],
                            ctypes.c_int64(a["max_len"]), a["k"], a["max_score"], a["idx"], None,
                            ctypes.c_size_t(0), None)


def test_topk_validation():
    assert _topk(idx=None) == ENULL
    assert _topk(k=0) == EUNSUP
    assert _topk(k=4097) == EUNSUP
    assert _topk(max_score=2049) == EUNSUP
    assert _topk(max_len=0) == ESHAPE


def test_sparse_and_dense_workspace_checks(lib):
    need = binding.workspace_bytes(binding.OP_SPARSE_DECODE, 1, 32, 8, 1024, 512)
    assert need > 0
    rc = binding.raw_call("hata_sparse_decode", A, A, A, 1, 32, 8, 128, ctypes.c_int64(1024), A, 512,
                          F(0.088), A, None, ctypes.c_size_t(0), None)
    assert rc == EWS
    rc = binding.raw_call("hata_sparse_decode", A, A, A, 1, 32, 8, 128, ctypes.c_int64(1024), A, 512,
                          F(0.088), A, A, ctypes.c_size_t(need - 1), None)
    assert rc == EWS
    rc = binding.raw_call("hata_sparse_decode", A, MIS, A, 1, 32, 8, 128, ctypes.c_int64(1024), A, 512,
                          F(0.088), A, A, ctypes.c_size_t(need), None)
    assert rc == EALIGN
    dneed = binding.workspace_bytes(binding.OP_DENSE_DECODE, 1, 32, 8, 4096, 1)
    assert dneed > 0
    rc = binding.raw_call("hata_dense_decode", A, A, A, 1, 32, 8, 128, ctypes.c_int64(4096), A,
                          ctypes.c_int64(4096), F(0.088), A, A, ctypes.c_size_t(dneed - 4), None)
    assert rc == EWS
    # top-k: the optional scratch of the many-workgroup selection (unit
    # histograms of G r + 1 bins, threshold and tie quota, per-chunk counts)
    U, nb, chunks = 8, 4 * 128 + 1, 1
    assert binding.workspace_bytes(binding.OP_TOPK, 1, 32, 8, 4096, 512) == 4 * (U * nb + 2 * U + 2 * U * chunks)


def test_decode_step_validation():
    def step(**kw):
        a = dict(q=A, K=A, V=A, W=A, codes=A, B=1, Hq=32, Hkv=8, d=128, r=128, cap=4096, seq=A,
                 max_len=4096, k=512, out=A)
        a.update(kw)
        return binding.raw_call("hata_decode_step", a["q"], a["K"], a["V"], a["W"], a["codes"], a["B"],
                                a["Hq"], a["Hkv"], a["d"], a["r"], ctypes.c_int64(a["cap"]), a["seq"],
                                ctypes.c_int64(a["max_len"]), a["k"], F(0.088), a["out"], None, A,
                                ctypes.c_size_t(1 << 30), None)
    assert step(W=None) == ENULL
    assert step(out=None) == ENULL
    assert step(d=96) == EUNSUP
    assert step(Hq=48, Hkv=4) == EUNSUP         # G = 12
    assert step(k=0) == EUNSUP
    assert step(max_len=8192) == ESHAPE
    assert step(codes=MIS) == EALIGN


def test_decode_step_qk_validation():
    def step(**kw):
        a = dict(q=A, K=A, V=A, Wq=A, Wk=A, codes=A, B=1, Hq=32, Hkv=8, d=128, r=128, cap=4096, seq=A,
                 max_len=4096, k=512, out=A)
        a.update(kw)
        return binding.raw_call("hata_decode_step_qk", a["q"], a["K"], a["V"], a["Wq"], a["Wk"], a["codes"],
                                a["B"], a["Hq"], a["Hkv"], a["d"], a["r"], ctypes.c_int64(a["cap"]), a["seq"],
                                ctypes.c_int64(a["max_len"]), a["k"], F(0.088), a["out"], None, A,
                                ctypes.c_size_t(1 << 30), None)
    assert step(Wq=None) == ENULL
    assert step(Wk=None) == ENULL
    assert step(d=96) == EUNSUP
    assert step(k=0) == EUNSUP
    assert step(max_len=8192) == ESHAPE
    assert step(codes=MIS) == EALIGN


def test_hash_labels_validation(lib):
    f = lib.hata_hash_labels
    ok = dict(q=A, k=A, pos=A, J=16, n=1024, d=128, pm=100, lab=A)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["q"], a["k"], a["pos"], a["J"], a["n"], a["d"], a["pm"], F(20.0), F(1.0), a["lab"], None)
    assert call(q=None) == ENULL
    assert call(lab=None) == ENULL
    assert call(d=64) == EUNSUP
    assert call(n=8193) == EUNSUP
    assert call(J=0) == ESHAPE
    assert call(pm=0) == ESHAPE
    assert call(pm=1001) == ESHAPE
    assert call(k=MIS2) == EALIGN
    assert call(q=MIS) == EALIGN
    assert call(k=MIS) == EALIGN


def test_hash_train_step_validation(lib):
    f = lib.hata_hash_train_step
    need = lib.hata_hash_train_workspace_bytes(64, 1024, 128, 128)
    assert need > 0
    assert lib.hata_hash_train_workspace_bytes(64, 1024, 128, 48) == 0
    assert lib.hata_hash_train_workspace_bytes(64, 1024, 96, 128) == 0

    def call(r=128, d=128, W=A, loss=A, ws_bytes=need, J=64, n=1024):
        return f(A, A, A, A, J, n, d, r, F(1.0), F(1.0), F(1.0), F(1.0), F(0.01), W, None, loss, A,
                 ctypes.c_size_t(ws_bytes), None)
    assert call(W=None) == ENULL
    assert call(loss=None) == ENULL
    assert call(d=96) == EUNSUP
    assert call(r=48) == EUNSUP
    assert call(r=512) == EUNSUP
    assert call(J=0) == ESHAPE
    assert call(ws_bytes=need - 1) == EWS


def _prefill(**kw):
    a = dict(q=A, K=A, V=A, W=A, codes=A, B=1, Hq=32, Hkv=8, d=128, r=128, q_rows=4096, cap=4096, seq=A,
             max_len=4096, out=A)
    a.update(kw)
    return binding.raw_call("hata_prefill", a["q"], a["K"], a["V"], a["W"], a["codes"], a["B"], a["Hq"],
                            a["Hkv"], a["d"], a["r"], ctypes.c_int64(a["q_rows"]), ctypes.c_int64(a["cap"]),
                            a["seq"], ctypes.c_int64(a["max_len"]), F(0.088), a["out"], None)


def test_prefill_validation():
    assert _prefill(q=None) == ENULL
    assert _prefill(codes=None) == ENULL
    assert _prefill(seq=None) == ENULL
    assert _prefill(out=None) == ENULL
    assert _prefill(d=64) == EUNSUP
    assert _prefill(r=96) == EUNSUP
    assert _prefill(Hq=48, Hkv=4) == EUNSUP      # G = 12
    assert _prefill(Hq=30, Hkv=8) == ESHAPE      # not a multiple
    assert _prefill(max_len=4097) == ESHAPE      # beyond cap
    assert _prefill(q_rows=4095) == ESHAPE       # queries shorter than max_len
    assert _prefill(max_len=0) == ESHAPE
    assert _prefill(q=MIS) == EALIGN
    assert _prefill(out=MIS) == EALIGN
    assert _prefill(codes=MIS2) == EALIGN


def _paged(**kw):
    a = dict(q=A, K=A, V=A, W=A, codes=A, bt=A, max_pages=256, num_pages=300, P=16, B=1, Hq=32, Hkv=8, d=128,
             r=128, seq=A, max_len=4096, k=512, out=A, ws_bytes=1 << 30)
    a.update(kw)
    return binding.raw_call("hata_decode_step_paged", a["q"], a["K"], a["V"], a["W"], a["codes"], a["bt"],
                            a["max_pages"], a["num_pages"], a["P"], a["B"], a["Hq"], a["Hkv"], a["d"], a["r"],
                            a["seq"], ctypes.c_int64(a["max_len"]), a["k"], F(0.088), a["out"], None, A,
                            ctypes.c_size_t(a["ws_bytes"]), None)


def test_decode_step_paged_validation(lib):
    # (the workspace size depends on the device's CU count, as for the
    # contiguous step, so it is not checked here)
    assert _paged(bt=None) == ENULL
    assert _paged(codes=None) == ENULL
    assert _paged(d=64) == EUNSUP
    assert _paged(P=24) == EUNSUP               # not a power of two
    assert _paged(P=8) == EUNSUP
    assert _paged(k=0) == EUNSUP
    assert _paged(max_pages=0) == ESHAPE
    assert _paged(num_pages=0) == ESHAPE
    assert _paged(max_len=4097) == ESHAPE       # beyond max_pages * page_rows
    assert _paged(codes=MIS) == EALIGN
    assert _paged(bt=MIS2) == EALIGN


def _prefill_paged(**kw):
    a = dict(q=A, K=A, V=A, W=A, codes=A, bt=A, max_pages=256, num_pages=300, P=16, B=1, Hq=32, Hkv=8, d=128,
             r=128, q_rows=4096, seq=A, max_len=4096, out=A)
    a.update(kw)
    return binding.raw_call("hata_prefill_paged", a["q"], a["K"], a["V"], a["W"], a["codes"], a["bt"],
                            a["max_pages"], a["num_pages"], a["P"], a["B"], a["Hq"], a["Hkv"], a["d"], a["r"],
                            ctypes.c_int64(a["q_rows"]), a["seq"], ctypes.c_int64(a["max_len"]), F(0.088), a["out"],
                            None)


def test_prefill_paged_validation():
    assert _prefill_paged(bt=None) == ENULL
    assert _prefill_paged(codes=None) == ENULL
    assert _prefill_paged(d=64) == EUNSUP
    assert _prefill_paged(P=48) == EUNSUP
    assert _prefill_paged(Hq=48, Hkv=4) == EUNSUP
    assert _prefill_paged(max_pages=0) == ESHAPE
    assert _prefill_paged(max_len=4097) == ESHAPE       # beyond max_pages * page_rows
    assert _prefill_paged(q_rows=100) == ESHAPE
    assert _prefill_paged(K=MIS) == EALIGN
    assert _prefill_paged(bt=MIS2) == EALIGN


def lib_stream_read_valid():
    return binding.load().hata_stream_read(A, ctypes.c_size_t(4096), A, ctypes.c_size_t(1024), P(None))


def test_stream_read_validation(lib):
    SZ = ctypes.c_size_t
    f = lib.hata_stream_read
    assert f(P(None), SZ(4096), A, SZ(1024), P(None)) == ENULL
    assert f(A, SZ(4096), P(None), SZ(1024), P(None)) == ENULL
    assert f(MIS, SZ(4096), A, SZ(1024), P(None)) == EALIGN
    assert f(A, SZ(4100), A, SZ(1024), P(None)) == EALIGN
    assert f(A, SZ(4096), A, SZ(1023), P(None)) == EWS


def test_forced_launch_failure_propagates():
    """With the test hook set, a fully valid call reports HATA_ERR_HIP before
    launching, and the binding raises it as HataError."""
    os.environ["HATA_TEST_FAIL_LAUNCH"] = "1"
    try:
        assert _ham() == EHIP
        assert "forced" in binding.last_error_message()
        assert _topk() == EHIP
        assert _enc() == EHIP
        assert lib_stream_read_valid() == EHIP
        assert _prefill() == EHIP
        assert _paged() == EHIP
        assert _prefill_paged() == EHIP
        with pytest.raises(binding.HataError) as ei:
            binding._check(_ham())
        assert ei.value.status == EHIP
    finally:
        del os.environ["HATA_TEST_FAIL_LAUNCH"]

"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, sizes its buffers as documented, and rejects bad arguments on the host
before anything is enqueued. No GPU is needed: every call below fails
validation (or is a pure size query) and never reaches the HIP runtime."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmhead.h")


@pytest.fixture(scope="module")
def lib():
    from lm_head_log_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from lm_head_log_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lmhead_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_signatures():
    from lm_head_log_amd import _lib
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_names_match_c_names():
    import lm_head_log_amd as m
    for name in declared_functions():
        assert callable(getattr(m, name)), name


def test_version_and_status_strings(lib):
    assert lib.lmhead_version() >= 100
    for s in range(6):
        assert lib.lmhead_status_string(s)
    assert b"unknown" in lib.lmhead_status_string(99)


def _align(x):
    return (x + 255) // 256 * 256


def test_saved_bytes_is_16_bytes_per_row_plus_header(lib):
    assert lib.lmhead_saved_bytes(-1) == 0
    assert lib.lmhead_saved_bytes(0) == 1024
    for N in (1, 100, 16384, 262144):
        assert lib.lmhead_saved_bytes(N) == 1024 + 4 * _align(4 * N)


def test_saved_state_is_far_below_one_full_vocab_activation(lib):
    """twinkle PR #283, Experiment results: at N=16384, V=151936 one full-vocab
    activation is 4.6 GiB (bf16). The saved state is per row, never per logit."""
    g = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "pages_figures.txt")):
        line = line.split("#", 1)[0]
        if "=" in line:
            k, v = line.split("=", 1)
            g[k.strip()] = float(v.split()[0])
    N, V = int(g["twinkle_N"]), int(g["twinkle_V"])
    full_bf16 = N * V * 2
    assert abs(full_bf16 / 2 ** 30 - g["twinkle_full_vocab_bf16_gib"]) < 0.05
    assert abs(2 * full_bf16 / 2 ** 30 - g["twinkle_full_vocab_fp32_gib"]) < 0.05
    assert lib.lmhead_saved_bytes(N) < full_bf16 / 10000


def _fwd_ws(N, H, V):
    nv = (V + 255) // 256
    up64 = lambda x: (x + 63) // 64 * 64
    rows = (N + 255) // 256 * 256
    return (_align(32) + _align(4 * rows) + _align(4 * N) + 3 * _align(nv * N * 4)
            + _align(H * up64(N) * 2))


MAX_N, MAX_H, MAX_V, MAX_CHUNK = 1 << 24, 1 << 20, 1 << 22, 1 << 22


def _bwd_ws(N, H, V, chunk):
    up = lambda x, m: (x + m - 1) // m * m
    ldz = up(V, 256) + 64  # dZ rows padded by 64 elements
    want = chunk if chunk > 0 else max(256, (8 << 30) // (2 * ldz) // 256 * 256)
    want = min(want, MAX_CHUNK)
    C = min(up(want, 256), up(N, 256)) if N > 0 else 0
    nchunks = (N + C - 1) // C if N > 0 else 1
    rows = up(N, 256)
    # partial dX tiles of a split tail: S pieces of each of at most 256 (S - 1) / S
    # tiles; S = 8 when 8 pieces of a multiple of 64 rows fit in V rounded to 256
    pieces = 1
    if V >= 2048:
        pieces = 8 if 8 * up(-(-V // 8), 64) <= up(V, 256) else 4
    tail = min(256 * (pieces - 1) // pieces, C // 256 * up(H, 256) // 256) if pieces > 1 else 0
    # checked copy of the saved header | queues | dz coefficients | targets |
    # one chunk of X_c^T (rows padded by 64 elements) | dZ of one chunk |
    # partial dX tiles
    return (256 + _align(nchunks * 4 * 32) + _align(16 * rows) + _align(4 * rows)
            + _align(H * (C + 64) * 2) + _align(C * ldz * 2)
            + tail * pieces * 256 * 256 * 4)


def test_workspace_sizes(lib):
    for (N, H, V) in ((16384, 4096, 131072), (128, 512, 8192), (10, 64, 1000), (0, 64, 5),
                      (262144, 5120, 152064), (700, 256, 20000), (16384, 2560, 151936)):
        assert lib.lmhead_fwd_workspace_bytes(N, H, V) == _fwd_ws(N, H, V)
        for chunk in (0, 100, 256, 8192, 1 << 20):
            assert lib.lmhead_bwd_workspace_bytes(N, H, V, chunk) == _bwd_ws(N, H, V, chunk)
    # default chunk: bf16 dZ within 8 GiB, i.e. the whole 16K batch at
    # V = 131072 (4 GiB)
    N, H, V = 16384, 4096, 131072
    assert _bwd_ws(N, H, V, 0) == _bwd_ws(N, H, V, 16384)
    # the 4096-row chunking holds one chunk of dZ (rows of V + 64) and of X_c^T
    # instead of the whole batch's, and four chunks' tile-queue counters
    # instead of one
    queues = _align(4 * 4 * 32) - _align(1 * 4 * 32)
    assert (_bwd_ws(N, H, V, 0) - _bwd_ws(N, H, V, 4096)
            == (16384 - 4096) * (V + 64 + H) * 2 - queues)
    assert _bwd_ws(262144, 4096, 152064, 0) == _bwd_ws(262144, 4096, 152064, 28160)
    # invalid sizes
    assert lib.lmhead_fwd_workspace_bytes(10, 100, 1000) == 0
    assert lib.lmhead_fwd_workspace_bytes(-1, 64, 1000) == 0
    assert lib.lmhead_bwd_workspace_bytes(10, 64, 0, 0) == 0
    assert lib.lmhead_fwd_workspace_bytes(10, 64, (1 << 22) + 1) == 0


def test_size_limits(lib):
    """N <= 2^24, H <= 2^20, V <= 2^22: every operand's buffer descriptors then
    stay below 2^31 bytes and every tile index inside int32; past them the
    size queries return 0 and the calls return LMHEAD_ERR_UNSUPPORTED."""
    assert lib.lmhead_fwd_workspace_bytes(MAX_N, 64, 1000) == _fwd_ws(MAX_N, 64, 1000)
    assert lib.lmhead_fwd_workspace_bytes(MAX_N + 1, 64, 1000) == 0
    assert lib.lmhead_fwd_workspace_bytes(16, MAX_H, 1000) > 0
    assert lib.lmhead_fwd_workspace_bytes(16, MAX_H + 64, 1000) == 0
    assert lib.lmhead_fwd_workspace_bytes(16, 64, MAX_V) > 0
    assert lib.lmhead_fwd_workspace_bytes(16, 64, MAX_V + 1) == 0
    assert lib.lmhead_bwd_workspace_bytes(MAX_N, 256, 1000, 0) == _bwd_ws(MAX_N, 256, 1000, 0)
    assert lib.lmhead_bwd_workspace_bytes(MAX_N + 1, 256, 1000, 0) == 0
    # the token chunk is clamped to 2^22 rows, whatever is asked for
    assert _bwd_ws(MAX_N, 256, 256, 0) == _bwd_ws(MAX_N, 256, 256, MAX_CHUNK)
    assert (lib.lmhead_bwd_workspace_bytes(MAX_N, 256, 256, 1 << 23)
            == lib.lmhead_bwd_workspace_bytes(MAX_N, 256, 256, MAX_CHUNK))
    assert _fwd(lib, N=MAX_N + 1) == 2
    assert _fwd(lib, entry="lmhead_fwd_blocksparse", N=MAX_N + 1) == 2
    assert _fwd(lib, V=MAX_V + 1) == 2
    assert _bwd(lib, N=MAX_N + 1) == 2
    assert _fwdp(lib, N=MAX_N + 1) == 2
    assert _bwdp(lib, N=MAX_N + 1) == 2
    assert _merge(lib, N=MAX_N + 1) == 1


FAKE = ctypes.c_void_p(0x10000)   # 16-byte aligned, never dereferenced
ODD = ctypes.c_void_p(0x10002)


def _fwd(lib, entry="lmhead_fwd", **kw):
    a = dict(hidden=FAKE, weight=FAKE, targets=FAKE, keep=None, N=8, H=64, V=100,
             ret=1, erg=1, logp=FAKE, ent=FAKE, saved=FAKE, saved_bytes=1 << 20,
             ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return getattr(lib, entry)(a["hidden"], a["weight"], a["targets"], a["keep"], a["N"], a["H"],
                          a["V"], a["ret"], a["erg"], a["logp"], a["ent"], a["saved"],
                          a["saved_bytes"], a["ws"], a["ws_bytes"], a["stream"])


def _bwd(lib, **kw):
    a = dict(hidden=FAKE, weight=FAKE, targets=FAKE, N=8, H=64, V=100, erg=1, saved=FAKE,
             saved_bytes=1 << 20, glp=FAKE, gh=FAKE, gX=FAKE, gW=FAKE, chunk=0, ws=FAKE,
             ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.lmhead_bwd(a["hidden"], a["weight"], a["targets"], a["N"], a["H"], a["V"],
                          a["erg"], a["saved"], a["saved_bytes"], a["glp"], a["gh"], a["gX"],
                          a["gW"], a["chunk"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), 1),
    (dict(V=0), 1),
    (dict(H=0), 1),
    (dict(H=100), 2),
    (dict(H=32), 2),
    (dict(hidden=None), 1),
    (dict(weight=None), 1),
    (dict(targets=None), 1),
    (dict(logp=None), 1),
    (dict(saved=None), 1),
    (dict(ent=None), 1),              # return_entropy without an entropy buffer
    (dict(ret=0), 1),                 # entropy buffer without return_entropy
    (dict(ret=0, ent=None), 1),       # entropy_requires_grad without return_entropy
    (dict(hidden=ODD), 1),            # misaligned
    (dict(saved_bytes=100), 3),
    (dict(ws_bytes=10), 3),
    (dict(ws=None), 3),
])
def test_fwd_host_validation(lib, kw, code):
    assert _fwd(lib, **kw) == code
    # the block-sparse forward takes the same arguments and checks them the same way
    assert _fwd(lib, entry="lmhead_fwd_blocksparse", **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(N=-5), 1),
    (dict(H=96), 2),
    (dict(saved=None), 1),
    (dict(gW=None), 1),
    (dict(gX=None), 1),
    (dict(glp=None), 1),
    (dict(gh=None), 1),               # entropy grad requested without its upstream grad
    (dict(erg=0), 1),                 # upstream entropy grad without the flag
    (dict(gX=ODD), 1),
    (dict(saved_bytes=8), 3),
    (dict(ws_bytes=0), 3),
    (dict(chunk=4, ws_bytes=10), 3),
])
def test_bwd_host_validation(lib, kw, code):
    assert _bwd(lib, **kw) == code


def test_sync_calls_reject_null(lib):
    n = ctypes.c_int64(0)
    assert lib.lmhead_read_n_kept(None, ctypes.byref(n), None) == 1
    assert lib.lmhead_read_n_kept(FAKE, None, None) == 1
    assert lib.lmhead_check_status(None, None) == 1


def test_missing_library_fails_loudly(tmp_path):
    from lm_head_log_amd import _lib
    with pytest.raises(ImportError):
        _lib.load(str(tmp_path / "nope.so"))


def test_binding_rejects_cpu_tensors():
    import torch
    import lm_head_log_amd as m
    h = torch.zeros(4, 64, dtype=torch.bfloat16)
    w = torch.zeros(10, 64, dtype=torch.bfloat16)
    t = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        m.lmhead_fwd(h, w, t)
    with pytest.raises(TypeError):
        m.lmhead_fwd(h.float(), w, t)


def _fwdp(lib, **kw):
    a = dict(hidden=FAKE, weight=FAKE, targets=FAKE, keep=None, N=8, H=64, Vs=100, v0=0, Vt=300,
             partial=FAKE, saved=FAKE, saved_bytes=1 << 20, ws=FAKE, ws_bytes=1 << 30,
             stream=None)
    a.update(kw)
    return lib.lmhead_fwd_partial(a["hidden"], a["weight"], a["targets"], a["keep"], a["N"],
                                  a["H"], a["Vs"], a["v0"], a["Vt"], a["partial"], a["saved"],
                                  a["saved_bytes"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), 1),
    (dict(Vs=0), 1),
    (dict(H=96), 2),
    (dict(v0=-1), 1),
    (dict(v0=250), 1),                # shard runs past the vocabulary
    (dict(Vt=(1 << 22) + 1), 1),
    (dict(partial=None), 1),
    (dict(partial=ODD), 1),
    (dict(weight=None), 1),
    (dict(saved=None), 1),
    (dict(saved_bytes=100), 3),
    (dict(ws_bytes=10), 3),
])
def test_fwd_partial_host_validation(lib, kw, code):
    assert _fwdp(lib, **kw) == code


def _merge(lib, **kw):
    a = dict(parts=FAKE, P=2, N=8, ret=1, erg=1, logp=FAKE, ent=FAKE, saved=FAKE,
             saved_bytes=1 << 20, stream=None)
    a.update(kw)
    return lib.lmhead_merge_partials(a["parts"], a["P"], a["N"], a["ret"], a["erg"], a["logp"],
                                     a["ent"], a["saved"], a["saved_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(P=0), 1),
    (dict(N=-1), 1),
    (dict(parts=None), 1),
    (dict(logp=None), 1),
    (dict(ent=None), 1),
    (dict(ret=0), 1),
    (dict(ret=0, ent=None), 1),
    (dict(parts=ODD), 1),
    (dict(saved=None), 1),
    (dict(saved_bytes=10), 3),
])
def test_merge_partials_host_validation(lib, kw, code):
    assert _merge(lib, **kw) == code


def _bwdp(lib, **kw):
    a = dict(hidden=FAKE, weight=FAKE, targets=FAKE, N=8, H=64, Vs=100, v0=200, erg=1, saved=FAKE,
             saved_bytes=1 << 20, glp=FAKE, gh=FAKE, gX=FAKE, gW=FAKE, chunk=0, ws=FAKE,
             ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.lmhead_bwd_partial(a["hidden"], a["weight"], a["targets"], a["N"], a["H"], a["Vs"],
                                  a["v0"], a["erg"], a["saved"], a["saved_bytes"], a["glp"],
                                  a["gh"], a["gX"], a["gW"], a["chunk"], a["ws"], a["ws_bytes"],
                                  a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(N=-5), 1),
    (dict(H=96), 2),
    (dict(v0=-1), 1),
    (dict(gW=None), 1),
    (dict(gh=None), 1),
    (dict(erg=0), 1),
    (dict(gX=ODD), 1),
    (dict(saved_bytes=8), 3),
    (dict(ws_bytes=0), 3),
])
def test_bwd_partial_host_validation(lib, kw, code):
    assert _bwdp(lib, **kw) == code


def _lfwd(lib, **kw):
    a = dict(logits=FAKE, dtype=0, N=8, V=100, targets=FAKE, keep=None, ret=1, logp=FAKE,
             ent=FAKE, stats=FAKE, stream=None)
    a.update(kw)
    return lib.lmhead_logits_fwd(a["logits"], a["dtype"], a["N"], a["V"], a["targets"], a["keep"],
                                 a["ret"], a["logp"], a["ent"], a["stats"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), 1),
    (dict(V=0), 1),
    (dict(dtype=2), 2),
    (dict(logits=None), 1),
    (dict(logits=ctypes.c_void_p(0x10001)), 1),   # odd address
    (dict(dtype=1, logits=ODD), 1),               # fp32 needs 4-byte alignment
    (dict(targets=None), 1),
    (dict(logp=None), 1),
    (dict(stats=None), 1),
    (dict(ent=None), 1),
    (dict(ret=0), 1),
])
def test_logits_fwd_host_validation(lib, kw, code):
    assert _lfwd(lib, **kw) == code


def _lbwd(lib, **kw):
    a = dict(logits=FAKE, dtype=0, N=8, V=100, targets=FAKE, keep=None, stats=FAKE, glp=FAKE,
             gh=FAKE, erg=1, grad=FAKE, stream=None)
    a.update(kw)
    return lib.lmhead_logits_bwd(a["logits"], a["dtype"], a["N"], a["V"], a["targets"], a["keep"],
                                 a["stats"], a["glp"], a["gh"], a["erg"], a["grad"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), 1),
    (dict(dtype=5), 2),
    (dict(stats=None), 1),
    (dict(glp=None), 1),
    (dict(gh=None), 1),
    (dict(erg=0), 1),
    (dict(grad=None), 1),
    (dict(grad=ctypes.c_void_p(0x10008)), 1),     # not the logits' offset modulo 16
])
def test_logits_bwd_host_validation(lib, kw, code):
    assert _lbwd(lib, **kw) == code


def _probe(lib, a=FAKE, a_elems=64, b=FAKE, b_elems=64, iters=10, ws=FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.lmhead_mfma_probe_workspace_bytes()
    return lib.lmhead_mfma_probe(a, a_elems, b, b_elems, iters, ws, ws_bytes, None, None, None,
                                 None)


def test_probe_workspace_covers_one_record_per_cu(lib):
    # a cycle count per workgroup (8 bytes) and a float per thread (256 threads),
    # one workgroup per CU; without a GPU the library assumes 256 CUs
    n = lib.lmhead_mfma_probe_workspace_bytes()
    assert n > 0 and n % (8 + 256 * 4) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(iters=0), 1),
    (dict(iters=(1 << 24) + 1), 1),
    (dict(a=None), 1),                # one operand array without the other
    (dict(b=None), 1),
    (dict(a_elems=4), 1),             # fewer than one fragment of 8 values
    (dict(b=ODD), 1),                 # misaligned
    (dict(ws=None), 1),
    (dict(ws_bytes=16), 3),
])
def test_probe_host_validation(lib, kw, code):
    assert _probe(lib, **kw) == code


def test_plain_c_caller(lib, tmp_path):
    """The header compiles as C and the library links and answers from a C
    program (size queries, status strings, host-side argument checks)."""
    import shutil
    import subprocess
    from lm_head_log_amd import _lib
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = tmp_path / "abi_client"
    libdir = os.path.dirname(_lib.LIB_PATH)
    src = os.path.join(ROOT, "tests", "c_client", "abi_client.c")
    r = subprocess.run([cc, "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        src, "-o", str(exe), "-L", libdir, "-llmhead", f"-Wl,-rpath,{libdir}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout

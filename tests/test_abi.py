"""Host-side checks of libswa.so: loading, exported symbols, status strings and
argument validation.  Every call here is rejected on the host before any
launch, so no GPU is needed (the device pointers are never dereferenced)."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import sliding_window_gqa_swa_amd as swa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swa.h")
FAKE = 0x7F0000000000  # 16-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swa_[a-z_0-9]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    names = declared_functions()
    assert names == sorted(["swa_abi_version", "swa_status_string", "swa_cache_write", "swa_prefill_chunk",
                            "swa_decode_workspace_size", "swa_decode", "swa_decode_step",
                            "swa_decode_step_noalloc", "swa_prefill_chunk_no_tile_skip"])
    lib = swa.lib()
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", swa.lib_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (swa_\w+)", out))
    assert set(names) <= exported


def test_library_shares_torchs_hip_runtime_when_loaded_first():
    """Loading libswa.so before anything has imported torch must still leave one HIP
    runtime in the process: torch's own copy, which the library then uses.  A second
    runtime would not know torch's device memory and streams."""
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import sliding_window_gqa_swa_amd as swa\n"
            "swa.lib()\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(sorted({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n") % ROOT
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    paths = eval(r.stdout.strip().splitlines()[-1])
    import torch
    assert len(paths) == 1, paths
    assert os.path.dirname(paths[0]) == os.path.join(os.path.dirname(torch.__file__), "lib"), paths


def test_abi_version_and_status_strings():
    text = open(HEADER).read()
    assert swa.swa_abi_version() == int(re.search(r"#define SWA_ABI_VERSION (\d+)", text).group(1)) == 3
    for code in range(6):
        s = swa.swa_status_string(code)
        assert s and isinstance(s, str)
    assert "unknown" in swa.swa_status_string(99)


def cache(**kw):
    base = dict(k=FAKE, v=FAKE + 4096, n_cache=4, n_kv_heads=8, head_dim=128, window=64, dtype=swa.SWA_DTYPE_BF16)
    base.update(kw)
    c = swa.SwaCacheC(base["k"], base["v"], base["n_cache"], base["n_kv_heads"], base["head_dim"], base["window"],
                      base["dtype"], base.get("reserved", 0))
    return c


class HostBatch:
    def __init__(self, lens, starts, rows=None, mirrors=True, **over):
        self.h_cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        self.h_sp = np.asarray(starts, np.int32)
        self.h_ci = None if rows is None else np.asarray(rows, np.int32)
        n = len(lens)
        vals = dict(num_seqs=n, total_tokens=int(self.h_cu[-1]), max_new_tokens=int(max(lens)) if n else 0)
        vals.update(over)
        self.c = swa.SwaBatchC(vals["num_seqs"], vals["total_tokens"], vals["max_new_tokens"],
                               vals.get("reserved", 0), FAKE + 0x100000, FAKE + 0x200000,
                               None if rows is None else FAKE + 0x300000,
                               self.h_cu.ctypes.data if mirrors else None,
                               self.h_sp.ctypes.data if mirrors else None,
                               None if (rows is None or not mirrors) else self.h_ci.ctypes.data)


def prefill(c, b, hq=32, scale=0.088, q=FAKE, kn=FAKE, vn=FAKE, out=FAKE):
    return swa.swa_prefill_chunk(c, b.c, q, hq, kn, vn, scale, out, stream=0, check=False)


def write(c, b, kn=FAKE, vn=FAKE):
    return swa.swa_cache_write(c, b.c, kn, vn, stream=0, check=False)


def decode(c, b, hq=32, scale=0.088, ws=None, wsb=0, q=FAKE, out=FAKE):
    return swa.swa_decode(c, b.c, q, hq, scale, out, ws, wsb, stream=0, check=False)


def step(c, b, hq=32, scale=0.088, ws=None, wsb=0, q=FAKE, kn=FAKE, vn=FAKE, out=FAKE):
    return swa.swa_decode_step(c, b.c, q, hq, kn, vn, scale, out, ws, wsb, stream=0, check=False)


INVALID, UNSUPPORTED, WORKSPACE = swa.SWA_ERR_INVALID_ARGUMENT, swa.SWA_ERR_UNSUPPORTED, swa.SWA_ERR_WORKSPACE


def test_null_structs_are_rejected():
    lib = swa.lib()
    b = HostBatch([3], [0])
    assert lib.swa_cache_write(None, ctypes.byref(b.c), FAKE, FAKE, None) == INVALID
    assert lib.swa_prefill_chunk(ctypes.byref(cache()), None, FAKE, 32, FAKE, FAKE, 0.1, FAKE, None) == INVALID
    assert lib.swa_decode(None, None, FAKE, 32, 0.1, FAKE, None, 0, None) == INVALID
    assert lib.swa_decode_step(None, None, FAKE, 32, FAKE, FAKE, 0.1, FAKE, None, 0, None) == INVALID


@pytest.mark.parametrize("field,value,code", [
    ("window", 0, INVALID), ("n_cache", 0, INVALID), ("n_kv_heads", 0, INVALID), ("head_dim", 0, INVALID),
    ("dtype", 7, INVALID), ("reserved", 1, INVALID), ("k", FAKE + 8, INVALID), ("v", None, INVALID),
    ("head_dim", 32, UNSUPPORTED), ("head_dim", 96, UNSUPPORTED), ("window", 2**30 + 1, UNSUPPORTED),
])
def test_bad_cache_descriptor(field, value, code):
    c = cache(**{field: value})
    assert write(c, HostBatch([3], [0])) == code


@pytest.mark.parametrize("dtype", [swa.SWA_DTYPE_BF16, swa.SWA_DTYPE_F32])
def test_supported_head_dims(dtype):
    for d in (16, 64, 128):
        c = cache(dtype=dtype, head_dim=d)
        # rejected only for the bad sequence metadata that follows, not the shape
        assert write(c, HostBatch([3], [-1])) == INVALID
        assert prefill(c, HostBatch([3], [-1])) == INVALID
    for d in (8, 32, 48, 256):
        assert write(cache(dtype=dtype, head_dim=d), HostBatch([3], [0])) == UNSUPPORTED


def test_bad_batch_metadata():
    c = cache()
    assert write(c, HostBatch([3, 2], [0, 5], total_tokens=6)) == INVALID          # cu[n] != total
    assert write(c, HostBatch([3, 2], [0, 5], max_new_tokens=2)) == INVALID        # a length > max
    assert write(c, HostBatch([3], [-1])) == INVALID                                # negative start
    assert write(c, HostBatch([3], [2**31 - 2])) == INVALID                         # position overflow
    assert write(c, HostBatch([1, 1], [0, 0], rows=[0, 4])) == INVALID              # row out of range
    assert write(c, HostBatch([1, 1], [0, 0], rows=[2, 2])) == INVALID              # shared row in a write
    assert write(c, HostBatch([1] * 5, [0] * 5)) == INVALID                         # more seqs than rows
    assert write(c, HostBatch([3], [0], reserved=1)) == INVALID
    assert write(c, HostBatch([3], [0], num_seqs=-1)) == INVALID
    assert write(c, HostBatch([3], [0]), kn=None) == INVALID
    assert write(c, HostBatch([3], [0]), vn=FAKE + 2) == INVALID


def test_no_tile_skip_variant_checks():
    c = cache()
    b = HostBatch([10, 4], [0, 3])
    nts = lambda cc, bb, **kw: swa.swa_prefill_chunk_no_tile_skip(cc, bb.c, kw.get("q", FAKE), kw.get("hq", 32),
                                                                  FAKE, FAKE, 0.088, FAKE, stream=0, check=False)
    assert nts(c, b, hq=12) == INVALID
    assert nts(c, b, q=None) == INVALID
    assert nts(cache(dtype=swa.SWA_DTYPE_F32, head_dim=16), HostBatch([3], [-1])) == INVALID
    assert nts(cache(dtype=swa.SWA_DTYPE_F32, head_dim=16), HostBatch([3], [0])) == UNSUPPORTED
    assert nts(c, HostBatch([], [])) == swa.SWA_OK


def test_prefill_argument_checks():
    c = cache()
    b = HostBatch([10, 4], [0, 3])
    assert prefill(c, b, hq=12) == INVALID           # not a multiple of n_kv_heads
    assert prefill(c, b, hq=8 * 16) == UNSUPPORTED   # group 16 not compiled for bf16
    assert prefill(c, b, scale=0.0) == INVALID
    assert prefill(c, b, scale=float("nan")) == INVALID
    assert prefill(c, b, scale=-1.0) == INVALID
    assert prefill(c, b, q=None) == INVALID
    assert prefill(c, b, out=FAKE + 4) == INVALID
    # no cache pointers: only when every start position is known to be 0
    nc = cache(k=None, v=None)
    assert prefill(nc, b) == INVALID
    assert prefill(nc, HostBatch([10], [0], mirrors=False)) == INVALID
    assert prefill(cache(k=None), HostBatch([10], [0])) == INVALID


def test_decode_argument_checks():
    c = cache(window=4096)
    one = HostBatch([1, 1], [5, 9])
    assert decode(c, HostBatch([2, 1], [5, 9])) == INVALID       # more than one token
    need = swa.swa_decode_workspace_size(c, 2, 32)
    assert need > 0
    assert decode(c, one, ws=None, wsb=0) == WORKSPACE
    assert decode(c, one, ws=FAKE, wsb=need - 1) == WORKSPACE
    assert decode(c, one, hq=33, ws=FAKE, wsb=need) == INVALID
    assert decode(c, one, scale=float("inf"), ws=FAKE, wsb=need) == INVALID
    assert decode(cache(v=None), one, ws=FAKE, wsb=need) == INVALID


def test_decode_step_argument_checks():
    c = cache(window=4096)
    one = HostBatch([1, 1], [5, 9])
    need = swa.swa_decode_workspace_size(c, 2, 32)
    # everything swa_decode rejects ...
    assert step(c, HostBatch([2, 1], [5, 9]), ws=FAKE, wsb=need) == INVALID
    assert step(c, one, ws=None, wsb=0) == WORKSPACE
    assert step(c, one, ws=FAKE, wsb=need - 1) == WORKSPACE
    assert step(c, one, hq=33, ws=FAKE, wsb=need) == INVALID
    assert step(c, one, scale=0.0, ws=FAKE, wsb=need) == INVALID
    assert step(cache(v=None, window=4096), one, ws=FAKE, wsb=need) == INVALID
    # ... plus the new token's rows and the write's distinct-row rule
    assert step(c, one, kn=None, ws=FAKE, wsb=need) == INVALID
    assert step(c, one, vn=None, ws=FAKE, wsb=need) == INVALID
    assert step(c, one, kn=FAKE + 8, ws=FAKE, wsb=need) == INVALID
    assert step(c, HostBatch([1, 1], [5, 9], rows=[3, 3]), ws=FAKE, wsb=need) == INVALID
    assert step(c, HostBatch([], [])) == swa.SWA_OK


def step_noalloc(c, b, hq=32, scale=0.088, q=FAKE, kn=FAKE, vn=FAKE, out=FAKE):
    return swa.swa_decode_step_noalloc(c, b.c, q, hq, kn, vn, scale, out, stream=0, check=False)


def test_decode_step_noalloc_argument_checks():
    """Rejected on the host like swa_decode_step (before the library's device array is looked up)."""
    c = cache(window=4096)
    one = HostBatch([1, 1], [5, 9])
    assert step_noalloc(c, HostBatch([2, 1], [5, 9])) == INVALID
    assert step_noalloc(c, one, hq=33) == INVALID
    assert step_noalloc(c, one, hq=8 * 16) == UNSUPPORTED
    assert step_noalloc(c, one, scale=0.0) == INVALID
    assert step_noalloc(cache(v=None, window=4096), one) == INVALID
    assert step_noalloc(c, one, kn=None) == INVALID
    assert step_noalloc(c, one, vn=None) == INVALID
    assert step_noalloc(c, one, kn=FAKE + 8) == INVALID
    assert step_noalloc(c, one, q=None) == INVALID
    assert step_noalloc(c, HostBatch([1, 1], [5, 9], rows=[3, 3])) == INVALID
    assert step_noalloc(c, HostBatch([1], [-4])) == INVALID
    assert step_noalloc(c, HostBatch([], [])) == swa.SWA_OK


def test_workspace_plan():
    c = cache(window=4096, n_cache=64)
    # 64 sequences x 8 KV heads (G = 4): 512 workgroups fill the chip, one per ring
    assert swa.swa_decode_workspace_size(c, 64, 32) == 0
    # 8 sequences (G = 4): stream mode, 512 workgroups x 2 partials x 4 heads x (D + 2) floats
    assert swa.swa_decode_workspace_size(c, 8, 32) == 512 * 2 * 4 * (128 + 2) * 4
    # two sequences, one KV head, G = 2: 2 x 4096 slots give 32 ranges of 256
    c1 = cache(window=4096, n_cache=2, n_kv_heads=1)
    assert swa.swa_decode_workspace_size(c1, 2, 2) == 32 * 2 * 2 * (128 + 2) * 4
    # one sequence (the same context in every KV head): split plan, 16 parts of 256 slots
    assert swa.swa_decode_workspace_size(c1, 1, 2) == 1 * 2 * 16 * (128 + 2) * 4
    # 65 sequences x 4 KV heads (G = 8): past the stream batch limit, split plan
    c8 = cache(window=4096, n_cache=65, n_kv_heads=4)
    sz8 = swa.swa_decode_workspace_size(c8, 65, 32)
    assert sz8 > 0 and sz8 % (65 * 32 * (128 + 2) * 4) == 0
    # G = 1 at head_dim 128 (VALU kernel) aims at more workgroups: 16 sequences already split
    sz1 = swa.swa_decode_workspace_size(cache(window=4096, n_cache=64, n_kv_heads=32), 16, 32)
    assert sz1 > 0 and sz1 % (16 * 32 * (128 + 2) * 4) == 0
    assert swa.swa_decode_workspace_size(c, 0, 32) == 0
    assert swa.swa_decode_workspace_size(cache(window=64), 2, 32) == 0      # too short to split
    assert swa.swa_decode_workspace_size(cache(window=511), 2, 32) == 0
    assert swa.swa_decode_workspace_size(cache(dtype=swa.SWA_DTYPE_F32), 2, 32) == 0
    assert swa.swa_decode_workspace_size(cache(window=0), 2, 32) == 0       # invalid -> 0


@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("window", [1, 127, 128, 255, 256, 511, 512, 1000, 4096, 4097, 32768, 2**20, 2**22])
@pytest.mark.parametrize("head_dim", [128, 64, 16])
def test_workspace_size_guarantees(group, window, head_dim):
    """The guarantees stated with swa_decode_workspace_size: the size is a whole
    number of partial results of head_dim + 2 floats, laid out by one of the two
    plans -- split (num_seqs x n_q_heads x S, 2 <= S <= W / 256) or stream (2 to
    64 sequences, matrix-core kernel at head_dim >= 64: N x 2 x G with N <= 512) -- none for
    W < 512 or once the batch alone gives 2048 (sequence, KV head) pairs, and
    never more than the stated maximum."""
    hkv = 32 // group
    on_valu = group == 1 and head_dim == 128
    c = cache(window=window, n_cache=65535, n_kv_heads=hkv, head_dim=head_dim)
    max_bytes = int(re.search(r"#define SWA_DECODE_WORKSPACE_MAX_BYTES \(\(size_t\)(\d+) << (\d+)\)",
                              open(HEADER).read()).group(1)) << 20
    for b in list(range(1, 70)) + [127, 128, 129, 255, 256, 511, 512, 513, 4095, 4096, 65535]:
        sz = swa.swa_decode_workspace_size(c, b, 32)
        assert sz <= max_bytes, (b, sz)
        if window < 512 or b * hkv >= 2048:
            assert sz == 0, b
        if sz == 0:
            continue
        part = (head_dim + 2) * 4
        assert sz % part == 0, (b, sz)
        parts = sz // part
        if not on_valu and head_dim >= 64 and 2 <= b <= 64:
            assert parts % (2 * group) == 0 and 1 <= parts // (2 * group) <= 512, (b, parts)
        else:
            assert parts % (b * 32) == 0, (b, parts)
            assert 2 <= parts // (b * 32) <= window // 256, (b, parts)
    assert swa.swa_decode_workspace_size(cache(window=window, dtype=swa.SWA_DTYPE_F32, n_kv_heads=hkv), 1, 32) == 0


def test_empty_batch_is_a_no_op():
    c = cache()
    assert write(c, HostBatch([], [])) == swa.SWA_OK
    assert prefill(c, HostBatch([], [])) == swa.SWA_OK
    assert decode(c, HostBatch([], [])) == swa.SWA_OK


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(swa, "_lib", None)
    monkeypatch.setattr(swa, "_LIB_PATH", str(tmp_path / "libswa.so"))
    with pytest.raises(swa.SwaLibraryMissing):
        swa.swa_abi_version()

"""CPU checks of the C ABI: the libraries load, export every function the
headers declare, and their host-only logic agrees with the oracle.  Calls that
would reach the GPU are not made here; argument errors are rejected before any
HIP call, so they are exercised with made-up pointer values."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import zero_partitioned_mixed_flat_amd as zs
from zero_partitioned_mixed_flat_amd import testkit

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DECL = re.compile(r"^(?:const\s+)?(?:unsigned\s+)?\w+\s*\*?\s*(zero_\w+)\s*\(", re.M)


def _declared(header):
    return DECL.findall(open(header).read())


CSRC = os.path.join(ROOT, "zero_partitioned_mixed_flat_amd", "csrc")


def test_public_headers_are_the_product_boundary():
    """include/ holds the product's C ABI only; the generators' and the
    probes' headers sit with their sources."""
    names = sorted(os.path.basename(h) for h in glob.glob(os.path.join(ROOT, "include", "*.h")))
    assert names == ["zero_host_adam.h", "zero_shard.h"]


def test_every_declared_symbol_is_exported():
    headers = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
    headers += [os.path.join(CSRC, "zero_testkit.h"), os.path.join(CSRC, "zero_probes.h")]
    from zero_partitioned_mixed_flat_amd import host_adam, probes
    libs = {"zero_shard.h": zs.library(), "zero_testkit.h": testkit.library(),
            "zero_host_adam.h": host_adam.library(), "zero_probes.h": probes.library()}
    for h in headers:
        names = _declared(h)
        assert names, h
        lib = libs[os.path.basename(h)]
        for name in names:
            assert hasattr(lib, name), f"{name} declared in {h} but not exported"


def test_shard_header_declares_the_path():
    names = set(_declared(os.path.join(ROOT, "include", "zero_shard.h")))
    assert {"zero_partition_layout", "zero_model_state_bytes", "zero_workspace_bytes",
            "zero_shard_grad_reduce", "zero_shard_grad_stats", "zero_shard_adam_step",
            "zero_shard_allgather", "zero_shard_adam_step_qwz", "zero_qwz_quantize", "zero_qwz_allgather",
            "zero_shard_adam_step_device_t", "zero_shard_adam_step_noalloc", "zero_status_string",
            "zero_last_error", "zero_shard_abi_version"} <= names


def test_abi_version_matches_header():
    text = open(os.path.join(ROOT, "include", "zero_shard.h")).read()
    version = int(re.search(r"#define ZERO_SHARD_ABI_VERSION (\d+)", text).group(1))
    assert zs.library().zero_shard_abi_version() == version
    from zero_partitioned_mixed_flat_amd import _native
    assert _native.ZERO_SHARD_ABI_VERSION == version


def test_layout_matches_oracle(orc):
    rng = np.random.default_rng(0)
    cases = [(psi, n, r, a) for psi in list(range(0, 200)) + [1023, 1024, 1025, 5000]
             for n in (1, 2, 3, 4, 7, 8, 64) for r in sorted({0, n // 2, n - 1})
             for a in (1, 4, 128)]
    cases += [(int(p), int(n), int(rng.integers(0, n)), int(2 ** rng.integers(0, 12)))
              for p, n in zip(rng.integers(0, 2**40, 2000), rng.integers(1, 1000, 2000))]
    cases += [(1_048_576, 4, 0, 128), (1_500_000_000, 4, 3, 128), (7_500_000_000, 64, 63, 128),
              (7_000_000_000, 8, 7, 128), (1_500_000_000, 1, 0, 128)]
    for psi, n, r, a in cases:
        st, ref = orc.partition_layout(psi, n, r, a)
        assert st == 0
        assert tuple(zs.partition_layout(psi, n, r, a)) == ref, (psi, n, r, a)


@pytest.mark.parametrize("args,status", [
    ((10, 0, 0, 1), -1), ((10, 4, 4, 1), -1), ((10, 4, 0, 3), -1), ((-1, 4, 0, 1), -1),
    ((2**62, 4, 0, 2**61), -5), ((2**63 - 1, 3, 0, 2**60), -5),
])
def test_layout_errors(args, status, orc):
    with pytest.raises(zs.ZeroError) as e:
        zs.partition_layout(*args)
    assert e.value.status == status == orc.partition_layout(*args)[0]


def test_model_state_bytes_matches_oracle(orc):
    for psi in (0.0, 1.5e9, 3e9, 7e9, 7.5e9, 70e9):
        for n in (1, 4, 8, 64):
            for stage in range(4):
                for K in (12.0, 4.0, 6.0):
                    a = zs.model_state_bytes(psi, n, stage, K)
                    b = orc.model_state_bytes(psi, n, stage, K)
                    assert abs(a - b) <= 1e-12 * max(1.0, b)
    with pytest.raises(zs.ZeroError):
        zs.model_state_bytes(1e9, 4, 4)


def test_workspace_and_status_strings():
    assert zs.workspace_bytes(0) >= 32768 and zs.workspace_bytes(-1) == 0
    for n in (1, 10**6, 117_187_584, 10**10):
        # 16-byte partials, one per 1024-element reduce tile plus one fold level
        assert zs.workspace_bytes(n) <= max(32768, 16 * (n // 1024 + n // (1024 * 4096) + 3))
        assert zs.workspace_bytes(n) >= 16 * (n // 1024)
    lib = zs.library()
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert lib.zero_status_string(code)


def _hp(lr=1e-4, b1=0.9, b2=0.999, eps=1e-8, mgn=0.0):
    from zero_partitioned_mixed_flat_amd._native import _HParams
    return _HParams(lr, b1, b2, eps, mgn)


A = 1 << 20  # made-up, 16-byte-aligned "device" addresses; never dereferenced


def _adam(lib, **kw):
    a = dict(grad=A, dt=1, s=1.0, master=2 * A, m=3 * A, v=4 * A, p16=5 * A, n=100, step=1,
             hp=_hp(), stats=6 * A, pre=1, ws=7 * A, wsn=1 << 16)
    a.update(kw)
    return lib.zero_shard_adam_step(a["grad"], a["dt"], a["s"], a["master"], a["m"], a["v"], a["p16"], a["n"],
                                    a["step"], ctypes.byref(a["hp"]) if a["hp"] is not None else None,
                                    a["stats"], a["pre"], a["ws"], a["wsn"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), -1), (dict(dt=3), -1), (dict(grad=None), -1), (dict(master=None), -1),
    (dict(stats=None), -1), (dict(hp=None), -1), (dict(step=0), -1),
    (dict(hp=_hp(lr=-1.0)), -1), (dict(hp=_hp(b1=1.0)), -1), (dict(hp=_hp(b2=-0.5)), -1),
    (dict(hp=_hp(eps=0.0)), -1), (dict(hp=_hp(lr=float("nan"))), -1), (dict(s=0.0), -1),
    (dict(hp=_hp(mgn=-1.0)), -1), (dict(hp=_hp(mgn=float("inf"))), -1),
    (dict(s=float("inf")), -1), (dict(m=3 * A + 4), -2), (dict(p16=5 * A + 8), -2),
    (dict(m=2 * A + 64), -1),                       # exp_avg overlaps master
    (dict(pre=0, ws=None), -1), (dict(pre=0, wsn=16), -3), (dict(pre=0, ws=7 * A + 8), -2),
    (dict(stats=2 * A + 96), -1),                   # stats inside master
    (dict(stats=A + 64), -1),                       # stats inside the gradient
    (dict(pre=0, ws=3 * A + 128), -1),              # workspace inside exp_avg
    (dict(pre=0, ws=6 * A - 1024, wsn=1 << 16), -1),  # workspace covers stats
])
def test_adam_step_rejects_bad_arguments(kw, status):
    lib = zs.library()
    assert _adam(lib, **kw) == status
    assert lib.zero_last_error()


def _adam_noalloc(lib, **kw):
    a = dict(grad=A, dt=1, s=1.0, master=2 * A, m=3 * A, v=4 * A, p16=5 * A, n=100, step=1,
             hp=_hp(), stats=6 * A, pre=0)
    a.update(kw)
    return lib.zero_shard_adam_step_noalloc(a["grad"], a["dt"], a["s"], a["master"], a["m"], a["v"], a["p16"],
                                            a["n"], a["step"],
                                            ctypes.byref(a["hp"]) if a["hp"] is not None else None,
                                            a["stats"], a["pre"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), -1), (dict(dt=3), -1), (dict(grad=None), -1), (dict(master=None), -1),
    (dict(stats=None), -1), (dict(hp=None), -1), (dict(step=0), -1), (dict(hp=_hp(b1=1.0)), -1),
    (dict(s=0.0), -1), (dict(m=3 * A + 4), -2), (dict(m=2 * A + 64), -1), (dict(stats=2 * A + 96), -1),
    (dict(stats=6 * A + 8), -2),
    (dict(pre=1, n=-1), -1), (dict(pre=1, step=0), -1),
])
def test_adam_step_noalloc_rejects_bad_arguments(kw, status):
    """The no-allocation step validates its arguments as the step does, and
    before it looks up its scratch (so no HIP call is made here)."""
    lib = zs.library()
    assert _adam_noalloc(lib, **kw) == status
    assert lib.zero_last_error()


def test_noalloc_scratch_size_in_header():
    text = open(os.path.join(ROOT, "include", "zero_shard.h")).read()
    size = int(re.search(r"#define ZERO_NOALLOC_SCRATCH_BYTES (\d+)", text).group(1))
    # the statistics kernel's most partials (2048) of 16 bytes each
    assert size == zs.ZERO_NOALLOC_SCRATCH_BYTES == 2048 * 16


def test_reduce_and_stats_reject_bad_arguments():
    lib = zs.library()
    ptrs = (ctypes.c_void_p * 65)(*[A * (i + 1) for i in range(65)])
    out = 100 * A
    f = lib.zero_shard_grad_reduce
    assert f(ptrs, 0, 10, out, None, 1.0, None, 0, None) == -1          # no slices
    assert f(ptrs, 65, 10, out, None, 1.0, None, 0, None) == -1         # too many
    assert f(ptrs, 4, -1, out, None, 1.0, None, 0, None) == -1
    assert f(ptrs, 4, 10, out, None, 0.0, None, 0, None) == -1          # bad scale
    assert f(ptrs, 4, 10, out + 4, None, 1.0, None, 0, None) == -2      # misaligned out
    assert f(ptrs, 4, 10, A, None, 1.0, None, 0, None) == -1            # out overlaps slice 0
    assert f(ptrs, 4, 10, out, 200 * A, 1.0, None, 0, None) == -1       # stats without workspace
    assert f(ptrs, 4, 10, out, 200 * A, 1.0, 300 * A, 8, None) == -3    # short workspace
    bad = (ctypes.c_void_p * 2)(A, A + 2)
    assert f(bad, 2, 10, out, None, 1.0, None, 0, None) == -2           # misaligned slice
    big = 1 << 16
    assert f(ptrs, 4, 10, out, 300 * A, 1.0, 300 * A - 1024, big, None) == -1   # workspace covers stats
    assert f(ptrs, 4, 10, out, 300 * A, 1.0, out, big, None) == -1              # workspace on out_sum
    assert f(ptrs, 4, 10, out, out + 16, 1.0, 300 * A, big, None) == -1         # stats inside out_sum
    assert f(ptrs, 4, 10, out, A, 1.0, 300 * A, big, None) == -1                # stats on slice 0
    assert f(ptrs, 4, 10, out, 300 * A, 1.0, 2 * A, big, None) == -1            # workspace on slice 1
    g = lib.zero_shard_grad_stats
    assert g(A, 1, 100, 1.0, A + 32, 3 * A, 1 << 16, None) == -1       # stats inside grad
    assert g(A, 1, 100, 1.0, 2 * A, A, 1 << 16, None) == -1            # workspace on grad
    assert g(A, 1, 100, 1.0, 2 * A, 2 * A - 1024, 1 << 16, None) == -1  # workspace covers stats
    assert g(A, 1, -5, 1.0, 2 * A, 3 * A, 1 << 16, None) == -1
    assert g(A, 9, 5, 1.0, 2 * A, 3 * A, 1 << 16, None) == -1
    assert g(A, 1, 5, float("nan"), 2 * A, 3 * A, 1 << 16, None) == -1
    assert g(A, 1, 5, 1.0, None, 3 * A, 1 << 16, None) == -1
    assert g(A, 1, 5, 1.0, 2 * A, 3 * A, 16, None) == -3
    assert g(A + 2, 1, 5, 1.0, 2 * A, 3 * A, 1 << 16, None) == -2


def test_allgather_rejects_bad_arguments():
    lib = zs.library()
    ptrs = (ctypes.c_void_p * 65)(*[A * (i + 1) for i in range(65)])
    rep = 100 * A
    f = lib.zero_shard_allgather
    assert f(ptrs, 0, 64, 10, rep, None) == -1          # no shards
    assert f(ptrs, 65, 64, 10, rep, None) == -1         # too many
    assert f(ptrs, 4, 60, 10, rep, None) == -1          # shard_len not a multiple of 8
    assert f(ptrs, 4, 64, 257, rep, None) == -1         # psi beyond N*shard_len
    assert f(ptrs, 4, 64, -1, rep, None) == -1
    assert f(ptrs, 4, 64, 200, rep + 2, None) == -2     # misaligned replica
    assert f(ptrs, 4, 64, 200, A, None) == -1           # replica overlaps shard 0
    bad = (ctypes.c_void_p * 2)(A, A + 2)
    assert f(bad, 2, 64, 100, rep, None) == -2          # misaligned shard


def _adam_qwz(lib, codes=8 * A, scales=9 * A, **kw):
    a = dict(grad=A, dt=1, s=1.0, master=2 * A, m=3 * A, v=4 * A, p16=5 * A, n=1000, step=1,
             hp=_hp(), stats=6 * A, pre=1, ws=7 * A, wsn=1 << 16)
    a.update(kw)
    return lib.zero_shard_adam_step_qwz(a["grad"], a["dt"], a["s"], a["master"], a["m"], a["v"], a["p16"], codes,
                                        scales, a["n"], a["step"], ctypes.byref(a["hp"]), a["stats"], a["pre"],
                                        a["ws"], a["wsn"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(codes=None), -1), (dict(scales=None), -1), (dict(codes=8 * A + 4), -2), (dict(scales=9 * A + 8), -2),
    (dict(codes=5 * A + 512), -1),                  # codes overlap param16
    (dict(scales=8 * A + 992), -1),                 # scales overlap codes (1000 bytes)
    (dict(n=-1), -1), (dict(step=0), -1), (dict(m=3 * A + 4), -2),
])
def test_adam_step_qwz_rejects_bad_arguments(kw, status):
    lib = zs.library()
    assert _adam_qwz(lib, **kw) == status
    assert lib.zero_last_error()


def test_qwz_quantize_and_allgather_reject_bad_arguments():
    lib = zs.library()
    q = lib.zero_qwz_quantize
    assert q(A, -1, 2 * A, 3 * A, None) == -1
    assert q(None, 10, 2 * A, 3 * A, None) == -1
    assert q(A, 10, None, 3 * A, None) == -1
    assert q(A, 10, 2 * A, None, None) == -1
    assert q(A + 2, 10, 2 * A, 3 * A, None) == -2
    assert q(A, 10, 2 * A + 4, 3 * A, None) == -2
    assert q(A, 1000, A + 1024, 3 * A, None) == -1     # codes inside x16 (2000 bytes)
    assert q(A, 1000, 2 * A, 2 * A + 992, None) == -1  # scales overlap codes
    assert q(A, 0, None, None, None) == 0              # empty: nothing to do, no device call
    codes = (ctypes.c_void_p * 65)(*[A * (i + 1) for i in range(65)])
    scales = (ctypes.c_void_p * 65)(*[A * (i + 101) for i in range(65)])
    rep = 300 * A
    g = lib.zero_qwz_allgather
    assert g(codes, scales, 0, 64, 10, rep, None) == -1
    assert g(codes, scales, 65, 64, 10, rep, None) == -1
    assert g(codes, scales, 4, 60, 10, rep, None) == -1      # shard_len not a multiple of 8
    assert g(codes, scales, 4, 64, 257, rep, None) == -1     # psi beyond N*shard_len
    assert g(codes, None, 4, 64, 10, rep, None) == -1
    assert g(codes, scales, 4, 64, 200, rep + 2, None) == -2
    assert g(codes, scales, 4, 64, 200, A, None) == -1       # replica overlaps codes of shard 0
    assert g(codes, scales, 4, 64, 200, 101 * A, None) == -1  # replica overlaps scales of shard 0
    bad = (ctypes.c_void_p * 2)(A, A + 4)
    assert g(bad, scales, 2, 64, 100, rep, None) == -2
    assert g(codes, scales, 4, 64, 0, rep, None) == 0        # psi = 0: nothing to do
    assert zs.qwz_scales_len(0) == 0 and zs.qwz_scales_len(1) == 1 and zs.qwz_scales_len(256) == 1
    assert zs.qwz_scales_len(257) == 2 and zs.ZERO_QWZ_BLOCK == 256


def test_philox_known_answers():
    # Known-answer vectors published with the Random123 Philox4x32-10
    # reference implementation (Salmon et al., SC'11).
    kat = [((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
           ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
           ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
            (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1))]
    for ctr, key, want in kat:
        got = testkit.philox_host(np.array([ctr], dtype=np.uint32), key)[0]
        assert tuple(int(x) for x in got) == want


def test_adam_step_device_t_rejects_bad_arguments():
    lib = zs.library()
    hp = _hp()

    def call(applied=8 * A, codes=None, scales=None, **kw):
        a = dict(grad=A, dt=1, s=1.0, master=2 * A, m=3 * A, v=4 * A, p16=5 * A, n=1000, stats=6 * A, pre=1)
        a.update(kw)
        return lib.zero_shard_adam_step_device_t(a["grad"], a["dt"], a["s"], a["master"], a["m"], a["v"], a["p16"],
                                                 codes, scales, a["n"], applied, ctypes.byref(hp), a["stats"],
                                                 a["pre"], None, 0, None)
    assert call(applied=None) == -1                      # no counter
    assert call(applied=8 * A + 8) == -2                 # misaligned counter
    assert call(applied=2 * A + 64) == -1                # counter inside master
    assert call(applied=6 * A) == -1                     # counter on the statistics
    assert call(codes=9 * A) == -1                       # codes without scales
    assert call(scales=10 * A) == -1
    assert call(dt=5) == -1
    assert call(n=-1) == -1


def _includes(path):
    return set(re.findall(r'^\s*#\s*include\s*[<"]([^>"]+)[>"]', open(path).read(), re.M))


def _imports(path):
    names = set()
    for line in open(path):
        m = re.match(r"\s*(?:from\s+(\S+)\s+import|import\s+(\S+))", line)
        if m:
            names.add((m.group(1) or m.group(2)).split(".")[0])
    return names


def test_oracle_generators_and_library_share_no_code():
    """The oracle, the seeded input generators and the HIP library are three
    separate code bases: no source of one includes or imports another (the
    probes of the library's own code are built with the library, apart from
    the generators)."""
    csrc = os.path.join(ROOT, "zero_partitioned_mixed_flat_amd", "csrc")
    library_headers = {"shard_kernels.hpp", "zero_shard.h", "zero_probes.h", "zero_host_adam.h"}
    assert _includes(os.path.join(csrc, "testkit.hip")) & (library_headers | {"zero_oracle.h"}) == set()
    assert _includes(os.path.join(csrc, "zero_testkit.h")) & library_headers == set()
    assert _includes(os.path.join(ROOT, "oracle", "zero_oracle.c")) & (library_headers | {"zero_testkit.h"}) == set()
    assert "zero_partitioned_mixed_flat_amd" not in _imports(os.path.join(ROOT, "oracle", "__init__.py"))
    for f in ("shard_kernels.hpp", "zero_shard.hip", "probes.hip", "host_adam.cpp"):
        assert _includes(os.path.join(csrc, f)) & {"zero_oracle.h", "zero_testkit.h"} == set(), f
    for f in glob.glob(os.path.join(ROOT, "zero_partitioned_mixed_flat_amd", "*.py")):
        assert "oracle" not in _imports(f), f"{f} imports the oracle"
    assert "testkit" not in " ".join(_imports(os.path.join(ROOT, "zero_partitioned_mixed_flat_amd", "_native.py")))

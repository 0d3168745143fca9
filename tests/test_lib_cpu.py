"""CPU-side checks of libkvcopy.so: exports, host planner parity with the
oracle's planning steps (bit-exact), argument validation.  No GPU needed:
every call here either is host-only or fails validation before any HIP call.
"""
import os
import re
import subprocess

import numpy as np
import pytest

import workloads as W
from oracle import plan as oplan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def K():
    from block_copy_amd import kvcopy
    return kvcopy


def _declared():
    names = []
    for h in os.listdir(os.path.join(ROOT, "include")):
        if h.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", h)).read()
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kvcopy_\w+)\s*\(", txt, re.M)
    return sorted(set(names))


def test_header_symbols_are_exported(K):
    declared = _declared()
    assert len(declared) >= 9
    assert sorted(K.EXPORTS) == declared
    out = subprocess.run(["nm", "-D", "--defined-only", K.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (kvcopy_\w+)", out))
    for name in declared:
        assert name in exported, name
        assert hasattr(K.lib, name)


@pytest.mark.parametrize("src", ["kvcopy_kernel.hip", "device_batch.hip", "order_kernel.hip"])
def test_kernels_have_no_scratch_or_spills(K, src):
    """No copy kernel may use private (scratch) memory or spill registers;
    every direction of every loop has its own symbol."""
    from block_copy_amd import build as B
    tmp = os.path.join(ROOT, "_build")
    os.makedirs(tmp, exist_ok=True)
    out = os.path.join(tmp, src + ".meta.s")
    subprocess.run(["hipcc", *B.HIPCC_FLAGS, "--cuda-device-only", "-S",
                    "-I" + os.path.join(ROOT, "include"),
                    "-I" + os.path.join(ROOT, "block_copy_amd", "csrc"),
                    os.path.join(ROOT, "block_copy_amd", "csrc", src), "-o", out],
                   check=True, capture_output=True)
    txt = open(out).read()
    sizes = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", txt)
    spills = re.findall(r"\.[sv]gpr_spill_count:\s+(\d+)", txt)
    assert sizes and all(int(s) == 0 for s in sizes)
    assert spills and all(int(s) == 0 for s in spills)
    names = set(re.findall(r"\.name:\s+_ZN3kvc12_GLOBAL__N_1\d+(kvcopy_\w+?_kernel)E", txt))
    if src == "kvcopy_kernel.hip":
        want = {f"kvcopy_{d}{v}_kernel" for d in ("h2d", "d2h", "d2d")
                for v in ("", "_sc1", "_pipe", "_dyn", "_inline", "_inline_sc1", "_wg",
                          "_wg_sc1")} | {
                    "kvcopy_pair_kernel", "kvcopy_pair_nt_kernel"}
    elif src == "device_batch.hip":
        want = {"kvcopy_device_plan_kernel", "kvcopy_device_copy_kernel"}
    else:
        want = {"kvcopy_order_count_kernel", "kvcopy_order_place_kernel"}
    assert names == want, names


# ---------------------------------------------------------------------------
# Planner parity with the oracle (integer work: bit-exact)
# ---------------------------------------------------------------------------

def _addr(wl, b):
    bases = [(i + 1) << 36 for i in range(len(wl.arenas))]
    return b.addresses(bases)


@pytest.mark.parametrize("make", [
    lambda: W.h2d_mixed(seed=0, n=16),
    lambda: W.h2d_mixed(seed=1, n=4096),
    lambda: W.h2d_mixed(seed=2, n=65536),
    lambda: W.kv_blocks(seed=0, directions="h2d"),
    lambda: W.moe_gather(seed=0, calls=1),
    lambda: W.irregular(seed=5, n=1000, zero_frac=0.1),
])
@pytest.mark.parametrize("chunk", [0, 16, 4096, 8192, 65536])
def test_plan_matches_oracle(K, make, chunk):
    wl = make()
    b = wl.batches[0]
    s, d = _addr(wl, b)
    p = K.kvcopy_plan(s, d, b.size, chunk)
    C = chunk or K.CHUNK_DEFAULT
    es, ed, ez = oplan.coalesce(s, d, b.size)
    assert p.n_in == b.n
    assert p.n_merged == len(ez)
    assert p.src.tolist() == es and p.dst.tolist() == ed and p.size.tolist() == ez
    assert p.chunk_begin.tolist() == oplan.chunk_begin(ez, C)
    assert p.n_chunks == p.chunk_begin[-1]
    assert p.total_bytes == int(b.size.sum())
    assert p.chunk_bytes == C


def test_coalesce_matches_oracle_and_golden(K):
    import json
    cases = json.load(open(os.path.join(ROOT, "tests", "golden", "coalesce_cases.json")))["cases"]
    for c in cases:
        a = np.array(c["in"], dtype=np.uint64).reshape(-1, 3)
        out = K.kvcopy_coalesce(a[:, 0], a[:, 1], a[:, 2])
        assert [list(map(int, x)) for x in zip(*out)] == c["out"], c["name"]
    rng = np.random.default_rng(9)
    for _ in range(300):
        n = int(rng.integers(0, 40))
        s = (8 * rng.integers(0, 50, n)).astype(np.uint64)
        d = (8 * rng.integers(0, 50, n)).astype(np.uint64)
        z = (8 * rng.integers(0, 3, n)).astype(np.uint64)
        # force some chains
        for i in range(1, n):
            if rng.random() < 0.4:
                s[i] = s[i - 1] + z[i - 1]
                d[i] = d[i - 1] + z[i - 1]
        got = K.kvcopy_coalesce(s, d, z)
        exp = oplan.coalesce(s, d, z)
        assert [g.tolist() for g in got] == [list(e) for e in exp]


def test_coalesce_in_place(K):
    import ctypes
    s = np.array([0, 8, 16, 100 * 8], np.uint64)
    d = np.array([64, 72, 80, 8], np.uint64)
    z = np.array([8, 8, 8, 8], np.uint64)
    m = ctypes.c_uint64()
    p = lambda x: x.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))  # noqa: E731
    rc = K.lib.kvcopy_coalesce(p(s), p(d), p(z), 4, p(s), p(d), p(z), ctypes.byref(m))
    assert rc == 0 and m.value == 2
    assert s[:2].tolist() == [0, 800] and d[:2].tolist() == [64, 8] and z[:2].tolist() == [24, 8]


# ---------------------------------------------------------------------------
# Argument validation: errors come back before anything touches the GPU
# ---------------------------------------------------------------------------

def test_batch_argument_errors(K):
    s = np.array([0x10000, 0x20000], np.uint64)
    d = np.array([0x30000, 0x40000], np.uint64)
    z = np.array([4096, 4096], np.uint64)
    call = lambda *a, **k: K.kvcopy_batch(*a, check=False, **k)  # noqa: E731
    assert call([], [], [], K.H2D) == K.OK                       # empty call
    assert call(s, d, np.zeros(2, np.uint64), K.H2D) == K.OK     # only zero sizes
    assert call(s, d, z + 4, K.H2D) == K.EALIGN                   # size not a multiple of 8
    assert call(s + 4, d, z, K.D2H) == K.EALIGN                   # misaligned source
    assert call(s, d + 12, z, K.D2D) == K.EALIGN                  # misaligned destination
    assert call(s, d, z, 3) == K.EINVAL                            # bad direction
    assert call(s, d, z, -1) == K.EINVAL
    assert call(s, d, z, K.H2D, -5) == K.EINVAL                    # max_wgs below WGS_AUTO
    assert call(s, d, z, K.H2D, -2) == K.EINVAL
    assert call(s, d, z, K.H2D, chunk_bytes=24) == K.EINVAL        # chunk not a multiple of 16
    assert call(s, d, z, K.H2D, chunk_bytes=(1 << 20) + 16) == K.EINVAL
    assert call(s, d, z, K.H2D, flags=0x1000) == K.EINVAL         # unknown flag
    assert call(s, d, z, K.H2D, flags=K.F_TAIL_BOUNDED | K.F_PIPELINE) == K.EINVAL
    assert call(s, d, z, K.H2D, flags=K.F_TAIL_BOUNDED | K.F_DYNAMIC) == K.EINVAL
    assert call(s, d, z, K.H2D, -5, flags=K.F_TAIL_BOUNDED) == K.EINVAL
    assert call(s, d, z + 4, K.H2D, flags=K.F_TAIL_BOUNDED) == K.EALIGN   # preset accepted
    assert call(s, d, z, K.H2D, flags=0x4) == K.EINVAL            # a retired flag value
    assert call(s, d, z, K.H2D, flags=K.F_PIPELINE | K.F_PER_CHUNK) == K.EINVAL  # two loops forced
    assert call(s, d, z, K.H2D, flags=K.F_DYNAMIC | K.F_PIPELINE) == K.EINVAL
    assert call(s, d, z, K.H2D, flags=K.F_DYNAMIC | K.F_PER_CHUNK) == K.EINVAL
    assert call(s, d, z, K.D2D, flags=K.F_WG_PER_CHUNK | K.F_PIPELINE) == K.EINVAL
    assert call(s, d, z, K.D2D, flags=K.F_WG_PER_CHUNK | K.F_DYNAMIC) == K.EINVAL
    assert call(s, d, z, K.D2D, flags=K.F_WG_PER_CHUNK | K.F_PER_CHUNK) == K.EINVAL
    assert call(s, d, z, K.D2D, flags=K.F_WG_PER_CHUNK | K.F_TAIL_BOUNDED) == K.EINVAL
    assert call(s, d, z, K.D2D, duty_on_ns=5000, duty_period_ns=20000,
                flags=K.F_WG_PER_CHUNK) == K.EINVAL
    assert call(s, d, z + 4, K.D2D, flags=K.F_WG_PER_CHUNK | K.F_STORE_SC1) == K.EALIGN  # accepted
    # store forms: one at a time, for the per-chunk loop only
    assert call(s, d, z, K.H2D, flags=K.F_STORE_SC1 | K.F_STORE_NT) == K.EINVAL
    assert call(s, d, z, K.H2D, flags=K.F_STORE_SC1 | K.F_PIPELINE) == K.EINVAL
    assert call(s, d, z, K.H2D, flags=K.F_STORE_NT | K.F_DYNAMIC) == K.EINVAL
    # duty cycle: 1 us <= on <= period <= 10 ms, per-chunk loop only
    assert call(s, d, z, K.H2D, duty_on_ns=999, duty_period_ns=10000) == K.EINVAL
    assert call(s, d, z, K.H2D, duty_on_ns=20000, duty_period_ns=10000) == K.EINVAL
    assert call(s, d, z, K.H2D, duty_on_ns=5000, duty_period_ns=10000001) == K.EINVAL
    assert call(s, d, z, K.H2D, duty_on_ns=5000, duty_period_ns=20000,
                flags=K.F_PIPELINE) == K.EINVAL
    assert call(s, d, z, K.H2D, duty_on_ns=5000, duty_period_ns=20000,
                flags=K.F_DYNAMIC) == K.EINVAL
    assert call(s, d, z, K.H2D, opts_size=24) == K.EINVAL          # unknown struct size
    assert call(s, d, z + 4, K.H2D, opts_size=K.OPTS_V1_SIZE) == K.EALIGN   # v1 layout accepted
    wrap = np.array([2**64 - 4096], np.uint64)
    assert call(wrap, d[:1], z[:1], K.H2D) == K.EINVAL             # address range wraps
    dup = np.array([0x30000, 0x30800], np.uint64)
    assert call(s, dup, z, K.H2D, flags=K.F_VALIDATE) == K.EOVERLAP  # destinations overlap
    over = np.array([0x30000, 0x10800], np.uint64)
    assert call(s, over, z, K.H2D, flags=K.F_VALIDATE) == K.EOVERLAP  # a destination overlaps a source


def test_pair_argument_errors(K):
    """kvcopy_batch_pair checks both lists before anything touches the GPU."""
    s = np.array([0x10000, 0x20000], np.uint64)
    d = np.array([0x30000, 0x40000], np.uint64)
    z = np.array([4096, 4096], np.uint64)
    s2, d2 = s + 0x100000, d + 0x100000
    e = np.zeros(0, np.uint64)
    call = lambda *a, **k: K.kvcopy_batch_pair(*a, check=False, **k)  # noqa: E731
    assert call(e, e, e, e, e, e) == K.OK                                  # both lists empty
    assert call(s, d, np.zeros(2, np.uint64), e, e, e) == K.OK             # only zero sizes
    assert call(s, d, z, s2 + 4, d2, z) == K.EALIGN                        # list b misaligned
    assert call(s, d, z + 4, s2, d2, z) == K.EALIGN                        # list a size
    assert call(s, d, z, s2, d2, z, -2) == K.EINVAL                        # max_wgs below AUTO
    assert call(s, d, z, s2, d2, z, flags=K.F_PIPELINE) == K.EINVAL        # loop flags: not here
    assert call(s, d, z, s2, d2, z, flags=K.F_DESC_UPLOAD) == K.EINVAL
    assert call(s, d, z, s2, d2, z, flags=K.F_STORE_SC1) == K.EINVAL       # sc1 is its default
    assert call(s, d, z, s2 + 4, d2, z, flags=K.F_STORE_NT) == K.EALIGN    # nt accepted
    wrap = np.array([2**64 - 4096], np.uint64)
    assert call(s, d, z, wrap, d2[:1], z[:1]) == K.EINVAL                  # list b wraps
    # The overlap rule spans both lists (validate mode only).
    assert call(s, d, z, s2, d, z, flags=K.F_VALIDATE) == K.EOVERLAP       # same destinations
    assert call(s, d, z, d + 0x800, d2, z, flags=K.F_VALIDATE) == K.EOVERLAP  # b reads a's dst
    assert call(s, d, z, s2[:1], s[:1], z[:1], flags=K.F_VALIDATE) == K.EOVERLAP  # b writes a's src
    import ctypes
    u = ctypes.POINTER(ctypes.c_uint64)()
    p = s.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))
    assert K.lib.kvcopy_batch_pair(p, p, p, 1, u, u, u, 2, 0, 0, None) == K.EINVAL   # null list b
    assert K.lib.kvcopy_batch_pair(u, u, u, 0, u, u, u, 0, 0, 0, None) == K.OK


def test_null_pointers_and_struct_size(K):
    import ctypes
    u = ctypes.POINTER(ctypes.c_uint64)()
    assert K.lib.kvcopy_batch(u, u, u, 3, 0, 0, None) == K.EINVAL
    assert K.lib.kvcopy_batch(u, u, u, 0, 0, 0, None) == K.OK
    o = K.Opts(ctypes.sizeof(K.Opts) - 4, 0, 0, 0, None, None)   # neither known size
    s = np.array([0], np.uint64)
    p = s.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))
    assert K.lib.kvcopy_batch_ex(p, p, p, 1, 0, 0, None, ctypes.byref(o)) == K.EINVAL
    m = ctypes.c_uint64()
    assert K.lib.kvcopy_coalesce(u, u, u, 2, u, u, u, ctypes.byref(m)) == K.EINVAL
    assert K.lib.kvcopy_coalesce(u, u, u, 0, u, u, u, None) == K.EINVAL
    assert K.lib.kvcopy_plan(u, u, u, 0, 0, None) == K.EINVAL
    assert K.lib.kvcopy_host_alloc_mapped(0, ctypes.byref(ctypes.c_void_p())) == K.EINVAL
    assert K.lib.kvcopy_host_free(None) == K.OK
    assert K.kvcopy_strerror(12345) == "unknown status"


def test_validate_env_is_strict(K, monkeypatch):
    s = np.array([0x10000, 0x20000], np.uint64)
    dup = np.array([0x30000, 0x30800], np.uint64)
    z = np.array([4096, 4096], np.uint64)
    monkeypatch.setenv("KVCOPY_VALIDATE", "1")
    assert K.kvcopy_batch(s, dup, z, K.H2D, check=False) == K.EOVERLAP
    with pytest.raises(K.KvcopyError):
        K.kvcopy_plan(s, dup, z)
    monkeypatch.setenv("KVCOPY_VALIDATE", "yes")                  # unknown value: rejected
    assert K.kvcopy_batch(s, dup, z, K.H2D, check=False) == K.EINVAL
    monkeypatch.setenv("KVCOPY_VALIDATE", "0")
    p = K.kvcopy_plan(s, dup, z)                                  # not validated: planned as given
    assert p.n_merged == 2


def test_plan_edge_cases(K):
    p = K.kvcopy_plan([], [], [])
    assert p.n_in == 0 and p.n_merged == 0 and p.n_chunks == 0 and p.chunk_begin.tolist() == [0]
    p = K.kvcopy_plan([8], [1 << 20], [K.CHUNK_MAX], K.CHUNK_MAX)
    assert p.n_chunks == 1
    p = K.kvcopy_plan([8], [1 << 20], [8], 16)
    assert p.n_chunks == 1 and p.size.tolist() == [8]
    with pytest.raises(K.KvcopyError):
        K.kvcopy_plan([8], [16], [8], 8)           # chunk must be a multiple of 16


def test_job_argument_errors(K):
    import ctypes
    s = np.array([0x10000, 0x20000], np.uint64)
    d = np.array([0x30000, 0x40000], np.uint64)
    z = np.array([4096, 4096], np.uint64)
    with pytest.raises(K.KvcopyError) as e:
        K.kvcopy_job_create(s, d, z + 4, K.H2D)
    assert e.value.code == K.EALIGN
    with pytest.raises(K.KvcopyError) as e:
        K.kvcopy_job_create(s, d, z, 7)
    assert e.value.code == K.EINVAL
    with pytest.raises(K.KvcopyError) as e:
        K.kvcopy_job_create(s, d, z, K.D2D, -2)
    assert e.value.code == K.EINVAL
    u = ctypes.POINTER(ctypes.c_uint64)()
    assert K.lib.kvcopy_job_create(u, u, u, 0, 0, 0, 0, None, None) == K.EINVAL
    assert K.lib.kvcopy_job_poll(None, ctypes.byref(ctypes.c_int())) == K.EINVAL
    assert K.lib.kvcopy_job_wait(None) == K.EINVAL
    K.lib.kvcopy_job_destroy(None)
    # an empty job is done at the first poll, without touching the GPU
    j = K.kvcopy_job_create([], [], [], K.D2D)
    assert K.kvcopy_job_poll(j) is True
    K.kvcopy_job_destroy(j)


def test_device_batch_argument_errors(K):
    call = lambda *a, **k: K.kvcopy_batch_device(*a, check=False, **k)  # noqa: E731
    assert call(0, 0, 0, 0, 0, K.D2D, 8, 0) == K.OK                 # max_n == 0: no-op
    assert call(0, 0, 0, 0, 10, K.D2D, 8, 0) == K.EINVAL            # NULL arrays
    good = dict(d_src=1 << 20, d_dst=2 << 20, d_sizes=3 << 20, d_n=4 << 20)
    assert call(*good.values(), 10, 9, 8, 5 << 20) == K.EINVAL      # bad dir
    assert call(*good.values(), 10, K.D2D, -2, 5 << 20) == K.EINVAL  # bad max_wgs
    assert call(*good.values(), 10, K.D2D, 8, (5 << 20) + 8) == K.EINVAL   # misaligned workspace
    assert call(*good.values(), 10, K.D2D, 8, 5 << 20, chunk_bytes=24) == K.EINVAL
    assert call(*good.values(), 2**31 + 1, K.D2D, 8, 5 << 20) == K.EINVAL
    # workspace: 32-byte header + 8 bytes per prefix entry, rounded up to 256
    assert K.kvcopy_device_workspace_bytes(0) == 256
    assert K.kvcopy_device_workspace_bytes(27) == 256
    assert K.kvcopy_device_workspace_bytes(28) == 512
    assert K.kvcopy_device_workspace_bytes(1000) == (32 + 8 * 1001 + 255) // 256 * 256


def test_autotune_rejects_bad_direction(K):
    import ctypes
    assert K.lib.kvcopy_autotune(3, None, None, None, None) == K.EINVAL
    assert K.lib.kvcopy_autotune(-1, None, None, ctypes.byref(ctypes.c_int()), None) == K.EINVAL


def test_latency_tool_is_built_and_checks_its_arguments(K):
    """The C-caller latency program is built next to the library and refuses
    to run without batch files (no GPU call is made before that check)."""
    exe = os.path.join(ROOT, "block_copy_amd", "kvcopy_latency")
    assert os.access(exe, os.X_OK)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr


def test_binding_matches_the_compiled_header(K, tmp_path):
    """Every constant and struct layout the Python binding restates equals
    what a C compiler reads from include/kvcopy.h (the argument marshalling
    depends on them)."""
    import ctypes
    consts = {"H2D": "KVCOPY_H2D", "D2H": "KVCOPY_D2H", "D2D": "KVCOPY_D2D", "OK": "KVCOPY_OK",
              "EINVAL": "KVCOPY_EINVAL", "EALIGN": "KVCOPY_EALIGN",
              "EOVERLAP": "KVCOPY_EOVERLAP", "ENOMEM": "KVCOPY_ENOMEM", "EHIP": "KVCOPY_EHIP",
              "WGS_ALL": "KVCOPY_WGS_ALL", "WGS_AUTO": "KVCOPY_WGS_AUTO",
              "CHUNK_DEFAULT": "KVCOPY_CHUNK_DEFAULT", "CHUNK_MAX": "KVCOPY_CHUNK_MAX",
              "OPTS_V1_SIZE": "KVCOPY_OPTS_V1_SIZE",
              "DEVICE_BAD_ALIGN": "KVCOPY_DEVICE_BAD_ALIGN",
              "DEVICE_TOO_MANY_CHUNKS": "KVCOPY_DEVICE_TOO_MANY_CHUNKS",
              "NOALLOC_MAX_N": "KVCOPY_NOALLOC_MAX_N"}
    hdr = open(os.path.join(ROOT, "include", "kvcopy.h")).read()
    flags = re.findall(r"#define (KVCOPY_F_(\w+)) 0x", hdr)
    assert len(flags) >= 11
    for macro, short in flags:
        consts["F_" + short] = macro
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "kvcopy.h"', "int main(void) {"]
    for name, macro in consts.items():
        src.append(f'    printf("{name} %lld\\n", (long long)({macro}));')
    for struct, fields in (("kvcopy_opts_t", K.Opts._fields_), ("kvcopy_plan_t", K._Plan._fields_)):
        src.append(f'    printf("sizeof {struct} %zu\\n", sizeof({struct}));')
        for f, _ in fields:
            src.append(f'    printf("offsetof {struct} {f} %zu\\n", offsetof({struct}, {f}));')
    src += ["    return 0;", "}"]
    c = tmp_path / "consts.c"
    c.write_text("\n".join(src) + "\n")
    exe = tmp_path / "consts"
    subprocess.run(["gcc", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    "-I" + os.path.join(ROOT, "include"), str(c), "-o", str(exe)],
                   check=True, capture_output=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True,
                               text=True).stdout.splitlines():
        key, val = line.rsplit(" ", 1)
        got[key] = int(val)
    for name in consts:
        assert getattr(K, name) == got[name], name
    for struct, cls in (("kvcopy_opts_t", K.Opts), ("kvcopy_plan_t", K._Plan)):
        assert ctypes.sizeof(cls) == got[f"sizeof {struct}"], struct
        for f, _ in cls._fields_:
            assert getattr(cls, f).offset == got[f"offsetof {struct} {f}"], (struct, f)

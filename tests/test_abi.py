"""Host-side checks of the C ABI (no GPU needed; nothing is launched).

The library loads, exports every function include/paged_attention.h
declares, sizes its workspace, and rejects bad arguments with the documented
status before touching the GPU.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attention.h")


@pytest.fixture(scope="module")
def lib():
    import paged_kv_cache_349_amd as pa
    if not os.path.exists(pa.LIB_PATH):
        from paged_kv_cache_349_amd.build import build
        build()
    return pa.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for n in ("pa_write_kv", "pa_decode", "pa_decode_workspace_bytes", "pa_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    import paged_kv_cache_349_amd as pa
    out = subprocess.run(["nm", "-D", "--defined-only", pa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in _declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings(lib):
    for code in range(5):
        assert lib.pa_status_string(code)
    assert lib.pa_status_string(99) == b"unknown status"
    assert lib.pa_status_str(3) == lib.pa_status_string(3)


def _align(n):
    return (n + 255) // 256 * 256


# planner control words: 32 ints + 32 claim counters, each in its own 128-byte line
CTRL = _align((32 + 32 * 32) * 4)


def test_workspace_sizes(lib):
    # one partition per sequence: planner outputs + work list + split list only
    assert lib.pa_decode_workspace_bytes_ex(4, 8, 8, 64, 4, 16, 0, 64) == \
        CTRL + _align(4 * 1 * 16) + _align(4 * 8)
    # 256 seqs, 64 heads / 8 KV heads, D=128, 285 blocks of 16, 512-token partitions -> 9
    n = lib.pa_decode_workspace_bytes_ex(256, 64, 8, 128, 285, 16, 1, 512)
    rows = 256 * 64 * 9
    assert n == (CTRL + _align(256 * 9 * 16) + _align(256 * 8) + _align(rows * 128 * 4) +
                 _align(rows * 8))
    # the library's choice is sized for its smallest partition (256 tokens)
    assert lib.pa_decode_workspace_bytes(256, 64, 8, 128, 285, 16, 1) == \
        lib.pa_decode_workspace_bytes_ex(256, 64, 8, 128, 285, 16, 1, 256)
    assert lib.pa_decode_workspace_bytes_ex(256, 64, 8, 128, 285, 16, 1, 24) == 0   # not a multiple
    assert lib.pa_decode_workspace_bytes(4, 6, 4, 64, 4, 16, 0) == 0                 # Hq % Hkv
    assert lib.pa_decode_partition_tokens(256, 8, 285, 16) == 256
    assert lib.pa_decode_partition_tokens(256, 8, 285, 32) == 256


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _decode(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, t=FAKE, l=FAKE, scale=0.125, bs=16, S=4, Hq=8,
             Hkv=2, D=128, maxb=8, NB=64, dt=1, ws=FAKE, wsb=1 << 30, pt=0, flags=0)
    a.update(kw)
    return lib.pa_decode_ex(a["out"], a["q"], a["k"], a["v"], a["t"], a["l"], a["scale"], a["bs"],
                            a["S"], a["Hq"], a["Hkv"], a["D"], a["maxb"], a["NB"], a["dt"],
                            a["ws"], a["wsb"], a["pt"], a["flags"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=6, Hkv=4), 1),
    (dict(Hq=0), 1),
    (dict(D=0), 1),
    (dict(NB=0), 1),
    (dict(S=-1), 1),
    (dict(maxb=0), 1),
    (dict(scale=float("nan")), 1),
    (dict(flags=8), 1),
    (dict(flags=4), 1),
    (dict(flags=2, dt=0), 2),            # packed-pool diagnostic: bf16 matrix-core kernel only
    (dict(flags=3), 2),
    (dict(pt=24), 1),
    (dict(out=None), 1),
    (dict(t=None), 1),
    (dict(q=FAKE + 4), 1),
    (dict(out=FAKE + 8), 1),
    (dict(D=96), 2),
    (dict(bs=8), 2),
    (dict(Hq=34, Hkv=2), 2),
    (dict(dt=7), 2),
    (dict(ws=None, maxb=100), 3),
    (dict(wsb=16, maxb=100), 3),
    (dict(ws=FAKE + 16), 3),
])
def test_decode_rejects_bad_arguments(lib, kw, status):
    assert _decode(lib, **kw) == status
    assert lib.pa_last_error()


def test_decode_empty_batch_is_noop(lib):
    assert _decode(lib, S=0, out=None, q=None) == 0


def _write(lib, **kw):
    a = dict(k=FAKE, v=FAKE, kn=FAKE, vn=FAKE, s=FAKE, T=4, NB=64, Hkv=2, D=128, bs=16, dt=1)
    a.update(kw)
    return lib.pa_write_kv(a["k"], a["v"], a["kn"], a["vn"], a["s"], a["T"], a["NB"], a["Hkv"],
                           a["D"], a["bs"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), 1), (dict(NB=0), 1), (dict(Hkv=0), 1), (dict(D=0), 1), (dict(bs=0), 1),
    (dict(k=None), 1), (dict(s=None), 1), (dict(D=2048), 2), (dict(dt=3), 2),
])
def test_write_rejects_bad_arguments(lib, kw, status):
    assert _write(lib, **kw) == status


def test_write_zero_tokens_is_noop(lib):
    assert _write(lib, T=0, k=None, v=None, kn=None, vn=None, s=None) == 0


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import paged_kv_cache_349_amd as pa
    monkeypatch.setattr(pa, "_lib", None)
    with pytest.raises(RuntimeError):
        pa.load_library(str(tmp_path / "missing.so"))


def test_kernel_timing_argument_errors(lib):
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int32(0)
    assert lib.pa_kernel_timing_begin(0) == 1
    assert lib.pa_kernel_timing_begin(-3) == 1
    assert lib.pa_kernel_timing_end(ctypes.byref(ms), ctypes.byref(n)) == 1   # not on
    assert lib.pa_kernel_timing_end(None, ctypes.byref(n)) == 1


def test_block_copy_argument_errors(lib):
    FAKE = 1 << 40
    args = dict(k=FAKE, v=FAKE, s=FAKE, d=FAKE, n=4, NB=16, Hkv=2, D=8, bs=4, dt=0)

    def call(**kw):
        a = {**args, **kw}
        return lib.pa_copy_blocks(a["k"], a["v"], a["s"], a["d"], a["n"], a["NB"], a["Hkv"],
                                  a["D"], a["bs"], a["dt"], None)
    assert call(n=-1) == 1
    assert call(dt=7) == 2
    assert call(NB=0) == 1
    assert call(s=None) == 1
    assert call(n=0, k=None, v=None, s=None, d=None) == 0
    assert lib.pa_swap_blocks(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 3, 0, 5, 2, 8, 4, 1, None) == 1
    assert lib.pa_swap_blocks(None, None, None, None, None, None, 0, 5, 5, 2, 8, 4, 1, None) == 0


def test_shared_prefix_workspace_and_errors(lib):
    parts = 11 + 1                # ceil(161 / 16) partitions, + 1 for the prefix cut
    rows = 128 * 32 * parts       # S * Hq * partitions
    n = lib.pa_decode_shared_prefix_workspace_bytes(128, 32, 8, 128, 161, 16, 1, 256)
    assert n == CTRL + _align(128 * parts * 16) + _align(128 * 8) + _align(rows * 128 * 4) + \
        _align(rows * 8) + _align(128 * parts * 16)
    assert lib.pa_decode_shared_prefix_workspace_bytes(4, 6, 4, 64, 4, 16, 1, 0) == 0
    FAKE = 1 << 40
    call = lambda dt, ng, S=4: lib.pa_decode_shared_prefix(
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ng, 0.5, 16, S, 8, 2, 128, 4, 64, dt,
        FAKE, 1 << 30, 0, None)
    assert call(0, 1) == 2            # fp32: not supported
    assert call(1, -1) == 1
    assert call(1, 1, S=9000) == 2    # more sequences than the planner keeps
    assert call(1, 1, S=0) == 0       # empty batch


def test_decode_step_argument_errors(lib):
    FAKE = 1 << 40
    def call(T=2, S=4, dt=1, Hq=8, ws=1 << 30):
        return lib.pa_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, T, FAKE, FAKE, FAKE, FAKE, 0.5, 16,
                                  S, Hq, 2, 128, 4, 64, dt, FAKE, ws, None)
    assert call(T=-1) == 1
    assert call(dt=5) == 2
    assert call(Hq=7) == 1          # Hq % Hkv
    assert call(ws=16) == 3         # workspace too small: nothing launched
    assert call(T=0, S=0) == 0      # empty step


def test_decode_check_argument_errors(lib):
    flag = 1 << 40
    assert lib.pa_decode_check(None, 1 << 20, flag, None) == 1
    assert lib.pa_decode_check(FAKE, 1 << 20, None, None) == 1
    assert lib.pa_decode_check(FAKE + 16, 1 << 20, flag, None) == 3      # misaligned workspace
    assert lib.pa_decode_check(FAKE, 64, flag, None) == 3                # smaller than any workspace
    assert lib.pa_decode_check(FAKE, 1 << 20, flag + 2, None) == 1       # misaligned flag
    assert lib.pa_last_error()


# A host program that calls the decode launcher with a launch-parameter size
# other than the one the library was compiled with, as an object built from
# an older version of the internal header would: the launcher must refuse
# before it launches anything (the check is the first thing it does, so this
# runs without a GPU).
_PARAMS_PROBE = r"""
#include <cstdio>
#include "pa_internal.h"
int main() {
  pa::DecodeParams p{};
  const hipError_t bad = pa::launch_decode(p, sizeof(p) + 8, pa::KvType::BF16, 128, 16, false,
                                           nullptr);
  const hipError_t bad2 = pa::launch_decode(p, sizeof(p) - 8, pa::KvType::F32, 64, 32, true,
                                            nullptr);
  std::printf("%d %d %d\n", (int)bad, (int)bad2, (int)hipErrorInvalidImage);
  return bad == hipErrorInvalidImage && bad2 == hipErrorInvalidImage ? 0 : 1;
}
"""


def test_launcher_refuses_a_mismatched_parameter_layout(lib, tmp_path):
    import shutil
    import paged_kv_cache_349_amd as pa
    from paged_kv_cache_349_amd import build as b
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    src = tmp_path / "params_probe.cpp"
    src.write_text(_PARAMS_PROBE)
    exe = tmp_path / "params_probe"
    libdir = os.path.dirname(pa.LIB_PATH)
    subprocess.run([gxx, "-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{b.ROCM}/include",
                    f"-I{b.CSRC}", f"-I{b.INCLUDE}", str(src), "-o", str(exe), f"-L{libdir}", "-lpa",
                    f"-Wl,-rpath,{libdir}", f"-L{b.ROCM}/lib", "-lamdhip64",
                    f"-Wl,-rpath,{b.ROCM}/lib"], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


def test_decode_noalloc_argument_errors(lib):
    """Checks that return before the library's array is touched (no GPU needed)."""
    def call(S=4, Hq=8, Hkv=2, D=128, maxb=8, bs=16, dt=1, out=FAKE):
        return lib.pa_decode_noalloc(out, FAKE, FAKE, FAKE, FAKE, FAKE, 0.125, bs, S, Hq, Hkv, D,
                                     maxb, 64, dt, None)
    assert call(S=4096, Hq=64, Hkv=8, maxb=2048) == 3     # too large for the array
    assert lib.pa_last_error().startswith(b"these shapes need")
    assert call(Hq=6, Hkv=4) == 1
    assert call(D=96) == 2
    assert call(dt=5) == 2
    assert call(out=None) == 1
    assert call(S=0, out=None) == 0                       # empty batch: nothing to do

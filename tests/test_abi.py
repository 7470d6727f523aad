"""The C ABI loads, exports every entry point its header declares, and rejects
bad arguments on the host before touching a device (CPU only)."""
import ctypes
import os
import re

import pytest

import int8_weight_gemm_amd as pf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libprefill.h")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pf_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared()
    for n in ("pf_quantize_act", "pf_gemm_i8_chunk", "pf_gemv_i8", "pf_prefill_stack",
              "pf_moe_chunk", "pf_status_string", "pf_init"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = pf.lib()
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, missing


def exported_c_functions():
    """Defined, exported text symbols of libprefill.so with C linkage (names that
    are not C++-mangled and not the toolchain's own)."""
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", pf.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    names = set()
    for line in out.splitlines():
        parts = line.split()
        if len(parts) == 3 and parts[1] in "TtWw" and not parts[2].startswith("_"):
            names.add(parts[2])
    return sorted(names)


def test_library_exports_exactly_the_header():
    """The C-linkage functions the library exports are the header's entry points,
    no more (internal helpers stay out of the ABI) and no fewer."""
    assert exported_c_functions() == declared()


def test_status_strings():
    assert pf.status_string(pf.PF_OK) == "PF_OK"
    assert "invalid" in pf.status_string(pf.PF_EINVAL)
    assert "unknown" in pf.status_string(42)


P = ctypes.c_void_p
FAKE = P(0x10000)     # aligned, never dereferenced: validation fails first


def test_gemm_rejects_bad_k_and_alignment():
    lib = pf.lib()
    # K not a multiple of 64
    assert lib.pf_gemm_i8_chunk(FAKE, FAKE, 64, 100, FAKE, FAKE, 4, P(0x20000), None, 0, None) == pf.PF_EINVAL
    # K too large for an exact int32 accumulator
    assert lib.pf_gemm_i8_chunk(FAKE, FAKE, 64, 131072 + 64, FAKE, FAKE, 4, P(0x20000), None, 0, None) == pf.PF_EINVAL
    # misaligned output
    assert lib.pf_gemm_i8_chunk(FAKE, FAKE, 64, 128, FAKE, FAKE, 4, P(0x20002), None, 0, None) == pf.PF_EINVAL
    assert lib.pf_gemm_i8_chunk(P(0x10008), FAKE, 64, 128, FAKE, FAKE, 4, P(0x20000), None, 0, None) == pf.PF_EINVAL
    # null pointer
    assert lib.pf_gemm_i8_chunk(None, FAKE, 64, 128, FAKE, FAKE, 4, P(0x20000), None, 0, None) == pf.PF_EINVAL
    # output overlapping the weights
    assert lib.pf_gemm_i8_chunk(FAKE, P(0x80000), 64, 128, P(0x90000), P(0xa0000), 4, P(0x10100), None, 0, None) == pf.PF_EINVAL
    # M = 0 is a no-op
    assert lib.pf_gemm_i8_chunk(FAKE, FAKE, 64, 128, FAKE, FAKE, 0, P(0x20000), None, 0, None) == pf.PF_OK
    # a weight matrix or token chunk of 2^32 bytes or more (32-bit offsets in the kernels)
    assert lib.pf_gemm_i8_chunk(FAKE, FAKE, 1 << 20, 4096, FAKE, FAKE, 4, P(0x20000), None, 0, None) == pf.PF_EINVAL
    # exactly 2^32 bytes at the largest K (one row fewer is the largest product taken)
    assert lib.pf_gemm_i8_chunk(FAKE, FAKE, 32768, 131072, FAKE, FAKE, 4, P(0x20000), None, 0, None) == pf.PF_EINVAL
    assert lib.pf_gemm_i8_chunk(FAKE, FAKE, 64, 4096, FAKE, FAKE, 1 << 20, P(0x20000), None, 0, None) == pf.PF_EINVAL


def test_quantize_and_gemv_validation():
    lib = pf.lib()
    assert lib.pf_quantize_act(FAKE, 4, 63, 63, P(0x20000), P(0x30000), None) == pf.PF_EINVAL
    assert lib.pf_quantize_act(FAKE, 4, 64, 32, P(0x20000), P(0x30000), None) == pf.PF_EINVAL
    assert lib.pf_quantize_act(FAKE, 0, 64, 64, None, None, None) == pf.PF_OK
    assert lib.pf_gemv_i8(FAKE, FAKE, 0, 64, FAKE, FAKE, P(0x20000), None) == pf.PF_EINVAL
    assert lib.pf_expf_cr(FAKE, -1, FAKE, None) == pf.PF_EINVAL


def test_no_device_here():
    # this container has no GPU: the device check answers PF_ENODEV
    if os.environ.get("PF_EXPECT_GPU"):
        pytest.skip("running on a GPU host")
    assert pf.lib().pf_init() == pf.PF_ENODEV
    assert pf.lib().pf_gemm_i8_chunk(FAKE, FAKE, 64, 128, P(0x30000), P(0x40000), 4, P(0x50000), None, 0, None) == pf.PF_ENODEV


def test_workspace_queries():
    lib = pf.lib()
    assert lib.pf_gemm_i8_chunk_workspace(1024, 4096, 32) > 0      # 16 row tiles: K split
    assert lib.pf_gemm_i8_chunk_workspace(16384, 4096, 32) == 0    # 256 row tiles fill the chip
    assert lib.pf_gemm_i8_chunk_workspace(4096, 4096, 128) > 0      # 16 tiles: K split
    assert lib.pf_gemm_i8_chunk_workspace(65536, 4096, 512) == 0    # 512 tiles fill the chip
    assert lib.pf_gemm_i8_chunk_workspace(4096, 100, 32) == 0
    layers = (pf._Layer * 2)()
    st = pf._Stack(2, 1024, 4096, ctypes.cast(layers, ctypes.POINTER(pf._Layer)))
    ws32 = lib.pf_prefill_stack_workspace(ctypes.byref(st), 32)
    assert ws32 >= 32 * (5 * 1024 + 2 * 4096) * 4
    m = pf._Moe(512, 10, 2048, 512, *[0x10000] * 7)
    assert lib.pf_moe_chunk_workspace(ctypes.byref(m), 512) >= 512 * 10 * 2048 * 4
    bad = pf._Moe(512, 10, 2000, 512, *[0x10000] * 7)
    assert lib.pf_moe_chunk_workspace(ctypes.byref(bad), 512) == 0


def test_stack_validation():
    lib = pf.lib()
    layers = (pf._Layer * 1)()
    st = pf._Stack(1, 128, 256, ctypes.cast(layers, ctypes.POINTER(pf._Layer)))
    # null weights in the layer table
    assert lib.pf_prefill_stack(ctypes.byref(st), FAKE, 4, 32, P(0x20000), None, None, P(0x40000), 1 << 20,
                                None, None) == pf.PF_EINVAL
    for j in range(7):
        layers[0].W[j] = 0x100000 + j * 0x10000
        layers[0].w_scale[j] = 0x200000 + j * 0x10000
    # workspace too small
    assert lib.pf_prefill_stack(ctypes.byref(st), P(0x300000), 4, 32, P(0x310000), None, None, P(0x400000), 16,
                                None, None) == pf.PF_EWORKSPACE
    # chunk must be positive
    assert lib.pf_prefill_stack(ctypes.byref(st), P(0x300000), 4, 0, P(0x310000), None, None, P(0x400000), 1 << 20,
                                None, None) == pf.PF_EINVAL


@pytest.mark.parametrize("L,H,F,chunk,P", [(16, 1024, 4096, 128, 40), (32, 4096, 11008, 256, 64),
                                           (3, 128, 320, 96, 75), (2, 1024, 4096, 32, 40)])
def test_stack_workspace_query_covers_short_prompts(L, H, F, chunk, P):
    """A prompt shorter than one chunk runs as a chunk of P tokens, whose layout
    (more slots and split partials up to 64 tokens) can exceed the layout of the
    requested chunk; the size query covers it, so the call gets past the
    workspace check with exactly the queried size (and then stops at the device
    check here, or runs on a GPU host)."""
    if os.environ.get("PF_EXPECT_GPU"):
        pytest.skip("running on a GPU host")
    lib = pf.lib()
    layers = (pf._Layer * L)()
    for l in range(L):
        for j in range(7):
            layers[l].W[j] = 0x1000000 + (l * 7 + j) * 0x10000
            layers[l].w_scale[j] = 0x8000000 + (l * 7 + j) * 0x10000
    st = pf._Stack(L, H, F, ctypes.cast(layers, ctypes.POINTER(pf._Layer)))
    need = lib.pf_prefill_stack_workspace(ctypes.byref(st), chunk)
    assert need > 0
    x, y, ws = P_(0x100000000), P_(0x200000000), P_(0x300000000)
    assert lib.pf_prefill_stack(ctypes.byref(st), x, P, chunk, y, None, None, ws, need, None, None) == pf.PF_ENODEV
    for p in range(1, chunk + 1):
        assert lib.pf_prefill_stack(ctypes.byref(st), x, p, chunk, y, None, None, ws, need, None, None) == pf.PF_ENODEV


P_ = ctypes.c_void_p


def test_noalloc_product_refuses_plans_beyond_its_array():
    """pf_gemm_i8_chunk_noalloc refuses, before touching a device, a product
    whose split plan needs more partials than its 64 MiB array holds (260 tiles
    of 256 x 256 over K = 131072: a two-way split of 520 MiB), and accepts
    the arguments of one that fits (then stops at the device check here)."""
    if os.environ.get("PF_EXPECT_GPU"):
        pytest.skip("running on a GPU host")
    lib = pf.lib()
    N, K, M = 3328, 131072, 5120
    assert lib.pf_gemm_i8_chunk_workspace(N, K, M) > pf.NOALLOC_SCRATCH_BYTES
    W, ws, q, s, y = (P_(a) for a in (0x1000000000, 0x2000000000, 0x3000000000, 0x4000000000,
                                      0x5000000000))
    assert lib.pf_gemm_i8_chunk_noalloc(W, ws, N, K, q, s, M, y, None) == pf.PF_EWORKSPACE
    assert lib.pf_gemm_i8_chunk_noalloc(W, ws, 4096, 4096, q, s, 512, y, None) == pf.PF_ENODEV
    assert lib.pf_gemm_i8_chunk_noalloc(W, ws, 4096, 100, q, s, 512, y, None) == pf.PF_EINVAL

"""Host-only checks of the C ABI (no GPU needed): the library loads, exports every
symbol include/tra.h declares, and rejects bad arguments with its status codes
before making any HIP call (so these run in a GPU-less container)."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tra.h")

OK, INVALID, UNSUPPORTED, HIPERR, CAPACITY = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
FAKE = 0x10000  # never dereferenced: every call below fails validation first
FAKE2 = 0x20000
FAKE3 = 0x30000
FAKE4 = 0x40000


@pytest.fixture(scope="module")
def lib():
    import entropy_adaptive_sparse_amd as tra
    if not os.path.exists(tra.library_path()):
        from entropy_adaptive_sparse_amd import build
        build.build()
    return tra.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(tra_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("tra_tile_major_permute", "tra_tile_major_unpermute", "tra_dense_attn_entropy",
              "tra_build_block_mask", "tra_block_sparse_attn", "tra_mask_prepare", "tra_status_string",
              "tra_dense_attn_entropy_mask", "tra_dense_attn_entropy_natural", "tra_block_sparse_attn_natural",
              "tra_dense_attn_entropy_mask_natural", "tra_natural_prepare", "tra_block_sparse_attn_fp8",
              "tra_sparse_schedule", "tra_block_sparse_attn_scheduled", "tra_build_block_mask_1d",
              "tra_mask_prepare_1d"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in ((0, b"TRA_OK"), (1, b"TRA_ERR_INVALID_ARG"), (2, b"TRA_ERR_UNSUPPORTED"),
                       (3, b"TRA_ERR_HIP"), (4, b"TRA_ERR_CAPACITY"), (99, b"TRA_ERR_UNKNOWN")):
        assert lib.tra_status_string(code) == name


def test_permute_validation(lib):
    f = lib.tra_tile_major_permute
    assert f(None, FAKE, 1, 2, 3, 4, 8, BF16, 8, 8, None) == INVALID
    assert f(FAKE, None, 1, 2, 3, 4, 8, BF16, 8, 8, None) == INVALID
    assert f(FAKE, FAKE, 1, 2, 3, 4, 8, BF16, 8, 8, None) == INVALID  # in place
    assert f(FAKE, FAKE2, 0, 2, 3, 4, 8, BF16, 8, 8, None) == INVALID
    assert f(FAKE, FAKE2, 1, 0, 3, 4, 8, BF16, 8, 8, None) == INVALID
    assert f(FAKE, FAKE2, 1, 2, 3, 4, 0, BF16, 8, 8, None) == INVALID
    assert f(FAKE, FAKE2, 1, 2, 3, 4, 8, 7, 8, 8, None) == INVALID
    assert f(FAKE, FAKE2, 1, 2, 3, 4, 8, BF16, 0, 8, None) == INVALID
    assert f(FAKE, FAKE2, 1, 2048, 2048, 2048, 8, BF16, 8, 8, None) == UNSUPPORTED
    assert lib.tra_tile_major_unpermute(FAKE, FAKE, 1, 2, 3, 4, 8, BF16, 8, 8, None) == INVALID


def test_dense_validation(lib):
    f = lib.tra_dense_attn_entropy
    args = [FAKE, FAKE2, FAKE3, FAKE4, None, None, 2, 1024, 128, BF16, 0.088, None]
    for i in range(4):
        a = list(args)
        a[i] = None
        assert f(*a) == INVALID
    a = list(args); a[3] = FAKE; assert f(*a) == INVALID         # o aliases q
    a = list(args); a[6] = 0; assert f(*a) == INVALID
    a = list(args); a[7] = 0; assert f(*a) == INVALID
    a = list(args); a[8] = 96; assert f(*a) == UNSUPPORTED
    a = list(args); a[9] = 5; assert f(*a) == INVALID
    a = list(args); a[10] = 0.0; assert f(*a) == INVALID
    a = list(args); a[10] = float("nan"); assert f(*a) == INVALID
    a = list(args); a[0] = FAKE + 2; assert f(*a) == INVALID     # misaligned


def _mask_args(**kw):
    a = dict(ent=FAKE, outer=2, F=4, H=16, W=16, tau=1.0, gamma=0.5, bq=64, bk=64, vote=1, th=8, tw=8,
             cnt=FAKE2, idx=FAKE3, cap=2 * 16 * 16, mask=None, s=None)
    a.update(kw)
    return list(a.values())


def test_mask_validation(lib):
    f = lib.tra_build_block_mask
    assert f(*_mask_args(ent=None)) == INVALID
    assert f(*_mask_args(cnt=None)) == INVALID
    assert f(*_mask_args(idx=None)) == INVALID
    assert f(*_mask_args(outer=0)) == INVALID
    assert f(*_mask_args(F=0)) == INVALID
    assert f(*_mask_args(tau=0.0)) == INVALID
    assert f(*_mask_args(tau=-1.0)) == INVALID
    assert f(*_mask_args(tau=float("inf"))) == INVALID
    assert f(*_mask_args(gamma=-0.1)) == INVALID
    assert f(*_mask_args(gamma=float("nan"))) == INVALID
    assert f(*_mask_args(vote=0)) == INVALID
    assert f(*_mask_args(bq=96)) == UNSUPPORTED
    assert f(*_mask_args(bk=128)) == UNSUPPORTED
    assert f(*_mask_args(th=0)) == INVALID
    assert f(*_mask_args(cap=2 * 16 * 16 - 1)) == CAPACITY
    assert f(*_mask_args(F=400, H=64, W=64, cap=10 ** 9)) == UNSUPPORTED  # LDS budget


def test_sparse_validation(lib):
    f = lib.tra_block_sparse_attn
    base = [FAKE, FAKE2, FAKE3, FAKE4, None, FAKE + 4096, FAKE2 + 4096, 2, 1024, 128, BF16, 0.088, 128, 64, None]
    a = list(base); a[5] = None; assert f(*a) == INVALID
    a = list(base); a[6] = None; assert f(*a) == INVALID
    a = list(base); a[12] = 32; assert f(*a) == UNSUPPORTED
    a = list(base); a[13] = 32; assert f(*a) == UNSUPPORTED
    a = list(base); a[12] = 0; assert f(*a) == INVALID
    a = list(base); a[9] = 80; assert f(*a) == UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    import entropy_adaptive_sparse_amd as tra
    x = torch.zeros(1, 8, 4)
    with pytest.raises(ValueError):
        tra.tile_major_permute(x, 1, 2, 4)


def test_fused_warmup_validation(lib):
    f = lib.tra_dense_attn_entropy_mask
    # q k v o H lse outer F H W D dt scale tau gamma bq bk vote th tw cnt idx cap mask stream
    base = [FAKE, FAKE2, FAKE3, FAKE4, None, None, 2, 4, 16, 16, 128, BF16, 0.088, 0.03, 0.5, 128, 64, 1, 8, 8,
            FAKE + 64, FAKE2 + 64, 2 * 8 * 16, None, None]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a20=None) == INVALID                         # kv_count
    assert call(a21=None) == INVALID                         # kv_index
    assert call(a0=None) == INVALID                          # q
    assert call(a3=FAKE) == INVALID                          # o aliases q
    assert call(a17=0) == INVALID                            # vote threshold
    assert call(a13=0.0) == INVALID                          # tau
    assert call(a11=F32) == UNSUPPORTED                      # fp32
    assert call(a10=64) == UNSUPPORTED                       # D = 64
    assert call(a15=64) == UNSUPPORTED                       # block_q = 64
    assert call(a16=32) == UNSUPPORTED                       # block_k
    assert call(a7=65, a8=8, a9=8) == UNSUPPORTED            # more frames than the tile buffers hold
    assert call(a22=2 * 8 * 16 - 1) == CAPACITY              # kv_index capacity


def test_natural_order_validation(lib):
    fd = lib.tra_dense_attn_entropy_natural
    # q k v o H lse outer F H W D dt scale th tw stream
    dense = [FAKE, FAKE2, FAKE3, FAKE4, None, None, 2, 4, 16, 16, 128, BF16, 0.088, 8, 8, None]
    fs = lib.tra_block_sparse_attn_natural
    # q k v o lse cnt idx outer F H W D dt scale bq bk th tw stream
    sparse = [FAKE, FAKE2, FAKE3, FAKE4, None, FAKE + 64, FAKE2 + 64, 2, 4, 16, 16, 128, BF16, 0.088, 128, 64, 8, 8,
              None]

    def call(f, base, **kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    for f, base in ((fd, dense), (fs, sparse)):
        assert call(f, base, a0=None) == INVALID                  # q
        assert call(f, base, a3=FAKE2) == INVALID                 # o aliases k
    assert call(fd, dense, a6=0) == INVALID                       # outer
    assert call(fd, dense, a7=0) == INVALID                       # F
    assert call(fs, sparse, a7=0) == INVALID                      # outer
    assert call(fs, sparse, a8=0) == INVALID                      # F
    assert call(fd, dense, a9=18) == UNSUPPORTED                  # W not a multiple of 4
    assert call(fd, dense, a14=6) == UNSUPPORTED                  # tile width not a multiple of 4
    assert call(fd, dense, a10=64) == UNSUPPORTED                 # D = 64
    assert call(fd, dense, a11=F32) == UNSUPPORTED                # fp32
    assert call(fd, dense, a13=0) == INVALID                      # tile height
    assert call(fs, sparse, a5=None) == INVALID                   # kv_count
    assert call(fs, sparse, a6=None) == INVALID                   # kv_index
    assert call(fs, sparse, a14=64) == UNSUPPORTED                # block_q = 64
    assert call(fs, sparse, a15=32) == UNSUPPORTED                # block_k
    assert call(fs, sparse, a10=18) == UNSUPPORTED                # W not a multiple of 4
    assert call(fs, sparse, a12=F32) == UNSUPPORTED               # fp32
    ff = lib.tra_dense_attn_entropy_mask_natural
    # q k v o H lse outer F H W D dt scale tau gamma bq bk vote th tw cnt idx cap mask stream
    fused = [FAKE, FAKE2, FAKE3, FAKE4, None, None, 2, 4, 16, 16, 128, BF16, 0.088, 0.03, 0.5, 128, 64, 1, 8, 8,
             FAKE + 64, FAKE2 + 64, 2 * 8 * 16, None, None]
    assert call(ff, fused, a20=None) == INVALID                   # kv_count
    assert call(ff, fused, a13=0.0) == INVALID                    # tau
    assert call(ff, fused, a9=18) == UNSUPPORTED                  # W not a multiple of 4
    assert call(ff, fused, a19=6) == UNSUPPORTED                  # tile width not a multiple of 4
    assert call(ff, fused, a11=F32) == UNSUPPORTED                # fp32
    assert call(ff, fused, a7=65, a8=8, a9=8) == UNSUPPORTED      # more frames than the tile buffers hold
    assert call(ff, fused, a22=2 * 8 * 16 - 1) == CAPACITY        # kv_index capacity


def test_sparse_fp8_validation(lib):
    f = lib.tra_block_sparse_attn_fp8
    # q k v o lse cnt idx order outer N D scale bq bk stream
    base = [FAKE, FAKE2, FAKE3, FAKE4, None, FAKE + 64, FAKE2 + 64, None, 2, 1024, 128, 0.088, 128, 64, None]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a0=None) == INVALID              # q
    assert call(a3=FAKE2) == INVALID             # o aliases k
    assert call(a5=None) == INVALID              # kv_count
    assert call(a6=None) == INVALID              # kv_index
    assert call(a11=0.0) == INVALID              # sm_scale
    assert call(a10=64) == UNSUPPORTED           # D = 64
    assert call(a12=64) == UNSUPPORTED           # block_q = 64
    assert call(a13=32) == UNSUPPORTED           # block_k
    assert call(a1=FAKE2 + 8) == INVALID         # k not 16-byte aligned


def test_schedule_validation(lib):
    f = lib.tra_sparse_schedule
    # cnt outer F H W bq bk th tw order cap stream
    base = [FAKE, 2, 4, 16, 16, 128, 64, 8, 8, FAKE2, 2 * 8, None]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a0=None) == INVALID              # kv_count
    assert call(a9=None) == INVALID              # order
    assert call(a1=0) == INVALID                 # outer
    assert call(a2=0) == INVALID                 # F
    assert call(a5=32) == UNSUPPORTED            # block_q
    assert call(a6=128) == UNSUPPORTED           # block_k
    assert call(a10=15) == CAPACITY              # order capacity
    g = lib.tra_block_sparse_attn_scheduled
    # q k v o lse cnt idx order outer N D dt scale bq bk stream
    sb = [FAKE, FAKE2, FAKE3, FAKE4, None, FAKE + 64, FAKE2 + 64, FAKE3 + 64, 2, 1024, 128, BF16, 0.088, 128, 64, None]
    a = list(sb); a[7] = None; assert g(*a) == INVALID       # order
    a = list(sb); a[6] = None; assert g(*a) == INVALID       # kv_index
    a = list(sb); a[14] = 32; assert g(*a) == UNSUPPORTED    # block_k
    a = list(sb); a[10] = 96; assert g(*a) == UNSUPPORTED    # D


def test_mask_1d_validation(lib):
    f = lib.tra_build_block_mask_1d
    # ent outer F H W tau bq bk vote th tw cnt idx cap mask stream
    base = [FAKE, 2, 4, 16, 16, 0.05, 128, 64, 1, 8, 8, FAKE2, FAKE3, 2 * 8 * 16, None, None]

    def call(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a0=None) == INVALID              # entropy
    assert call(a11=None) == INVALID             # kv_count
    assert call(a1=0) == INVALID                 # outer
    assert call(a5=0.0) == INVALID               # tau
    assert call(a5=float("inf")) == INVALID      # tau
    assert call(a8=0) == INVALID                 # vote threshold
    assert call(a6=96) == UNSUPPORTED            # block_q
    assert call(a7=32) == UNSUPPORTED            # block_k
    assert call(a13=2 * 8 * 16 - 1) == CAPACITY  # kv_index capacity
    assert lib.tra_mask_prepare_1d(4, 16, 16, -1.0, 128, 64, 8, 8) == INVALID


def test_natural_prepare_validation(lib):
    f = lib.tra_natural_prepare
    assert f(0, 16, 16, 8, 8) == INVALID            # F
    assert f(4, 16, 16, 0, 8) == INVALID            # tile height
    assert f(4, 16, 18, 8, 8) == UNSUPPORTED        # W not a multiple of 4
    assert f(4, 16, 16, 8, 6) == UNSUPPORTED        # tile width not a multiple of 4


def test_header_is_plain_c(tmp_path):
    # the ABI header compiles as C99 and as C++17 on its own (the HIP runtime API header
    # supplies hipStream_t; no HIP compiler involved)
    import shutil
    import subprocess
    inc = "/opt/rocm/include"
    if shutil.which("gcc") is None or not os.path.exists(os.path.join(inc, "hip", "hip_runtime_api.h")):
        pytest.skip("gcc or the ROCm headers are not available")
    src = tmp_path / "use.c"
    src.write_text('#include "tra.h"\nint main(void) { return (int)TRA_OK + (tra_status_string(TRA_OK) == 0); }\n')
    for cc, std in (("gcc", "-std=c99"), ("g++", "-std=c++17")):
        lang = ["-x", "c++"] if cc == "g++" else []
        r = subprocess.run([cc, std, *lang, "-D__HIP_PLATFORM_AMD__", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                            "-I", os.path.join(ROOT, "include"), "-I", inc, str(src)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr

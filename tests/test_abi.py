"""The C-ABI library loads, exports every symbol include/binattn.h declares, and rejects
bad arguments before touching a device (no compute calls are made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "binattn.h")
LIB = os.path.join(ROOT, "diffusion_transformers_amd", "libbinattn.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libbinattn.so not built (run __graft_entry__.build())")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(binattn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from diffusion_transformers_amd import binding
    return binding.lib()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"binattn_pack_qk", "binattn_quant_v", "binattn_forward", "binattn_scores_i32"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} missing from libbinattn.so"
    from diffusion_transformers_amd import binding
    assert sorted(binding.EXPORTS) == names


def test_header_has_no_torch_types():
    text = open(HEADER).read()
    assert "torch" not in text.lower().replace("pytorch", "")
    assert "extern \"C\"" in text


def test_small_helpers(lib):
    assert lib.binattn_abi_version() == 1
    assert [lib.binattn_words(d) for d in (1, 32, 33, 64, 72, 128)] == [1, 1, 2, 2, 3, 4]
    assert [lib.binattn_vq_ld(n) for n in (1, 64, 65, 197, 577, 16384)] == [64, 64, 128, 256, 640, 16384]
    assert lib.binattn_strerror(-2) and lib.binattn_strerror(12345) == b"unknown error"


P = ctypes.c_void_p


def _a(x):
    return P(x)


def test_pack_and_quant_validation(lib):
    ok = (_a(256), 1, 2, 3, 5, 64, _a(512), _a(1024), None)
    # null pointers / sizes / dtype / d / alignment are all rejected before any device call
    assert lib.binattn_pack_qk(None, *ok[1:]) == -1
    assert lib.binattn_pack_qk(ok[0], 1, 0, 3, 5, 64, ok[6], ok[7], None) == -1
    assert lib.binattn_pack_qk(ok[0], 1, 2, 3, -5, 64, ok[6], ok[7], None) == -1
    assert lib.binattn_pack_qk(ok[0], 7, 2, 3, 5, 64, ok[6], ok[7], None) == -2
    assert lib.binattn_pack_qk(ok[0], 1, 2, 3, 5, 60, ok[6], ok[7], None) == -2
    assert lib.binattn_pack_qk(ok[0], 1, 2, 3, 5, 136, ok[6], ok[7], None) == -2
    assert lib.binattn_pack_qk(ok[0], 1, 2, 3, 70000, 64, ok[6], ok[7], None) == -2
    assert lib.binattn_pack_qk(_a(258), 1, 2, 3, 5, 64, ok[6], ok[7], None) == -3
    assert lib.binattn_quant_v(ok[0], 1, 2, 3, 5, 64, None, ok[7], None) == -1
    assert lib.binattn_quant_v(ok[0], 1, 2, 3, 5, 64, _a(520), ok[7], None) == -3
    assert lib.binattn_vq_canonical(None, 2, 3, 5, 64, ok[6], None) == -1
    assert lib.binattn_vq_canonical(ok[0], 2, 0, 5, 64, ok[6], None) == -1
    assert lib.binattn_vq_canonical(ok[0], 2, 3, 5, 60, ok[6], None) == -2
    assert lib.binattn_vq_canonical(ok[0], 2, 3, 5, 64, _a(520), None) == -3


def _fwd(lib, **kw):
    args = dict(qb=_a(256), qm=_a(512), kb=_a(768), km=_a(1024), vq=_a(1280), vs=_a(1536), kind=0, bdt=1,
                bias=None, ld=0, gh=0, gw=0, B=2, H=3, N=256, d=64, out=_a(2048), odt=1, stream=None)
    args.update(kw)
    return lib.binattn_forward(*args.values())


def test_forward_validation(lib):
    assert _fwd(lib, qb=None) == -1
    assert _fwd(lib, kind=0, bias=_a(4096)) == -1            # bias given with kind NONE
    assert _fwd(lib, kind=1, bias=None, ld=256) == -1        # dense without data
    assert _fwd(lib, kind=1, bias=_a(4096), ld=255) == -1    # ld < N
    assert _fwd(lib, kind=1, bias=_a(4096), ld=260, N=257) == -3  # 520-byte rows are not 16-byte multiples
    assert _fwd(lib, kind=1, bias=_a(4100), ld=256) == -3    # misaligned base
    # a dense bias whose 16-row byte extent does not fit a 32-bit buffer extent
    assert _fwd(lib, kind=1, bias=_a(4096), ld=1 << 26) == -2           # fp16: 16 * 2^27 bytes = 2^31
    assert _fwd(lib, kind=1, bias=_a(4096), ld=1 << 25, bdt=0) == -2    # fp32: 16 * 2^27 bytes
    assert _fwd(lib, kind=1, bias=_a(4096), ld=(1 << 62)) == -2         # no 64-bit wrap in the check
    assert _fwd(lib, kind=2, bias=_a(4096), gh=16, gw=15) == -1   # grid does not cover N
    assert _fwd(lib, kind=2, bias=_a(4096), N=344, gh=2, gw=172) == -2  # staged table rows of one tile too wide
    assert _fwd(lib, kind=2, bias=_a(4096), N=1024, gh=1, gw=1024) == -2  # window of one tile too wide
    assert _fwd(lib, kind=2, bias=_a(4096), N=1056, gh=6, gw=176) == -2
    assert _fwd(lib, kind=3, bias=_a(4096)) == -2
    assert _fwd(lib, odt=5) == -2
    assert _fwd(lib, d=72, out=_a(2056)) == -3
    assert lib.binattn_scores_i32(_a(256), None, 1, 1, 4, 64, _a(512), None) == -1
    assert lib.binattn_qk_rowstats(_a(256), _a(512), 1, 1, 4, 64, 0, None, _a(768), None) == -1
    assert lib.binattn_qk_rowstats(_a(256), _a(512), 1, 1, 4, 64, 2, _a(1024), _a(768), None) == -2
    assert lib.binattn_qk_rowstats(_a(256), _a(516), 1, 1, 4, 64, 1, _a(1024), _a(768), None) == -3


def test_prepare_and_attention_validation(lib):
    import ctypes as C
    lib.binattn_attention_workspace.restype = C.c_int64
    ws = lib.binattn_attention_workspace(2, 3, 197, 64)
    # bits (2 x 1182 tokens x 2 words), mu (2 x 1182), V^ (6 x 64 x 256), absmax, each 256-aligned
    up = lambda x: (x + 255) // 256 * 256
    assert ws == 2 * up(1182 * 8) + 2 * up(1182 * 4) + up(6 * 64 * 256) + up(6 * 64 * 4)
    assert lib.binattn_attention_workspace(2, 3, 197, 60) == -1
    P = C.c_void_p
    i64 = C.c_int64
    pre = [P(256), P(512), P(768), 1, 2, 3, 197, 64, P(1024), P(1280), P(1536), P(1792), P(2048), P(2304), None]
    bad = list(pre); bad[0] = None
    assert lib.binattn_prepare(*bad) == -1
    bad = list(pre); bad[3] = 9
    assert lib.binattn_prepare(*bad) == -2
    bad = list(pre); bad[8] = P(1028)
    assert lib.binattn_prepare(*bad) == -3
    att = [P(256), P(512), P(768), 1, 0, 1, None, i64(0), 0, 0, 2, 3, 197, 64, P(4096), 1, P(1 << 20), i64(ws), None]
    lib.binattn_attention.argtypes = [P, P, P, C.c_int, C.c_int, C.c_int, P, C.c_int64, C.c_int, C.c_int, C.c_int,
                                      C.c_int, C.c_int, C.c_int, P, C.c_int, P, C.c_int64, P]
    bad = list(att); bad[17] = i64(ws - 1)
    assert lib.binattn_attention(*bad) == -1          # workspace too small
    bad = list(att); bad[16] = P((1 << 20) + 16)
    assert lib.binattn_attention(*bad) == -3          # workspace not 256-byte aligned
    bad = list(att); bad[16] = None
    assert lib.binattn_attention(*bad) == -1
    bad = list(att); bad[4] = 1                        # dense bias kind without data
    assert lib.binattn_attention(*bad) == -1


def test_attention_one_kernel_query(lib):
    """Which way binattn_attention runs is a pure function of the shapes (no device needed):
    one kernel for fp16 rows of <= 256 keys at d of 56..80 or 120..128, else prepare + forward."""
    q = lib.binattn_attention_one_kernel
    F32, F16, NONE, DENSE, REL = 0, 1, 0, 1, 2
    assert q(F16, DENSE, F16, 0, 0, 64, 6, 197, 64) == 1      # DeiT-S
    assert q(F16, REL, F16, 16, 16, 64, 16, 256, 72) == 1     # DiT-XL/2
    assert q(F16, NONE, F16, 0, 0, 1, 1, 1, 128) == 1
    assert q(F16, DENSE, F16, 0, 0, 32, 12, 577, 64) == 0     # DeiT-B/384: rows of 577 keys
    assert q(F32, DENSE, F32, 0, 0, 1, 3, 197, 64) == 0       # fp32 inputs
    assert q(F16, NONE, F16, 0, 0, 2, 2, 100, 32) == 0        # d = 32
    assert q(F16, NONE, F16, 0, 0, 2, 2, 257, 64) == 0
    assert q(F16, NONE, F16, 0, 0, 2, 2, 100, 60) == -2       # d not a multiple of 8
    assert q(F16, REL, F16, 32, 8, 2, 2, 256, 64) == 0        # grid width not a multiple of 16: two launches
    assert q(F16, REL, F16, 14, 14, 2, 2, 196, 64) == 0       # the 14 x 14 grid of a 224^2 image, 16-pixel patches
    assert q(F16, REL, F16, 2, 172, 2, 2, 344, 64) == -2      # staged table rows of one tile too wide
    assert q(F16, REL, F16, 16, 16, 2, 2, 255, 64) == -1      # grid does not cover N
    assert q(7, NONE, F16, 0, 0, 2, 2, 100, 64) == -2


def _noalloc(lib, **kw):
    args = dict(q=_a(256), k=_a(512), v=_a(768), dt=1, kind=0, bdt=1, bias=None, ld=0, gh=0, gw=0, B=2, H=3, N=1000,
                d=64, out=_a(1024), odt=1, stream=None)
    args.update(kw)
    return lib.binattn_attention_noalloc(*args.values())


def test_noalloc_validation(lib):
    """binattn_attention_noalloc checks its arguments as binattn_attention does, and refuses a
    batch item whose packed inputs exceed the scratch, all before touching a device."""
    import ctypes as C
    lib.binattn_attention_noalloc.argtypes = [C.c_void_p] * 3 + [C.c_int] * 3 + [C.c_void_p, C.c_int64] + \
        [C.c_int] * 6 + [C.c_void_p, C.c_int, C.c_void_p]
    lib.binattn_attention_workspace.restype = C.c_int64
    assert _noalloc(lib, q=None) == -1
    assert _noalloc(lib, out=None) == -1
    assert _noalloc(lib, B=0) == -1
    assert _noalloc(lib, dt=3) == -2
    assert _noalloc(lib, d=60) == -2
    assert _noalloc(lib, v=_a(770)) == -3
    assert _noalloc(lib, kind=1, bias=None, ld=1000) == -1
    # one batch item of 64 heads x 8192 tokens x 128 channels: V^ alone fills the 64 MiB scratch
    assert lib.binattn_attention_workspace(1, 64, 8192, 128) > 64 << 20
    assert _noalloc(lib, B=1, H=64, N=8192, d=128) == -2
    assert _noalloc(lib, B=4, H=64, N=8192, d=128) == -2


def _qkv(lib, **kw):
    args = dict(x=_a(256), w=_a(512), bias=None, B=2, N=5, H=3, d=64, qb=_a(768), qm=_a(1024), kb=_a(1280),
                km=_a(1536), v=_a(1792), q=None, k=None, stream=None)
    args.update(kw)
    return lib.binattn_qkv_pack(*args.values())


def test_qkv_pack_validation(lib):
    assert _qkv(lib, x=None) == -1 and _qkv(lib, w=None) == -1 and _qkv(lib, v=None) == -1
    assert _qkv(lib, km=None) == -1
    assert _qkv(lib, B=0) == -1 and _qkv(lib, N=-1) == -1
    assert _qkv(lib, d=60) == -2 and _qkv(lib, d=136) == -2 and _qkv(lib, N=70000) == -2
    assert _qkv(lib, x=_a(258)) == -3 and _qkv(lib, bias=_a(260)) == -3 and _qkv(lib, q=_a(262)) == -3


def test_valid_arguments_without_a_device_report_enodevice(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    assert lib.binattn_pack_qk(_a(256), 1, 2, 3, 5, 64, _a(512), _a(1024), None) == -4
    assert lib.binattn_vq_canonical(_a(256), 2, 3, 5, 64, _a(512), None) == -4
    assert _fwd(lib) == -4
    assert _fwd(lib, kind=2, bias=_a(4096), gh=16, gw=16) == -4
    assert _fwd(lib, kind=1, bias=_a(4096), ld=(1 << 26) - 8) == -4  # the largest fp16 dense-bias stride accepted
    assert _qkv(lib) == -4 and _qkv(lib, bias=_a(2048), q=_a(2304), k=_a(2560)) == -4
    assert _noalloc(lib) == -4                    # two-launch shape, batch items fit the scratch
    assert _noalloc(lib, B=64, H=16, N=4096) == -4  # several chunks of batch items
    assert _noalloc(lib, N=197) == -4             # one kernel, no scratch
    assert lib.binattn_prepare(_a(256), _a(512), _a(768), 1, 2, 3, 197, 64, _a(1024), _a(1280), _a(1536),
                               _a(1792), _a(2048), _a(2304), None) == -4


def _plan_cover(nheads, nqb, plan):
    """(head, query block) -> how many workgroups of the launch compute it: the launch's
    workgroup-to-work mapping (XCD = workgroup % 8, a contiguous eighth of the heads per XCD,
    first the `a` segments of f blocks of each head, then the `b` segments of r blocks)."""
    a, f, b, r = plan
    grid = 8 * (-(-nheads // 8)) * (a + b)
    cover = {}
    for w in range(grid):
        xcd, slot = w % 8, w // 8
        hx0 = nheads * xcd // 8
        hx = nheads * (xcd + 1) // 8 - hx0
        if slot < hx * a:
            bh, lo, ln = hx0 + slot // a, (slot % a) * f, f
        else:
            s2 = slot - hx * a
            if s2 >= hx * b:
                continue
            bh, lo, ln = hx0 + s2 // b, a * f + (s2 % b) * r, r
        for qb in range(lo, min(nqb, lo + ln)):
            cover[(bh, qb)] = cover.get((bh, qb), 0) + 1
    return cover


@pytest.mark.parametrize("fused", [0, 1])
def test_keep_plan_covers_every_block_once(lib, fused):
    """The head-resident forward's workgroup plan (host logic, no device): for head counts
    below, at and above the XCD count and the model shapes (DeiT-S 384, DiT-XL/2 1024 heads),
    rows of 1..10 query blocks and 2..4 resident workgroups per CU, every (head, block) is
    computed by exactly one workgroup."""
    from diffusion_transformers_amd import binding
    for nheads in (1, 3, 8, 13, 100, 384, 1024):
        for nqb in range(1, 11):
            for slots in (512, 768, 1024):
                plan = binding.keep_plan(nheads, nqb, slots, fused)
                a, f, b, r = plan
                assert a >= 1 and f >= 1 and b >= 0 and r >= 1, plan
                assert a * f + b * r >= nqb, plan
                cover = _plan_cover(nheads, nqb, plan)
                assert len(cover) == nheads * nqb and set(cover.values()) == {1}, (nheads, nqb, slots, plan)


def test_keep_plan_shapes_and_validation(lib):
    """Whole heads where they fill the device; split heads where whole ones would leave most
    resident slots idle; argument checks."""
    from diffusion_transformers_amd import binding
    assert binding.keep_plan(1024, 4, 768, True) == (1, 4, 0, 1)   # DiT-XL/2 one kernel: whole heads
    a, f, b, r = binding.keep_plan(8, 10, 512, False)              # 8 heads of 10 blocks on 512 slots
    assert a + b > 1                                                # split, not one workgroup per head
    out = (ctypes.c_int * 4)()
    assert lib.binattn_keep_plan(0, 4, 512, 0, out) == -1
    assert lib.binattn_keep_plan(8, 0, 512, 0, out) == -1
    assert lib.binattn_keep_plan(8, 4, 0, 0, out) == -1
    assert lib.binattn_keep_plan(8, 4, 512, 0, None) == -1
    assert lib.binattn_keep_plan(8, 11, 512, 0, out) == -2

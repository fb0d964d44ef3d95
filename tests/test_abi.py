"""The C-ABI library loads, exports every symbol include/pkv.h declares, and
rejects bad arguments on the host before launching anything (no GPU needed:
every call here fails validation, or has no work, before any HIP call)."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_fill_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkv.library_path()):
        from paged_kv_cache_fill_amd import _build
        _build.build()
    return pkv.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_operations():
    names = declared_functions()
    for op in ("pkv_fill_slots", "pkv_cache_write_k_fused", "pkv_cache_write_v",
               "pkv_paged_decode_attn"):
        assert op in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_signatures_cover_the_header(lib):
    from paged_kv_cache_fill_amd import _SIGNATURES
    assert sorted(_SIGNATURES) == declared_functions()


def test_binding_argument_counts_match_the_prototypes():
    from paged_kv_cache_fill_amd import _SIGNATURES
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name, (args, _) in _SIGNATURES.items():
        m = re.search(r"\b" + name + r"\s*\(([^)]*)\)", text)
        params = m.group(1).strip()
        n = 0 if params in ("", "void") else params.count(",") + 1
        assert n == len(args), name


def test_version(lib):
    assert re.fullmatch(r"\d+\.\d+\.\d+", lib.pkv_version().decode())


def _err(lib):
    return lib.pkv_last_error().decode()


def test_zero_work_returns_ok_without_pointers(lib):
    assert lib.pkv_fill_slots(None, None, 0, None, None, 0, 0, 16, None) == 0
    assert lib.pkv_cache_write_v(None, 0, 0, None, 0, 8, 128, 16, 1, None, 0, 1.0, None) == 0
    assert lib.pkv_cache_write_k_fused(None, 0, 0, None, 1e-6, None, None, None, 1e4, 0, 128, 0,
                                       None, 0, 8, 128, 16, 1, None, 0, 1.0, None) == 0
    assert lib.pkv_paged_decode_attn(None, 0, 0, None, 0, 1.0, None, 0, 1.0, 0.0, None, 1, None,
                                     0, 1, 8, 8, 128, 128, 16, 0.1, 0, None, 0, 1e4, 0, 0, None,
                                     None, 0, None, 0, None) == 0
    assert _err(lib) == ""


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation


def test_null_pointers_are_invalid(lib):
    assert lib.pkv_fill_slots(None, FAKE, 4, FAKE, FAKE, 1, 10, 16, None) == -1
    assert "non-NULL" in _err(lib)
    assert lib.pkv_cache_write_v(FAKE, 0, 1024, None, 10, 8, 128, 16, 4, FAKE, 0, 1.0,
                                 None) == -1


def test_bad_dtypes_and_shapes(lib):
    def vw(ind, cd, vs=1.0, stride=1024):
        return lib.pkv_cache_write_v(FAKE, ind, stride, FAKE, 10, 8, 128, 16, 4, FAKE, cd, vs,
                                     None)
    assert vw(1, 1) == -2                         # FP8 V input is not a V write input dtype
    assert vw(0, 2) == -2                         # BF16 -> FP32 is not a V store
    assert vw(7, 7) == -1                         # bad enum
    assert vw(0, 1, 0.0) == -1                    # E4M3 store needs a positive finite v_scale
    assert vw(2, 1, float("inf")) == -1
    assert vw(0, 1, 0.5, stride=512) == -1        # token stride smaller than a row
    # head_dim 96 unsupported by the K write
    assert lib.pkv_cache_write_k_fused(FAKE, 0, 768, None, 1e-6, FAKE, None, None, 1e4, 0, 96,
                                       0, FAKE, 10, 8, 96, 16, 4, FAKE, 0, 1.0, None) == -2
    # rotary_dim past the head
    assert lib.pkv_cache_write_k_fused(FAKE, 0, 1024, None, 1e-6, FAKE, None, None, 1e4, 64,
                                       128, 0, FAKE, 10, 8, 128, 16, 4, FAKE, 0, 1.0, None) == -1
    # pos_h without pos_w
    assert lib.pkv_cache_write_k_fused(FAKE, 0, 1024, None, 1e-6, FAKE, FAKE, None, 1e4, 0,
                                       128, 0, FAKE, 10, 8, 128, 16, 4, FAKE, 0, 1.0, None) == -1
    # FP8 store needs a positive finite k_scale that is a normal number (its
    # reciprocal is folded into the row factor); FLT_MIN itself is accepted
    # up to the launch, which this fake pointer set never reaches
    for bad in (0.0, -1.0, float("inf"), float("nan"), 2.0 ** -127, 2.0 ** -149):
        assert lib.pkv_cache_write_k_fused(FAKE, 0, 1024, None, 1e-6, FAKE, None, None, 1e4, 0,
                                           128, 0, FAKE, 10, 8, 128, 16, 4, FAKE, 1, bad,
                                           None) == -1, bad
    # token stride smaller than a row
    assert lib.pkv_cache_write_k_fused(FAKE, 0, 512, None, 1e-6, FAKE, None, None, 1e4, 0,
                                       128, 0, FAKE, 10, 8, 128, 16, 4, FAKE, 0, 1.0, None) == -1


def test_decode_validation(lib):
    def call(**kw):
        a = dict(q=FAKE, qd=0, qs=32 * 128, k=FAKE, kd=0, ks=1.0, v=FAKE, vd=0, vs=1.0, spv=0.0,
                 bt=FAKE, M=4, sl=FAKE, S=2, nb=8, Hq=32, Hkv=8, Dqk=128, Dv=128, B=16, scale=0.1,
                 win=0, sinks=None, qr=0, qt=1e4, qo=0, qdim=0, gate=None, out=FAKE, split=0,
                 ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.pkv_paged_decode_attn(*a.values(), None)
    assert call(Hq=30) == -1                      # Hq % Hkv
    assert call(B=32) == -2                       # block size 16 only
    assert call(kd=2) == -2                       # (BF16, FP32, BF16) not a supported set
    assert call(kd=1, ks=0.0) == -1               # FP8 K needs a scale
    assert call(vd=1, vs=-1.0) == -1              # FP8 V needs a scale
    assert call(vd=2) == -2                       # (BF16, BF16, FP32) not a supported set
    for bad in (-0.1, 1.0, float("nan"), float("inf")):
        assert call(vd=pkv.TQ3, spv=bad) == -1    # sparse-V threshold in [0, 1)
    assert "sparse_v_threshold" in _err(lib)
    assert call(spv=0.01) == -2                   # the sparse-V skip is for TQ V only
    assert call(vd=1, spv=0.01) == -2
    assert "TQ" in _err(lib)
    assert call(Dqk=192, qs=32 * 192) == -2       # BF16 caches need Dqk == Dv
    assert call(qr=1, qdim=64) == -2              # query rotation: FP32 path only
    assert call(M=512, wsb=16) == -3              # workspace too small
    assert "workspace" in _err(lib)
    assert call(qs=100) == -1                     # q stride smaller than a row
    for bad in (0.0, -0.1, float("nan"), float("inf")):
        assert call(scale=bad) == -1              # softmax scale finite and > 0
    assert "scale" in _err(lib)
    # the split index is a grid dimension: at most 65535 splits per sequence
    assert call(M=70000, split=16, wsb=1 << 40) == -2
    assert "splits" in _err(lib)
    # FP32 caches put the sequence in a grid dimension too
    f32 = dict(qd=2, kd=2, vd=2, Hq=8, Hkv=8, qs=8 * 128)
    assert call(S=70000, **f32) == -2
    assert "65535 sequences" in _err(lib)


def test_decode_noalloc_validation(lib):
    """The no-allocation decode rejects, before any device call, what the
    workspace entry point rejects, and a plan whose split partials exceed
    the library's static scratch."""
    def call(**kw):
        a = dict(q=FAKE, qd=0, qs=32 * 128, k=FAKE, kd=0, ks=1.0, v=FAKE, vd=0, vs=1.0, spv=0.0,
                 bt=FAKE, M=4, sl=FAKE, S=2, nb=8, Hq=32, Hkv=8, Dqk=128, Dv=128, B=16, scale=0.1,
                 win=0, sinks=None, qr=0, qt=1e4, qo=0, qdim=0, gate=None, out=FAKE, split=0)
        a.update(kw)
        return lib.pkv_paged_decode_attn_noalloc(*a.values(), None)
    assert call(S=0) == 0                         # no work: nothing launched
    assert call(Hq=30) == -1
    assert call(B=32) == -2
    assert call(scale=float("nan")) == -1
    # 1024 sequences x 64 query heads x 4096-block tables: the balanced plan's
    # partials are far beyond 32 MiB
    need = lib.pkv_decode_workspace_bytes(1024, 64, 8, 128, 4096, 16, 0, 0)
    assert need > pkv.DECODE_SCRATCH_BYTES
    assert call(S=1024, Hq=64, qs=64 * 128, M=4096) == -3
    assert "scratch" in _err(lib)
    # an explicit split size too (FP32 path, 16-token splits of a long table)
    assert lib.pkv_decode_workspace_bytes(64, 64, 64, 128, 65535, 16, 0, 16) > \
        pkv.DECODE_SCRATCH_BYTES
    assert call(S=64, Hq=64, Hkv=64, qs=64 * 128, M=65535, split=16, qd=2, kd=2, vd=2) == -3


def test_decode_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define PKV_DECODE_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == pkv.DECODE_SCRATCH_BYTES


def test_workspace_query(lib):
    assert lib.pkv_decode_workspace_bytes(1, 4, 2, 64, 4, 16, 0, 0) == 0     # one split
    n = lib.pkv_decode_workspace_bytes(256, 32, 8, 128, 512, 16, 0, 0)
    assert n > 0 and n % 16 == 0
    # explicit split size: 1024 tokens = 64 blocks -> 2 splits of a 128-block table
    assert lib.pkv_decode_workspace_bytes(2, 4, 1, 64, 128, 16, 0, 1024) == 2 * 2 * 4 * 66 * 4
    assert lib.pkv_decode_workspace_bytes(2, 4, 1, 64, 64, 16, 0, 1024) == 0
    # a window of W tokens touches at most ceil((W - 1) / 16) + 1 blocks of 16:
    # 64 for W = 1009 (one 64-block split), 65 for W = 1010 (two)
    assert lib.pkv_decode_workspace_bytes(2, 4, 1, 64, 128, 16, 1009, 1024) == 0
    assert lib.pkv_decode_workspace_bytes(2, 4, 1, 64, 128, 16, 1010, 1024) == 2 * 2 * 4 * 66 * 4
    # a window never asks for more than no window
    assert lib.pkv_decode_workspace_bytes(256, 32, 8, 128, 512, 16, 100000, 0) == n
    # balanced plan (automatic split size, no window, <= 1024 sequences): 1024
    # sequences of at most 8 blocks, 4 kv groups -> max(ceil(8192 / 512), 768 / 4)
    # = 192 ranges: partial rows for ranges + sequences, plus the prefix sums;
    # the split plan needs nothing here (one split per sequence), and with a
    # window the split plan is the only one
    assert lib.pkv_decode_workspace_bytes(1024, 32, 8, 128, 8, 16, 0, 0) == \
        (192 + 1024) * 32 * 130 * 4 + 1025 * 4
    assert lib.pkv_decode_workspace_bytes(1024, 32, 8, 128, 8, 16, 64, 0) == 0
    # past 1024 sequences only the split plan
    assert lib.pkv_decode_workspace_bytes(1025, 32, 8, 128, 8, 16, 0, 0) == 0


def test_prefill_and_mla_validation(lib):
    def pre(**kw):
        a = dict(q=FAKE, qd=0, qs=32 * 128, cu=FAKE, mql=8, tq=64, k=FAKE, kd=0, ks=1.0, v=FAKE,
                 vd=0, vs=1.0, bt=FAKE, M=4, sl=FAKE, S=2, nb=8, Hq=32, Hkv=8, Dqk=128, Dv=128,
                 B=16, scale=0.1, win=0, sinks=None, out=FAKE)
        a.update(kw)
        return lib.pkv_paged_prefill_attn(*a.values(), None)
    assert pre(S=0) == 0 and pre(mql=0) == 0       # no work
    assert pre(out=None) == -1
    assert pre(Hq=30) == -1                       # Hq % Hkv
    assert pre(Hq=24) == -2                       # group of 3 does not divide 16
    assert pre(Dqk=192, Dv=192, qs=32 * 192) == -2
    assert pre(qd=2) == -2                        # FP32 q not supported here
    assert pre(kd=1, ks=0.0) == -1
    assert pre(vd=1, vs=float("nan")) == -1
    assert pre(qs=100) == -1
    assert pre(scale=-0.5) == -1 and pre(scale=0.0) == -1
    assert pre(B=32) == -2
    assert _err(lib) != ""

    def mla(**kw):
        a = dict(lat=FAKE, rope_p=FAKE, dt=0, ls=512, rs=64, slots=FAKE, T=4, lora=512, rope=64,
                 dim=576, B=16, nb=4, kc=FAKE, vc=FAKE)
        a.update(kw)
        return lib.pkv_mla_cache_assemble(*a.values(), None)
    assert mla(T=0) == 0
    assert mla(slots=None) == -1
    assert mla(dim=512) == -1                     # kv_lora + rope > cache_dim
    assert mla(ls=500) == -1                      # latent stride below the row
    assert mla(lora=500, ls=500, dim=576) == -2   # 1000 bytes: not a 16-byte multiple
    assert mla(dt=1) == -2                        # E4M3 not an MLA cache dtype here


def test_tq_queries_match_the_oracle(lib):
    import oracle
    for bits in (2, 3, 4):
        got = pkv.tq_codebook(bits)
        assert got == bytes(oracle.tq_codebook(bits))
        for B, H, D in ((16, 8, 128), (16, 1, 16), (32, 3, 64)):
            assert pkv.v_block_bytes(bits + 1, B, H, D) == oracle.tq_block_bytes(bits, B, H, D)
    assert pkv.v_block_bytes(pkv.TQ3, 16, 8, 128) == 16 * 8 * 128 * 3 // 8 + 16 * 8 * 8
    assert pkv.v_block_bytes(pkv.TQ2, 16, 8, 120) == 0          # head_dim % 16
    assert pkv.v_block_bytes(pkv.BF16, 16, 8, 128) == 16 * 8 * 128 * 2
    assert pkv.v_block_bytes(9, 16, 8, 128) == 0
    buf = (ctypes.c_uint8 * 8)()
    assert lib.pkv_tq_codebook(pkv.FP8_E4M3, buf) == -1
    assert lib.pkv_tq_codebook(pkv.TQ2, None) == -1


def test_tq_validation(lib):
    def vw(ind=0, cd=pkv.TQ3, H=8, D=128, B=16, stride=1024):
        return lib.pkv_cache_write_v(FAKE, ind, stride, FAKE, 10, H, D, B, 4, FAKE, cd, 1.0,
                                     None)
    assert vw(D=120, stride=960) == -2            # head_dim % 16
    assert vw(H=1, D=16, B=3, stride=16) == -2    # blocks would break the stores' alignment
    assert vw(ind=1) == -2                        # E4M3 input
    assert vw(stride=512) == -1                   # token stride smaller than a row

    def dec(**kw):
        a = dict(q=FAKE, qd=0, qs=32 * 128, k=FAKE, kd=0, ks=1.0, v=FAKE, vd=pkv.TQ3, vs=1.0,
                 spv=0.0, bt=FAKE, M=4, sl=FAKE, S=2, nb=8, Hq=32, Hkv=8, Dqk=128, Dv=128, B=16, scale=0.1,
                 win=0, sinks=None, qr=0, qt=1e4, qo=0, qdim=0, gate=None, out=FAKE, split=0,
                 ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.pkv_paged_decode_attn(*a.values(), None)
    assert dec(Dqk=64, Dv=64, qs=32 * 64) == -2   # TQ V decode: head dim 128 only
    assert dec(qd=2, kd=2) == -2                  # FP32 q/K with TQ V
    assert dec(Dqk=64, Dv=64, qs=32 * 64, spv=0.01) == -2
    assert dec(spv=1.5) == -1
    pre = lib.pkv_paged_prefill_attn(FAKE, 0, 32 * 128, FAKE, 8, 64, FAKE, 0, 1.0, FAKE, pkv.TQ3,
                                     1.0, FAKE, 4, FAKE, 2, 8, 32, 8, 128, 128, 16, 0.1, 0, None,
                                     FAKE, None)
    assert pre in (-1, -2) and _err(lib) != ""    # prefill reads BF16 / E4M3 V only

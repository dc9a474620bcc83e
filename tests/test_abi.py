"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch.

Every rejection case below fails host validation, so no kernel is ever
enqueued; the tests still refuse to run where a GPU is visible, so that a
mistake in a case can never send a fake pointer to a device.
"""
import ctypes
import os
import re

import pytest
import torch

from block_sparse_attention_sparge_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparge.h")

pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="host-only rejection tests (no device pointers)")

FAKE = 0x10000          # 16-byte aligned address that validation must never hand to a kernel


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        from block_sparse_attention_sparge_amd import build
        build.build(verbose=False)
    return ops.load_library()


def test_library_exports_every_declared_function(lib):
    names = header_functions()
    assert set(names) == set(ops.EXPORTED_SYMBOLS), names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version(lib):
    assert lib.sparge_abi_version() == ops.ABI_VERSION == 7


def _s3(a, b, c):
    return ops._I64x3(a, b, c)


def _arr(vals):
    return (ctypes.c_float * len(vals))(*vals)


def _err(lib):
    return lib.sparge_last_error().decode()


def test_workspace_size(lib):
    n = lib.sparge_build_block_map_workspace(2, 32, 16384, 16384, 128, 64, 64)
    # q_mean + k_mean (fp32) + Q gate flags (u8) + K block similarities (fp32)
    # + K-mean partials (16 chunks of 1024 rows per head, fp32), each rounded
    # up to 256 bytes; sized for as many K heads as Q heads
    assert n == (2 * (2 * 32 * 256 * 128 * 4) + 2 * 32 * 256 + 2 * 32 * 256 * 4
                 + 2 * 32 * 16 * 128 * 4)
    # A length that is not a multiple of 64 counts its partial last block.
    assert (lib.sparge_build_block_map_workspace(1, 1, 100, 65, 64, 64, 64)
            == lib.sparge_build_block_map_workspace(1, 1, 128, 128, 64, 64, 64) > 0)
    assert lib.sparge_build_block_map_workspace(1, 1, 64, 64, 96, 64, 64) == 0


def _bm(lib, **kw):
    args = dict(q=FAKE, k=FAKE, dt=ops.SPARGE_F16, b=1, h=2, hkv=2, s_q=512, s_k=512, d=64,
                qs=_s3(65536, 32768, 64), ks=_s3(65536, 32768, 64), blk_q=64, blk_k=64,
                topk=_arr([0.5, 0.5]), cdf=None, sim=_arr([0.001, 0.001]), scale=0.0, flags=0,
                lut=FAKE, cnt=FAKE, q8=None, q8s=None, k8=None, k8s=None, ws=FAKE, ws_bytes=1 << 20)
    args.update(kw)
    return lib.sparge_build_block_map(
        args["q"], args["k"], args["dt"], args["b"], args["h"], args["hkv"], args["s_q"], args["s_k"], args["d"],
        args["qs"], args["ks"], args["blk_q"], args["blk_k"], args["topk"], args["cdf"], args["sim"],
        args["scale"], args["flags"], args["lut"], args["cnt"], None, None, None, None, None, None,
        args["q8"], args["q8s"], args["k8"], args["k8s"], args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ops.SPARGE_ERR_INVALID),
    (dict(lut=None), ops.SPARGE_ERR_INVALID),
    (dict(dt=ops.SPARGE_F32), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(d=96), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(flags=ops.SPARGE_FLAG_CAUSAL, s_q=500, s_k=520), ops.SPARGE_ERR_UNSUPPORTED),   # ragged, causal, unequal
    (dict(blk_q=128), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(h=0), ops.SPARGE_ERR_INVALID),
    (dict(b=0), ops.SPARGE_ERR_INVALID),                             # empty batch
    (dict(hkv=0), ops.SPARGE_ERR_INVALID),
    (dict(h=3, hkv=2, topk=_arr([0.5] * 3), sim=_arr([0.0] * 3)), ops.SPARGE_ERR_INVALID),   # 3 not a multiple of 2
    (dict(s_q=0), ops.SPARGE_ERR_INVALID),                           # empty sequence
    (dict(s_k=0), ops.SPARGE_ERR_INVALID),
    (dict(h=200), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(s_k=64 * 1025), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(s_k=64 * 1024 + 1), ops.SPARGE_ERR_UNSUPPORTED),           # 1025 blocks, the last partial
    (dict(qs=_s3(65536, 32768, 60)), ops.SPARGE_ERR_INVALID),
    (dict(topk=_arr([1.5, 0.5])), ops.SPARGE_ERR_INVALID),
    (dict(topk=_arr([float("nan"), 0.5])), ops.SPARGE_ERR_INVALID),
    (dict(topk=_arr([0.0, 0.5])), ops.SPARGE_ERR_INVALID),          # cdf mode without cdfthreshd
    (dict(topk=_arr([0.0, 0.5]), cdf=_arr([1.5, 0.5])), ops.SPARGE_ERR_INVALID),
    (dict(sim=_arr([float("inf"), 0.0])), ops.SPARGE_ERR_INVALID),
    (dict(ws_bytes=16), ops.SPARGE_ERR_INVALID),
    (dict(ws=FAKE + 16), ops.SPARGE_ERR_INVALID),
    (dict(q=FAKE + 2), ops.SPARGE_ERR_INVALID),
    (dict(scale=-1.0), ops.SPARGE_ERR_INVALID),
    (dict(flags=8), ops.SPARGE_ERR_INVALID),                         # unknown flag bit
    (dict(flags=ops.SPARGE_FLAG_CAUSAL, s_k=1024), ops.SPARGE_ERR_UNSUPPORTED),   # causal, s_q != s_k
    (dict(q8=FAKE), ops.SPARGE_ERR_INVALID),                                      # int8 outputs: all or none
    (dict(q8=FAKE, q8s=FAKE, k8=FAKE), ops.SPARGE_ERR_INVALID),
    (dict(q8=FAKE + 8, q8s=FAKE, k8=FAKE, k8s=FAKE), ops.SPARGE_ERR_INVALID),     # misaligned codes
    (dict(flags=ops.SPARGE_FLAG_QUANT_FP8), ops.SPARGE_ERR_INVALID),              # fp8 codes need the outputs
])
def test_block_map_rejections(lib, kw, status):
    st = _bm(lib, **kw)
    assert st == status, _err(lib)
    assert _err(lib) != ""


def _bm_noalloc(lib, **kw):
    args = dict(q=FAKE, k=FAKE, dt=ops.SPARGE_F16, b=1, h=2, hkv=2, s_q=512, s_k=512, d=64,
                qs=_s3(65536, 32768, 64), ks=_s3(65536, 32768, 64), blk_q=64, blk_k=64,
                topk=_arr([0.5, 0.5]), cdf=None, sim=_arr([0.001, 0.001]), scale=0.0, flags=0,
                lut=FAKE, cnt=FAKE)
    args.update(kw)
    h = args["h"]
    return lib.sparge_build_block_map_noalloc(
        args["q"], args["k"], args["dt"], args["b"], h, args["hkv"], args["s_q"], args["s_k"], args["d"],
        args["qs"], args["ks"], args["blk_q"], args["blk_k"], args["topk"], args["cdf"], args["sim"],
        args["scale"], args["flags"], args["lut"], args["cnt"], None, None, None, None, None, None,
        None, None, None, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ops.SPARGE_ERR_INVALID),
    (dict(d=96), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(b=0), ops.SPARGE_ERR_INVALID),
    (dict(topk=_arr([1.5, 0.5])), ops.SPARGE_ERR_INVALID),
    (dict(flags=8), ops.SPARGE_ERR_INVALID),
    # b4 h32 s16384 d128 needs about 34 MiB of scratch, beyond the 32 MiB held
    (dict(b=4, h=32, hkv=32, s_q=16384, s_k=16384, d=128, qs=_s3(32 << 21, 1 << 21, 128),
          ks=_s3(32 << 21, 1 << 21, 128), topk=_arr([0.4] * 32), sim=_arr([0.001] * 32)),
     ops.SPARGE_ERR_UNSUPPORTED),
])
def test_block_map_noalloc_rejections(lib, kw, status):
    # Host validation runs in full before the scratch array is looked up, so
    # none of these reaches the device.
    assert _bm_noalloc(lib, **kw) == status, _err(lib)
    assert _err(lib) != ""


def test_noalloc_scratch_fits_the_headline_block_map(lib):
    need = lib.sparge_build_block_map_workspace(2, 32, 16384, 16384, 128, 64, 64)
    assert need <= ops.NOALLOC_SCRATCH_BYTES < lib.sparge_build_block_map_workspace(4, 32, 16384, 16384, 128, 64, 64)


def _fmha(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dt=ops.SPARGE_BF16, odt=ops.SPARGE_BF16,
             b=1, hq=8, hkv=2, sq=512, sk=512, d=128, qs=_s3(8 * 512 * 128, 512 * 128, 128),
             ks=_s3(2 * 512 * 128, 512 * 128, 128), vs=_s3(2 * 512 * 128, 512 * 128, 128),
             os=_s3(8 * 512 * 128, 512 * 128, 128), bq=64, bk=64, lut=FAKE, cnt=FAKE, L=8,
             lh=8, scale=0.0, flags=0, pv=0.0, splits=1, sst=0)
    a.update(kw)
    return lib.sparse_fmha_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dt"], a["odt"], a["b"],
                               a["hq"], a["hkv"], a["sq"], a["sk"], a["d"], a["qs"], a["ks"], a["vs"],
                               a["os"], a["bq"], a["bk"], a["lut"], a["cnt"], a["L"], a["lh"],
                               a["scale"], a["flags"], a["pv"], a["splits"], a["sst"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ops.SPARGE_ERR_INVALID),
    (dict(o=None), ops.SPARGE_ERR_INVALID),
    (dict(hkv=3), ops.SPARGE_ERR_INVALID),
    (dict(d=80), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(dt=ops.SPARGE_F32), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(odt=ops.SPARGE_F16), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(flags=ops.SPARGE_FLAG_CAUSAL, sq=500, sk=520), ops.SPARGE_ERR_UNSUPPORTED),   # ragged, causal, unequal
    (dict(bq=128, bk=128), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(bq=64, bk=1), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(lh=4), ops.SPARGE_ERR_INVALID),
    (dict(L=0), ops.SPARGE_ERR_INVALID),
    (dict(b=0), ops.SPARGE_ERR_INVALID),                             # empty inputs
    (dict(sq=0), ops.SPARGE_ERR_INVALID),
    (dict(sk=0), ops.SPARGE_ERR_INVALID),
    (dict(splits=0), ops.SPARGE_ERR_INVALID),
    (dict(splits=2, lse=None), ops.SPARGE_ERR_INVALID),
    (dict(splits=2, sst=12), ops.SPARGE_ERR_INVALID),
    (dict(ks=_s3(2 * 512 * 128, 512 * 128, 130)), ops.SPARGE_ERR_INVALID),
    (dict(vs=_s3(-8, 512 * 128, 128)), ops.SPARGE_ERR_INVALID),
    (dict(k=FAKE + 8), ops.SPARGE_ERR_INVALID),
    (dict(lut=None, cnt=FAKE), ops.SPARGE_ERR_INVALID),
    (dict(scale=float("nan")), ops.SPARGE_ERR_INVALID),
    (dict(vs=_s3(2 * 512 * 128, 512 * 128, 1 << 24)), ops.SPARGE_ERR_UNSUPPORTED),   # 64 rows span 2^31 bytes
    (dict(qs=_s3(8 * 512 * 128, 512 * 128, 1 << 24)), ops.SPARGE_ERR_UNSUPPORTED),   # 64 Q rows likewise
    (dict(flags=ops.SPARGE_FLAG_SMOOTH_K), ops.SPARGE_ERR_INVALID),                  # block-map flag only
    (dict(flags=ops.SPARGE_FLAG_CAUSAL, sk=1024), ops.SPARGE_ERR_UNSUPPORTED),       # causal, s_q != s_k
    (dict(flags=ops.SPARGE_FLAG_CAUSAL, bq=1, bk=1, cnt=None, lh=2), ops.SPARGE_ERR_INVALID),   # token mode
    (dict(pv=-1.0), ops.SPARGE_ERR_INVALID),
    (dict(pv=float("inf")), ops.SPARGE_ERR_INVALID),
    (dict(pv=float("nan")), ops.SPARGE_ERR_INVALID),
    (dict(pv=4.0, bq=1, bk=1, cnt=None, lh=2), ops.SPARGE_ERR_UNSUPPORTED),   # token mode
    (dict(pv=4.0, splits=2, sst=8 * 512 * 128), ops.SPARGE_ERR_UNSUPPORTED),   # one pass per row
    # token-list mode
    (dict(bq=1, bk=1, lut=None, cnt=None), ops.SPARGE_ERR_INVALID),
    (dict(bq=1, bk=1, cnt=FAKE, lh=2), ops.SPARGE_ERR_INVALID),
    (dict(bq=1, bk=1, cnt=None, lh=8), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(bq=1, bk=1, cnt=None, lh=2, sq=16385), ops.SPARGE_ERR_UNSUPPORTED),   # 65540 rows per KV head (limit 65536)
    # a (b, KV head) slice of 2^20 rows of 1024-element stride spans 2^31 bytes
    (dict(bq=1, bk=1, cnt=None, lh=2, sk=1 << 20, ks=_s3(1 << 31, 1 << 30, 1024)), ops.SPARGE_ERR_UNSUPPORTED),
])
def test_fmha_rejections(lib, kw, status):
    st = _fmha(lib, **kw)
    assert st == status, _err(lib)


def _fmha8(lib, entry="sparse_fmha_fwd_qk_int8", **kw):
    a = dict(q=FAKE, qsc=FAKE, k=FAKE, ksc=FAKE, v=FAKE, o=FAKE, lse=FAKE, vdt=ops.SPARGE_BF16,
             odt=ops.SPARGE_BF16, b=1, hq=8, hkv=2, sq=512, sk=512, d=128,
             qs=_s3(8 * 512 * 128, 512 * 128, 128), ks=_s3(2 * 512 * 128, 512 * 128, 128),
             vs=_s3(2 * 512 * 128, 512 * 128, 128), os=_s3(8 * 512 * 128, 512 * 128, 128),
             lut=FAKE, cnt=FAKE, L=8, lh=8, scale=0.0, flags=0, splits=1, sst=0)
    a.update(kw)
    return getattr(lib, entry)(a["q"], a["qsc"], a["k"], a["ksc"], a["v"], a["o"], a["lse"],
                                       a["vdt"], a["odt"], a["b"], a["hq"], a["hkv"], a["sq"], a["sk"],
                                       a["d"], a["qs"], a["ks"], a["vs"], a["os"], a["lut"], a["cnt"],
                                       a["L"], a["lh"], a["scale"], a["flags"], a["splits"], a["sst"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(qsc=None), ops.SPARGE_ERR_INVALID),
    (dict(b=0), ops.SPARGE_ERR_INVALID),
    (dict(sq=0), ops.SPARGE_ERR_INVALID),
    (dict(ksc=None), ops.SPARGE_ERR_INVALID),
    (dict(v=None), ops.SPARGE_ERR_INVALID),
    (dict(vdt=ops.SPARGE_F32), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(odt=ops.SPARGE_F16), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(d=96), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(flags=ops.SPARGE_FLAG_CAUSAL, sq=500, sk=520), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(hkv=3), ops.SPARGE_ERR_INVALID),
    (dict(qs=_s3(8 * 512 * 128, 512 * 136, 136)), ops.SPARGE_ERR_INVALID),       # 136 B rows: not 16-aligned steps
    (dict(k=FAKE + 4), ops.SPARGE_ERR_INVALID),
    (dict(flags=ops.SPARGE_FLAG_ATTN_SINK), ops.SPARGE_ERR_INVALID),
    (dict(flags=ops.SPARGE_FLAG_CAUSAL, sk=1024), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(splits=2, lse=None), ops.SPARGE_ERR_INVALID),
    (dict(lut=None, cnt=FAKE), ops.SPARGE_ERR_INVALID),
    (dict(lh=4), ops.SPARGE_ERR_INVALID),
    (dict(vs=_s3(2 * 512 * 128, 512 * 128, 1 << 24)), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(qs=_s3(8 * 512 * 128, 512 * 128, 1 << 25)), ops.SPARGE_ERR_UNSUPPORTED),   # 64 Q code rows span 2^31 bytes
])
@pytest.mark.parametrize("entry", ["sparse_fmha_fwd_qk_int8", "sparse_fmha_fwd_qk_fp8"])
def test_fmha_qk_int8_rejections(lib, kw, status, entry):
    st = _fmha8(lib, entry=entry, **kw)
    assert st == status, _err(lib)


@pytest.mark.parametrize("kw,status", [
    (dict(parts=None), ops.SPARGE_ERR_INVALID),
    (dict(n=0), ops.SPARGE_ERR_INVALID),
    (dict(b=0), ops.SPARGE_ERR_INVALID),
    (dict(s=0), ops.SPARGE_ERR_INVALID),
    (dict(n=1025), ops.SPARGE_ERR_INVALID),
    (dict(d=32), ops.SPARGE_ERR_UNSUPPORTED),
    (dict(stride=100), ops.SPARGE_ERR_INVALID),
    (dict(pdt=7), ops.SPARGE_ERR_INVALID),
    (dict(o=FAKE + 4), ops.SPARGE_ERR_INVALID),
])
def test_combine_rejections(lib, kw, status):
    a = dict(parts=FAKE, pdt=ops.SPARGE_F32, lse=FAKE, n=2, b=1, h=2, s=16, d=64,
             stride=2 * 16 * 64, o=FAKE, odt=ops.SPARGE_F32, lse_out=FAKE)
    a.update(kw)
    st = lib.attn_combine(a["parts"], a["pdt"], a["lse"], a["n"], a["b"], a["h"], a["s"], a["d"],
                          a["stride"], a["o"], a["odt"], a["lse_out"], None)
    assert st == status, _err(lib)


def test_validate_lut_rejections(lib):
    assert lib.sparge_validate_lut(None, None, 4, 4, 4, FAKE, None) == ops.SPARGE_ERR_INVALID
    assert lib.sparge_validate_lut(FAKE, None, 0, 4, 4, FAKE, None) == ops.SPARGE_ERR_INVALID


def test_error_message_is_per_call(lib):
    assert _bm(lib, d=96) == ops.SPARGE_ERR_UNSUPPORTED
    assert "head dim" in _err(lib)


def test_python_binding_rejects_cpu_tensors(lib):
    q = torch.zeros(1, 1, 64, 64, dtype=torch.float16)
    with pytest.raises(ops.SpargeError):
        ops.sparse_fmha_fwd(q, q, q)
    with pytest.raises(ops.SpargeError):
        ops.build_block_map(q, q, [0.5], [0.001])


def _meta(*shape, dtype=torch.float16):
    return torch.empty(shape, dtype=dtype, device="meta")


@pytest.mark.parametrize("case", [
    dict(k=_meta(2, 2, 256, 64)),                       # k batch differs from q
    dict(k=_meta(1, 2, 256, 128), v=_meta(1, 2, 256, 128)),   # k head dim differs
    dict(v=_meta(1, 2, 200, 64)),                       # v shorter than k
    dict(v=_meta(1, 4, 256, 64)),                       # v heads differ from k
    dict(v=_meta(1, 2, 256, 128)),                      # v head dim differs
    dict(o=_meta(1, 4, 128, 64)),                       # o too short
    dict(o=_meta(1, 4, 256, 64), splits=2),             # split partials need [S, ...]
    dict(o=_meta(3, 1, 4, 256, 64), splits=2),          # wrong split count
    dict(lse=_meta(1, 4, 255, dtype=torch.float32)),    # lse too short
    dict(lse=_meta(1, 4, 256, dtype=torch.float16)),    # lse not fp32
    dict(lse=_meta(1, 4, 256, dtype=torch.float32), splits=2),
    dict(lse=_meta(256, 4, dtype=torch.float32).t()[None]),   # not contiguous
])
def test_binding_rejects_mismatched_attention_shapes(case):
    # q [1, 4, 256, 64]; k, v [1, 2, 256, 64].  The C ABI takes one b, s_k and
    # d for all tensors, so the binding must refuse anything else before a
    # launch could read or write past a buffer.
    a = dict(k=_meta(1, 2, 256, 64), v=_meta(1, 2, 256, 64), o=None, lse=None, splits=1)
    a.update(case)
    with pytest.raises(ops.SpargeError):
        ops._check_attn_shapes(_meta(1, 4, 256, 64), a["k"], a["v"], a["o"], a["lse"], a["splits"])


def test_binding_accepts_matching_attention_shapes():
    q, k = _meta(1, 4, 256, 64), _meta(1, 2, 256, 64)
    ops._check_attn_shapes(q, k, k, _meta(1, 4, 256, 64), _meta(1, 4, 256, dtype=torch.float32), 1)
    ops._check_attn_shapes(q, k, k, _meta(3, 1, 4, 256, 64, dtype=torch.float32),
                           _meta(3, 1, 4, 256, dtype=torch.float32), 3)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ops.SpargeError):
        ops.load_library(str(tmp_path / "nope.so"))

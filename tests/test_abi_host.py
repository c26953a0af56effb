"""Host-only tests of the C ABI: the library loads, exports every declared entry
point, and rejects bad arguments before touching the GPU.  No compute calls."""
import ctypes
import os
import re

import pytest

from compressed_attention_long_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")

FAKE = 0x10000          # an aligned, never-dereferenced stand-in for a device pointer


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(csa_[a-z_0-9]+|hca_[a-z_0-9]+)\s*\(", src, flags=re.M)


def test_library_exports_every_declared_symbol():
    lib = L.load()
    names = declared_functions()
    assert set(names) == set(L.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.csa_abi_version() == 1


def cache(dtype=L.CSA_BF16, cap=64, C=512, window=8, stride=4, scales=True, sb=64):
    quant = dtype in (L.CSA_FP8_E4M3, L.CSA_FP4_E2M1)
    return L.CCache(FAKE, FAKE if (quant and scales) else None, FAKE, FAKE, dtype, cap, C, sb, window, stride)


def rc_msg(rc):
    return rc, L.last_error()


def compress(out, kv=FAKE, logits=FAKE, ld_tok=512, ld_seq=512 * 64, B=1, T=64, first=0, n_new=4,
             inv=FAKE, rope=64):
    lib = L.load()
    return rc_msg(lib.csa_compress(kv, logits, ld_tok, ld_seq, B, T, first, n_new, ctypes.byref(out), inv, rope, None))


def test_compress_validation():
    c = cache()
    assert compress(c, kv=None)[0] == L.CSA_EINVAL
    rc, msg = compress(c, logits=None)
    assert rc == L.CSA_EINVAL and "logits" in msg
    assert compress(c, T=15, n_new=4)[0] == L.CSA_EINVAL          # needs (4-1)*4 + 8 = 20 rows
    assert compress(c, first=62, n_new=4)[0] == L.CSA_EINVAL      # past cap
    assert compress(c, rope=63)[0] == L.CSA_EINVAL
    assert compress(c, inv=None)[0] == L.CSA_EINVAL
    assert compress(c, kv=FAKE + 4)[0] == L.CSA_EINVAL            # misaligned
    assert compress(cache(C=520))[0] == L.CSA_ENOTSUP
    assert compress(cache(dtype=7))[0] == L.CSA_ENOTSUP
    assert compress(cache(dtype=L.CSA_FP8_E4M3, scales=False))[0] == L.CSA_EINVAL
    assert compress(cache(dtype=L.CSA_FP8_E4M3, sb=24))[0] == L.CSA_EINVAL   # does not divide C
    assert compress(cache(dtype=L.CSA_FP8_E4M3, sb=1024, C=1024), ld_tok=1024, ld_seq=1024 * 64)[0] == L.CSA_ENOTSUP
    # fp4 (MXFP4) caches: scales required, 32-channel blocks only
    assert compress(cache(dtype=L.CSA_FP4_E2M1, scales=False, sb=32))[0] == L.CSA_EINVAL
    rc, msg = compress(cache(dtype=L.CSA_FP4_E2M1, sb=64))
    assert rc == L.CSA_EINVAL and "32" in msg
    assert compress(cache(dtype=L.CSA_FP4_E2M1, sb=32), n_new=0) == (L.CSA_OK, "")
    # nothing to do is a success with no launch
    rc, msg = compress(c, n_new=0)
    assert rc == L.CSA_OK and msg == ""


def test_compress_batch_validation():
    lib = L.load()
    c = cache()
    empty = L.CCompressCall(FAKE, FAKE, 512, 512 * 64, 1, 64, 0, 0, ctypes.pointer(c), FAKE, 64)
    bad = L.CCompressCall(None, FAKE, 512, 512 * 64, 1, 64, 0, 4, ctypes.pointer(c), FAKE, 64)
    arr = (L.CCompressCall * 2)(empty, bad)
    rc, msg = rc_msg(lib.csa_compress_batch(arr, 2, None))
    assert rc == L.CSA_EINVAL and msg.startswith("call 1:") and "kv" in msg
    assert rc_msg(lib.csa_compress_batch(arr, 1, None)) == (L.CSA_OK, "")   # only empty calls: no launch
    assert lib.csa_compress_batch(None, 0, None) == L.CSA_OK
    assert lib.csa_compress_batch(None, 1, None) == L.CSA_EINVAL
    assert lib.csa_compress_batch(arr, -1, None) == L.CSA_EINVAL


def index(keys, topk=16, B=1, Tq=1, Hi=64, ws=None, wsb=0, scores=None, q=FAKE):
    lib = L.load()
    return rc_msg(lib.csa_index_topk(q, FAKE, FAKE, B, Tq, Hi, ctypes.byref(keys), topk, FAKE, scores, ws, wsb, None))


def test_index_topk_validation():
    k = cache(C=128)
    assert index(k, topk=65)[0] == L.CSA_EINVAL                    # topk > cap
    assert index(k, topk=0)[0] == L.CSA_EINVAL
    assert index(cache(C=128, cap=10000), topk=4097)[0] == L.CSA_EINVAL     # topk above 4,096
    assert index(k, Hi=65)[0] == L.CSA_ENOTSUP
    assert index(cache(C=256))[0] == L.CSA_ENOTSUP
    assert index(cache(C=128, dtype=L.CSA_FP8_E4M3, sb=64))[0] == L.CSA_ENOTSUP
    rc, msg = index(cache(C=128, dtype=L.CSA_FP4_E2M1, sb=32))
    assert rc == L.CSA_ENOTSUP and "fp4" in msg
    need = L.index_topk_workspace_bytes(1, 1, 64, 64, 16)
    assert need >= 64 * 4
    rc, msg = index(k, ws=FAKE, wsb=need - 1)
    assert rc == L.CSA_EWORKSPACE and str(need) in msg
    assert index(k, ws=FAKE + 16, wsb=need)[0] == L.CSA_EINVAL     # misaligned workspace
    assert index(k, q=None)[0] == L.CSA_EINVAL
    assert index(k, B=0)[0] == L.CSA_OK
    # rows longer than 16384 entries select in two stages, whose candidates need a workspace
    # even when the scores go to scores_out
    long_keys = cache(C=128, cap=100000)
    assert index(long_keys, topk=1024, scores=FAKE)[0] == L.CSA_EWORKSPACE
    # (a row that fits one block passes validation; without a GPU the launch itself then fails)
    assert index(cache(C=128, cap=16384), topk=1024, scores=FAKE)[0] not in (L.CSA_EWORKSPACE, L.CSA_EINVAL,
                                                                              L.CSA_ENOTSUP)


def test_index_topk_compress_validation():
    lib = L.load()
    keys = cache(C=128)
    out = cache()
    ok_call = L.CCompressCall(FAKE, FAKE, 512, 512 * 64, 1, 64, 0, 4, ctypes.pointer(out), FAKE, 64)
    bad_call = L.CCompressCall(None, FAKE, 512, 512 * 64, 1, 64, 0, 4, ctypes.pointer(out), FAKE, 64)

    def run(calls, n, B=1, keys_=keys):
        arr = (L.CCompressCall * max(len(calls), 1))(*calls)
        return rc_msg(lib.csa_index_topk_compress(arr, n, FAKE, FAKE, FAKE, B, 1, 64, ctypes.byref(keys_), 16,
                                                  FAKE, FAKE, None, 0, None))

    rc, msg = run([ok_call, bad_call], 2)
    assert rc == L.CSA_EINVAL and msg.startswith("call 1:")
    assert run([ok_call], 1, keys_=cache(C=256))[0] == L.CSA_ENOTSUP          # the indexer's own checks
    # a compress output that is the key cache itself (same device address) is refused
    alias = cache()
    alias.data = keys.data
    alias_call = L.CCompressCall(FAKE, FAKE, 512, 512 * 64, 1, 64, 0, 4, ctypes.pointer(alias), FAKE, 64)
    rc, msg = run([alias_call], 1)
    assert rc == L.CSA_EINVAL and "overlaps" in msg
    assert lib.csa_index_topk_compress(None, 0, FAKE, FAKE, FAKE, 0, 1, 64, ctypes.byref(keys), 16, FAKE, FAKE,
                                       None, 0, None) == L.CSA_OK              # nothing to do: no launch
    assert lib.csa_index_topk_compress(None, 1, FAKE, FAKE, FAKE, 0, 1, 64, ctypes.byref(keys), 16, FAKE, FAKE,
                                       None, 0, None) == L.CSA_EINVAL


def attend(kv, win, topk=16, H=128, W=128, ws=None, wsb=0, out_dtype=L.CSA_FP32, rope=64, hca=False, B=32):
    lib = L.load()
    if hca:
        return rc_msg(lib.hca_attend(FAKE, FAKE, B, 1, H, ctypes.byref(kv), ctypes.byref(win), W, FAKE, FAKE, rope,
                                     0.04, FAKE, out_dtype, None, ws, wsb, None))
    return rc_msg(lib.csa_attend(FAKE, FAKE, B, 1, H, ctypes.byref(kv), FAKE, topk, ctypes.byref(win), W, FAKE,
                                 FAKE, rope, 0.04, FAKE, out_dtype, None, ws, wsb, None))


def test_attend_validation():
    kv = cache(cap=2048)
    win = cache(cap=160, window=1, stride=1)
    assert attend(kv, win, topk=4096)[0] == L.CSA_EINVAL
    assert attend(kv, cache(cap=160, window=2, stride=1))[0] == L.CSA_EINVAL
    assert attend(cache(cap=2048, C=256), win)[0] == L.CSA_ENOTSUP
    assert attend(kv, win, out_dtype=9)[0] == L.CSA_ENOTSUP
    assert attend(kv, win, W=-1)[0] == L.CSA_EINVAL
    need = L.csa_attend_workspace_bytes(32, 1, 128, 16, 128)
    assert need > 0                                               # 32 rows cannot fill the GPU: split
    assert attend(kv, win, ws=FAKE, wsb=need - 1)[0] == L.CSA_EWORKSPACE
    assert attend(kv, win, ws=None, wsb=0)[0] == L.CSA_EWORKSPACE
    hneed = L.hca_attend_workspace_bytes(32, 1, 128, 2048, 128)
    assert attend(kv, win, hca=True, ws=FAKE, wsb=hneed - 256)[0] == L.CSA_EWORKSPACE
    assert attend(kv, win, B=0)[0] == L.CSA_OK
    fp4 = cache(cap=2048, dtype=L.CSA_FP4_E2M1, sb=32)
    assert attend(fp4, win, B=0)[0] == L.CSA_OK                   # fp4 entries are accepted
    assert attend(cache(cap=2048, dtype=L.CSA_FP4_E2M1, sb=32, scales=False), win)[0] == L.CSA_EINVAL
    assert attend(kv, cache(cap=160, window=1, stride=1, dtype=L.CSA_FP4_E2M1, sb=32))[0] == L.CSA_ENOTSUP
    # fp8 entries: scales per 64 channels (or a multiple); finer blocks are not supported
    rc, msg = attend(cache(cap=2048, dtype=L.CSA_FP8_E4M3, sb=32), win, ws=FAKE, wsb=1 << 40)
    assert rc == L.CSA_ENOTSUP and "scale_block" in msg
    assert attend(cache(cap=2048, dtype=L.CSA_FP8_E4M3, sb=64), win, ws=FAKE, wsb=1 << 40)[0] not in (
        L.CSA_ENOTSUP, L.CSA_EINVAL, L.CSA_EWORKSPACE)


def test_attend_noalloc_rejects_calls_beyond_its_scratch():
    # an fp4 cache with a 20,000-entry selection over 64 query rows needs far more than the
    # library's scratch: refused on the host, before anything touches a GPU
    lib = L.load()
    kv = cache(cap=30000, dtype=L.CSA_FP4_E2M1, sb=32)
    win = cache(cap=160, window=1, stride=1)
    assert L.csa_attend_workspace_bytes(64, 1, 128, 20000, 128) > L.CSA_NOALLOC_SCRATCH_BYTES
    rc = lib.csa_attend_noalloc(FAKE, FAKE, 64, 1, 128, ctypes.byref(kv), FAKE, 20000, ctypes.byref(win), 128,
                                FAKE, FAKE, 64, 0.04, FAKE, L.CSA_FP32, None, None)
    assert rc == L.CSA_EWORKSPACE and "scratch" in L.last_error()


def test_workspace_sizes_scale_with_work():
    assert L.csa_attend_workspace_bytes(4096, 1, 128, 1024, 128) == 0   # enough rows: no split partials
    a = L.hca_attend_workspace_bytes(16, 1, 128, 8192, 128)
    b = L.hca_attend_workspace_bytes(16, 1, 128, 4096, 128)
    assert a > 0 and b > 0
    assert L.index_topk_workspace_bytes(32, 1, 64, 16383, 1024) >= 32 * 16383 * 4
    # scores plus the stage-1 candidates of 16 chunks of 16,384 entries (key + index each)
    assert L.index_topk_workspace_bytes(4, 1, 64, 262143, 1024) >= 4 * 262143 * 4 + 4 * 16 * 1024 * 8


def test_rotary_tables_agree_with_the_oracle():
    """Host logic: the tables handed to the kernels equal the oracle's own, written separately."""
    import numpy as np
    from compressed_attention_long_amd import rope
    from oracle import csa_oracle as O
    np.testing.assert_allclose(rope.rope_inv_freq(160000.0, 64, "cpu").numpy(), O.rope_inv_freq(160000.0, 64),
                               rtol=1e-15, atol=0)
    np.testing.assert_allclose(rope.yarn_inv_freq(160000.0, 64, 16.0, 65536, "cpu").numpy(),
                               O.yarn_inv_freq(160000.0, 64, 16.0, 65536), rtol=1e-14, atol=0)
    assert abs(rope.yarn_logit_scale(16.0) - O.yarn_logit_scale(16.0)) < 1e-15
    assert rope.yarn_logit_scale(1.0) == 1.0


def out_proj(o=FAKE, o_dt=L.CSA_BF16, T=32, H=128, D=512, G=16, wa=FAKE, R=1024, wb=FAKE, hidden=7168, y=FAKE,
             y_dt=L.CSA_FP32, ws=FAKE, ws_bytes=None):
    lib = L.load()
    if ws_bytes is None:
        ws_bytes = lib.csa_out_proj_workspace_bytes(T, G, R, hidden)
    return rc_msg(lib.csa_out_proj(o, o_dt, T, H, D, G, wa, R, wb, hidden, y, y_dt, ws, ws_bytes, None))


def test_out_proj_validation():
    lib = L.load()
    assert lib.csa_out_proj_workspace_bytes(32, 16, 1024, 7168) == 32 * 16 * 1024 * 4 + 4 * 32 * 7168 * 4
    assert lib.csa_out_proj_workspace_bytes(3, 2, 65, 32) == 1792 + 4 * 3 * 32 * 4   # codes: 1560 B, 256-aligned
    assert lib.csa_out_proj_workspace_bytes(0, 16, 1024, 7168) == 0
    assert out_proj(T=0, o=None) == (L.CSA_OK, "")                # nothing to do, nothing launched
    assert out_proj(o=None)[0] == L.CSA_EINVAL
    assert out_proj(wb=None)[0] == L.CSA_EINVAL
    rc, msg = out_proj(G=12)
    assert rc == L.CSA_EINVAL and "multiple of G" in msg           # 128 heads do not split in 12 groups
    assert out_proj(D=6)[0] == L.CSA_ENOTSUP                      # (H / G) D = 48: not a multiple of 32
    assert out_proj(R=1000)[0] == L.CSA_ENOTSUP
    assert out_proj(hidden=7000)[0] == L.CSA_ENOTSUP
    assert out_proj(o_dt=7)[0] == L.CSA_ENOTSUP
    assert out_proj(y_dt=L.CSA_FP8_E4M3)[0] == L.CSA_ENOTSUP
    assert out_proj(wa=FAKE + 8)[0] == L.CSA_EINVAL               # misaligned
    assert out_proj(ws=None)[0] == L.CSA_EWORKSPACE
    rc, msg = out_proj(ws_bytes=1024)
    assert rc == L.CSA_EWORKSPACE and "5767168" in msg
    assert out_proj(ws=FAKE + 64)[0] == L.CSA_EINVAL              # workspace not 256-byte aligned

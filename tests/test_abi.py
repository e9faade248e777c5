"""The C ABI (include/lac.h) on the CPU: the library loads, exports every
declared function, sizes workspaces with pure host arithmetic, and rejects
invalid arguments before touching the device (no kernel runs here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "lac.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(?:int32_t|size_t|const char\*)\s+(\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    import long_context_attention_compressor_amd as L
    return L


def test_header_declares_the_five_operations():
    names = _declared()
    for fn in ("csa_compress", "hca_compress", "indexer_topk", "csa_attend", "hca_attend"):
        assert fn in names


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L.lib, name), name


def test_workspace_sizes_are_host_arithmetic(L):
    a = L.indexer_topk_workspace_size(4, 1, 262144, 2048)
    assert a >= 4 * 262144 * 4                      # fp32 scores at least
    assert L.indexer_topk_workspace_size(4, 1, 262144, 2048) == a
    assert L.indexer_topk_workspace_size(1, 4096, 66560, 2048) >= 4096 * 66560 * 4
    assert L.indexer_topk_workspace_size(1, 1, 0, 16) >= 0
    assert L.indexer_topk_workspace_size(-1, 1, 10, 16) == 0
    w1 = L.attend_workspace_size(4, 1, 64, 512, 64, L.LAC_KV_E4M3_ROPE_BF16, 2048, 128)
    assert w1 >= 4 * 128 * 576                      # rotated window copy
    assert L.attend_workspace_size(4, 1, 64, 512, 64, L.LAC_BF16, 2048, 0) >= 0
    assert L.attend_workspace_size(1, 1, 0, 512, 64, L.LAC_BF16, 16, 8) == 0


def _err(L):
    return L.lib.lac_last_error().decode()


def test_compress_rejects_bad_arguments(L):
    f = L.lib.csa_compress
    fake = ctypes.c_void_p(0x10000)
    # dtype, sizes, rope dims, positions, null pointers, alignment
    assert f(fake, fake, 7, fake, 1, 1, 16, 128, 4, 64, 1e4, None, 16, 16, 4, None) == 2
    assert "in_dtype" in _err(L)
    assert f(fake, fake, 1, fake, 1, 1, 16, 100, 4, 64, 1e4, None, 16, 16, 4, None) == 1
    assert f(fake, fake, 1, fake, 1, 1, 16, 128, 0, 64, 1e4, None, 16, 16, 4, None) == 1
    assert f(fake, fake, 1, fake, 1, 1, 16, 128, 4, 60, 1e4, None, 16, 16, 4, None) == 1
    pos = (ctypes.c_int64 * 1)(6)
    assert f(fake, fake, 1, fake, 1, 1, 16, 128, 4, 64, 1e4, pos, 16, 16, 4, None) == 1
    assert "multiple of m" in _err(L)
    assert f(None, fake, 1, fake, 1, 1, 16, 128, 4, 64, 1e4, None, 16, 16, 4, None) == 1
    assert f(ctypes.c_void_p(0x10004), fake, 1, fake, 1, 1, 16, 128, 4, 64, 1e4, None, 16, 16, 4,
             None) == 1
    assert "aligned" in _err(L)
    # nothing to do (T < m) is not an error and touches nothing
    assert f(None, None, 1, None, 1, 1, 3, 128, 4, 64, 1e4, None, 3, 3, 0, None) == 0
    assert L.lib.hca_compress(fake, fake, 1, fake, 1, 1, 256, 128, 300, 64, 1e4, None, 256, 256,
                              1, None) == 1


def test_indexer_rejects_bad_arguments(L):
    f = L.lib.indexer_topk
    fake = ctypes.c_void_p(0x10000)
    ws = ctypes.c_void_p(0x100000)
    args = [fake, fake, fake, 1, 2, 1, 64, 128, 1000, None, 4, 16, fake, None, ws, 1 << 30, None]

    def call(**kw):
        a = list(args)
        names = ["q", "w", "K", "dtype", "B", "Tq", "HI", "dI", "N", "pos", "m", "k", "idx",
                 "score", "ws", "wsb", "st"]
        for k_, v in kw.items():
            a[names.index(k_)] = v
        return f(*a)

    assert call(dtype=5) == 2
    assert call(HI=48) == 2 and "H_I" in _err(L)
    assert call(dI=96) == 2
    assert call(k=0) == 1 and call(k=9000) == 1
    assert call(m=0) == 1
    assert call(B=200) == 1
    assert call(ws=None) == 3
    assert call(wsb=16) == 3 and "workspace" in _err(L)
    assert call(ws=ctypes.c_void_p(0x100010)) == 3
    assert call(idx=None) == 1
    neg = (ctypes.c_int64 * 2)(5, -1)
    assert call(pos=neg) == 1
    assert call(dtype=0, HI=64, dI=256) == 2
    # E4M3 queries (LAC_Q_E4M3) go with MXFP4 keys only, at d_I = 128
    assert call(dtype=L.LAC_BF16 | L.LAC_Q_E4M3) == 2 and "LAC_Q_E4M3" in _err(L)
    assert call(dtype=L.LAC_E4M3 | L.LAC_Q_E4M3) == 2
    assert call(dtype=L.LAC_MXFP4 | L.LAC_Q_E4M3, dI=64) == 2 and "d_I = 128" in _err(L)


def test_attend_rejects_bad_arguments(L):
    f = L.lib.csa_attend
    fake = ctypes.c_void_p(0x10000)
    ws = ctypes.c_void_p(0x100000)
    qp = (ctypes.c_int64 * 1)(1000)
    rp_ok = (ctypes.c_int64 * 1)(1000 - 127)
    rp_bad = (ctypes.c_int64 * 1)(1000 - 100)
    base = dict(q=fake, qd=1, kv=fake, kvd=1, N=500, idx=fake, k=64, raw=fake, T_raw=128,
                rp=rp_ok, W=128, sink=None, sc=0.0, B=1, Tq=1, H=64, D=512, r=64, th=1e4,
                qp=qp, out=fake, ws=ws, wsb=1 << 30, st=None)
    order = list(base)

    def call(**kw):
        d = dict(base, **kw)
        return f(*[d[k_] for k_ in order])

    assert call(qd=0) == 2                           # f32 q with a bf16 cache
    assert call(D=384) == 2
    assert call(H=48) == 2
    assert call(r=12) == 1
    assert call(rp=rp_bad) == 1 and "raw window" in _err(L)
    assert call(raw=None) == 1
    assert call(idx=None) == 1
    assert call(wsb=100) == 3
    assert call(sc=float("nan")) == 1
    h = L.lib.hca_attend
    assert h(fake, 1, fake, 1, 64, 0, fake, 128, rp_ok, 128, None, 0.0, 1, 1, 64, 512, 64, 1e4,
             qp, fake, ws, 1 << 30, None) == 1


def test_timer_rejects_unknown_kernel(L):
    assert L.lib.lac_time_next_launch(99, None, None) == 1
    assert L.lib.lac_time_next_launch(1, None, None) == 0    # disarm


# ---------------------------------------------------------------- launch groups
def _csa_compress_args(fake, stream=None):
    # a valid call: bf16 in, bf16 out, B = 1, T = 16, D = 128, m = 4, r = 64
    return (fake, fake, 1, fake, 1, 1, 16, 128, 4, 64, 1e4, None, 16, 16, 4, stream)


def _hca_attend_args(fake, ws, stream=None):
    # q, q_dtype, hkv, kv_dtype, N, m, raw, T_raw, raw_pos0, W, sink, scale, B, Tq, H, D, r,
    # theta, q_pos0, out, ws, ws_bytes, stream
    return (fake, 1, fake, 1, 8, 128, fake, 16, None, 16, None, 0.0, 1, 1, 64, 512, 64, 1e4,
            (ctypes.c_int64 * 1)(15), fake, ws, 1 << 24, stream)


def test_group_state_machine(L):
    lib = L.lib
    fake = ctypes.c_void_p(0x10000)
    assert lib.lac_group_end(None) == 1 and "no launch group" in _err(L)
    assert lib.lac_group_cancel() == 1
    assert lib.lac_group_begin(None) == 0
    assert lib.lac_group_begin(None) == 1 and "already open" in _err(L)
    # recorded, not launched: valid calls return OK without a device
    assert lib.csa_compress(*_csa_compress_args(fake)) == 0
    # validation is unchanged inside a group
    bad = list(_csa_compress_args(fake))
    bad[7] = 100
    assert lib.csa_compress(*bad) == 1
    # another stream than the group's
    assert lib.csa_compress(*_csa_compress_args(fake, ctypes.c_void_p(0x20000))) == 1
    assert "stream" in _err(L)
    # entry points that cannot be recorded
    assert lib.grouped_output_projection(fake, fake, fake, 1, 8, 128, 1, 256, 256, fake, fake,
                                         1 << 20, None) == 1
    assert "launch group" in _err(L)
    assert lib.indexer_topk(fake, fake, fake, 1, 1, 1, 64, 128, 64, None, 4, 16, fake, None,
                            fake, 1 << 20, None) == 1
    assert lib.lac_group_cancel() == 0         # drops the recorded call
    assert lib.lac_group_cancel() == 1
    assert lib.lac_group_begin(None) == 0
    assert lib.lac_group_end(None) == 0        # empty group: nothing to enqueue


def test_group_refuses_shared_attention_workspace(L):
    lib = L.lib
    fake = ctypes.c_void_p(0x10000)
    ws = ctypes.c_void_p(0x1000000)
    assert lib.lac_group_begin(None) == 0
    assert lib.hca_attend(*_hca_attend_args(fake, ws)) == 0
    assert lib.hca_attend(*_hca_attend_args(fake, ws)) == 0
    assert lib.lac_group_end(None) == 3 and "workspace" in _err(L)
    assert lib.lac_group_end(None) == 1        # the failed end closed the group


def test_group_end_on_another_stream_closes_the_group(L):
    lib = L.lib
    fake = ctypes.c_void_p(0x10000)
    assert lib.lac_group_begin(None) == 0
    assert lib.csa_compress(*_csa_compress_args(fake)) == 0
    assert lib.lac_group_end(ctypes.c_void_p(0x20000)) == 1
    assert lib.lac_group_end(None) == 1


def test_indexer_prepare_validation_and_grouping(L):
    lib = L.lib
    fake = ctypes.c_void_p(0x1000000)
    need = L.indexer_topk_workspace_size(4, 1, 262144, 2048)
    # bad sizes, workspace missing, misaligned or small
    assert lib.indexer_topk_prepare(4, 1, 262144, 0, fake, need, None) == 1
    assert lib.indexer_topk_prepare(-1, 1, 262144, 2048, fake, need, None) == 1
    assert lib.indexer_topk_prepare(4, 1, 262144, 2048, None, need, None) == 3
    assert lib.indexer_topk_prepare(4, 1, 262144, 2048, ctypes.c_void_p(0x1000010), need, None) == 3
    assert lib.indexer_topk_prepare(4, 1, 262144, 2048, fake, need - 1, None) == 3
    # inside a group it is recorded (nothing enqueued), on the group's stream only
    assert lib.lac_group_begin(None) == 0
    assert lib.indexer_topk_prepare(4, 1, 262144, 2048, fake, need, None) == 0
    assert lib.indexer_topk_prepare(4, 1, 262144, 2048, fake, need, ctypes.c_void_p(0x20000)) == 1
    assert lib.lac_group_cancel() == 0
    # the flag needs a caller's workspace
    q = ctypes.c_void_p(0x10000)
    assert lib.indexer_topk_noalloc(q, q, q, 1 | L.LAC_TOPK_PREPARED, 1, 1, 64, 128, 64, None, 4,
                                    16, q, None, None) == 1
    assert "LAC_TOPK_PREPARED" in _err(L)

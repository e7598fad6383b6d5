"""The C ABI: the library loads, exports every declared entry point, and rejects
bad arguments before it touches the device (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dualkv.h")

b = pytest.importorskip("sparse_kv_retrieval_amd.binding",
                        reason="libdualkv.so not built (python -m sparse_kv_retrieval_amd.build)")
lib = b.lib

FAKE = ctypes.c_void_p(0x1000)        # 16-byte aligned, never dereferenced by a failing call
MIS = ctypes.c_void_p(0x1004)         # misaligned
NULL = None
S0 = b.dk_strides(0, 0, 0)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dk_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 22, names
    for n in names:
        assert hasattr(lib, n), n
    assert {n for n, _, _ in b.EXPORTS} == set(names)


def test_abi_version():
    assert lib.dk_abi_version() == 14


def err():
    return lib.dk_last_error().decode()


def landmarks(K=FAKE, dt=1, ks=b.dk_strides(1 << 20, 1 << 16, 128), B=1, H=1, L=64, d=128, chunk=32,
              lm=FAKE):
    return lib.dk_build_landmarks(K, dt, ks, B, H, L, d, chunk, lm, None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=NULL), 1), (dict(lm=NULL), 1), (dict(dt=7), 1), (dict(B=0), 1), (dict(chunk=0), 1),
    (dict(L=65), 1), (dict(d=12), 2), (dict(d=1024), 2), (dict(K=MIS), 2),
    (dict(ks=b.dk_strides(1 << 20, 1 << 16, 100)), 2),
])
def test_landmarks_rejects(kw, status):
    assert landmarks(**kw) == status
    assert err().startswith("dk_build_landmarks")


def score(q=FAKE, B=2, T=2, Hq=32, lm=FAKE, lmdt=0, ls=b.dk_strides(1 << 22, 1 << 19, 128), Hkv=8,
          C=1024, d=128, k=64, scale=0.088, reduce=0, shadow=None, idx=FAKE, sc=FAKE, ws=FAKE,
          wsb=1 << 30):
    return lib.dk_score_topk(q, B, T, Hq, lm, lmdt, ls, Hkv, C, d, k, scale, reduce, shadow, idx, sc,
                             ws, wsb, None)


SH_OK = b.dk_landmark_shadow(0x1000, 0x1000, 0x1000)
SH_NULL = b.dk_landmark_shadow(0x1000, 0x1000, 0)
SH_MIS = b.dk_landmark_shadow(0x1008, 0x1000, 0x1000)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), 1), (dict(idx=NULL), 1), (dict(T=3), 1), (dict(T=0), 1), (dict(Hq=30), 1),
    (dict(k=0), 1), (dict(k=1025), 1), (dict(reduce=5), 1), (dict(scale=float("nan")), 1),
    (dict(lmdt=7), 2), (dict(d=96), 2), (dict(C=70000, k=64), 2), (dict(reduce=1, Hq=24), 2),
    # bf16 per-token indexer keys: mean only, no shadow, C % 4 == 0, their own workspace size
    (dict(lmdt=1, reduce=1), 2), (dict(lmdt=1, shadow=ctypes.byref(SH_OK)), 2), (dict(lmdt=1, C=1022), 2),
    (dict(lmdt=1, d=96), 2), (dict(lmdt=1, wsb=16), 1), (dict(lmdt=1, ws=NULL), 1), (dict(lmdt=1, k=1025), 1),
    (dict(lmdt=1, ls=b.dk_strides(1 << 22, 1 << 19, 129)), 2),
    (dict(ws=NULL), 1), (dict(wsb=16), 1), (dict(lm=MIS), 2),
    (dict(shadow=ctypes.byref(SH_NULL)), 1), (dict(shadow=ctypes.byref(SH_MIS)), 2),
    (dict(shadow=ctypes.byref(SH_OK), C=8192), 2), (dict(shadow=ctypes.byref(SH_OK), C=6145), 2),
])
def test_score_topk_rejects(kw, status):
    assert score(**kw) == status, err()
    assert err().startswith("dk_score_topk")


def score_union(uid=FAKE, mem=FAKE, cnt=FAKE, ov=NULL, **kw):
    a = dict(q=FAKE, B=2, T=2, Hq=32, lm=FAKE, lmdt=0, ls=b.dk_strides(1 << 22, 1 << 19, 128), Hkv=8,
             C=1024, d=128, k=64, scale=0.088, reduce=0, shadow=None, idx=FAKE, sc=FAKE, ws=FAKE,
             wsb=1 << 30)
    a.update(kw)
    return lib.dk_score_topk_union(a["q"], a["B"], a["T"], a["Hq"], a["lm"], a["lmdt"], a["ls"], a["Hkv"],
                                   a["C"], a["d"], a["k"], a["scale"], a["reduce"], a["shadow"], a["idx"],
                                   a["sc"], uid, mem, cnt, ov, a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(uid=NULL), 1), (dict(mem=NULL), 1), (dict(cnt=NULL), 1), (dict(q=NULL), 1), (dict(T=3), 1),
    (dict(k=0), 1), (dict(wsb=16), 1), (dict(d=96), 2), (dict(lm=MIS), 2),
    (dict(shadow=ctypes.byref(SH_NULL)), 1), (dict(shadow=ctypes.byref(SH_OK), C=8192), 2),
    (dict(C=65536, k=4097), 2), (dict(lmdt=1, C=131072, k=4097), 2), (dict(lmdt=1, uid=NULL), 1),
])
def test_score_topk_union_rejects(kw, status):
    # every case fails its checks, so nothing is launched
    assert score_union(**kw) == status, err()
    assert err().startswith("dk_score_topk_union")


def test_score_topk_workspace_sizes():
    # 64 x 8 (b, g) rows over 4096 chunks: 4 ranges of 1024, 64 candidates each
    assert lib.dk_score_topk_workspace_size(64, 8, 2, 4096, 64, 0) == 64 * 8 * 2 * 4 * 64 * 8
    # with a shadow one block per (b, g) scores and selects in LDS: no workspace
    assert lib.dk_score_topk_workspace_size(64, 8, 2, 4096, 64, 1) == 0
    assert lib.dk_score_topk_workspace_size(1, 1, 2, 128, 8, 0) > 0
    assert lib.dk_score_topk_workspace_size(1, 1, 2, 128, 0, 0) == 0


def test_index_topk_workspace_size():
    # fp32 scores of every token of every (b, g, t), then the per-block score
    # minima and maxima (1024 tokens per block), then one union arrival counter
    # per (b, g), each region 256-byte aligned
    # scores, per-block minima and maxima, arrival counters; rows of >= 32768 positions also
    # get the split selection's regions (8 slices: histograms, ordered lists, candidates,
    # counts, flags; each 256-byte aligned)
    rows, P = 32 * 2, 8
    split = rows * P * (2048 * 4 + 2 * 4096 * 4 + 2 * 2048 * 4 + 2 * 4) + 256
    assert lib.dk_index_topk_workspace_size(32, 1, 2, 131072) == 32 * 2 * 131072 * 4 + 2 * 32 * 2 * 128 * 4 + 256 + split
    assert lib.dk_index_topk_workspace_size(1, 1, 1, 2048) == 2048 * 4 + 2 * 256 + 256
    assert lib.dk_index_topk_workspace_size(1, 1, 3, 2048) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(lm=NULL), 1), (dict(C=0), 1), (dict(d=96), 2), (dict(lm8=MIS), 2), (dict(cs=NULL), 1), (dict(sm=NULL), 1),
])
def test_shadow_rejects(kw, status):
    a = dict(lm=FAKE, ls=b.dk_strides(1 << 22, 1 << 19, 128), B=2, H=8, C=1024, d=128, lm8=FAKE, cs=FAKE,
             sm=FAKE)
    a.update(kw)
    assert lib.dk_build_landmark_shadow(a["lm"], a["ls"], a["B"], a["H"], a["C"], a["d"], a["lm8"], a["cs"],
                                        a["sm"], None) == status
    assert err().startswith("dk_build_landmark_shadow")


def union(idx=FAKE, B=2, H=8, T=2, k=64, C=1024, uo=FAKE, mo=FAKE, cnt=FAKE, ov=FAKE, plan=None):
    return lib.dk_union_select(idx, B, H, T, k, C, uo, mo, cnt, ov, plan, None)


@pytest.mark.parametrize("kw,status", [
    (dict(idx=NULL), 1), (dict(uo=NULL), 1), (dict(T=3), 1), (dict(k=0), 1), (dict(k=2000), 1),
    (dict(k=5000, C=100000), 2),
])
def test_union_rejects(kw, status):
    assert union(**kw) == status
    assert err().startswith("dk_union_select")


def test_union_plan_rejects_small_cache():
    p = b.dk_cache_plan(0x1000, 100, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    assert union(plan=ctypes.byref(p)) == 1 and "slots" in err()
    p = b.dk_cache_plan(0x1000, 128, 0, 0x1000, 0x1000, 0x1000, 0x1000)
    assert union(plan=ctypes.byref(p)) == 1


def attn(q=FAKE, B=2, T=2, Hq=32, Hkv=8, K=FAKE, V=FAKE, dt=1, ks=b.dk_strides(1 << 22, 1 << 19, 128),
         vs=b.dk_strides(1 << 22, 1 << 19, 128), dk=128, dv=128, chunk=32, ids=FAKE, mem=FAKE, cnt=FAKE,
         N=128, pool=1024, scale=0.088, out=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 30):
    return lib.dk_sparse_decode_attn(q, B, T, Hq, Hkv, K, V, dt, ks, vs, dk, dv, chunk, ids, mem, cnt, N,
                                     pool, scale, out, lse, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), 1), (dict(ids=NULL), 1), (dict(out=NULL), 1), (dict(mem=NULL), 1), (dict(T=3), 1),
    (dict(Hq=33), 1), (dict(N=0), 1), (dict(dt=9), 1), (dict(scale=float("inf")), 1),
    (dict(dk=96, dv=96), 2), (dict(dk=128, dv=64), 2), (dict(Hq=80, Hkv=8), 2), (dict(K=MIS), 2),
    (dict(vs=b.dk_strides(1 << 22, 1 << 19, 100)), 2), (dict(ws=NULL), 1), (dict(wsb=8), 1),
])
def test_attention_rejects(kw, status):
    assert attn(**kw) == status, err()
    assert err().startswith("dk_sparse_decode_attn")


def test_attention_member_optional_for_one_query():
    # T == 1 without a member array gets past the member check and stops at the
    # (deliberately too small) workspace, so nothing is launched.
    assert attn(T=1, mem=NULL, wsb=8) == 1
    assert "workspace" in err()


def gather(Ks=FAKE, Vs=FAKE, dt=1, ss=b.dk_strides(1 << 22, 1 << 19, 128), B=2, H=8, chunk=32, d=128,
           src=FAKE, dst=NULL, cnt=NULL, N=16, sb=1024, Kd=FAKE, Vd=FAKE, ds=b.dk_strides(1 << 16, 1 << 13, 128),
           db=64, host=0):
    return lib.dk_gather_kv(Ks, Vs, dt, ss, B, H, chunk, d, src, dst, cnt, N, sb, Kd, Vd, ds, db, host, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Ks=NULL), 1), (dict(src=NULL), 1), (dict(N=-1), 1), (dict(host=3), 1), (dict(host=-1), 1),
    (dict(dt=3), 1),
    (dict(Kd=MIS), 2), (dict(d=4), 2), (dict(ss=b.dk_strides(-8, 0, 128)), 1),
])
def test_gather_rejects(kw, status):
    assert gather(**kw) == status
    assert err().startswith("dk_gather_kv")


def test_gather_empty_is_ok():
    assert gather(N=0) == 0


@pytest.mark.parametrize("host", [1, 2])
def test_gather_host_kinds_need_pinned_host_memory(host):
    # FAKE is no pinned host allocation: both host kinds refuse it before any copy
    # or launch (with or without a GPU present).
    assert gather(host=host) == 1
    assert "pinned host memory" in err()


def attn_tail(extra=None, **kw):
    a = dict(q=FAKE, B=2, T=2, Hq=32, Hkv=8, K=FAKE, V=FAKE, dt=1, ks=b.dk_strides(1 << 22, 1 << 19, 128),
             vs=b.dk_strides(1 << 22, 1 << 19, 128), dk=128, dv=128, chunk=32, ids=FAKE, mem=FAKE, cnt=FAKE,
             N=128, pb=4096, scale=0.088, out=FAKE, lse=FAKE, ws=FAKE, wsb=16)
    a.update(kw)
    ex = ctypes.byref(extra) if extra is not None else None
    return lib.dk_sparse_decode_attn_tail(a["q"], a["B"], a["T"], a["Hq"], a["Hkv"], a["K"], a["V"], a["dt"],
                                          a["ks"], a["vs"], a["dk"], a["dv"], a["chunk"], a["ids"], a["mem"],
                                          a["cnt"], a["N"], a["pb"], ex, a["scale"], a["out"], a["lse"], a["ws"],
                                          a["wsb"], None)


def extra(Kt=FAKE, Vt=FAKE, tmax=8, Kn=FAKE, Vn=FAKE, ts=b.dk_strides(8192, 1024, 128)):
    return b.dk_attn_extra(Kt, Vt, ts, ts, 0, tmax, Kn, Vn)


@pytest.mark.parametrize("kw,ex,status", [
    (dict(), None, 1),                               # no extra
    (dict(), extra(Vt=NULL), 1),                     # half a tail
    (dict(), extra(Vn=NULL), 1),                     # half the new rows
    (dict(), extra(tmax=-1), 1),
    (dict(dk=96, dv=96), extra(), 2),
    (dict(), extra(Kt=MIS), 2),
    (dict(), extra(ts=b.dk_strides(8192, 1024, 100)), 2),
    (dict(), extra(), 1),                            # the (16-byte) workspace is too small
])
def test_attention_tail_rejects(kw, ex, status):
    # every case fails its checks, so nothing is launched
    assert attn_tail(ex, **kw) == status, err()
    assert err().startswith("dk_sparse_decode_attn_tail")


def test_attention_tail_workspace_size():
    # one more partial slot than the ranges: 1 range per (b, g) at 512 of them + the tail
    assert lib.dk_attn_tail_workspace_size(64, 8, 2, 32, 128, 128, 32) == 64 * 8 * 2 * 8 * 130 * 4
    # 16 x 8 (b, g): 2 ranges (about 256 blocks) + the tail
    assert lib.dk_attn_tail_workspace_size(16, 8, 2, 32, 128, 128, 32) == 16 * 8 * 3 * 8 * 130 * 4
    # a single range still needs partials once a tail is attended
    assert lib.dk_attn_tail_workspace_size(1, 1, 2, 4, 128, 4, 32) == 1 * 1 * 2 * 8 * 130 * 4


def test_attention_workspace_sizes():
    # 16 x 8 (b, g) rows, 2 ranges each (about 256 blocks), 8 query rows of 128
    # values plus (m, l)
    assert lib.dk_attn_workspace_size(16, 8, 2, 32, 128, 128, 32) == 16 * 8 * 2 * 8 * 130 * 4
    # 256 or 512 (b, g): one range each, no merge, no workspace
    assert lib.dk_attn_workspace_size(32, 8, 2, 32, 128, 128, 32) == 0
    assert lib.dk_attn_workspace_size(64, 8, 2, 32, 128, 128, 32) == 0
    # a single (b, g) with few entries: one range, no workspace
    assert lib.dk_attn_workspace_size(1, 1, 2, 4, 128, 4, 32) == 0
    assert lib.dk_attn_workspace_size(64, 8, 2, 30, 128, 128, 32) == 0


def minmax_topk(q=FAKE, B=2, T=2, Hq=32, mn=FAKE, mx=FAKE, dt=1, ss=b.dk_strides(1 << 19, 1 << 16, 128), Hkv=8,
                C=1024, d=128, k=64, scale=0.088, reduce=0, idx=FAKE, sc=FAKE, uid=NULL, mem=NULL, cnt=NULL,
                ov=NULL, ws=FAKE, wsb=1 << 30):
    return lib.dk_score_topk_minmax(q, B, T, Hq, mn, mx, dt, ss, Hkv, C, d, k, scale, reduce, idx, sc, uid, mem,
                                    cnt, ov, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), 1), (dict(mn=NULL), 1), (dict(idx=NULL), 1), (dict(T=3), 1), (dict(k=0), 1),
    (dict(k=1025), 1), (dict(reduce=4), 1), (dict(scale=float("inf")), 1), (dict(dt=5), 1),
    (dict(uid=FAKE), 1), (dict(d=96), 2), (dict(C=1022, k=8), 2), (dict(reduce=1, Hq=64), 2),
    (dict(mx=MIS), 2),
    (dict(wsb=16), 1), (dict(ws=NULL), 1), (dict(uid=FAKE, mem=FAKE, cnt=FAKE, k=4000, C=8192), 2),
])
def test_minmax_topk_rejects(kw, status):
    assert minmax_topk(**kw) == status, err()
    assert err().startswith("dk_score_topk_minmax")


@pytest.mark.parametrize("kw,status", [
    (dict(K=NULL), 1), (dict(L=1000), 1), (dict(d=96), 2), (dict(mn=MIS), 2), (dict(dt=9), 1),
])
def test_build_minmax_rejects(kw, status):
    a = dict(K=FAKE, dt=1, ks=b.dk_strides(1 << 22, 1 << 19, 128), B=2, Hkv=8, L=4096, d=128, chunk=32, mn=FAKE,
             mx=FAKE)
    a.update(kw)
    assert lib.dk_build_minmax(a["K"], a["dt"], a["ks"], a["B"], a["Hkv"], a["L"], a["d"], a["chunk"], a["mn"],
                               a["mx"], None) == status, err()
    assert err().startswith("dk_build_minmax")


def coverage(q=FAKE, B=2, T=2, Hq=32, lm=FAKE, dt=0, ls=b.dk_strides(1 << 22, 1 << 19, 128), Hkv=8, C=1024,
             d=128, scale=0.088, reduce=0, gamma=0.9, k_max=64, idx=FAKE, cnt=FAKE, sc=NULL, uid=NULL, mem=NULL,
             ucnt=NULL, ov=NULL, ws=FAKE, wsb=1 << 30):
    return lib.dk_score_coverage(q, B, T, Hq, lm, dt, ls, Hkv, C, d, scale, reduce, gamma, k_max, idx, cnt, sc, uid,
                                 mem, ucnt, ov, ws, wsb, None)


# every case breaks exactly one rule, so no call reaches a launch
@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), 1), (dict(lm=NULL), 1), (dict(idx=NULL), 1), (dict(cnt=NULL), 1), (dict(T=3), 1),
    (dict(k_max=0), 1), (dict(k_max=1025), 1), (dict(gamma=0.0), 1), (dict(gamma=1.5), 1),
    (dict(gamma=float("nan")), 1), (dict(reduce=4), 1), (dict(scale=float("inf")), 1), (dict(dt=5), 1),
    (dict(uid=FAKE), 1), (dict(Hq=30), 1), (dict(d=96), 2), (dict(C=16385, k_max=8), 2),
    (dict(reduce=1, Hq=64), 2), (dict(lm=MIS), 2), (dict(ls=b.dk_strides(1 << 22, 1 << 19, 129)), 2),
    (dict(wsb=16), 1), (dict(ws=NULL), 1),
])
def test_coverage_rejects(kw, status):
    assert coverage(**kw) == status, err()
    assert err().startswith("dk_score_coverage")


def test_coverage_workspace_size():
    # fp32 score rows [B*Hkv*T, C], per-block minima and maxima, one counter per (b, g); 256-byte aligned
    assert lib.dk_coverage_workspace_size(64, 8, 2, 4096) == 1024 * 4096 * 4 + 2 * 16384 + 2048
    assert lib.dk_coverage_workspace_size(1, 1, 1, 100) == 512 + 2 * 256 + 256
    assert lib.dk_coverage_workspace_size(1, 1, 3, 100) == 0
    assert lib.dk_coverage_workspace_size(0, 1, 1, 100) == 0


def capped(ids=FAKE, sc=NULL, cnt=NULL, B=2, Hkv=8, N=64, stride=64, cstride=1, res=FAKE, st=FAKE, S=128, cap=8,
           step=3, slot=FAKE, ac=FAKE, asl=FAKE, acnt=FAKE, hc=NULL):
    return lib.dk_capped_plan(ids, sc, cnt, B, Hkv, N, stride, cstride, res, st, S, cap, step, slot, ac, asl, acnt,
                              hc, None)


@pytest.mark.parametrize("kw,status", [
    (dict(ids=NULL), 1), (dict(res=NULL), 1), (dict(st=NULL), 1), (dict(slot=NULL), 1), (dict(acnt=NULL), 1),
    (dict(B=0), 1), (dict(N=0), 1), (dict(S=0), 1), (dict(stride=63), 1), (dict(cnt=FAKE, cstride=0), 1),
    (dict(cap=-1), 1), (dict(cap=(1 << 20) + 1), 1), (dict(ac=NULL), 1), (dict(asl=NULL), 1),
    (dict(N=4097, stride=4097), 2), (dict(S=4097), 2),
])
def test_capped_plan_rejects(kw, status):
    assert capped(**kw) == status, err()
    assert err().startswith("dk_capped_plan")



def decode_step(q=FAKE, B=64, T=2, Hq=32, Hkv=8, lm=FAKE, lmdt=0, ls=b.dk_strides(1 << 22, 1 << 19, 128), C=4096,
                d=128, k=64, scale=0.088, reduce=0, shadow=None, K=FAKE, V=FAKE, kvdt=1,
                ks=b.dk_strides(1 << 30, 1 << 27, 128), vs=b.dk_strides(1 << 30, 1 << 27, 128), chunk=32,
                idx=FAKE, sc=FAKE, uid=FAKE, mem=FAKE, cnt=FAKE, ov=FAKE, out=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 30,
                ex=None):
    exp = ctypes.byref(ex) if ex is not None else None
    return lib.dk_decode_step(q, B, T, Hq, Hkv, lm, lmdt, ls, C, d, k, scale, reduce, shadow, K, V, kvdt, ks, vs,
                              chunk, exp, idx, sc, uid, mem, cnt, ov, out, lse, ws, wsb, None)


def test_decode_step_workspace_size():
    # the two calls run in turn on one workspace: the larger of their sizes
    for B, Hkv, C, k, sh in [(64, 8, 4096, 64, 1), (16, 8, 1024, 64, 1), (16, 8, 1024, 64, 0), (2, 8, 512, 16, 0)]:
        want = max(lib.dk_score_topk_workspace_size(B, Hkv, 2, C, k, sh),
                   lib.dk_attn_workspace_size(B, Hkv, 2, 32, 128, 2 * k, 32))
        assert lib.dk_decode_step_workspace_size(B, Hkv, 2, 32, C, 128, k, 32, sh, 0) == want
        # with the tail rows the attention's share is the tail attention's size
        want_t = max(lib.dk_score_topk_workspace_size(B, Hkv, 2, C, k, sh),
                     lib.dk_attn_tail_workspace_size(B, Hkv, 2, 32, 128, 2 * k, 32))
        assert lib.dk_decode_step_workspace_size(B, Hkv, 2, 32, C, 128, k, 32, sh, 1) == want_t
    assert lib.dk_decode_step_workspace_size(0, 8, 2, 32, 4096, 128, 64, 32, 1, 0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(q=NULL), 1), (dict(lmdt=1), 2), (dict(T=3), 1), (dict(uid=NULL), 1), (dict(cnt=NULL), 1),
    (dict(out=NULL), 1), (dict(K=NULL), 1), (dict(d=96), 2), (dict(k=0), 1), (dict(k=5000), 1),
    (dict(Hq=30), 1), (dict(chunk=0), 1), (dict(ws=NULL, wsb=0, B=16), 1),
    # the tail attention's checks: a half-given pair, a negative tail length, misaligned rows
    (dict(ex=extra(Vt=NULL)), 1), (dict(ex=extra(Kn=NULL)), 1), (dict(ex=extra(tmax=-1)), 1),
    (dict(ex=extra(Kn=ctypes.c_void_p(0x1008))), 2),
])
def test_decode_step_rejects(kw, status):
    assert decode_step(**kw) == status, err()
    assert err().startswith("dk_decode_step")

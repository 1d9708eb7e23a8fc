"""The C-ABI boundary on the CPU: the library loads, exports what the header
declares, sizes its workspace affinely in T, and rejects bad arguments on the
host before any HIP call (so none of these tests touches a GPU)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kdloss.h")

kdl = pytest.importorskip("chunked_kl_loss_logit_amd")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kdl.LIB_PATH):
        pytest.fail("libkdloss.so is not built (run __graft_entry__.build())")
    return kdl.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kd_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert len(names) == 31
    for n in names:
        assert hasattr(L, n), f"{n} declared in kdloss.h but not exported"
    assert sorted(kdl.EXPORTS) == names


def test_status_strings_and_version(L):
    for code, name in kdl._binding.STATUS.items():
        assert L.kd_status_string(code).decode() == name
    assert L.kd_version() == 10400


# ---------------------------------------------------------------- workspace sizing
def ws_topk(T, d=3072, V=128256, K=64, dt=kdl.KD_BF16, chunk=0):
    out = ctypes.c_size_t()
    st = kdl.lib().kd_topk_kl_workspace_size(T, d, V, K, dt, chunk, ctypes.byref(out))
    return st, out.value


def ws_full(T, d=3072, dtt=4096, V=128256, dt=kdl.KD_BF16, chunk=0):
    out = ctypes.c_size_t()
    st = kdl.lib().kd_full_kl_workspace_size(T, d, dtt, V, dt, chunk, ctypes.byref(out))
    return st, out.value


def test_workspace_zero_rows(L):
    assert ws_topk(0) == (0, 0)
    assert ws_full(0) == (0, 0)


def test_workspace_is_affine_in_T_with_small_slope(L):
    # extra device memory = the workspace: a constant (the chunk buffers) plus a
    # per-token part (teacher data and split partials), never a [T, V] buffer
    Ts = [16384, 65536, 262144]
    sizes = [ws_topk(T)[1] for T in Ts]
    slope = (sizes[2] - sizes[1]) / (Ts[2] - Ts[1])
    assert slope <= 1024, slope  # bytes per token
    assert slope >= 10 * 64      # at least the sorted teacher data
    pred = sizes[1] + slope * (Ts[0] - Ts[1])
    assert abs(pred - sizes[0]) / sizes[0] < 0.01
    # a bf16 [T, V] buffer alone would be 250 KiB per token
    assert sizes[2] < 262144 * 128256 * 2 / 40
    fs = [ws_full(T)[1] for T in Ts]
    assert (fs[2] - fs[1]) / (Ts[2] - Ts[1]) <= 1024


def test_workspace_chunk_rows(L):
    s_small = ws_topk(32768, chunk=1024)[1]
    s_big = ws_topk(32768, chunk=8192)[1]
    assert s_small < s_big
    # chunk rows round up to 256 and clamp to the rows present
    assert ws_topk(1000, chunk=100000)[1] == ws_topk(1000, chunk=1024)[1]
    assert ws_topk(4096, chunk=300)[1] == ws_topk(4096, chunk=512)[1]


# ---------------------------------------------------------------- argument errors
FAKE = 0x10000  # 64 KiB: aligned to 256, never dereferenced (calls fail before any HIP call)


def fwd(T=8, d=64, V=256, K=4, dt=kdl.KD_BF16, tau=1.0, H=FAKE, W=FAKE, idx=FAKE, lg=FAKE, kl=FAKE, lse=FAKE,
        z=None, ws=FAKE, wsb=0):
    L = kdl.lib()
    vp = ctypes.c_void_p
    return L.kd_topk_kl_fwd(vp(H), vp(W), vp(idx), vp(lg), None, ctypes.c_float(tau), T, d, V, K, dt, vp(kl),
                            vp(lse), vp(z) if z else None, vp(ws) if ws else None, wsb, None)


def bwd(T=8, d=64, V=256, K=4, dt=kdl.KD_BF16, tau=1.0, dH=FAKE, dW=FAKE, chunk=0, ws=FAKE, wsb=0, lse=FAKE):
    L = kdl.lib()
    vp = ctypes.c_void_p
    return L.kd_topk_kl_bwd(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(tau), T, d, V, K, dt,
                            vp(lse) if lse else None, vp(FAKE), vp(dH) if dH else None, vp(dW) if dW else None,
                            chunk, vp(ws) if ws else None, wsb, None)


def full_fwd(T=8, d=64, dtt=64, V=256, dt=kdl.KD_BF16, tau=1.0, Ht=FAKE, wsb=0):
    L = kdl.lib()
    vp = ctypes.c_void_p
    return L.kd_full_kl_fwd(vp(FAKE), vp(FAKE), vp(Ht) if Ht else None, vp(FAKE), None, ctypes.c_float(tau), T, d,
                            dtt, V, dt, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), wsb, None)


def last_error():
    return kdl.lib().kd_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(K=0), 1), (dict(K=300), 1), (dict(T=-1), 1), (dict(d=0), 1), (dict(V=0), 1),
    (dict(tau=0.0), 1), (dict(tau=-1.0), 1), (dict(tau=math.nan), 1), (dict(tau=math.inf), 1),
    (dict(dt=7), 1), (dict(H=0), 1), (dict(W=0), 1), (dict(idx=0), 1), (dict(lg=0), 1), (dict(kl=0), 1),
    (dict(lse=0), 1),
    (dict(d=60), 2), (dict(V=260), 2), (dict(V=20000, K=9000), 2), (dict(d=6, dt=kdl.KD_F32), 2),
    (dict(H=FAKE + 8), 3), (dict(W=FAKE + 4), 3), (dict(kl=FAKE + 2), 3), (dict(z=FAKE + 1), 3),
    (dict(ws=FAKE + 128, wsb=1 << 40), 3),
    (dict(wsb=16), 4),
])
def test_topk_fwd_rejects(L, kw, code):
    assert fwd(**kw) == code
    assert last_error() != ""


def test_fp32_allows_multiples_of_four(L):
    # d = 12, V = 260 are fine for fp32 (4 per 16 bytes) but not bf16
    assert fwd(d=12, V=260, dt=kdl.KD_F32, wsb=16) == 4  # reaches the workspace check
    assert fwd(d=12, V=260, dt=kdl.KD_BF16, wsb=16) == 2


def test_zero_rows_forward_is_a_noop(L):
    assert fwd(T=0, H=0, W=0, idx=0, lg=0, kl=0, lse=0, ws=0) == 0
    assert last_error() == ""
    assert full_fwd(T=0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dW=0), 1), (dict(dH=0), 1), (dict(lse=0), 1), (dict(chunk=-1), 1), (dict(dW=FAKE + 4), 3),
    (dict(dH=FAKE + 8), 3), (dict(wsb=16), 4), (dict(tau=0.0), 1), (dict(K=0), 1),
])
def test_topk_bwd_rejects(L, kw, code):
    assert bwd(**kw) == code


def fwd_bwd(T=8, d=64, V=256, K=4, dt=kdl.KD_BF16, tau=1.0, g=FAKE, kl=FAKE, lse=FAKE, dH=FAKE, dW=FAKE, chunk=0,
            wsb=0):
    vp = ctypes.c_void_p
    L = kdl.lib()
    return L.kd_topk_kl_fwd_bwd(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(tau), T, d, V, K, dt,
                                vp(g) if g else None, vp(kl) if kl else None, vp(lse) if lse else None, None,
                                vp(dH) if dH else None, vp(dW) if dW else None, chunk, vp(FAKE), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(g=0), 1), (dict(kl=0), 1), (dict(lse=0), 1), (dict(dH=0), 1), (dict(dW=0), 1), (dict(chunk=-1), 1),
    (dict(dW=FAKE + 4), 3), (dict(dH=FAKE + 8), 3), (dict(wsb=16), 4), (dict(tau=0.0), 1), (dict(K=0), 1),
    (dict(d=12), 2),
])
def test_topk_fwd_bwd_rejects(L, kw, code):
    assert fwd_bwd(**kw) == code


def test_fwd_bwd_workspace_adds_one_fp32_logit_chunk(L):
    # same per-row buffers and backward chunk buffers as the two-call path, plus
    # per-chunk forward partials, the chunk's fp32 logits [C, roundup(V, 256)]
    # and the gathered logits at the sorted entries [T, K + 1] (for z_topk)
    for T, chunk in ((4096, 0), (10000, 1024), (300, 0)):
        out = ctypes.c_size_t(0)
        assert L.kd_topk_kl_fwd_bwd_workspace_size(T, 3072, 128256, 64, kdl.KD_BF16, chunk, ctypes.byref(out)) == 0
        C = min(4096 if chunk == 0 else chunk, (T + 255) // 256 * 256)
        two_call = ws_topk(T, chunk=chunk)[1]
        zsort = T * 65 * 4
        assert two_call + C * 128256 * 4 <= out.value <= two_call + C * 128256 * 4 + 256 * C * 16 + zsort + (1 << 20)
    out = ctypes.c_size_t(0)
    assert L.kd_topk_kl_fwd_bwd_workspace_size(0, 3072, 128256, 64, kdl.KD_BF16, 0, ctypes.byref(out)) == 0
    assert out.value == 0


def test_full_fwd_rejects(L):
    assert full_fwd(Ht=0) == 1
    assert full_fwd(dtt=60) == 2
    assert full_fwd(tau=0.0) == 1
    assert full_fwd(Ht=FAKE + 8) == 3
    assert full_fwd(wsb=16) == 4


def test_workspace_query_rejects(L):
    assert ws_topk(8, K=0)[0] == 1
    assert ws_topk(8, d=12)[0] == 2
    assert L.kd_topk_kl_workspace_size(8, 64, 256, 4, 1, 0, None) == 1


def test_profile_api_without_gpu(L):
    assert L.kd_profile_enable(0) == 0
    assert L.kd_profile_reset() == 0
    assert L.kd_profile_count() == 0
    assert L.kd_profile_get(0, None, None, None) == 1


def test_binding_refuses_cpu_tensors(L):
    import torch
    H = torch.zeros(8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kdl._binding._ptr(H)


def full_fwd_bwd(T=8, d=64, dtt=64, V=256, dt=kdl.KD_BF16, tau=1.0, Ht=FAKE, g=FAKE, kl=FAKE, dH=FAKE, dW=FAKE,
                 chunk=0, wsb=0):
    vp = ctypes.c_void_p
    L = kdl.lib()
    return L.kd_full_kl_fwd_bwd(vp(FAKE), vp(FAKE), vp(Ht) if Ht else None, vp(FAKE), None, ctypes.c_float(tau), T,
                                d, dtt, V, dt, vp(g) if g else None, vp(kl) if kl else None, vp(FAKE), vp(FAKE),
                                vp(dH) if dH else None, vp(dW) if dW else None, chunk, vp(FAKE), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Ht=0), 1), (dict(g=0), 1), (dict(kl=0), 1), (dict(dH=0), 1), (dict(dW=0), 1), (dict(chunk=-1), 1),
    (dict(tau=0.0), 1), (dict(dtt=60), 2), (dict(V=260), 2), (dict(dW=FAKE + 4), 3), (dict(dH=FAKE + 8), 3),
    (dict(Ht=FAKE + 8), 3), (dict(wsb=16), 4),
])
def test_full_fwd_bwd_rejects(L, kw, code):
    assert full_fwd_bwd(**kw) == code
    assert last_error() != ""


def test_full_fwd_bwd_zero_rows_needs_only_dw(L):
    assert full_fwd_bwd(T=0, Ht=0, g=0, kl=0, dH=0, dW=0) == 1  # dW is still written
    out = ctypes.c_size_t(7)
    assert L.kd_full_kl_fwd_bwd_workspace_size(0, 3072, 4096, 128256, kdl.KD_BF16, 0, ctypes.byref(out)) == 0
    assert out.value == 0


def test_full_fwd_bwd_workspace_adds_two_fp32_logit_chunks(L):
    # the two-call path's buffers, per-chunk partials, and the chunk's student
    # and teacher logits, fp32 [C, roundup(V, 256)] each
    for T, chunk in ((16384, 0), (10000, 2048), (300, 0)):
        out = ctypes.c_size_t(0)
        assert L.kd_full_kl_fwd_bwd_workspace_size(T, 3072, 4096, 128256, kdl.KD_BF16, chunk,
                                                   ctypes.byref(out)) == 0
        C = min(4096 if chunk == 0 else chunk, (T + 255) // 256 * 256)
        two_call = ws_full(T, chunk=chunk)[1]
        extra = 2 * C * 128256 * 4
        assert two_call + extra <= out.value <= two_call + extra + 256 * C * 32 + (1 << 20)


# ---------------------------------------------------------------- top-K options
def fwd_ex(opts, T=8, d=64, V=256, K=4, wsb=0):
    vp = ctypes.c_void_p
    L = kdl.lib()
    ref = None if opts is None else ctypes.byref(opts)
    return L.kd_topk_kl_fwd_ex(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(1.0), ref, T, d, V, K,
                               kdl.KD_BF16, vp(FAKE), vp(FAKE), None, vp(FAKE), wsb, None)


def opts(tau_rows=0, teacher_lse=0, labels=0, ce_weight=0.0, check=0, rev=0.0, z=0):
    return kdl._binding.KdTopkOpts(tau_rows or None, teacher_lse or None, labels or None, ce_weight, check, rev,
                                   z or None)


def test_topk_opts_layout_matches_the_header(L):
    # three pointers, the CE weight, the index-check flag, the reverse-KL
    # weight and the forward's z_topk
    assert ctypes.sizeof(kdl._binding.KdTopkOpts) == 48
    assert kdl._binding.KdTopkOpts.check_indices.offset == 28
    assert kdl._binding.KdTopkOpts.rev_weight.offset == 32
    assert kdl._binding.KdTopkOpts.z_topk.offset == 40


def test_index_check_is_an_option_of_the_whole_head_only(L):
    # a valid request reaches the workspace check (nothing is enqueued before it)
    assert fwd_ex(opts(check=1)) == 4
    # a shard does not know the whole head's width
    vp = ctypes.c_void_p
    o = ctypes.byref(opts(check=1))
    assert L.kd_topk_kl_fwd_shard(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(1.0), o, 8, 64, 256,
                                  512, 4, kdl.KD_BF16, vp(FAKE), vp(FAKE), None, vp(FAKE), 0, None) == 2
    assert "check_indices" in last_error()
    assert L.kd_topk_kl_bwd_shard(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(1.0), o, 8, 64, 256,
                                  512, 4, kdl.KD_BF16, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 0, vp(FAKE), 0,
                                  None) == 2


@pytest.mark.parametrize("o,code", [
    (opts(ce_weight=0.5), 1),                                     # a CE weight needs labels
    (opts(labels=FAKE, ce_weight=-0.1), 1), (opts(labels=FAKE, ce_weight=1.5), 1),
    (opts(labels=FAKE, ce_weight=math.nan), 1), (opts(labels=FAKE, ce_weight=math.inf), 1),
    (opts(tau_rows=FAKE + 2), 3), (opts(teacher_lse=FAKE + 1), 3), (opts(labels=FAKE + 2, ce_weight=0.5), 3),
    (opts(tau_rows=FAKE, teacher_lse=FAKE, labels=FAKE, ce_weight=0.5), 4),  # valid: reaches the workspace
    (None, 4), (opts(), 4), (opts(labels=FAKE), 4),                # labels without a weight are ignored
])
def test_topk_options_checks(L, o, code):
    assert fwd_ex(o) == code
    assert last_error() != ""


def test_topk_options_label_needs_room_for_one_more_entry(L):
    o = opts(labels=FAKE, ce_weight=0.5)
    assert fwd_ex(o, V=16384, K=kdl.KD_MAX_K) == 2
    assert fwd_ex(o, V=16384, K=kdl.KD_MAX_K - 1) == 4
    assert fwd_ex(None, V=16384, K=kdl.KD_MAX_K) == 4


def test_topk_reverse_option_checks(L):
    vp = ctypes.c_void_p
    L_ = kdl.lib()

    def fwd(o, z):
        return L_.kd_topk_kl_fwd_ex(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(1.0),
                                    ctypes.byref(o), 8, 64, 256, 4, kdl.KD_BF16, vp(FAKE), vp(FAKE),
                                    vp(z) if z else None, vp(FAKE), 0, None)

    def bwd(o):
        return L_.kd_topk_kl_bwd_ex(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(1.0),
                                    ctypes.byref(o), 8, 64, 256, 4, kdl.KD_BF16, vp(FAKE), vp(FAKE), vp(FAKE),
                                    vp(FAKE), 0, vp(FAKE), 0, None)

    def one(o, z):
        return L_.kd_topk_kl_fwd_bwd_ex(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(1.0),
                                        ctypes.byref(o), 8, 64, 256, 4, kdl.KD_BF16, vp(FAKE), vp(FAKE), vp(FAKE),
                                        vp(z) if z else None, vp(FAKE), vp(FAKE), 0, vp(FAKE), 0, None)

    for r in (-0.1, 1.5, math.nan, math.inf):
        assert fwd(opts(rev=r), FAKE) == 1 and "rev_weight" in last_error()
    # the forward and the single call need their z_topk output, the backward the forward's
    assert fwd(opts(rev=0.5), 0) == 1 and "z_topk" in last_error()
    assert one(opts(rev=0.5), 0) == 1 and "z_topk" in last_error()
    assert bwd(opts(rev=0.5)) == 1 and "z_topk" in last_error()
    assert bwd(opts(rev=0.5, z=FAKE + 2)) == 3
    # valid requests reach the workspace check
    assert fwd(opts(rev=0.5), FAKE) == 4 and one(opts(rev=1.0), FAKE) == 4 and bwd(opts(rev=0.5, z=FAKE)) == 4
    assert fwd(opts(rev=0.0), 0) == 4  # no reverse part: z_topk stays optional
    # a vocabulary shard cannot form the reverse part
    o = ctypes.byref(opts(rev=0.5, z=FAKE))
    assert L_.kd_topk_kl_fwd_shard(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(1.0), o, 8, 64, 256,
                                   512, 4, kdl.KD_BF16, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 0, None) == 2
    assert "rev_weight" in last_error()
    assert L_.kd_topk_kl_bwd_shard(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(1.0), o, 8, 64, 256,
                                   512, 4, kdl.KD_BF16, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 0, vp(FAKE), 0,
                                   None) == 2


def test_topk_ex_calls_check_their_options_too(L):
    vp = ctypes.c_void_p
    bad = ctypes.byref(opts(ce_weight=0.5))
    assert L.kd_topk_kl_bwd_ex(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(1.0), bad, 8, 64, 256, 4,
                               kdl.KD_BF16, vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 0, vp(FAKE), 0, None) == 1
    assert L.kd_topk_kl_fwd_bwd_ex(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(1.0), bad, 8, 64,
                                   256, 4, kdl.KD_BF16, vp(FAKE), vp(FAKE), vp(FAKE), None, vp(FAKE), vp(FAKE), 0,
                                   vp(FAKE), 0, None) == 1


# ---------------------------------------------------------------- full-vocabulary options
def full_fwd_ex(o, kl_rev=FAKE, wsb=0):
    vp = ctypes.c_void_p
    ref = None if o is None else ctypes.byref(o)
    return kdl.lib().kd_full_kl_fwd_ex(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(1.0), ref, 8, 64,
                                       64, 256, kdl.KD_BF16, vp(FAKE), vp(FAKE), vp(FAKE),
                                       vp(kl_rev) if kl_rev else None, vp(FAKE), wsb, None)


def full_bwd_ex(o, kl_rev=FAKE):
    vp = ctypes.c_void_p
    ref = None if o is None else ctypes.byref(o)
    return kdl.lib().kd_full_kl_bwd_ex(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(1.0), ref, 8, 64,
                                       64, 256, kdl.KD_BF16, vp(FAKE), vp(FAKE), vp(kl_rev) if kl_rev else None,
                                       vp(FAKE), vp(FAKE), vp(FAKE), 0, vp(FAKE), 0, None)


def fopts(tau_rows=0, rev_weight=0.0):
    return kdl._binding.KdFullOpts(tau_rows or None, rev_weight)


@pytest.mark.parametrize("o,kr,code", [
    (fopts(rev_weight=-0.5), FAKE, 1), (fopts(rev_weight=1.01), FAKE, 1), (fopts(rev_weight=math.nan), FAKE, 1),
    (fopts(tau_rows=FAKE + 2), FAKE, 3), (fopts(), FAKE + 2, 3),
    (fopts(rev_weight=0.5), 0, 4), (fopts(tau_rows=FAKE, rev_weight=1.0), FAKE, 4), (None, 0, 4),
])
def test_full_options_checks(L, o, kr, code):
    assert full_fwd_ex(o, kl_rev=kr) == code
    assert last_error() != ""


def test_full_backward_needs_kl_rev_when_mixing(L):
    assert full_bwd_ex(fopts(rev_weight=0.5), kl_rev=0) == 1
    assert "kl_rev" in last_error()
    assert full_bwd_ex(fopts(rev_weight=0.5)) == 4
    assert full_bwd_ex(fopts(), kl_rev=0) == 4


def test_bf16_chunks_stay_within_the_direct_load_reach(L):
    # a chunk's bf16 dZ buffer must stay under 4 GiB (16640 rows at V = 128256),
    # and the cap is rounded down to a multiple of the default chunk: 16384
    big = ws_topk(65536, chunk=32768)[1]
    assert big == ws_topk(65536, chunk=16384)[1] == ws_topk(65536, chunk=16640)[1] == ws_topk(65536, chunk=20000)[1]
    assert ws_topk(65536, chunk=16128)[1] < big
    # fp32 has no such limit (its mainloop is not the direct-load one)
    assert ws_topk(65536, chunk=32768, dt=kdl.KD_F32)[1] > ws_topk(65536, chunk=16640, dt=kdl.KD_F32)[1]


# ---------------------------------------------------------------- one vocabulary shard
def fwd_shard(T=8, d=64, V=256, v0=512, K=4, dt=kdl.KD_BF16, tau=1.0, rec=FAKE, trow=FAKE, wsb=0):
    vp = ctypes.c_void_p
    return kdl.lib().kd_topk_kl_fwd_shard(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(tau), None,
                                          T, d, V, v0, K, dt, vp(rec) if rec else None,
                                          vp(trow) if trow else None, None, vp(FAKE), wsb, None)


def bwd_shard(T=8, d=64, V=256, v0=512, K=4, dH=FAKE, dW=FAKE, wsb=0):
    vp = ctypes.c_void_p
    return kdl.lib().kd_topk_kl_bwd_shard(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(1.0), None,
                                          T, d, V, v0, K, kdl.KD_BF16, vp(FAKE), vp(FAKE), vp(dH) if dH else None,
                                          vp(dW) if dW else None, 0, vp(FAKE), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(v0=-1), 1), (dict(rec=0), 1), (dict(trow=0), 1), (dict(K=0), 1),
    (dict(v0=(1 << 30) - 100), 2), (dict(K=kdl.KD_MAX_K + 1), 2),
    (dict(rec=FAKE + 8), 3), (dict(trow=FAKE + 4), 3),
    (dict(wsb=16), 4), (dict(K=300, wsb=16), 4),  # K may exceed the shard's width
])
def test_topk_fwd_shard_rejects(L, kw, code):
    assert fwd_shard(**kw) == code
    assert last_error() != ""


@pytest.mark.parametrize("kw,code", [
    (dict(v0=-1), 1), (dict(dH=0), 1), (dict(dW=0), 1), (dict(dH=FAKE + 8), 3), (dict(wsb=16), 4),
    (dict(K=300, wsb=16), 4),
])
def test_topk_bwd_shard_rejects(L, kw, code):
    assert bwd_shard(**kw) == code


def test_shard_combine_checks(L):
    vp = ctypes.c_void_p
    comb = kdl.lib().kd_topk_kl_shard_combine
    assert comb(vp(FAKE), 8, vp(FAKE), None, 0, None, None, None) == 0  # T = 0: nothing to do
    assert comb(vp(FAKE), 0, vp(FAKE), None, 16, vp(FAKE), vp(FAKE), None) == 1
    assert comb(vp(FAKE), 8, vp(FAKE), None, -1, vp(FAKE), vp(FAKE), None) == 1
    assert comb(None, 8, vp(FAKE), None, 16, vp(FAKE), vp(FAKE), None) == 1
    assert comb(vp(FAKE + 8), 8, vp(FAKE), None, 16, vp(FAKE), vp(FAKE), None) == 3
    assert comb(vp(FAKE), 8, vp(FAKE + 4), None, 16, vp(FAKE), vp(FAKE), None) == 3
    assert comb(vp(FAKE), 1 << 20, vp(FAKE), None, 1 << 12, vp(FAKE), vp(FAKE), None) == 2


def test_shard_workspace_is_the_plain_size_at_the_shard_width(L):
    for T, d, V, K, chunk in ((4096, 3072, 16032, 64, 0), (300, 256, 168, 16, 256)):
        assert (kdl.kd_topk_kl_shard_workspace_size(T, d, V, 3 * V, K, kdl.torch.bfloat16, chunk)
                == kdl.kd_topk_kl_workspace_size(T, d, V, K, kdl.torch.bfloat16, chunk))
    # more cached entries than the shard has columns
    assert kdl.kd_topk_kl_shard_workspace_size(64, 64, 8, 0, 16, kdl.torch.bfloat16) > 0


def test_full_shard_checks(L):
    vp = ctypes.c_void_p
    f = kdl.lib()
    fwd = lambda rec=FAKE, T=8: f.kd_full_kl_fwd_shard(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None,
                                                        ctypes.c_float(1.0), None, T, 64, 64, 256, kdl.KD_BF16,
                                                        vp(rec) if rec else None, vp(FAKE), 16, None)
    assert fwd(rec=0) == 1 and fwd(rec=FAKE + 8) == 3 and fwd() == 4  # reaches the workspace check
    assert fwd(rec=0, T=0) == 0
    comb = lambda R=8, T=16, r=0.0, rec=FAKE, kr=None: f.kd_full_kl_shard_combine(
        vp(rec) if rec else None, R, None, T, ctypes.c_float(r), vp(FAKE), vp(FAKE), vp(FAKE), kr, None)
    assert comb(R=0) == 1 and comb(T=-1) == 1 and comb(r=1.5) == 1 and comb(r=math.nan) == 1
    assert comb(rec=0) == 1 and comb(rec=FAKE + 8) == 3 and comb(kr=vp(FAKE + 2)) == 3
    assert comb(R=1 << 20, T=1 << 12) == 2
    assert comb(T=0) == 0
    bwd = lambda dH=FAKE: f.kd_full_kl_bwd_shard(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(1.0),
                                                 None, 8, 64, 64, 256, kdl.KD_BF16, vp(FAKE), vp(FAKE), None,
                                                 vp(FAKE), vp(dH) if dH else None, vp(FAKE), 0, vp(FAKE), 16, None)
    assert bwd(dH=0) == 1 and bwd(dH=FAKE + 8) == 3 and bwd() == 4


# ---------------------------------------------------------------- the forward without a workspace
def noalloc(T=8, d=64, V=256, K=4, dt=kdl.KD_BF16, tau=1.0, kl=FAKE):
    vp = ctypes.c_void_p
    return kdl.lib().kd_topk_kl_fwd_noalloc(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, ctypes.c_float(tau), T, d,
                                            V, K, dt, vp(kl) if kl else None, vp(FAKE), None, None)


def test_noalloc_forward_rejects_shapes_beyond_its_scratch(L):
    # checked on the host before the scratch array is looked up or anything is
    # enqueued: 64 MiB holds the forward of ~37,000 rows of the output head
    assert noalloc(T=200000, d=3072, V=128256, K=64) == 2
    msg = last_error()
    assert "KD_NOALLOC_SCRATCH_BYTES" in msg and "needs" in msg
    assert noalloc(T=-1) == 1
    assert noalloc(tau=0.0) == 1
    assert noalloc(K=0) == 1
    assert noalloc(d=12) == 2
    assert noalloc(T=0) == 0  # nothing to do, nothing touched
    assert kdl.KD_NOALLOC_SCRATCH_BYTES == 64 << 20

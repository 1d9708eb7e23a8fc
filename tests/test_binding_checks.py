"""The Python binding checks shapes, dtypes and devices before it takes any
pointer: the C ABI sees only pointers and sizes, so a short topk_logits, a W of
the wrong width or int64 indices would otherwise be read on the device as if
they were right.  Every case here runs on the CPU: a call whose arguments pass
the checks stops at the "must be on the GPU" test that follows them, so each
rejection is told apart from that one by its message."""
import pytest
import torch

kd = pytest.importorskip("chunked_kl_loss_logit_amd")
B = kd._binding

T, D, V, K, DT = 6, 16, 40, 4, 24
bf, f32, i32, u8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8


def z(*shape, dtype=f32, device="cpu"):
    return torch.zeros(*shape, dtype=dtype, device=device)


def on_gpu_only(fn):
    """The arguments passed every check: the call stops at the device test."""
    with pytest.raises(ValueError, match="on the GPU"):
        fn()


def rejected(fn, err, match):
    with pytest.raises(err, match=match):
        fn()


# ---------------------------------------------------------------- top-K forward
def topk_fwd_args(**over):
    a = dict(H=z(T, D, dtype=bf), W=z(D, V, dtype=bf), topk_idx=z(T, K, dtype=i32), topk_logits=z(T, K),
             mask=z(T, dtype=u8), tau=1.0, kl=z(T), lse=z(T), z_topk=z(T, K), workspace=z(64, dtype=u8))
    a.update(over)
    return a


def test_topk_fwd_good_arguments_reach_the_device_test():
    on_gpu_only(lambda: B.kd_topk_kl_fwd(**topk_fwd_args()))
    on_gpu_only(lambda: B.kd_topk_kl_fwd(**topk_fwd_args(mask=None, z_topk=None)))
    on_gpu_only(lambda: B.kd_topk_kl_fwd(**topk_fwd_args(mask=z(T, dtype=torch.bool))))
    on_gpu_only(lambda: B.kd_topk_kl_fwd(**topk_fwd_args(H=z(T, D), W=z(D, V))))  # fp32 head


@pytest.mark.parametrize("over,err,match", [
    (dict(topk_idx=z(T, K, dtype=torch.int64)), TypeError, r"topk_idx must be torch.int32.*\.int\(\)"),
    (dict(topk_logits=z(T, K, dtype=bf)), TypeError, "topk_logits must be torch.float32"),
    (dict(topk_logits=z(T, K - 1)), ValueError, "topk_logits must have shape"),
    (dict(topk_idx=z(T + 1, K, dtype=i32)), ValueError, "topk_idx must have 6 rows"),
    (dict(W=z(D + 8, V, dtype=bf)), ValueError, "W must have 16 rows"),
    (dict(W=z(D, V)), TypeError, "W must be torch.bfloat16"),
    (dict(H=z(T, D, dtype=torch.float16)), TypeError, "H must be"),
    (dict(H=z(T * D, dtype=bf)), ValueError, "H must be 2-D"),
    (dict(mask=z(T + 1, dtype=u8)), ValueError, "mask must have shape"),
    (dict(mask=z(T, dtype=i32)), TypeError, "mask must be"),
    (dict(kl=z(T + 1)), ValueError, "kl must have shape"),
    (dict(kl=None), ValueError, "kl is required"),
    (dict(lse=z(T, dtype=torch.float64)), TypeError, "lse must be torch.float32"),
    (dict(z_topk=z(T, K + 1)), ValueError, "z_topk must have shape"),
    (dict(H=[[0.0] * D] * T), TypeError, "H must be a torch.Tensor"),
    (dict(kl=z(T, device="meta")), ValueError, "one device"),
    (dict(workspace=z(64, dtype=u8, device="meta")), ValueError, "one device"),
])
def test_topk_fwd_rejects(over, err, match):
    rejected(lambda: B.kd_topk_kl_fwd(**topk_fwd_args(**over)), err, match)
    opts = B.topk_opts(tau_rows=z(T))
    rejected(lambda: B.kd_topk_kl_fwd_ex(**{**topk_fwd_args(**over), "opts": opts}), err, match)


@pytest.mark.parametrize("kw,err,match", [
    (dict(tau_rows=z(T + 1)), ValueError, "tau_rows must have shape"),
    (dict(tau_rows=z(T, dtype=bf)), TypeError, "tau_rows must be torch.float32"),
    (dict(teacher_lse=z(T - 1)), ValueError, "teacher_lse must have shape"),
    (dict(labels=z(T, dtype=torch.int64), ce_weight=0.5), TypeError, "labels must be torch.int32"),
    (dict(labels=z(T, 2, dtype=i32), ce_weight=0.5), ValueError, "labels must be 1-D"),
    (dict(tau_rows=z(T, device="meta")), ValueError, "one device"),
    (dict(rev_weight=0.5, z_topk=z(T, K + 1)), ValueError, "z_topk must have shape"),
    (dict(rev_weight=0.5, z_topk=z(T * K)), ValueError, "z_topk must be 2-D"),
    (dict(rev_weight=0.5, z_topk=z(T, K, dtype=bf)), TypeError, "z_topk must be torch.float32"),
])
def test_topk_options_are_checked_against_the_call(kw, err, match):
    def call():
        return B.kd_topk_kl_fwd_ex(**{**topk_fwd_args(), "opts": B.topk_opts(**kw)})
    rejected(call, err, match)


def test_topk_options_good_reach_the_device_test():
    o = B.topk_opts(tau_rows=z(T), teacher_lse=z(T), labels=z(T, dtype=i32), ce_weight=0.25)
    on_gpu_only(lambda: B.kd_topk_kl_fwd_ex(**{**topk_fwd_args(), "opts": o}))
    o = B.topk_opts(rev_weight=0.5, z_topk=z(T, K))
    on_gpu_only(lambda: B.kd_topk_kl_bwd_ex(**{**topk_bwd_args(), "opts": o}))
    assert B.topk_opts() is None


# ---------------------------------------------------------------- top-K backward and single call
def topk_bwd_args(**over):
    a = dict(H=z(T, D, dtype=bf), W=z(D, V, dtype=bf), topk_idx=z(T, K, dtype=i32), topk_logits=z(T, K),
             mask=None, tau=1.0, lse=z(T), grad_kl=z(T), dH=z(T, D, dtype=bf), dW=z(D, V), chunk_rows=0,
             workspace=z(64, dtype=u8))
    a.update(over)
    return a


@pytest.mark.parametrize("over,err,match", [
    (dict(), None, None),
    (dict(dH=z(T, D)), TypeError, "dH must be torch.bfloat16"),
    (dict(dH=z(T, D + 8, dtype=bf)), ValueError, "dH must have shape"),
    (dict(dW=z(D, V, dtype=bf)), TypeError, "dW must be torch.float32"),
    (dict(dW=z(D, V - 8)), ValueError, "dW must have shape"),
    (dict(grad_kl=z(T - 1)), ValueError, "grad_kl must have shape"),
    (dict(lse=None), ValueError, "lse is required"),
    (dict(topk_idx=z(T, K, dtype=torch.int64)), TypeError, "topk_idx must be torch.int32"),
    (dict(dW=z(D, V, device="meta")), ValueError, "one device"),
])
def test_topk_bwd_checks(over, err, match):
    call = lambda: B.kd_topk_kl_bwd(**topk_bwd_args(**over))
    if err is None:
        on_gpu_only(call)
    else:
        rejected(call, err, match)


def single_args(**over):
    a = dict(H=z(T, D, dtype=bf), W=z(D, V, dtype=bf), topk_idx=z(T, K, dtype=i32), topk_logits=z(T, K),
             mask=None, tau=1.0, grad_kl=z(T), kl=z(T), lse=z(T), z_topk=None, dH=z(T, D, dtype=bf), dW=z(D, V),
             chunk_rows=0, workspace=z(64, dtype=u8))
    a.update(over)
    return a


@pytest.mark.parametrize("over,err,match", [
    (dict(), None, None),
    (dict(kl=z(T, 1)), ValueError, "kl must have shape"),
    (dict(dH=z(T, D)), TypeError, "dH must be torch.bfloat16"),
    (dict(topk_logits=z(T, K, dtype=torch.float64)), TypeError, "topk_logits must be torch.float32"),
])
def test_topk_single_call_checks(over, err, match):
    for fn in (B.kd_topk_kl_fwd_bwd, lambda **a: B.kd_topk_kl_fwd_bwd_ex(**a, opts=None)):
        call = lambda: fn(**single_args(**over))
        if err is None:
            on_gpu_only(call)
        else:
            rejected(call, err, match)


# ---------------------------------------------------------------- top-K shards
def test_topk_shard_checks():
    base = dict(H=z(T, D, dtype=bf), W=z(D, V, dtype=bf), v0=8, topk_idx=z(T, K, dtype=i32), topk_logits=z(T, K),
                mask=None, tau=1.0, opts=None, rec=z(T, 4), trow=z(T, 2), z_topk=None, workspace=z(64, dtype=u8))
    on_gpu_only(lambda: B.kd_topk_kl_fwd_shard(**base))
    rejected(lambda: B.kd_topk_kl_fwd_shard(**{**base, "rec": z(T, 2)}), ValueError, "rec must have shape")
    rejected(lambda: B.kd_topk_kl_fwd_shard(**{**base, "trow": z(T, 4)}), ValueError, "trow must have shape")
    comb = dict(rec=z(8, T, 4), trow=z(T, 2), mask=None, kl=z(T), lse=z(T))
    on_gpu_only(lambda: B.kd_topk_kl_shard_combine(**comb))
    rejected(lambda: B.kd_topk_kl_shard_combine(**{**comb, "rec": z(T, 4)}), ValueError, "rec must have shape")
    rejected(lambda: B.kd_topk_kl_shard_combine(**{**comb, "trow": z(T + 1, 2)}), ValueError, "trow must have")
    bw = dict(topk_bwd_args(dH=z(T, D)), v0=8, opts=None)
    on_gpu_only(lambda: B.kd_topk_kl_bwd_shard(**bw))
    # a shard's dH is an fp32 partial, whatever the head's dtype
    rejected(lambda: B.kd_topk_kl_bwd_shard(**{**bw, "dH": z(T, D, dtype=bf)}), TypeError, "dH must be torch.float32")


# ---------------------------------------------------------------- full vocabulary
def full_fwd_args(**over):
    a = dict(H=z(T, D, dtype=bf), Ws=z(D, V, dtype=bf), Ht=z(T, DT, dtype=bf), Wt=z(DT, V, dtype=bf), mask=None,
             tau=1.0, kl=z(T), lse_s=z(T), lse_t=z(T), workspace=z(64, dtype=u8))
    a.update(over)
    return a


@pytest.mark.parametrize("over,err,match", [
    (dict(), None, None),
    (dict(Wt=z(DT, V + 8, dtype=bf)), ValueError, "Wt must have shape"),
    (dict(Wt=z(D, V, dtype=bf)), ValueError, "Wt must have shape"),
    (dict(Ht=z(T + 1, DT, dtype=bf)), ValueError, "Ht must have 6 rows"),
    (dict(Ht=z(T, DT)), TypeError, "Ht must be torch.bfloat16"),
    (dict(Ws=z(D, V)), TypeError, "Ws must be torch.bfloat16"),
    (dict(Ws=z(DT, V, dtype=bf)), ValueError, "Ws must have 16 rows"),
    (dict(lse_t=z(2 * T)), ValueError, "lse_t must have shape"),
    (dict(mask=z(T, 1, dtype=u8)), ValueError, "mask must have shape"),
    (dict(Wt=z(DT, V, dtype=bf, device="meta")), ValueError, "one device"),
])
def test_full_fwd_checks(over, err, match):
    call = lambda: B.kd_full_kl_fwd(**full_fwd_args(**over))
    if err is None:
        on_gpu_only(call)
    else:
        rejected(call, err, match)
    call_ex = lambda: B.kd_full_kl_fwd_ex(**full_fwd_args(**over), opts=B.full_opts(tau_rows=z(T)), kl_rev=None)
    if err is None:
        on_gpu_only(call_ex)
    else:
        rejected(call_ex, err, match)


def test_full_bwd_and_single_call_checks():
    bw = dict(H=z(T, D, dtype=bf), Ws=z(D, V, dtype=bf), Ht=z(T, DT, dtype=bf), Wt=z(DT, V, dtype=bf), mask=None,
              tau=1.0, lse_s=z(T), lse_t=z(T), grad_kl=z(T), dH=z(T, D, dtype=bf), dWs=z(D, V), chunk_rows=0,
              workspace=z(64, dtype=u8))
    on_gpu_only(lambda: B.kd_full_kl_bwd(**bw))
    rejected(lambda: B.kd_full_kl_bwd(**{**bw, "dWs": z(DT, V)}), ValueError, "dWs must have shape")
    rejected(lambda: B.kd_full_kl_bwd(**{**bw, "dH": z(T, DT, dtype=bf)}), ValueError, "dH must have shape")
    ex = {**bw, "opts": B.full_opts(rev_weight=0.5), "kl_rev": z(T)}
    on_gpu_only(lambda: B.kd_full_kl_bwd_ex(**ex))
    rejected(lambda: B.kd_full_kl_bwd_ex(**{**ex, "kl_rev": z(T + 1)}), ValueError, "kl_rev must have shape")
    rejected(lambda: B.kd_full_kl_bwd_ex(**{**ex, "opts": B.full_opts(tau_rows=z(T - 1))}), ValueError,
             "tau_rows must have shape")
    sc = {k: v for k, v in bw.items() if k not in ("lse_s", "lse_t")}
    sc.update(kl=z(T), lse_s=z(T), lse_t=z(T))
    on_gpu_only(lambda: B.kd_full_kl_fwd_bwd(**sc))
    rejected(lambda: B.kd_full_kl_fwd_bwd(**{**sc, "grad_kl": z(T, dtype=bf)}), TypeError, "grad_kl must be")
    on_gpu_only(lambda: B.kd_full_kl_fwd_bwd_ex(**sc, opts=None, kl_rev=None))
    rejected(lambda: B.kd_full_kl_fwd_bwd_ex(**sc, opts=None, kl_rev=z(T, 2)), ValueError, "kl_rev must have")


def test_full_shard_checks():
    fw = dict(H=z(T, D, dtype=bf), Ws=z(D, V, dtype=bf), Ht=z(T, DT, dtype=bf), Wt=z(DT, V, dtype=bf), mask=None,
              tau=1.0, opts=None, rec=z(T, 8), workspace=z(64, dtype=u8))
    on_gpu_only(lambda: B.kd_full_kl_fwd_shard(**fw))
    rejected(lambda: B.kd_full_kl_fwd_shard(**{**fw, "rec": z(T, 4)}), ValueError, "rec must have shape")
    comb = dict(rec=z(4, T, 8), mask=None, rev_weight=0.0, kl=z(T), lse_s=z(T), lse_t=z(T), kl_rev=None)
    on_gpu_only(lambda: B.kd_full_kl_shard_combine(**comb))
    rejected(lambda: B.kd_full_kl_shard_combine(**{**comb, "rec": z(4, T, 4)}), ValueError, "rec must have shape")
    bw = dict(H=z(T, D, dtype=bf), Ws=z(D, V, dtype=bf), Ht=z(T, DT, dtype=bf), Wt=z(DT, V, dtype=bf), mask=None,
              tau=1.0, opts=None, lse_s=z(T), lse_t=z(T), kl_rev=None, grad_kl=z(T), dH=z(T, D), dWs=z(D, V),
              chunk_rows=0, workspace=z(64, dtype=u8))
    on_gpu_only(lambda: B.kd_full_kl_bwd_shard(**bw))
    rejected(lambda: B.kd_full_kl_bwd_shard(**{**bw, "dH": z(T, D, dtype=bf)}), TypeError, "dH must be torch.float32")


# ---------------------------------------------------------------- the allocating wrappers
def test_wrappers_check_before_allocating_on_the_device():
    # the torch-level wrappers size and allocate with torch, then call the
    # checked mirrors; int64 indices from torch.topk are refused, not reinterpreted
    H, W = z(T, D, dtype=bf), z(D, V, dtype=bf)
    I64 = torch.zeros(T, K, dtype=torch.int64)
    with pytest.raises(TypeError, match="topk_idx must be torch.int32"):
        kd.topk_kl_forward(H, W, I64, z(T, K), workspace=z(64, dtype=u8))

"""The Python binding's argument checks, on the CPU with the library stubbed.

Every tensor a call hands to the C ABI is checked against the call's sizes
(bs, k, num_experts, hidden, capacity_rows) before the library is touched, so
a wrong shape, dtype or length raises ValueError instead of becoming an
out-of-bounds access on the device.  Here the binding's device type is set to
"cpu" and load_library() returns a stub that records calls; each bad variant
must raise and leave the stub uncalled, and the good call must reach it once.
check=True turns status bits written by the (stubbed) call into
MoeStatusError.
"""

import ctypes

import pytest
import torch

import combine_moe_dispatch_layout_amd as moe
import oracle

BS, K, E, H = 600, 8, 64, 256   # 4800 pairs: the layout needs a workspace
WS_BYTES = 4096


class StubLib:
    """Stands in for libmoe_dispatch.so: size queries answer like the real
    library, launches are recorded and return 0 (optionally writing a status
    word first)."""

    def __init__(self):
        self.calls = []
        self.status_to_write = 0

    def moe_dispatch_capacity(self, bs, k, e, align):
        if oracle.check_layout_args(bs, k, e, align) != oracle.OK:
            return -1
        return oracle.capacity(bs, k, e, align)

    def moe_dispatch_layout_workspace_size(self, bs, k, e):
        return WS_BYTES if bs * k > 2048 else 0

    def moe_status_string(self, rc):
        return b"stub"

    def __getattr__(self, name):
        if not name.startswith("moe_"):
            raise AttributeError(name)

        def call(*args):
            self.calls.append(name)
            # the status word the call writes (the layout calls overwrite it)
            ptr = args[STATUS_ARG[name]] if name in STATUS_ARG else None
            if ptr:
                ctypes.c_int32.from_address(ptr).value = self.status_to_write
            return 0
        return call


# Position of the status pointer in each entry point's C signature.
STATUS_ARG = {"moe_dispatch_layout": 8, "moe_dispatch": 14, "moe_dispatch_fused": 16,
              "moe_combine": 14, "moe_combine_fp8": 15, "moe_dispatch_layout_ep": 10,
              "moe_dispatch_layout_replicated": 13, "moe_dispatch_fused_replicated": 20}


@pytest.fixture
def stub(monkeypatch):
    lib = StubLib()
    monkeypatch.setattr(moe, "_DEVICE_TYPE", "cpu")
    monkeypatch.setattr(moe, "load_library", lambda: lib)
    monkeypatch.setattr(moe, "_stream", lambda t: None)
    return lib


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def cap():
    return oracle.capacity(BS, K, E, 128)


def layout_out(e=E, n=BS * K):
    return moe.Layout(i32(e), i32(e + 1), i32(n), i32(1))


def expect_refused(stub, fn, match):
    with pytest.raises(ValueError, match=match):
        fn()
    assert stub.calls == [], "a refused call reached the library"


# ------------------------------------------------------------------ layout

def test_layout_good_call_reaches_the_library(stub):
    moe.moe_dispatch_layout(i32(BS, K), E, out=layout_out(), workspace=torch.zeros(WS_BYTES,
                                                                                   dtype=torch.uint8))
    assert stub.calls == ["moe_dispatch_layout"]


@pytest.mark.parametrize("bad,match", [
    (lambda: moe.moe_dispatch_layout(torch.zeros((BS, K), dtype=torch.int64), E), "int32"),
    (lambda: moe.moe_dispatch_layout(i32(BS * K), E), r"\[BS, K\]"),
    (lambda: moe.moe_dispatch_layout(i32(K, BS).t(), E), "contiguous"),
    (lambda: moe.moe_dispatch_layout(i32(BS, K), E, out=layout_out(n=BS * K - 1)),
     "expand_idx holds"),
    (lambda: moe.moe_dispatch_layout(i32(BS, K), E, out=layout_out(e=E - 1)), "holds"),
    (lambda: moe.moe_dispatch_layout(i32(BS, K), E, out=moe.Layout(
        f32(E), i32(E + 1), i32(BS * K), i32(1))), "expert_counts must be"),
    (lambda: moe.moe_dispatch_layout(i32(BS, K), E, workspace=torch.zeros(
        WS_BYTES - 1, dtype=torch.uint8)), "workspace holds"),
    (lambda: moe.moe_dispatch_layout([[0] * K] * BS, E), "must be a tensor"),
])
def test_layout_refusals(stub, bad, match):
    expect_refused(stub, bad, match)


def test_layout_ep_and_replicated_refusals(stub):
    expect_refused(stub, lambda: moe.moe_dispatch_layout_ep(
        i32(BS, K), E, 8, rank_offsets=i32(8)), "rank_offsets holds")
    expect_refused(stub, lambda: moe.moe_dispatch_layout_replicated(
        i32(BS, K), E, i32(E), i32(2 * E), 7), "replica_offsets holds")
    expect_refused(stub, lambda: moe.moe_dispatch_layout_replicated(
        i32(BS, K), E, i32(E + 1), f32(2 * E), 7), "replica_thresholds must be")
    expect_refused(stub, lambda: moe.moe_dispatch_layout_replicated(
        i32(BS, K), E, i32(E + 1), i32(2 * E), 7, replica_ids=i32(BS, K - 1)),
        "replica_ids holds")
    moe.moe_dispatch_layout_ep(i32(BS, K), E, 8)
    moe.moe_dispatch_layout_replicated(i32(BS, K), E, i32(E + 1),
                                       torch.zeros(2 * E, dtype=torch.uint32), 7)
    assert stub.calls == ["moe_dispatch_layout_ep", "moe_dispatch_layout_replicated"]


# ------------------------------------------------------------------ dispatch

def dispatch_args(**kw):
    args = dict(x=bf16(BS, H), expert_ids=i32(BS, K), expand_idx=i32(BS * K),
                ep_send_counts=i32(E + 1), num_experts=E)
    args.update(kw)
    return args


def test_dispatch_good_calls_reach_the_library(stub):
    moe.moe_dispatch(**dispatch_args())
    moe.moe_dispatch(**dispatch_args(), out_dtype="fp8")
    moe.moe_dispatch(**dispatch_args(), capacity_rows=cap() - 100,   # short buffer: allowed
                     expand_x=bf16(cap() - 100, H))
    assert stub.calls == ["moe_dispatch"] * 3


@pytest.mark.parametrize("kw,match", [
    (dict(expand_x=bf16(cap() - 1, H), capacity_rows=cap()), "expand_x has"),
    (dict(expand_x=bf16(cap(), H + 8)), "columns"),
    (dict(expand_x=torch.zeros((cap(), H), dtype=torch.uint8)), "expand_x must be"),
    (dict(out_dtype="fp8", expand_x=bf16(cap(), H)), "expand_x must be"),
    (dict(out_dtype="fp8", quant_scales=f32(cap() - 1, H // 128)), "quant_scales has"),
    (dict(out_dtype="fp8", quant_scales=f32(cap(), H // 128 + 1)), "columns"),
    (dict(out_dtype="int8"), "out_dtype"),
    (dict(expert_ids=i32(BS - 1, K)), "rows, x has"),
    (dict(expand_idx=i32(BS * K - 1)), "expand_idx holds"),
    (dict(ep_send_counts=i32(E)), "ep_send_counts holds"),
    (dict(status=torch.zeros(1, dtype=torch.int64)), "status must be"),
    (dict(x=torch.zeros((BS, H), dtype=torch.float16)), "x must be"),
    (dict(capacity_rows=-1), "capacity_rows"),
])
def test_dispatch_refusals(stub, kw, match):
    args = dispatch_args()
    extra = {k: v for k, v in kw.items() if k not in args}
    args.update({k: v for k, v in kw.items() if k in args})
    expect_refused(stub, lambda: moe.moe_dispatch(**args, **extra), match)


def test_dispatch_fused_refusals(stub):
    x, ids = bf16(BS, H), i32(BS, K)
    expect_refused(stub, lambda: moe.moe_dispatch_fused(
        x, ids, E, capacity_rows=cap() + 1, expand_x=bf16(cap(), H)), "expand_x has")
    expect_refused(stub, lambda: moe.moe_dispatch_fused(x, i32(BS + 1, K), E), "rows, x has")
    expect_refused(stub, lambda: moe.moe_dispatch_fused(
        x, ids, E, out=layout_out(n=BS * K - 8)), "expand_idx holds")
    expect_refused(stub, lambda: moe.moe_dispatch_fused(
        x, ids, E, workspace=torch.zeros(16, dtype=torch.uint8)), "workspace holds")
    expect_refused(stub, lambda: moe.moe_dispatch_fused_replicated(
        x, ids, E, i32(E + 1), i32(2 * E), 3, capacity_rows=10, expand_x=bf16(9, H)),
        "expand_x has")
    moe.moe_dispatch_fused(x, ids, E)
    moe.moe_dispatch_fused_replicated(x, ids, E, i32(E + 1), i32(2 * E), 3)
    assert stub.calls == ["moe_dispatch_fused", "moe_dispatch_fused_replicated"]


# ------------------------------------------------------------------ combine

def combine_args(**kw):
    args = dict(expand_x=bf16(cap(), H), expert_ids=i32(BS, K), expand_idx=i32(BS * K),
                ep_send_counts=i32(E + 1), expert_scales=f32(BS, K),
                shared_expert_x=bf16(BS, H), num_experts=E)
    args.update(kw)
    return args


def test_combine_good_calls_reach_the_library(stub):
    moe.moe_combine(**combine_args())
    moe.moe_combine(**combine_args(shared_expert_x=None), out=bf16(BS, H))
    moe.moe_combine_fp8(**combine_args(expand_x=torch.zeros((cap(), H), dtype=torch.uint8)),
                        quant_scales=f32(cap(), H // 128))
    assert stub.calls == ["moe_combine", "moe_combine", "moe_combine_fp8"]


@pytest.mark.parametrize("kw,match", [
    (dict(expert_scales=f32(BS * K - 1)), "expert_scales holds"),
    (dict(expert_scales=torch.zeros((BS, K), dtype=torch.float64)), "expert_scales must be"),
    (dict(shared_expert_x=bf16(BS - 1, H)), "shared_expert_x has"),
    (dict(shared_expert_x=bf16(BS, H - 32)), "columns"),
    (dict(expand_idx=i32(BS * K - 1)), "expand_idx holds"),
    (dict(ep_send_counts=i32(E)), "ep_send_counts holds"),
    (dict(expand_x=f32(cap(), H)), "expand_x must be"),
    (dict(out=bf16(BS, H + 32)), r"out must be \["),
    (dict(out=bf16(BS - 1, H)), r"out must be \["),
])
def test_combine_refusals(stub, kw, match):
    args = combine_args()
    extra = {k: v for k, v in kw.items() if k not in args}
    args.update({k: v for k, v in kw.items() if k in args})
    expect_refused(stub, lambda: moe.moe_combine(**args, **extra), match)


def test_combine_fp8_refusals(stub):
    codes = torch.zeros((cap(), H), dtype=torch.uint8)
    expect_refused(stub, lambda: moe.moe_combine_fp8(
        **combine_args(expand_x=codes), quant_scales=f32(cap() - 1, H // 128)), "quant_scales")
    expect_refused(stub, lambda: moe.moe_combine_fp8(
        **combine_args(expand_x=torch.zeros((cap(), 96), dtype=torch.uint8),
                       shared_expert_x=bf16(BS, 96)),
        quant_scales=f32(cap(), 1)), "multiple of 128")


# ------------------------------------------------------------------ check=True

def test_check_raises_on_status_bits(stub):
    stub.status_to_write = moe.MOE_FLAG_GUARD
    with pytest.raises(moe.MoeStatusError, match="GUARD") as err:
        moe.moe_dispatch(**dispatch_args(), check=True)
    assert err.value.flags == moe.MOE_FLAG_GUARD
    stub.status_to_write = moe.MOE_FLAG_ID_RANGE | moe.MOE_FLAG_DUP_ID
    with pytest.raises(moe.MoeStatusError, match="ID_RANGE\\|DUP_ID"):
        moe.moe_dispatch_layout(i32(BS, K), E, check=True)
    stub.status_to_write = moe.MOE_FLAG_GUARD
    with pytest.raises(moe.MoeStatusError):
        moe.moe_combine(**combine_args(), check=True)
    with pytest.raises(moe.MoeStatusError):
        moe.moe_dispatch_fused(bf16(BS, H), i32(BS, K), E, check=True)
    stub.status_to_write = 0
    moe.moe_dispatch_fused(bf16(BS, H), i32(BS, K), E, check=True)   # clean: no raise


def test_check_is_off_by_default(stub):
    stub.status_to_write = moe.MOE_FLAG_GUARD
    moe.moe_dispatch(**dispatch_args(), status=i32(1))
    moe.moe_dispatch_fused(bf16(BS, H), i32(BS, K), E)
    assert stub.calls == ["moe_dispatch", "moe_dispatch_fused"]


def test_prepare_records_one_launch_and_repeats_it(stub):
    """prepare() runs every check and allocates the outputs once, records the
    entry point's one library launch instead of making it, and each call of
    the result makes exactly that launch again."""
    x, ids = bf16(BS, H), i32(BS, K)
    call = moe.prepare(moe.moe_dispatch_fused, x, ids, E, workspace=torch.zeros(WS_BYTES,
                                                                                  dtype=torch.uint8))
    assert stub.calls == []
    lay, ex = call.result
    assert ex.shape == (oracle.capacity(BS, K, E, 128), H)
    for n in range(1, 4):
        assert call() is call.result
        assert stub.calls == ["moe_dispatch_fused"] * n
    with pytest.raises(ValueError):
        moe.prepare(moe.moe_dispatch_fused, x, i32(BS - 1, K), E)   # the checks still run
    with pytest.raises(ValueError):
        moe.prepare(moe.moe_dispatch_layout, ids, E, check=True)     # synchronises: refused
    with pytest.raises(ValueError):
        moe.prepare(moe.moe_dispatch_capacity, BS, K, E)             # launches nothing
    assert stub.calls == ["moe_dispatch_fused"] * 3

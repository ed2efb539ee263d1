"""The Python binding checks every buffer's shape and element type against
q and k before calling the library: the C entry points receive bare pointers
and cannot know buffer sizes, so a mismatched v, o, lse, dO or gradient
buffer would otherwise be read or written out of bounds on the device.

Runs on the CPU: with host tensors a well-formed call gets past every check
and stops at the first device-pointer conversion ("must be a device
tensor"); a malformed one must raise earlier, naming the operand."""

import math

import numpy as np
import pytest
import torch

import segmented_causal_attention_amd as sa

T, HQ, HKV, D = 96, 4, 2, 64
BF, F32 = torch.bfloat16, torch.float32
ITEMS = np.array([[0, 0, T, 0, T]], np.int64)


def qkv(dtype=BF):
    q = torch.zeros(T, HQ, D, dtype=dtype)
    k = torch.zeros(T, HKV, D, dtype=dtype)
    return q, k, torch.zeros_like(k), torch.zeros_like(q)


def stats(odt=BF):
    return torch.zeros(T, HQ, D, dtype=odt), torch.zeros(HQ, T, dtype=F32)


def reaches_device_check(fn):
    with pytest.raises(TypeError, match="must be a device tensor"):
        fn()


# ------------------------------------------------------------------ forward

def test_fwd_well_formed_reaches_device_check():
    q, k, v, _ = qkv()
    o, lse = stats(F32)
    reaches_device_check(lambda: sa.segattn_fwd(q, k, v, ITEMS, o=o, lse=lse))


@pytest.mark.parametrize("what", ["v_shape", "v_dtype", "o_shape", "o_dtype", "lse_shape", "lse_dtype"])
def test_fwd_rejects(what):
    q, k, v, _ = qkv()
    o, lse = stats()
    if what == "v_shape":
        v = torch.zeros(T, HQ, D, dtype=BF)
    elif what == "v_dtype":
        v = v.float()
    elif what == "o_shape":
        o = torch.zeros(T, HKV, D, dtype=BF)
    elif what == "o_dtype":
        o = o.half()
    elif what == "lse_shape":
        lse = torch.zeros(T, HQ, dtype=F32)
    elif what == "lse_dtype":
        lse = lse.double()
    name = what.split("_")[0]
    with pytest.raises((ValueError, TypeError), match=rf"^{name} must"):
        sa.segattn_fwd(q, k, v, ITEMS, o=o, lse=lse)


# ----------------------------------------------------------------- backward

def test_bwd_well_formed_reaches_device_check():
    q, k, v, do = qkv()
    o, lse = stats()
    reaches_device_check(lambda: sa.segattn_bwd(q, k, v, o, lse, do, ITEMS))
    reaches_device_check(lambda: sa.segattn_bwd(q, k, v, o, lse, do, ITEMS, g_dtype=F32, accumulate=True))


@pytest.mark.parametrize("what", ["v_shape", "do_shape", "do_dtype", "o_shape", "lse_shape", "dq_shape",
                                  "dk_dtype", "dv_shape", "dq_dtype"])
def test_bwd_rejects(what):
    q, k, v, do = qkv()
    o, lse = stats()
    g = dict(dq=torch.zeros(T, HQ, D, dtype=F32), dk=torch.zeros(T, HKV, D, dtype=F32),
             dv=torch.zeros(T, HKV, D, dtype=F32))
    if what == "v_shape":
        v = torch.zeros(T + 1, HKV, D, dtype=BF)
    elif what == "do_shape":
        do = torch.zeros(T, HKV, D, dtype=BF)
    elif what == "do_dtype":
        do = do.float()
    elif what == "o_shape":
        o = torch.zeros(T, HQ, D // 2, dtype=BF)
    elif what == "lse_shape":
        lse = torch.zeros(HQ, T - 1, dtype=F32)
    elif what == "dq_shape":
        g["dq"] = torch.zeros(T, HKV, D, dtype=F32)
    elif what == "dk_dtype":
        g["dk"] = g["dk"].to(BF)  # bf16 dK beside fp32 dQ: the kernel would write fp32 past its end
    elif what == "dv_shape":
        g["dv"] = torch.zeros(T, HQ, D, dtype=F32)
    elif what == "dq_dtype":
        g["dq"] = g["dq"].half()
    name = what.split("_")[0]
    with pytest.raises((ValueError, TypeError), match=rf"^{name} must"):
        sa.segattn_bwd(q, k, v, o, lse, do, ITEMS, **g)


def test_bwd_accumulate_needs_fp32():
    q, k, v, do = qkv()
    o, lse = stats()
    with pytest.raises(TypeError, match="accumulate"):
        sa.segattn_bwd(q, k, v, o, lse, do, ITEMS, g_dtype=BF, accumulate=True)


def test_preprocess_rejects():
    q, k, v, do = qkv()
    o, _ = stats()
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    reaches_device_check(lambda: sa.segattn_bwd_preprocess(q, k, o, do, ITEMS, ws))
    with pytest.raises(TypeError, match="^do must"):
        sa.segattn_bwd_preprocess(q, k, o, do.float(), ITEMS, ws)
    with pytest.raises(ValueError, match="^o must"):
        sa.segattn_bwd_preprocess(q, k, o[:, :1], do, ITEMS, ws)
    with pytest.raises(ValueError, match="workspace too small"):
        sa.segattn_bwd_preprocess(q, k, o, do, ITEMS, torch.zeros(16, dtype=torch.uint8))


# -------------------------------------------------------------------- merge

def _partials(rows=T, h=HQ, d=D, stride=None):
    stride = rows if stride is None else stride
    return (torch.zeros(rows, h, d), torch.zeros(h, stride), torch.zeros(rows, h, d), torch.zeros(h, stride))


def test_merge_well_formed_reaches_device_check():
    oa, la, ob, lb = _partials()
    reaches_device_check(lambda: sa.segattn_merge(oa, la, ob, lb))
    oa, la, ob, lb = _partials(stride=T + 32)
    reaches_device_check(lambda: sa.segattn_merge(oa, la, ob, lb, rows=T))
    # a row sub-range of larger partials: lse views keep the full row stride
    r0 = 10
    reaches_device_check(lambda: sa.segattn_merge(oa[r0:], la[:, r0:], ob[r0:], lb[:, r0:], o_out=oa[r0:],
                                                  lse_out=la[:, r0:], rows=T - r0, lse_stride=T + 32))


@pytest.mark.parametrize("what", ["o_b", "o_out", "lse_b", "lse_out", "rows", "stride", "dtype"])
def test_merge_rejects(what):
    oa, la, ob, lb = _partials()
    kw = {}
    if what == "o_b":
        ob = torch.zeros(T, HQ, D + 4)
    elif what == "o_out":
        kw["o_out"] = torch.zeros(T - 1, HQ, D)
    elif what == "lse_b":
        lb = torch.zeros(HQ + 1, T)
    elif what == "lse_out":
        kw["lse_out"] = torch.zeros(HQ, T - 1)
    elif what == "rows":
        kw["rows"] = T + 1
    elif what == "stride":
        kw["lse_stride"] = T + 8
    elif what == "dtype":
        ob = ob.to(BF)
    with pytest.raises((ValueError, TypeError)):
        sa.segattn_merge(oa, la, ob, lb, **kw)


# ------------------------------------------------------------------ prepared forward

def test_fwd_prepare_checks_like_fwd():
    q, k, v, _ = qkv()
    o, lse = stats(F32)
    reaches_device_check(lambda: sa.segattn_fwd_prepare(q, k, v, ITEMS, o=o, lse=lse))
    with pytest.raises(ValueError, match="lse"):
        sa.segattn_fwd_prepare(q, k, v, ITEMS, o=o, lse=torch.zeros(T, HQ, dtype=F32))
    with pytest.raises(TypeError, match="v"):
        sa.segattn_fwd_prepare(q, k, v.float(), ITEMS, o=o, lse=lse)

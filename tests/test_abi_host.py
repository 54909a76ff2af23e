"""Host-side tests of the C ABI (no GPU): the library loads, exports every entry
point include/moe.h declares, rejects bad arguments before touching the device,
and its blob packer round-trips every weight format."""
import ctypes
import os
import re

import numpy as np
import pytest

import expert_grouped_quantized_amd as M
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # an aligned non-null address; only passed where a check must fail first


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(M.LIB_PATH)
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert M.moe_abi_version() == 2
    assert M.moe_status_str(0) == "ok"
    assert M.moe_status_str(-3) == "workspace too small"
    assert M.moe_status_str(12345) == "unknown status"


def _desc(**kw):
    base = dict(d=2560, n_experts=512, ffn=1024, n_shared=1, shared_ffn=1024, act="bf16",
                expert_w="i4g32", shared_w="i8row")
    base.update(kw)
    return M.make_desc(**base)


def _route(desc, T=4, k=10, hidden=FAKE, rw=FAKE, bias=None, logits=FAKE, ids=FAKE, w=FAKE):
    return M.lib().moe_route(ctypes.byref(desc), T, k, hidden, rw, bias, logits, ids, w, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(n_experts=0), M.MOE_EINVAL, "n_experts"),
    (dict(n_experts=1025), M.MOE_EINVAL, "n_experts"),
    (dict(n_shared=2), M.MOE_EINVAL, "n_shared"),
    (dict(d=2500), M.MOE_EUNSUPPORTED, "d % 256"),
    (dict(ffn=1000), M.MOE_EUNSUPPORTED, "ffn"),
    (dict(ffn=1152), M.MOE_EUNSUPPORTED, "4-bit routed experts need ffn % 256"),
    (dict(act="i4g32"), M.MOE_EUNSUPPORTED, "act"),
    (dict(expert_w="i8row"), M.MOE_EUNSUPPORTED, "routed"),
    (dict(shared_w="i4g32"), M.MOE_EUNSUPPORTED, "shared"),
    (dict(act="f32"), M.MOE_EUNSUPPORTED, "F32"),
])
def test_desc_validation(kw, status, msg):
    rc = _route(_desc(**kw))
    assert rc == status
    assert msg in M.moe_last_error()


def test_null_desc():
    assert M.lib().moe_route(None, 4, 2, FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == M.MOE_EINVAL
    assert "desc is NULL" in M.moe_last_error()


@pytest.mark.parametrize("T,k,msg", [(-1, 10, "negative"), (4, 0, "k=0"), (4, 33, "k=33"),
                                     (1 << 27, 10, "2^30")])
def test_T_and_k_validation(T, k, msg):
    assert _route(_desc(), T=T, k=k) == M.MOE_EINVAL
    assert msg in M.moe_last_error()


def test_k_above_E_rejected():
    assert _route(_desc(n_experts=4), k=5) == M.MOE_EINVAL


@pytest.mark.parametrize("field", ["hidden", "rw", "logits", "ids", "w"])
def test_null_and_misaligned_pointers(field):
    assert _route(_desc(), **{field: None}) == M.MOE_EINVAL
    assert "NULL" in M.moe_last_error()
    assert _route(_desc(), **{field: FAKE + 4}) == M.MOE_EINVAL
    assert "aligned" in M.moe_last_error()


def test_T_zero_is_ok_and_launches_nothing():
    # no GPU here: any launch would fail, so OK proves nothing was enqueued
    assert _route(_desc(), T=0) == M.MOE_OK
    desc = _desc()
    ws = M.moe_workspace_bytes(desc, 0, 10)
    L = M.lib()
    assert L.moe_permute(ctypes.byref(desc), 0, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws,
                         None) == 0
    assert L.moe_combine(ctypes.byref(desc), 0, 10, FAKE, FAKE, FAKE, FAKE, None) == 0


def test_workspace_too_small():
    desc = _desc()
    need = M.moe_workspace_bytes(desc, 64, 10)
    rc = M.lib().moe_permute(ctypes.byref(desc), 64, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             need - 1, None)
    assert rc == M.MOE_EWORKSPACE
    assert "workspace" in M.moe_last_error()
    rc = M.lib().moe_permute(ctypes.byref(desc), 64, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16,
                             need, None)
    assert rc == M.MOE_EINVAL  # workspace must be 256-byte aligned
    rc = M.lib().moe_permute(ctypes.byref(desc), 64, 10, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                             need, None)
    assert rc == M.MOE_EINVAL and "hidden" in M.moe_last_error()



def _route_plan(desc, T=16, k=10, ws_bytes=None, **ptrs):
    p = dict(hidden=FAKE, rw=FAKE, bias=None, logits=FAKE, ids=FAKE, w=FAKE, offsets=FAKE,
             perm=FAKE, inv=FAKE, ws=FAKE)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = M.moe_workspace_bytes(desc, T, k)
    return M.lib().moe_route_plan(ctypes.byref(desc), T, k, p["hidden"], p["rw"], p["bias"],
                                  p["logits"], p["ids"], p["w"], p["offsets"], p["perm"],
                                  p["inv"], p["ws"], ws_bytes, None)


@pytest.mark.parametrize("field", ["hidden", "rw", "logits", "ids", "w", "offsets", "perm", "inv"])
def test_route_plan_pointer_checks(field):
    assert _route_plan(_desc(), **{field: None}) == M.MOE_EINVAL
    assert "NULL" in M.moe_last_error()
    assert _route_plan(_desc(), **{field: FAKE + 4}) == M.MOE_EINVAL
    assert "aligned" in M.moe_last_error()


def test_route_plan_workspace_and_T_zero():
    desc = _desc()
    for T in (16, 32, 33, 4096):
        need = M.moe_workspace_bytes(desc, T, 10)
        assert _route_plan(desc, T=T, ws_bytes=need - 1) == M.MOE_EWORKSPACE
        assert "workspace" in M.moe_last_error()
        assert _route_plan(desc, T=T, ws=FAKE + 16) == M.MOE_EINVAL  # 256-byte alignment
    assert _route_plan(desc, k=0, ws_bytes=1 << 30) == M.MOE_EINVAL
    # no GPU here: any launch would fail, so OK proves nothing was enqueued
    assert _route_plan(desc, T=0) == M.MOE_OK


def test_shared_pointers_must_match_n_shared():
    desc = _desc(n_shared=0)
    ws = M.moe_workspace_bytes(desc, 8, 10)
    rc = M.lib().moe_grouped_ffn(ctypes.byref(desc), 8, 10, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, FAKE, FAKE, ws, None)
    assert rc == M.MOE_EINVAL and "n_shared == 0" in M.moe_last_error()


def test_workspace_grows_with_T():
    desc = _desc()
    sizes = [M.moe_workspace_bytes(desc, T, 10) for T in (1, 16, 512, 4096, 16384)]
    assert sizes == sorted(sizes)
    # holds at least h (bf16) for every routed and shared row
    assert sizes[3] >= (4096 * 10 * 1024 + 4096 * 1024) * 2


def test_blob_bytes_formulas():
    desc = _desc()
    r = M.moe_blob_bytes(desc, M.MOE_BLOB_ROUTED)
    s = M.moe_blob_bytes(desc, M.MOE_BLOB_SHARED)
    per_w = 3 * 1024 * 2560
    assert r == 512 * per_w * 9 // 16            # int4 codes + one fp16 per 32 weights
    assert s == per_w + 2 * 2 * 1024 + 2 * 2560  # int8 codes + one fp16 per row
    assert M.moe_blob_bytes(_desc(expert_w="bf16"), 0) == 512 * per_w * 2


def _rand_expert(fmt, rows, K, n, rng):
    w = rng.standard_normal((n, rows, K)).astype(np.float32) * 0.05
    parts = [W.store(w[i], fmt) for i in range(n)]
    q = np.stack([p[0] for p in parts])
    s = None if parts[0][1] is None else np.stack([p[1] for p in parts])
    return q, s


@pytest.mark.parametrize("act,fmt,kind", [("bf16", "bf16", 0), ("bf16", "i4g32", 0),
                                          ("bf16", "i8row", 1), ("bf16", "bf16", 1),
                                          ("f32", "f32", 0), ("f32", "f32", 1)]
                         + [("bf16", f, 0) for f in W.IG32.values()] + [("bf16", "mxfp4", 0)])
def test_pack_unpack_roundtrip(act, fmt, kind):
    rng = np.random.default_rng(hash((act, fmt, kind)) % 2**32)
    d, F, E = (256, 256, 3) if act == "bf16" else (128, 64, 2)
    desc = M.make_desc(d, E, F, 1, F, act=act, expert_w=fmt if kind == 0 else act,
                       shared_w=fmt if kind == 1 else act)
    n = E if kind == 0 else 1
    g, gs = _rand_expert(fmt, F, d, n, rng)
    u, us = _rand_expert(fmt, F, d, n, rng)
    dn, ds = _rand_expert(fmt, d, F, n, rng)
    if kind == 1:
        g, u, dn = g[0], u[0], dn[0]
        gs, us, ds = (None if x is None else x[0] for x in (gs, us, ds))
    blob = np.empty(M.moe_blob_bytes(desc, kind), np.uint8)
    M.moe_pack_experts(desc, kind, g, gs, u, us, dn, ds, blob)
    outs = [np.zeros_like(a) if a is not None else None for a in (g, gs, u, us, dn, ds)]
    M.moe_unpack_experts(desc, kind, blob, *outs)
    for a, b in zip((g, gs, u, us, dn, ds), outs):
        if a is not None:
            assert np.array_equal(a, b)
    # the blob is a permutation of the information: every byte is determined
    assert blob.nbytes == M.moe_blob_bytes(desc, kind)


@pytest.mark.parametrize("d,F", [(16384, 256), (256, 16384)])
@pytest.mark.parametrize("fmt,kind", [("bf16", 0), ("i4g32", 0), ("i8row", 1), ("mxfp4", 0)]
                         + [(f, 0) for f in W.IG32.values()])
def test_pack_unpack_roundtrip_max_widths(fmt, kind, d, F):
    """Round trip at the largest widths the ABI takes (d or ffn = 16384): the
    tile and bit-stream offsets of the packer span the whole index range."""
    rng = np.random.default_rng(abs(hash((fmt, kind, d))) % 2**32)
    desc = M.make_desc(d, 1, F, 1, F, act="bf16", expert_w=fmt if kind == 0 else "bf16",
                       shared_w=fmt if kind == 1 else "bf16")
    g, gs = _rand_expert(fmt, F, d, 1, rng)
    u, us = _rand_expert(fmt, F, d, 1, rng)
    dn, ds = _rand_expert(fmt, d, F, 1, rng)
    if kind == 1:
        g, u, dn = g[0], u[0], dn[0]
        gs, us, ds = (None if x is None else x[0] for x in (gs, us, ds))
    blob = np.empty(M.moe_blob_bytes(desc, kind), np.uint8)
    M.moe_pack_experts(desc, kind, g, gs, u, us, dn, ds, blob)
    outs = [np.zeros_like(a) if a is not None else None for a in (g, gs, u, us, dn, ds)]
    M.moe_unpack_experts(desc, kind, blob, *outs)
    for a, b in zip((g, gs, u, us, dn, ds), outs):
        if a is not None:
            assert np.array_equal(a, b)


def test_pack_rejects_int4_minus_eight():
    desc = M.make_desc(256, 1, 256, 0, 0, act="bf16", expert_w="i4g32")
    q = np.zeros((1, 256, 256), np.int8)
    q[0, 5, 7] = -8
    g = W.pack_int4(q)
    s = np.full((1, 256, 8), 0x3C00, np.uint16)
    dq = W.pack_int4(np.zeros((1, 256, 256), np.int8))
    dsc = np.full((1, 256, 8), 0x3C00, np.uint16)
    blob = np.empty(M.moe_blob_bytes(desc, 0), np.uint8)
    with pytest.raises(M.MoeError) as ei:
        M.moe_pack_experts(desc, 0, g, s, g, s, dq, dsc, blob)
    assert ei.value.status == M.MOE_EINVAL and "outside [-7, 7]" in str(ei.value)


@pytest.mark.parametrize("b", sorted(W.IG32))
def test_pack_rejects_codes_outside_the_symmetric_range(b):
    lim = (1 << (b - 1)) - 1
    desc = M.make_desc(256, 1, 256, 0, 0, act="bf16", expert_w=W.IG32[b])
    s = np.full((1, 256, 8), 0x3C00, np.uint16)
    z = np.zeros((1, 256, 256), np.int8)
    blob = np.empty(M.moe_blob_bytes(desc, 0), np.uint8)
    M.moe_pack_experts(desc, 0, z + lim, s, z - lim, s, z, s, blob)  # the extremes are fine
    for bad in (lim + 1, -lim - 1):
        if not -128 <= bad <= 127:  # 8-bit: only -128 lies outside and fits a byte
            continue
        q = z.copy()
        q[0, 3, 200] = bad
        with pytest.raises(M.MoeError) as ei:
            M.moe_pack_experts(desc, 0, z, s, z, s, q, s, blob)
        assert ei.value.status == M.MOE_EINVAL and f"[{-lim}, {lim}]" in str(ei.value)


@pytest.mark.parametrize("b", sorted(W.IG32))
def test_blob_bytes_of_bbit_codes(b):
    desc = _desc(expert_w=W.IG32[b])
    per_w = 3 * 1024 * 2560
    # b bits per weight plus one fp16 scale per 32 weights, nothing else
    assert M.moe_blob_bytes(desc, M.MOE_BLOB_ROUTED) == 512 * per_w * (2 * b + 1) // 16


def test_bbit_formats_only_for_routed_weights_and_2bit_needs_ffn_256():
    with pytest.raises(M.MoeError) as ei:
        M.moe_blob_bytes(_desc(shared_w="i5g32"), 0)
    assert ei.value.status == M.MOE_EUNSUPPORTED
    with pytest.raises(M.MoeError) as ei:
        M.moe_blob_bytes(M.make_desc(256, 4, 384, 0, 0, act="bf16", expert_w="i2g32"), 0)
    assert ei.value.status == M.MOE_EUNSUPPORTED and "256" in str(ei.value)
    M.moe_blob_bytes(M.make_desc(256, 4, 384, 0, 0, act="bf16", expert_w="i3g32"), 0)


def test_mxfp4_blob_bytes_rejections_and_width():
    """MXFP4: 4 bits a weight plus one E8M0 byte per 32; routed weights only;
    d and ffn multiples of 256; a NaN scale (255) is rejected."""
    per_w = 3 * 1024 * 2560
    assert M.moe_blob_bytes(_desc(expert_w="mxfp4"), M.MOE_BLOB_ROUTED) == 512 * per_w * 17 // 32
    with pytest.raises(M.MoeError) as ei:
        M.moe_blob_bytes(_desc(shared_w="mxfp4"), 0)
    assert ei.value.status == M.MOE_EUNSUPPORTED
    with pytest.raises(M.MoeError) as ei:
        M.moe_blob_bytes(M.make_desc(256, 4, 384, 0, 0, act="bf16", expert_w="mxfp4"), 0)
    assert ei.value.status == M.MOE_EUNSUPPORTED and "256" in str(ei.value)
    desc = M.make_desc(256, 2, 256, 0, 0, act="bf16", expert_w="mxfp4")
    q = np.zeros((2, 256, 128), np.uint8)
    s = np.full((2, 256, 8), 127, np.uint8)
    blob = np.empty(M.moe_blob_bytes(desc, 0), np.uint8)
    M.moe_pack_experts(desc, 0, q, s, q, s, q, s, blob)
    bad = s.copy()
    bad[1, 17, 3] = 255
    with pytest.raises(M.MoeError) as ei:
        M.moe_pack_experts(desc, 0, q, s, q, s, q, bad, blob)
    assert ei.value.status == M.MOE_EINVAL and "expert 1" in str(ei.value) and "255" in str(ei.value)


def _i4_expert_arrays(desc, scale_bits):
    """One int4 expert (d=256, F=256) with every code 7 and every group scale
    set to the fp16 bit pattern scale_bits."""
    d, F = desc.d, desc.ffn
    q = np.full((desc.n_experts, F, d // 2), 0x77, np.uint8)
    qd = np.full((desc.n_experts, d, F // 2), 0x77, np.uint8)
    sg = np.full((desc.n_experts, F, d // 32), scale_bits, np.uint16)
    sd = np.full((desc.n_experts, d, F // 32), scale_bits, np.uint16)
    return q, sg, qd, sd


@pytest.mark.parametrize("scale,ok", [(9352.0, True), (9360.0, False), (65504.0, False),
                                      (2.0 ** -24, True), (2.0 ** -16, True), (1.0, True),
                                      (np.inf, False), (np.nan, False), (-9352.0, True),
                                      (-9360.0, False)])
def test_pack_checks_int4_group_scales(scale, ok):
    """A group scale must be finite and keep 7 * scale finite in fp16 (the
    gate/up products take fp16(code * scale) as their weights)."""
    desc = _desc(d=256, ffn=256, n_experts=2, n_shared=0, shared_ffn=0)
    bits = int(np.array([scale], np.float16).view(np.uint16)[0])
    q, sg, qd, sd = _i4_expert_arrays(desc, bits)
    blob = np.empty(M.moe_blob_bytes(desc, 0), np.uint8)
    if ok:
        M.moe_pack_experts(desc, 0, q, sg, q, sg, qd, sd, blob)
    else:
        with pytest.raises(M.MoeError) as ei:
            M.moe_pack_experts(desc, 0, q, sg, q, sg, qd, sd, blob)
        assert ei.value.status == M.MOE_EINVAL
        assert "group scale" in str(ei.value)


@pytest.mark.parametrize("b,scale,ok", [(8, 515.5, True), (8, 516.0, False), (2, 65504.0, True),
                                        (2, np.inf, False), (5, 4364.0, True),
                                        (5, 4368.0, False)])
def test_pack_checks_bbit_group_scales(b, scale, ok):
    desc = _desc(d=256, ffn=256, n_experts=1, n_shared=0, shared_ffn=0, expert_w=W.IG32[b])
    d, F = 256, 256
    bits = int(np.array([scale], np.float16).view(np.uint16)[0])
    q = np.ones((1, F, d), np.int8)
    qd = np.ones((1, d, F), np.int8)
    sg = np.full((1, F, d // 32), bits, np.uint16)
    sd = np.full((1, d, F // 32), bits, np.uint16)
    blob = np.empty(M.moe_blob_bytes(desc, 0), np.uint8)
    if ok:
        M.moe_pack_experts(desc, 0, q, sg, q, sg, qd, sd, blob)
    else:
        with pytest.raises(M.MoeError, match="group scale"):
            M.moe_pack_experts(desc, 0, q, sg, q, sg, qd, sd, blob)


@pytest.mark.parametrize("scale,ok", [(65504.0, True), (np.inf, False), (np.nan, False)])
def test_pack_checks_int8_row_scales(scale, ok):
    desc = _desc(d=256, ffn=256, n_experts=1, n_shared=1, shared_ffn=256)
    d, Fs = 256, 256
    bits = int(np.array([scale], np.float16).view(np.uint16)[0])
    q = np.ones((Fs, d), np.int8)
    qd = np.ones((d, Fs), np.int8)
    s1 = np.full(Fs, 0x3c00, np.uint16)
    s1[17] = bits
    sd = np.full(d, 0x3c00, np.uint16)
    blob = np.empty(M.moe_blob_bytes(desc, 1), np.uint8)
    if ok:
        M.moe_pack_experts(desc, 1, q, s1, q, s1, qd, sd, blob)
    else:
        with pytest.raises(M.MoeError, match="row scale"):
            M.moe_pack_experts(desc, 1, q, s1, q, s1, qd, sd, blob)

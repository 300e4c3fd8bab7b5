"""Host-side checks of the C ABI, no GPU needed: the library loads, exports
every function include/muon.h declares, and rejects invalid plans and calls
with the documented status before touching any device memory."""
import ctypes
import os
import re

import numpy as np
import pytest

from matrix_aware_optimizer_muon_amd import _lib as L
from matrix_aware_optimizer_muon_amd import workloads as WL

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "muon.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert set(names) == set(L.EXPORTED), names


def test_library_exports_every_declared_symbol():
    lib = L.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_default_hparams_are_the_pages_values():
    hp = L.default_hparams()
    assert hp.momentum == pytest.approx(0.95) and hp.nesterov == 1 and hp.ns_steps == 5
    assert (hp.a, hp.b, hp.c) == pytest.approx((3.4445, -4.7750, 2.0315))
    assert hp.scale_coeff == pytest.approx(0.2) and hp.rownorm_eps == pytest.approx(1e-8)


def test_status_strings():
    for code, name in [(0, "MUON_OK"), (1, "MUON_ERR_INVALID_ARGUMENT"), (2, "MUON_ERR_UNSUPPORTED"),
                       (3, "MUON_ERR_WORKSPACE_TOO_SMALL"), (4, "MUON_ERR_HIP")]:
        assert L.status_string(code) == name


def plan_status(shapes, **kw):
    try:
        L.Plan(shapes, **kw)
        return 0
    except L.MuonError as e:
        return e.status


def test_plan_rejects_bad_descriptions():
    assert plan_status([]) == L.MUON_ERR_INVALID_ARGUMENT
    assert plan_status([(0, 5)]) == L.MUON_ERR_INVALID_ARGUMENT
    assert plan_status([(5, -1)]) == L.MUON_ERR_INVALID_ARGUMENT
    assert plan_status([(1 << 25, 4)]) == L.MUON_ERR_UNSUPPORTED
    assert plan_status([(70000, 70000)]) == L.MUON_ERR_UNSUPPORTED
    hp = L.default_hparams(); hp.ns_steps = 0
    assert plan_status([(4, 4)], hp=hp) == L.MUON_ERR_INVALID_ARGUMENT
    hp = L.default_hparams(); hp.ns_steps = 17
    assert plan_status([(4, 4)], hp=hp) == L.MUON_ERR_UNSUPPORTED
    assert plan_status([(4, 4)], ns_dtype="f32", hp=hp) == L.MUON_ERR_UNSUPPORTED
    # the 16-bit path stops at N = 12 (its accuracy bound), the fp32 path at 16
    hp = L.default_hparams(); hp.ns_steps = 13
    assert plan_status([(4, 4)], hp=hp) == L.MUON_ERR_UNSUPPORTED
    assert plan_status([(4, 4)], ns_dtype="f32", hp=hp) == 0
    hp = L.default_hparams(); hp.ns_steps = 16
    assert plan_status([(4, 4)], ns_dtype="f32", hp=hp) == 0
    hp = L.default_hparams(); hp.ns_steps = 12
    assert plan_status([(4, 4)], hp=hp) == 0
    hp = L.default_hparams(); hp.rownorm_eps = 0.0
    assert plan_status([(4, 4)], hp=hp) == L.MUON_ERR_INVALID_ARGUMENT
    hp = L.default_hparams(); hp.momentum = float("nan")
    assert plan_status([(4, 4)], hp=hp) == L.MUON_ERR_INVALID_ARGUMENT
    assert plan_status([(4, 4)], max_workspace_bytes=-1) == L.MUON_ERR_INVALID_ARGUMENT
    lib = L.load()
    h = ctypes.c_void_p()
    assert lib.muon_plan(None, ctypes.byref(h), None) == L.MUON_ERR_INVALID_ARGUMENT
    desc = L.PlanDesc(); desc.num_matrices = 1; desc.grad_dtype = 7
    assert lib.muon_plan(ctypes.byref(desc), ctypes.byref(h), None) == L.MUON_ERR_INVALID_ARGUMENT


def test_plan_buckets_and_chunks():
    p = L.Plan(WL.config(3).shapes)
    assert p.info() == (4, 4)  # 3584^2, 512x3584, 18944x3584, 3584x18944
    p4 = L.Plan(WL.config(4).shapes, grad_dtype="bf16")
    nb, nc = p4.info()
    assert nb == 4 and nc >= 4
    small = L.Plan(WL.config(4).shapes, grad_dtype="bf16", max_workspace_bytes=1)
    assert small.info() == (4, 196)  # a single matrix always fits
    assert small.workspace_bytes < p4.workspace_bytes
    p2 = L.Plan(WL.config(2).shapes)
    assert p2.info() == (2, 2)


def test_fused_recursion_rule():
    # the one-launch r x r recursion: Gram form on the 16-bit path with tiles
    # below 256 and r padded to <= 128
    b2 = {tuple(b["shape"]): b for b in L.Plan(WL.config(2).shapes).buckets()}
    assert b2[(128, 3584)]["fused"] and b2[(128, 3584)]["tile"] == 64
    # square: the direct form, as one launch (padded squares of 128 / 256)
    assert b2[(256, 256)]["fused"] and b2[(256, 256)]["formulation"] == "direct"
    assert not any(b["fused"] for b in L.Plan(WL.config(3).shapes).buckets())
    assert not L.Plan([(128, 3584)], ns_dtype="f32").buckets()[0]["fused"]  # fp32 path
    assert L.Plan([(3584, 64)]).buckets()[0]["fused"]  # tall: r = 64
    assert not L.Plan([(200, 900)]).buckets()[0]["fused"]  # r_pad = 256
    assert L.Plan([(64, 80)]).buckets()[0]["fused"]  # c > 1.125 r: Gram form
    assert not L.Plan([(64, 72)]).buckets()[0]["fused"]  # near-square: direct form


def test_fused_direct_rule():
    # the one-launch direct form: padded squares of 128 or 256 (rows <= cols)
    # on the small-tile 16-bit path
    def b(shapes, **kw):
        return L.Plan(shapes, **kw).buckets()[0]
    assert b([(256, 256)] * 64)["formulation"] == "direct" and b([(256, 256)] * 64)["fused"]
    assert b([(120, 128)])["fused"] and b([(250, 256)])["fused"] and b([(100, 110)])["fused"]
    assert not b([(240, 270)])["fused"]  # direct, but c_pad 320 != r_pad 256
    assert not b([(64, 64)])["fused"]  # r_pad 64
    assert not b([(256, 256)], ns_dtype="f32")["fused"]  # fp32 path
    assert not b([(3584, 3584)] * 2)["fused"]  # 256-wide tiles
    assert not b([(256, 256)], hints={(256, 256): {"tile": 256}})["fused"]
    assert b([(256, 256)], hints={(256, 256): {"tile": 128}})["fused"]


def _scales(n, ns_dtype="bf16", **coef):
    hp = L.default_hparams()
    hp.ns_steps = n
    for k, v in coef.items():
        setattr(hp, k, v)
    return L.Plan([(100, 900)], ns_dtype=ns_dtype, hp=hp).buckets()[0]["scales"]


def test_operand_scales_follow_the_iteration_bounds():
    # Default coefficients: p(g) = a + b g + c g^2 peaks at g = 0 on the
    # singular-value range, so Q = P_N...P_1 is bounded by a^N (reached in
    # padding and rank-deficient directions) and its fp16 scale is the
    # largest power of two with 1.05 a^N s <= 65504, capped at 64; the other
    # bounds do not depend on N and keep their scales.
    a = float(np.float32(3.4445))
    assert _scales(5) == (16384.0, 16384.0, 8192.0, 64.0, 256.0)
    for n in range(1, 13):
        expect = 64.0
        while 1.05 * a ** n * expect > 65504.0:
            expect /= 2
        s = _scales(n)
        assert s[3] == expect, (n, s)
        assert (s[0], s[1], s[4]) == (16384.0, 16384.0, 256.0)
    assert _scales(8)[3] == 2.0 and _scales(12)[3] == 2.0 ** -6
    assert _scales(5, ns_dtype="f32") == (1.0,) * 5


def test_coefficients_the_16bit_path_cannot_scale():
    # c = 0 (a cubic): the 256-tile quintic product folds b G into c G^2 as
    # (b / c) G; the fp32 path takes it
    assert plan_status([(4, 4)], hp=_hp(c=0.0)) == L.MUON_ERR_UNSUPPORTED
    assert plan_status([(4, 4)], ns_dtype="f32", hp=_hp(c=0.0)) == 0
    # an iteration that grows without limit (f(1) = 4 and beyond): no fp16
    # scale holds it
    assert plan_status([(4, 4)], hp=_hp(a=2.0, b=1.0, c=1.0)) == L.MUON_ERR_UNSUPPORTED
    # the cubic of classic Newton-Schulz written as a quintic with a tiny c
    s = _scales(5, a=1.5, b=-0.5, c=1e-6)
    assert all(v >= 2.0 ** -14 for v in s)


def _hp(**coef):
    hp = L.default_hparams()
    for k, v in coef.items():
        setattr(hp, k, v)
    return hp


def test_default_cap_keeps_the_qwen_buckets_whole():
    # The default 32 GiB scratch cap holds the largest Qwen2.5-7B bucket
    # (56 x 18944 x 3584, ~401 MB of scratch per matrix) in one chunk; a
    # 16 GiB cap splits it into two equal chunks of 28.
    p4 = L.Plan(WL.config(4).shapes, grad_dtype="bf16")
    assert [b["chunks"] for b in p4.buckets()] == [1, 1, 1, 1]
    assert p4.workspace_bytes <= 32 << 30
    p16 = L.Plan(WL.config(4).shapes, grad_dtype="bf16", max_workspace_bytes=16 << 30)
    assert {tuple(b["shape"]): b["chunks"] for b in p16.buckets()}[(18944, 3584)] == 2
    assert p16.workspace_bytes < p4.workspace_bytes


def test_step_validation_happens_before_device_work():
    # Fake (never dereferenced) device pointers: every call must fail in host
    # validation, so nothing reaches the GPU (none exists here).
    p = L.Plan([(16, 32), (32, 16)])
    fake = [0x1000, 0x2000]
    ws = 0x10000
    lib = L.load()

    def call(fn, W, M, G, lr=0.02, wd=0.1, wsp=ws, wsb=None):
        wsb = p.workspace_bytes if wsb is None else wsb
        try:
            fn(W, M, G, lr, wd, wsp, wsb)
            return 0
        except L.MuonError as e:
            return e.status

    for fn in (p.step_ptrs, p.rownorm_ptrs):
        assert call(fn, fake, fake, [0x3000, 0]) == L.MUON_ERR_INVALID_ARGUMENT
        assert call(fn, fake, fake, fake, lr=float("inf")) == L.MUON_ERR_INVALID_ARGUMENT
        assert call(fn, fake, fake, fake, wd=float("nan")) == L.MUON_ERR_INVALID_ARGUMENT
        assert call(fn, fake, fake, fake, wsp=0) == L.MUON_ERR_INVALID_ARGUMENT
        assert call(fn, fake, fake, fake, wsp=ws + 16) == L.MUON_ERR_INVALID_ARGUMENT
        assert call(fn, fake, fake, fake, wsb=p.workspace_bytes - 1) == L.MUON_ERR_WORKSPACE_TOO_SMALL
    assert lib.muon_step_batched(None, None, None, None, 0.0, 0.0, None, 0, None, None) == \
        L.MUON_ERR_INVALID_ARGUMENT
    # the allocation-free step: argument checks, then the size of the plan's
    # single-stream workspace against the library's scratch, before any HIP call
    for kw in ({"lr": float("nan")}, {"G": [0x3000, 0]}):
        args = dict(W=fake, M=fake, G=fake, lr=0.02)
        args.update(kw)
        with pytest.raises(L.MuonError) as e:
            p.step_noalloc_ptrs(args["W"], args["M"], args["G"], args["lr"], 0.1)
        assert e.value.status == L.MUON_ERR_INVALID_ARGUMENT
    big = L.Plan([(4096, 4096)])
    assert big.workspace_bytes > L.NOALLOC_WORKSPACE_BYTES
    with pytest.raises(L.MuonError) as e:
        big.step_noalloc_ptrs([0x1000], [0x2000], [0x3000], 0.02, 0.1)
    assert e.value.status == L.MUON_ERR_WORKSPACE_TOO_SMALL
    capped = L.Plan([(128, 3584)] * 200, max_workspace_bytes=L.NOALLOC_WORKSPACE_BYTES - (8 << 20))
    assert capped.workspace_bytes <= L.NOALLOC_WORKSPACE_BYTES
    assert lib.muon_plan_destroy(None) == L.MUON_OK


def test_workspace_size_query_matches_plan():
    p = L.Plan([(100, 300)] * 3)
    n = ctypes.c_size_t()
    assert L.load().muon_plan_workspace_size(p._handle, ctypes.byref(n)) == L.MUON_OK
    assert n.value == p.workspace_bytes > 0


def test_formulation_choice_and_validation():
    # AUTO plans the Gram form for buckets with c > 1.125 r and the direct
    # form for near-square ones on the 16-bit path; DIRECT keeps X and X^T
    # twice plus two r x r buffers, all on 256-wide tiles.
    rect = [(600, 1000), (1000, 600)]
    assert L.Plan(rect, formulation="auto").workspace_bytes == \
        L.Plan(rect, formulation="gram").workspace_bytes
    sq = [(1024, 1024)] * 2
    assert L.Plan(sq, formulation="auto").workspace_bytes == \
        L.Plan(sq, formulation="direct").workspace_bytes
    # on the fp32 path AUTO stays with the Gram form
    assert L.Plan(sq, "f32", "f32", formulation="auto").workspace_bytes == \
        L.Plan(sq, "f32", "f32", formulation="gram").workspace_bytes
    shapes = [(1200, 1024), (600, 1000), (1000, 600)]
    gram = L.Plan(shapes, formulation="gram")
    direct = L.Plan(shapes, formulation="direct")
    assert direct.info() == gram.info() == (3, 3)
    r_pad = {(1200, 1024): 1024, (600, 1000): 768, (1000, 600): 768}
    c_pad = {(1200, 1024): 1280, (600, 1000): 1024, (1000, 600): 1024}
    per_mat = [4 * r_pad[s] * c_pad[s] * 2 + 2 * r_pad[s] ** 2 * 2 for s in shapes]
    assert direct.workspace_bytes >= max(per_mat)
    # unknown formulation; direct form on the fp32 path
    assert plan_status([(64, 64)], formulation=3) == L.MUON_ERR_INVALID_ARGUMENT
    assert plan_status([(64, 64)], formulation=-1) == L.MUON_ERR_INVALID_ARGUMENT
    with pytest.raises(L.MuonError) as e:
        L.Plan([(64, 64)], "f32", "f32", formulation="direct")
    assert e.value.status == L.MUON_ERR_UNSUPPORTED
    L.Plan([(64, 64)], "f32", "f32", formulation="gram")


def test_near_square_buckets_take_the_direct_form():
    # c <= 1.125 r: the Gram form's fp16 recursion resolves the small
    # singular values of near-square inputs too coarsely for the 2e-2 bound,
    # so AUTO takes the direct form and a forced Gram form is refused on the
    # 16-bit path (the fp32 path keeps it)
    uns = L.MUON_ERR_UNSUPPORTED
    for m, n, direct in [(64, 72, True), (64, 73, False), (100, 112, True), (100, 113, False),
                         (127, 128, True), (128, 129, True), (63, 64, True), (1, 1, True),
                         (3584, 4032, True), (3584, 4033, False), (512, 768, False)]:
        for shape in ((m, n), (n, m)):
            b = L.Plan([shape]).buckets()[0]
            assert (b["formulation"] == "direct") == direct, (shape, b)
            g = plan_status([shape], formulation="gram")
            assert g == (uns if direct else 0), (shape, g)
            assert plan_status([shape], formulation="gram", hints={shape: {"formulation": "gram"}}) == g
            assert plan_status([shape], grad_dtype="f32", ns_dtype="f32", formulation="gram") == 0
    # a plan-wide Gram form with one near-square bucket is refused as a whole
    assert plan_status([(256, 1024), (300, 300)], formulation="gram") == uns


def test_kernel_class_enum_matches_binding():
    text = open(HEADER).read()
    names = re.findall(r"MUON_K_(\w+)\s*=\s*(\d+)", text)
    classes = {n.lower(): int(v) for n, v in names if n != "COUNT"}
    count = int(dict(names)["COUNT"])
    assert count == len(L.KERNEL_CLASSES)
    assert [k for k, _ in sorted(classes.items(), key=lambda kv: kv[1])] == list(L.KERNEL_CLASSES)


def test_bucket_info_reports_the_planner_rule():
    shapes = [(256, 1024), (1024, 256), (256, 1024), (1024, 1024), (1000, 300), (3584, 18944)]
    b = L.Plan(shapes).buckets()
    assert [x["shape"] for x in b] == [(256, 1024), (1024, 256), (1024, 1024), (1000, 300),
                                       (3584, 18944)]
    assert [x["count"] for x in b] == [2, 1, 1, 1, 1]
    assert [x["transposed"] for x in b] == [False, True, False, True, False]
    # squares take the direct form on the 16-bit path, 256-wide tiles above r = 768
    assert [x["formulation"] for x in b] == ["gram", "gram", "direct", "gram", "gram"]
    assert [x["tile"] for x in b] == [64, 64, 256, 64, 256]
    assert all(x["chunks"] == 1 for x in b)
    f = L.Plan(shapes, "f32", "f32").buckets()
    assert all(x["formulation"] == "gram" and x["tile"] in (64, 128) for x in f)
    lib = L.load()
    info = L.BucketInfo()
    plan = L.Plan(shapes)
    assert lib.muon_plan_bucket_info(plan._handle, 5, ctypes.byref(info)) == L.MUON_ERR_INVALID_ARGUMENT
    assert lib.muon_plan_bucket_info(plan._handle, -1, ctypes.byref(info)) == L.MUON_ERR_INVALID_ARGUMENT
    assert lib.muon_plan_bucket_info(plan._handle, 0, None) == L.MUON_ERR_INVALID_ARGUMENT
    assert lib.muon_plan_bucket_info(None, 0, ctypes.byref(info)) == L.MUON_ERR_INVALID_ARGUMENT


def test_bucket_hints_override_tile_and_formulation():
    shapes = [(3584, 18944), (1024, 1280), (384, 1000), (700, 300)]
    hints = {(3584, 18944): {"tile": 128}, (1024, 1280): {"formulation": "gram"},
             (384, 1000): {"tile": 256, "formulation": "gram"},
             (700, 300): {"formulation": "direct"},
             (5, 5): {"tile": 64}}                     # matches no matrix: ignored
    b = {x["shape"]: x for x in L.Plan(shapes, hints=hints).buckets()}
    assert (b[(3584, 18944)]["tile"], b[(3584, 18944)]["formulation"]) == (128, "gram")
    assert (b[(1024, 1280)]["tile"], b[(1024, 1280)]["formulation"]) == (256, "gram")
    assert (b[(384, 1000)]["tile"], b[(384, 1000)]["formulation"]) == (256, "gram")
    assert (b[(700, 300)]["tile"], b[(700, 300)]["formulation"]) == (64, "direct")
    # a 128-wide tile on a 3584-row bucket keeps fp32 master copies: more workspace
    assert L.Plan([(3584, 18944)], hints={(3584, 18944): {"tile": 128}}).workspace_bytes > \
        L.Plan([(3584, 18944)]).workspace_bytes
    # the fp32 path takes 64 / 128 tile hints
    f = L.Plan([(300, 700)], "f32", "f32", hints={(300, 700): {"tile": 128}}).buckets()
    assert f[0]["tile"] == 128


def test_bucket_hints_validation():
    bad = L.MUON_ERR_INVALID_ARGUMENT
    assert plan_status([(64, 64)], hints={(64, 64): {"tile": 32}}) == bad
    assert plan_status([(64, 64)], hints={(64, 64): {"tile": -1}}) == bad
    assert plan_status([(64, 64)], hints={(64, 64): {"formulation": 3}}) == bad
    assert plan_status([(64, 64)], hints={(0, 64): {"tile": 64}}) == bad
    # two hints for one shape
    lib = L.load()
    rows = (ctypes.c_int64 * 1)(64)
    cols = (ctypes.c_int64 * 1)(80)
    harr = (L.BucketHint * 2)(L.BucketHint(64, 80, 64, 1), L.BucketHint(64, 80, 128, 1))
    desc = L.PlanDesc()
    desc.num_matrices = 1
    desc.rows = ctypes.cast(rows, ctypes.POINTER(ctypes.c_int64))
    desc.cols = ctypes.cast(cols, ctypes.POINTER(ctypes.c_int64))
    desc.grad_dtype, desc.ns_dtype = L.MUON_F32, L.MUON_BF16
    desc.hp = L.default_hparams()
    desc.hints = ctypes.cast(harr, ctypes.POINTER(L.BucketHint))
    handle = ctypes.c_void_p()
    for n, want in ((2, bad), (-1, bad), (1, L.MUON_OK)):
        desc.num_hints = n
        st = lib.muon_plan(ctypes.byref(desc), ctypes.byref(handle), None)
        assert st == want, (n, st)
        if st == L.MUON_OK:
            lib.muon_plan_destroy(handle)
    desc.hints = None
    desc.num_hints = 1
    assert lib.muon_plan(ctypes.byref(desc), ctypes.byref(handle), None) == bad
    # combinations the kernels do not provide
    uns = L.MUON_ERR_UNSUPPORTED
    assert plan_status([(64, 64)], grad_dtype="f32", ns_dtype="f32", hints={(64, 64): {"tile": 256}}) == uns
    assert plan_status([(64, 64)], grad_dtype="f32", ns_dtype="f32",
                       hints={(64, 64): {"formulation": "direct"}}) == uns
    assert plan_status([(512, 512)], hints={(512, 512): {"tile": 128}}) == 0   # small-tile direct form
    assert plan_status([(512, 640)], hints={(512, 640): {"tile": 128, "formulation": "gram"}}) == 0
    assert plan_status([(512, 512)], hints={(512, 512): {"tile": 128, "formulation": "gram"}}) == uns
    assert plan_status([(300, 700)], hints={(300, 700): {"tile": 64, "formulation": "direct"}}) == 0


def test_concurrent_bucket_layout_and_cap_fallback():
    # small buckets get one scratch region per internal stream; a cap below
    # their sum (but above each bucket's own need) falls back to one region
    small = [(640, 640)] * 2 + [(512, 1536)] * 2 + [(1536, 512)] + [(300, 700)] * 3 + [(96, 2000)]
    each = max(L.Plan([s] * small.count(s)).workspace_bytes for s in dict.fromkeys(small))
    conc = L.Plan(small).workspace_bytes
    seq = L.Plan(small, max_workspace_bytes=each).workspace_bytes
    assert conc > seq and seq <= each + (1 << 20)
    # a bucket that fills the device keeps every bucket on the caller's stream
    big = small + [(3584, 3584)] * 8
    assert L.Plan(big).workspace_bytes <= L.Plan([(3584, 3584)] * 8).workspace_bytes + (1 << 20)


def test_kernel_knob_hints():
    # tile-order group, XCD run length and wave count of the 256-wide kernels
    shape = (3584, 18944)
    b = L.Plan([shape], grad_dtype="bf16",
               hints={shape: {"group": 16, "xcd_chunk": -1, "waves": 4}}).buckets()[0]
    assert (b["tile"], b["group"], b["xcd_chunk"], b["waves"]) == (256, 16, -1, 4)
    b = L.Plan([shape]).buckets()[0]
    assert (b["group"], b["xcd_chunk"], b["waves"]) == (0, 0, 0)
    bad, uns = L.MUON_ERR_INVALID_ARGUMENT, L.MUON_ERR_UNSUPPORTED
    for h in ({"group": -1}, {"group": 65}, {"xcd_chunk": -2}, {"xcd_chunk": 65537}, {"waves": 6},
              {"waves": 2}):
        assert plan_status([shape], hints={shape: h}) == bad, h
    # the knobs need the 256-wide kernels
    assert plan_status([shape], hints={shape: {"tile": 128, "group": 4}}) == uns
    assert plan_status([(300, 900)], hints={(300, 900): {"waves": 4}}) == uns  # small tiles by rule
    assert plan_status([shape], grad_dtype="f32", ns_dtype="f32", hints={shape: {"xcd_chunk": 64}}) == uns
    assert plan_status([(4096, 4096)], hints={(4096, 4096): {"group": 2, "waves": 8}}) == 0

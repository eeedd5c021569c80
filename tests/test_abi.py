"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and rejects bad arguments before anything reaches the device."""
import ctypes
import os
import re
import subprocess

import pytest

from mixture_experts_layer_50_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.lib_path()):
        from mixture_experts_layer_50_amd.build import build
        build()
    return B.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(B.EXPORTS)


def declared_parameters():
    """{function: [kind of each parameter]} from the header's prototypes;
    kinds: ptr (pointers and the stream handle), size, int, float."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for name, params in re.findall(r"\b(moe_[a-z_0-9]+)\s*\(([^)]*)\)\s*;", src):
        kinds = []
        for prm in [q.strip() for q in params.split(",")]:
            if prm in ("", "void"):
                continue
            if "*" in prm or prm.startswith("moe_stream_t"):
                kinds.append("ptr")
            elif prm.startswith("size_t"):
                kinds.append("size")
            elif prm.startswith("float"):
                kinds.append("float")
            else:
                kinds.append("int")
        out[name] = kinds
    return out


def _kind(ct):
    if ct is ctypes.c_size_t:
        return "size"
    if ct is ctypes.c_float:
        return "float"
    if ct is ctypes.c_int:
        return "int"
    return "ptr"


def test_binding_argtypes_match_the_prototypes(lib):
    """Every binding's ctypes argument list has the header prototype's
    length and kinds, position by position (a missing pointer shifts the
    size and the stream handle, which the library cannot detect)."""
    decl = declared_parameters()
    assert sorted(decl) == declared_functions()
    for name, kinds in decl.items():
        f = getattr(lib, name)
        if f.argtypes is None:  # no arguments set: the prototype must take none
            assert kinds == [], name
            continue
        assert [_kind(t) for t in f.argtypes] == kinds, name


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in declared_functions():
        assert name in syms, name
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for code, name in B.STATUS.items():
        assert lib.moe_status_string(code).decode() == name
    assert b"gfx950" in lib.moe_version()


FAKE = 1 << 20   # 16-byte aligned, never dereferenced: validation fails first


def shape(**kw):
    base = dict(T=64, d=128, E=8, k=2, I=256, dtype="bf16", gate="softmax_topk")
    base.update(kw)
    return B.MoEShape.make(**base)


def call_route(lib, s, **ptrs):
    p = dict(x=FAKE, w=FAKE, b=None, logits=FAKE, idx=FAKE, g=FAKE)
    p.update(ptrs)
    st = lib.moe_route(ctypes.byref(s) if s is not None else None, p["x"], p["w"], p["b"],
                       p["logits"], p["idx"], p["g"], None)
    return B.STATUS[st], lib.moe_last_error().decode()


@pytest.mark.parametrize("kw,status,text", [
    (dict(k=9), "MOE_ERR_ARG", "k=9 > E=8"),
    (dict(T=0), "MOE_ERR_SHAPE", "positive"),
    (dict(dtype=7), "MOE_ERR_DTYPE", "dtype"),
    (dict(gate=5), "MOE_ERR_ARG", "gate"),
    (dict(d=96), "MOE_ERR_UNSUPPORTED", "multiples of 64"),
    (dict(I=100), "MOE_ERR_UNSUPPORTED", "multiples of 64"),
    (dict(E=12, k=2), "MOE_ERR_UNSUPPORTED", "E % 8"),
    (dict(E=1024, k=2), "MOE_ERR_UNSUPPORTED", "E > 512"),
    (dict(E=64, k=33), "MOE_ERR_UNSUPPORTED", "k > 32"),
    (dict(e_lo=4, e_hi=2), "MOE_ERR_ARG", "local experts"),
    (dict(e_lo=0, e_hi=9), "MOE_ERR_ARG", "local experts"),
    (dict(R_cap=129), "MOE_ERR_SHAPE", "R_cap"),
    (dict(E=8, k=3, gate="balanced"), "MOE_ERR_ARG", "k | E"),
    (dict(T=1 << 28, k=8), "MOE_ERR_SHAPE", "overflows"),
])
def test_route_rejects_bad_shapes(lib, kw, status, text):
    st, msg = call_route(lib, shape(**kw))
    assert st == status, msg
    assert text in msg


def test_null_and_misaligned_pointers(lib):
    st, msg = call_route(lib, None)
    assert st == "MOE_ERR_ARG" and "shape is NULL" in msg
    st, msg = call_route(lib, shape(), logits=None)
    assert st == "MOE_ERR_ARG" and "logits is NULL" in msg
    st, msg = call_route(lib, shape(), x=FAKE + 2)
    assert st == "MOE_ERR_UNSUPPORTED" and "aligned" in msg
    st, msg = call_route(lib, shape(), b=FAKE + 8)
    assert st == "MOE_ERR_UNSUPPORTED" and "bias" in msg


def test_workspace_sizes_and_short_workspace(lib):
    s = shape(T=4096, d=2048, E=128, k=8, I=768, gate="balanced")
    R = 4096 * 8
    assert B.workspace_size(s, "route") == 0
    assert B.workspace_size(s, "combine") == 0
    assert B.workspace_size(s, "permute") == 16 * 128 * 4          # 16 blocks of 256 tokens
    def table(bm):  # one tile table per M-tile height, 256-byte aligned
        return -(-(1 + 2 * (R // bm + 128)) * 4 // 256) * 256
    # + weight-gradient cost prefix [E_loc + 1] + token row of each routed row (gathered calls)
    tiles = table(256) + table(128) + 768 + R * 4
    assert B.workspace_size(s, "ffn_fwd") == tiles
    # [dHg | dHu] + the tables + the gate gradient's fp32 shares [R][I / 32]
    assert B.workspace_size(s, "ffn_bwd") == R * 2 * 768 * 2 + tiles + R * (768 // 32) * 4
    assert B.workspace_size(s, "route_bwd") == 0                    # balanced gate: no dL copy
    n = B.workspace_size(shape(T=4096, d=2048, E=128, k=8, I=768), "route_bwd")
    # bf16 copy of dL, column sums per 32 tokens, 8 split-K partials of x^T dL (fp32)
    assert n == 4096 * 128 * 2 + 128 * 128 * 4 + 8 * 2048 * 128 * 4
    with pytest.raises(B.MoEError) as ei:
        B.workspace_size(s, 99)
    assert ei.value.status_name == "MOE_ERR_ARG"
    st = lib.moe_permute(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100, None)
    assert B.STATUS[st] == "MOE_ERR_WORKSPACE"
    assert "workspace" in lib.moe_last_error().decode()


def test_every_entry_point_validates_before_launch(lib):
    s = shape(k=9)   # invalid: k > E
    P = FAKE
    calls = [
        lambda: lib.moe_permute(ctypes.byref(s), P, P, P, P, P, P, P, 1 << 20, None),
        lambda: lib.moe_grouped_ffn_fwd(ctypes.byref(s), P, P, P, P, P, P, P, P, P, 1 << 20, None),
        lambda: lib.moe_combine(ctypes.byref(s), P, P, P, P, None),
        lambda: lib.moe_combine_bwd(ctypes.byref(s), P, P, P, P, P, P, None),
        lambda: lib.moe_grouped_ffn_bwd(ctypes.byref(s), P, P, P, P, P, P, P, P, P, P, P, P, P,
                                        1 << 30, None),
        lambda: lib.moe_permute_bwd(ctypes.byref(s), P, P, P, None),
        lambda: lib.moe_grouped_ffn_fwd_gather(ctypes.byref(s), P, P, P, P, P, P, P, P, P, P,
                                               1 << 20, None),
        lambda: lib.moe_grouped_ffn_bwd_gather(ctypes.byref(s), P, P, P, P, P, P, P, P, P, P, P,
                                               P, P, P, 1 << 30, None),
        lambda: lib.moe_route_bwd(ctypes.byref(s), P, P, P, P, P, P, P, P, P, P, 1 << 20, None),
    ]
    for c in calls:
        assert B.STATUS[c()] == "MOE_ERR_ARG"
    good = shape()
    st = lib.moe_grouped_ffn_fwd(ctypes.byref(good), P, P, P, P, P, None, None, P, P, 1 << 20, None)
    assert B.STATUS[st] == "MOE_ERR_ARG" and "a_save" in lib.moe_last_error().decode()
    st = lib.moe_grouped_ffn_bwd(ctypes.byref(good), P, P, P, P, P, None, P, P, P, P, P, P, P,
                                 1 << 30, None)
    assert B.STATUS[st] == "MOE_ERR_ARG" and "h_save" in lib.moe_last_error().decode()


def test_profiler_api_without_gpu(lib):
    B.prof_enable(False)
    B.prof_reset()
    assert B.prof_read("ffn_gateup_fwd") == (0.0, 0)
    assert B.prof_names() == []


def test_gathered_ffn_validation(lib):
    """The gathered FFN calls need perm, check the 32-bit offsets of x, and
    moe_permute runs without xp (the sort alone)."""
    P = FAKE
    good = shape()
    st = lib.moe_grouped_ffn_fwd_gather(ctypes.byref(good), P, None, P, P, P, P, P, P, P, P,
                                        1 << 20, None)
    assert B.STATUS[st] == "MOE_ERR_ARG" and "perm" in lib.moe_last_error().decode()
    st = lib.moe_grouped_ffn_fwd_gather(ctypes.byref(good), None, P, P, P, P, P, P, P, P, P,
                                        1 << 20, None)
    assert B.STATUS[st] == "MOE_ERR_ARG" and "x is NULL" in lib.moe_last_error().decode()
    st = lib.moe_grouped_ffn_bwd_gather(ctypes.byref(good), P, None, P, P, P, P, P, P, P, P, P,
                                        P, P, P, 1 << 30, None)
    assert B.STATUS[st] == "MOE_ERR_ARG" and "perm" in lib.moe_last_error().decode()
    # x of 2^31 bytes or more: the gathered form is refused, the plain one is not limited
    big = shape(T=65536, d=16384, E=8, k=2, I=64)
    st = lib.moe_grouped_ffn_fwd_gather(ctypes.byref(big), P, P, P, P, P, P, P, P, P, P,
                                        1 << 40, None)
    assert B.STATUS[st] == "MOE_ERR_UNSUPPORTED" and "2^31" in lib.moe_last_error().decode()
    st = lib.moe_grouped_ffn_bwd_gather(ctypes.byref(big), P, P, P, P, P, P, P, P, P, P, P, P,
                                        P, P, 1 << 40, None)
    assert B.STATUS[st] == "MOE_ERR_UNSUPPORTED"
    # permute: xp NULL is the sort alone (x may then be NULL); validation still runs
    s = shape(k=9)
    assert B.STATUS[lib.moe_permute(ctypes.byref(s), P, None, P, P, P, None, P, 1 << 20,
                                    None)] == "MOE_ERR_ARG"
    st = lib.moe_permute(ctypes.byref(good), P, None, P, P, P, P, P, 1 << 20, None)
    assert B.STATUS[st] == "MOE_ERR_ARG" and "x is NULL" in lib.moe_last_error().decode()


def test_small_batch_ffn_validation(lib):
    """moe_ffn_small_fwd: its size limits, no row capacity, its workspace."""
    P = FAKE
    s = shape(T=64, d=128, E=8, k=2, I=256)
    n = B.workspace_size(s, "small_fwd")
    # fp32 [Hg | Hu] partials (one K range at d = 128), the slot outputs
    # [T*k, d] in bf16, the combine's arrival counters [T][d / 64] int32
    assert n == 128 * 2 * 256 * 4 + 128 * 128 * 2 + 64 * 2 * 4
    # at the Qwen3 shape d = 2048 splits in 4 ranges of 512 rows
    n1 = B.workspace_size(shape(T=1, d=2048, E=128, k=8, I=768), "small_fwd")
    assert n1 == 8 * 4 * 2 * 768 * 4 + 8 * 2048 * 2 + 256  # counters: 32 int32, padded

    def call(sh, ws_bytes=1 << 30, y=P):
        return B.STATUS[lib.moe_ffn_small_fwd(ctypes.byref(sh), P, P, P, P, P, P, y, P, ws_bytes,
                                               None)], lib.moe_last_error().decode()

    assert call(s, y=None) == ("MOE_ERR_ARG", "moe_ffn_small_fwd: y is NULL")
    st, msg = call(shape(T=2049, d=128, E=8, k=2, I=256))
    assert st == "MOE_ERR_UNSUPPORTED" and "T*k" in msg
    assert call(shape(T=2048, d=128, E=8, k=2, I=256), ws_bytes=0)[0] == "MOE_ERR_WORKSPACE"
    st, msg = call(shape(T=4, d=8256, E=8, k=2, I=256))
    assert st == "MOE_ERR_UNSUPPORTED" and "<=" in msg
    st, msg = call(shape(T=64, d=128, E=8, k=2, I=256, R_cap=100))
    assert st == "MOE_ERR_UNSUPPORTED" and "capacity" in msg
    st, msg = call(s, ws_bytes=n - 1)
    assert st == "MOE_ERR_WORKSPACE"
    assert B.STATUS[lib.moe_ffn_small_fwd(ctypes.byref(shape(k=9)), P, P, P, P, P, P, P, P,
                                          1 << 20, None)] == "MOE_ERR_ARG"


def test_aux_loss_validation(lib):
    """moe_aux_loss / moe_route_bwd_aux: natural gate only, required buffers,
    finite alpha, the workspace of per-32-token partials."""
    P = FAKE
    s = shape(T=100, d=128, E=16, k=2, I=256)
    n = B.workspace_size(s, "aux_loss")
    # column sums of the probabilities and expert counts per 32 tokens (4 blocks)
    assert n == 2 * 256
    assert B.workspace_size(shape(T=4096, d=2048, E=128, k=8, I=768), "aux_loss") == 2 * 128 * 128 * 4

    def aux(sh, alpha=0.01, logits=P, loss=P, ws_bytes=1 << 20):
        return B.STATUS[lib.moe_aux_loss(ctypes.byref(sh), logits, P, ctypes.c_float(alpha), loss, P,
                                         P, ws_bytes, None)], lib.moe_last_error().decode()

    assert aux(s, logits=None) == ("MOE_ERR_ARG", "moe_aux_loss: logits is NULL")
    assert aux(s, loss=None) == ("MOE_ERR_ARG", "moe_aux_loss: loss is NULL")
    st, msg = aux(s, alpha=float("nan"))
    assert st == "MOE_ERR_ARG" and "alpha" in msg
    st, msg = aux(shape(T=100, d=128, E=16, k=2, I=256, gate="balanced"))
    assert st == "MOE_ERR_ARG" and "balanced" in msg
    assert aux(s, ws_bytes=n - 1)[0] == "MOE_ERR_WORKSPACE"

    def bwd(sh, logits=P, aux_w=P):
        return B.STATUS[lib.moe_route_bwd_aux(ctypes.byref(sh), P, P, P, P, P, logits, aux_w, P, P,
                                              None, P, P, 1 << 30, None)], \
            lib.moe_last_error().decode()

    assert bwd(s, aux_w=None) == ("MOE_ERR_ARG", "moe_route_bwd_aux: aux_w is NULL")
    assert bwd(s, logits=None) == ("MOE_ERR_ARG", "moe_route_bwd_aux: logits is NULL")
    st, msg = bwd(shape(T=100, d=128, E=16, k=2, I=256, gate="balanced"))
    assert st == "MOE_ERR_ARG" and "balanced" in msg


def test_noalloc_rejects_shapes_beyond_its_scratch(lib):
    """The entry point without a workspace refuses a shape whose tile and
    token tables exceed its static scratch, before any device work."""
    s = shape(T=262144, d=128, E=8, k=8)        # R_cap = 2M rows: 8 MiB of token table
    st = lib.moe_grouped_ffn_fwd_gather_noalloc(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE,
                                                FAKE, None, FAKE, FAKE, None)
    assert B.STATUS[st] == "MOE_ERR_UNSUPPORTED"
    assert "static scratch" in lib.moe_last_error().decode()


def test_small_routed_fwd_validation(lib):
    """moe_small_fwd: workspace = the few-token router's partial logits (softmax
    gate, T <= 16) + the small-batch FFN's; the router's pointers are required
    under the softmax gate only; the FFN's limits hold."""
    P = FAKE
    q1 = shape(T=1, d=2048, E=128, k=8, I=768)
    n_ffn = B.workspace_size(q1, "small_fwd")
    # d / 64 partial logit rows of [T][E] fp32
    assert B.workspace_size(q1, "small_routed_fwd") == 32 * 1 * 128 * 4 + n_ffn
    q17 = shape(T=17, d=2048, E=128, k=2, I=768)  # more tokens: the MFMA router, no partials
    assert B.workspace_size(q17, "small_routed_fwd") == B.workspace_size(q17, "small_fwd")
    qb = shape(T=4, d=2048, E=128, k=8, I=768, gate="balanced")
    assert B.workspace_size(qb, "small_routed_fwd") == B.workspace_size(qb, "small_fwd")

    def call(sh, wr=P, logits=P, y=P, ws_bytes=1 << 30):
        st = lib.moe_small_fwd(ctypes.byref(sh), P, wr, None, logits, P, P, P, P, P, y, P,
                               ws_bytes, None)
        return B.STATUS[st], lib.moe_last_error().decode()

    assert call(q1, wr=None) == ("MOE_ERR_ARG", "moe_small_fwd: w_router is NULL")
    assert call(q1, logits=None) == ("MOE_ERR_ARG", "moe_small_fwd: logits is NULL")
    assert call(q1, y=None) == ("MOE_ERR_ARG", "moe_small_fwd: y is NULL")
    st, msg = call(shape(T=2049, d=128, E=8, k=2, I=256))
    assert st == "MOE_ERR_UNSUPPORTED" and "T*k" in msg
    st, msg = call(shape(T=64, d=128, E=8, k=2, I=256, R_cap=100))
    assert st == "MOE_ERR_UNSUPPORTED" and "capacity" in msg
    st, _ = call(q1, ws_bytes=B.workspace_size(q1, "small_routed_fwd") - 1)
    assert st == "MOE_ERR_WORKSPACE"
    # the balanced gate reads no router weights and writes no logits: its
    # argument checks pass with them NULL and only the workspace is short
    st, _ = call(qb, wr=None, logits=None, ws_bytes=0)
    assert st == "MOE_ERR_WORKSPACE"


def test_small_path_size_rule():
    """The layer takes the small-batch forward for inference with at most
    fewer than E_loc / 2 routed pairs and no row capacity, the grouped path
    otherwise."""
    from mixture_experts_layer_50_amd.layer import small_path_fits
    q = lambda T, **kw: B.MoEShape.make(T, 2048, 128, 8, 768, **kw)
    assert small_path_fits(q(1), training=False)
    assert small_path_fits(q(7), training=False)
    assert not small_path_fits(q(8), training=False)
    assert not small_path_fits(q(1), training=True)
    assert not small_path_fits(q(8, R_cap=40), training=False)
    assert small_path_fits(B.MoEShape.make(3, 2048, 128, 8, 768, e_lo=64, e_hi=128), False)
    assert not small_path_fits(B.MoEShape.make(4, 2048, 128, 8, 768, e_lo=64, e_hi=128), False)
    # wider than the small kernels take
    assert not small_path_fits(B.MoEShape.make(1, 8256, 128, 8, 768), False)


def test_combine_ffn_bwd_gather_validation(lib):
    """moe_combine_ffn_bwd_gather checks its arguments before any launch: an
    invalid shape, each NULL input of the combine backward, and x of 2^31
    bytes or more."""
    P = FAKE
    bad = shape(k=9)
    args = [P] * 19  # x .. ws
    st = lib.moe_combine_ffn_bwd_gather(ctypes.byref(bad), *args, 1 << 30, None)
    assert B.STATUS[st] == "MOE_ERR_ARG"
    good = shape()
    for i, name in ((2, "inv"), (4, "topk_w"), (10, "yp"), (11, "dy"), (12, "dyp"),
                    (13, "dtopk_w")):
        a = list(args)
        a[i] = None
        st = lib.moe_combine_ffn_bwd_gather(ctypes.byref(good), *a, 1 << 30, None)
        assert B.STATUS[st] == "MOE_ERR_ARG" and f"{name} is NULL" in lib.moe_last_error().decode()
    big = shape(T=65536, d=16384, E=8, k=2, I=64)
    st = lib.moe_combine_ffn_bwd_gather(ctypes.byref(big), *args, 1 << 40, None)
    assert B.STATUS[st] == "MOE_ERR_UNSUPPORTED" and "2^31" in lib.moe_last_error().decode()


def test_check_routing_validation(lib):
    s = shape(T=100, E=16, k=4, e_lo=4, e_hi=12)
    assert B.workspace_size(s, "check_routing") == 256          # 8 local group sizes, aligned
    assert B.workspace_size(shape(E=512, k=2), "check_routing") == 512 * 4
    P = FAKE
    st = lib.moe_check_routing(ctypes.byref(s), None, None, P, None, 0, None)
    assert B.STATUS[st] == "MOE_ERR_ARG" and "topk_idx" in lib.moe_last_error().decode()
    st = lib.moe_check_routing(ctypes.byref(s), P, None, None, None, 0, None)
    assert B.STATUS[st] == "MOE_ERR_ARG" and "flags" in lib.moe_last_error().decode()
    # the group sizes need the workspace only when offsets are checked
    st = lib.moe_check_routing(ctypes.byref(s), P, P, P, None, 0, None)
    assert B.STATUS[st] == "MOE_ERR_WORKSPACE"
    st = lib.moe_check_routing(ctypes.byref(s), P, P, P, P, 16, None)
    assert B.STATUS[st] == "MOE_ERR_WORKSPACE"
    st = lib.moe_check_routing(ctypes.byref(shape(k=9)), P, None, P, None, 0, None)
    assert B.STATUS[st] == "MOE_ERR_ARG"

"""The C-ABI library without a GPU: it loads, exports exactly the symbols the
header declares, and rejects invalid requests before any HIP call (so these
run on a host with no device).  Validation order and codes follow the
Diffusers TP page, §Restrições e verificação (tp_degree divides the heads and
every packed block, checked before any weight is touched) and §Limitações
(an error, never a silent fallback)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as O
import tensor_dit_transformer_amd as tp
from tensor_dit_transformer_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp_shard.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tp.LIB_PATH):
        from tensor_dit_transformer_amd import build
        build.build(verbose=False)
    return tp.lib()


def header_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^TP_API[^(]*?\b(tp_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    syms = header_symbols()
    assert syms == sorted(binding.EXPORTED)


def test_library_exports_exactly_the_header_symbols(L):
    out = subprocess.run(["nm", "-D", "--defined-only", tp.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines()
                       if l.split() and l.split()[-2] in ("T", "W") and not l.split()[-1].startswith("_")})
    assert exported == header_symbols()
    for s in header_symbols():
        assert hasattr(L, s)


def _create(L, cfg, weights=None):
    w = tp.TpBlockWeights()
    keep = []
    for k, a in (weights or {}).items():
        keep.append(a)
        setattr(w, k, a.ctypes.data)
    out = ctypes.c_void_p(12345)
    st = L.tp_block_shard_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(out))
    return st, out.value


def _tiny_weights(D, H, d, F, dtype=np.uint16):
    HD = H * d
    w = {}
    if H:
        for k in ("w_q", "w_k", "w_v"):
            w[k] = np.zeros((HD, D), dtype)
        w["w_o"] = np.zeros((D, HD), dtype)
    if F:
        w["w_up"] = np.zeros((F, D), dtype)
        w["w_down"] = np.zeros((D, F), dtype)
    return w


@pytest.mark.parametrize("P,r,D,H,d,F,want", [
    (5, 0, 24 * 8, 24, 8, 0, tp.TP_ERR_DIVISIBILITY),     # P does not divide the heads
    (4, 0, 24 * 8, 24, 8, 1022, tp.TP_ERR_DIVISIBILITY),  # ... nor the FFN width
    (2, 0, 100, 4, 8, 0, tp.TP_ERR_DIVISIBILITY),         # heads * head_dim != hidden
    (4, 4, 32, 4, 8, 64, tp.TP_ERR_ARG),                  # rank out of range
    (4, -1, 32, 4, 8, 64, tp.TP_ERR_ARG),
    (0, 0, 32, 4, 8, 64, tp.TP_ERR_ARG),                  # tp_degree < 1
    (1, 0, 32, 0, 0, 0, tp.TP_ERR_ARG),                   # neither attention nor MLP
    (1, 0, 0, 0, 0, 64, tp.TP_ERR_ARG),                   # hidden <= 0
    (2, 0, 36, 0, 0, 64, tp.TP_ERR_UNSUPPORTED),          # hidden not a multiple of 8
    (4, 0, 64, 0, 0, 40, tp.TP_ERR_UNSUPPORTED),          # ffn / tp not a multiple of 8
])
def test_create_rejects_before_touching_weights(L, P, r, D, H, d, F, want):
    # No weights at all: the checks that fail must come before any weight is read.
    st, out = _create(L, tp.make_config(P, r, D, H, d, F, tp.TP_BF16))
    assert st == want, tp.tp_last_error_detail()
    assert out is None
    assert tp.tp_last_error_detail()


def test_create_rejects_missing_weights_and_nulls(L):
    st, out = _create(L, tp.make_config(2, 0, 32, 4, 8, 64, tp.TP_BF16))
    assert st == tp.TP_ERR_ARG and out is None and "missing" in tp.tp_last_error_detail()
    w = tp.TpBlockWeights()
    assert L.tp_block_shard_create(None, ctypes.byref(w), ctypes.byref(ctypes.c_void_p())) == tp.TP_ERR_ARG
    cfg = tp.make_config(2, 0, 32, 4, 8, 64, tp.TP_BF16)
    assert L.tp_block_shard_create(ctypes.byref(cfg), None, ctypes.byref(ctypes.c_void_p())) == tp.TP_ERR_ARG
    assert L.tp_block_shard_create(ctypes.byref(cfg), ctypes.byref(w), None) == tp.TP_ERR_ARG
    cfg.dtype = 7
    st, _ = _create(L, cfg, _tiny_weights(32, 4, 8, 64))
    assert st == tp.TP_ERR_ARG


@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 6, 8, 12, 24])
@pytest.mark.parametrize("H,F", [(24, 24 * 8 * 4), (24, 1000), (12, 0), (0, 96)])
def test_create_agrees_with_oracle_constraints(L, P, H, F):
    """The library's accept/reject decision matches the oracle's constraint
    check (sizes chosen so every accepted case also meets the 8-alignment)."""
    d = 8
    D = H * d if H else 192
    try:
        O.check_config(P, 0, D, H, d, F)
        oracle_kind = None
    except O.ShardConfigError as e:
        oracle_kind = e.kind
    st, out = _create(L, tp.make_config(P, 0, D, H, d, F, tp.TP_BF16), _tiny_weights(D, H, d, F))
    if out:
        L.tp_block_shard_destroy(out)
    if oracle_kind == "divisibility":
        assert st == tp.TP_ERR_DIVISIBILITY
    elif oracle_kind == "argument":
        assert st == tp.TP_ERR_ARG
    else:
        # accepted: either created (device present) or failed in the HIP runtime,
        # or a multiple-of-8 requirement of this library
        assert st in (tp.TP_OK, tp.TP_ERR_HIP, tp.TP_ERR_UNSUPPORTED, tp.TP_ERR_OOM)
        if st == tp.TP_ERR_UNSUPPORTED:
            assert (D // P) % 8 or (F // P) % 8


def test_calls_reject_null_shard(L):
    vp = ctypes.c_void_p(0x10000)
    assert L.tp_colwise_linear(None, tp.TP_QKV, 8, vp, 64, vp, 64, None) == tp.TP_ERR_ARG
    assert L.tp_colwise_qkv_up(None, 8, vp, 64, vp, 64, vp, 64, None) == tp.TP_ERR_ARG
    assert L.tp_attn_heads(None, 8, vp, 64, vp, 64, None) == tp.TP_ERR_ARG
    assert L.tp_rowwise_linear_partial(None, tp.TP_BLOCK_OUT, 8, vp, 64, vp, 64, 0, None) == tp.TP_ERR_ARG
    L.tp_block_shard_destroy(None)  # ignored


def _reduce(L, parts, n_p, ldp, biases, n_b, T, D, out, ldo):
    P = (ctypes.c_void_p * max(1, len(parts)))(*parts)
    B = (ctypes.c_void_p * max(1, len(biases)))(*biases) if biases is not None else None
    return L.tp_partial_reduce(P, n_p, ldp, B, n_b, T, D, out, ldo, None)


def test_reduce_validation_without_device(L):
    a, b, c, o = 0x100000, 0x200000, 0x300000, 0x400000   # never dereferenced
    ok = dict(parts=[a, b], n_p=2, ldp=64, biases=[c], n_b=1, T=0, D=64, out=o, ldo=64)
    assert _reduce(L, **ok) == tp.TP_OK                           # tokens == 0: no-op
    assert _reduce(L, **{**ok, "n_p": 0}) == tp.TP_ERR_ARG
    assert _reduce(L, **{**ok, "n_p": 17}) == tp.TP_ERR_UNSUPPORTED
    assert _reduce(L, **{**ok, "n_b": 5}) == tp.TP_ERR_UNSUPPORTED
    assert _reduce(L, **{**ok, "n_b": -1}) == tp.TP_ERR_ARG
    assert _reduce(L, **{**ok, "biases": None}) == tp.TP_ERR_ARG
    assert _reduce(L, **{**ok, "T": -1}) == tp.TP_ERR_ARG
    assert _reduce(L, **{**ok, "D": 62, "ldp": 64, "ldo": 64}) == tp.TP_ERR_ARG  # hidden % 4
    assert _reduce(L, **{**ok, "parts": [a + 8, b]}) == tp.TP_ERR_ARG            # misaligned
    assert _reduce(L, **{**ok, "parts": [0, b]}) == tp.TP_ERR_ARG                # NULL
    assert _reduce(L, **{**ok, "ldp": 60}) == tp.TP_ERR_ARG                      # ld < width
    assert _reduce(L, **{**ok, "ldo": 66}) == tp.TP_ERR_ARG                      # 16-byte rows
    assert _reduce(L, **{**ok, "out": 0}) == tp.TP_ERR_ARG
    # overlap: out on top of partials[1] is rejected; exact alias of partials[0] is allowed
    live = {**ok, "T": 4}
    assert _reduce(L, **{**live, "out": b}) == tp.TP_ERR_ARG
    assert _reduce(L, **{**live, "out": c - 64}) == tp.TP_ERR_ARG                # covers the bias
    assert "overlap" in tp.tp_last_error_detail()


def test_status_strings(L):
    for code in (tp.TP_OK, tp.TP_ERR_ARG, tp.TP_ERR_DIVISIBILITY, tp.TP_ERR_UNSUPPORTED,
                 tp.TP_ERR_HIP, tp.TP_ERR_OOM):
        assert tp.tp_status_string(code).startswith("TP_")
    assert tp.tp_status_string(42) == "unknown tp_status"


def test_binding_raises_with_detail(L):
    with pytest.raises(tp.TpError) as e:
        tp.tp_block_shard_create(tp.make_config(5, 0, 192, 24, 8, 0, tp.TP_BF16),
                                 _tiny_weights(192, 24, 8, 0))
    assert e.value.status == tp.TP_ERR_DIVISIBILITY
    assert "divide" in str(e.value)


def _swiglu_weights(D, H, d, F, dtype=np.uint16):
    w = _tiny_weights(D, H, d, F, dtype)
    w["w_up"] = np.zeros((2 * F, D), dtype)
    return w


def test_create_rejects_swiglu_and_stride_errors(L):
    sw = tp.TP_MLP_SWIGLU
    # ffn / tp = 40 is a multiple of 8 but not of 32: SwiGLU's paired tiles need 32
    st, out = _create(L, tp.make_config(2, 0, 64, 0, 0, 80, tp.TP_BF16, sw), _swiglu_weights(64, 0, 0, 80))
    assert st == tp.TP_ERR_UNSUPPORTED and out is None and "32" in tp.tp_last_error_detail()
    # ... while GELU accepts it (past validation: created, or a HIP error without a device)
    st, out = _create(L, tp.make_config(2, 0, 64, 0, 0, 80, tp.TP_BF16), _tiny_weights(64, 0, 0, 80))
    assert st != tp.TP_ERR_UNSUPPORTED
    if out:
        L.tp_block_shard_destroy(out)
    # unknown activation
    st, out = _create(L, tp.make_config(1, 0, 64, 0, 0, 64, tp.TP_BF16, 5), _tiny_weights(64, 0, 0, 64))
    assert st == tp.TP_ERR_ARG and "mlp_act" in tp.tp_last_error_detail()
    # row strides of the rowwise weights shorter than their rows
    for field, msg in (("ld_o", "ld_o"), ("ld_down", "ld_down")):
        cfg = tp.make_config(2, 0, 32, 4, 8, 64, tp.TP_BF16)
        weights = _tiny_weights(32, 4, 8, 64)
        w = tp.TpBlockWeights()
        for k, a in weights.items():
            setattr(w, k, a.ctypes.data)
        setattr(w, field, 16)
        out = ctypes.c_void_p()
        st = L.tp_block_shard_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(out))
        assert st == tp.TP_ERR_ARG and msg in tp.tp_last_error_detail()


def test_struct_layouts_match_the_header(tmp_path):
    """ctypes mirrors of tp_block_config / tp_block_weights have the C
    compiler's sizes and field offsets."""
    src = tmp_path / "layout.c"
    fields_c = ["tp_degree", "rank", "hidden", "num_heads", "head_dim", "ffn", "dtype", "mlp_act", "mod_in", "mod_out"]
    fields_w = list(binding._WEIGHT_FIELDS) + ["ld_o", "ld_down"]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "tp_shard.h"', 'int main(void) {',
             'printf("%zu\\n", sizeof(tp_block_config));', 'printf("%zu\\n", sizeof(tp_block_weights));']
    lines += [f'printf("%zu\\n", offsetof(tp_block_config, {f}));' for f in fields_c]
    lines += [f'printf("%zu\\n", offsetof(tp_block_weights, {f}));' for f in fields_w]
    lines += ['return 0; }']
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [ctypes.sizeof(tp.TpBlockConfig), ctypes.sizeof(tp.TpBlockWeights)]
    want += [getattr(tp.TpBlockConfig, f).offset for f in fields_c]
    want += [getattr(tp.TpBlockWeights, f).offset for f in fields_w]
    assert got == want


def test_binding_packed_weights_address_the_blocks():
    """A packed input projection and a packed output projection are passed as
    pointers into the blocks, with the output projection's row stride."""
    H, d, F, D = 4, 8, 96, 32
    HD = H * d
    cfg = tp.make_config(2, 0, D, H, d, F, tp.TP_BF16, tp.TP_MLP_SWIGLU)
    w_in = np.zeros((3 * HD + 2 * F, D), np.uint16)
    b_in = np.zeros(3 * HD + 2 * F, np.uint16)
    w_out = np.zeros((D, HD + F), np.uint16)
    w, keep = binding._host_weights({"w_in": w_in, "b_in": b_in, "w_out": w_out}, cfg)
    base = keep[0].ctypes.data
    assert [w.w_q, w.w_k, w.w_v, w.w_up] == [base + i * HD * D * 2 for i in range(4)]
    bb = keep[1].ctypes.data
    assert [w.b_q, w.b_k, w.b_v, w.b_up] == [bb + i * HD * 2 for i in range(4)]
    ob = keep[2].ctypes.data
    assert (w.w_o, w.w_down, w.ld_o, w.ld_down) == (ob, ob + HD * 2, HD + F, HD + F)
    with pytest.raises(ValueError):      # a GELU config expects W_up [F, D], not [2F, D]
        binding._host_weights({"w_in": w_in}, tp.make_config(2, 0, D, H, d, F, tp.TP_BF16))


@pytest.mark.parametrize("P,mi,mo,want", [
    (4, 30, 64, tp.TP_ERR_DIVISIBILITY),     # tp_degree does not divide the modulation input
    (4, 64, 0, tp.TP_ERR_ARG),               # mod_in without mod_out
    (4, 0, 64, tp.TP_ERR_ARG),               # mod_out without mod_in
    (4, -8, 64, tp.TP_ERR_ARG),
    (4, 96, 64, None),                       # mod_in / tp = 24, a multiple of 8: accepted
    (4, 64, 36, tp.TP_ERR_UNSUPPORTED),      # mod_out not a multiple of 8
    (4, 80, 64, tp.TP_ERR_UNSUPPORTED),      # mod_in / tp = 20 not a multiple of 8
])
def test_create_modulation_checks(L, P, mi, mo, want):
    cfg = tp.make_config(P, 0, 64, 0, 0, 0, tp.TP_BF16, mod_in=mi, mod_out=mo)
    w = {"w_mod": np.zeros((max(mo, 1), max(mi, 1)), np.uint16)}
    st, out = _create(L, cfg, w)
    if (mi, mo) == (96, 64):
        assert st != tp.TP_ERR_UNSUPPORTED and st != tp.TP_ERR_ARG   # valid: created or HIP error
        if out:
            L.tp_block_shard_destroy(out)
        return
    assert st == want, tp.tp_last_error_detail()
    assert out is None


def test_create_modulation_needs_its_weight(L):
    st, out = _create(L, tp.make_config(4, 0, 64, 0, 0, 0, tp.TP_BF16, mod_in=64, mod_out=64))
    assert st == tp.TP_ERR_ARG and "w_mod" in tp.tp_last_error_detail()


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("mi", [64, 96, 100])
def test_modulation_create_agrees_with_oracle(L, P, mi):
    try:
        O.check_config(P, 0, 64, 0, 0, 0, mod_in=mi)
        kind = None
    except O.ShardConfigError as e:
        kind = e.kind
    st, out = _create(L, tp.make_config(P, 0, 64, 0, 0, 0, tp.TP_BF16, mod_in=mi, mod_out=64),
                      {"w_mod": np.zeros((64, mi), np.uint16)})
    if out:
        L.tp_block_shard_destroy(out)
    if kind == "divisibility":
        assert st == tp.TP_ERR_DIVISIBILITY
    else:
        assert st in (tp.TP_OK, tp.TP_ERR_HIP, tp.TP_ERR_UNSUPPORTED, tp.TP_ERR_OOM)
        if st == tp.TP_ERR_UNSUPPORTED:
            assert (mi // P) % 8


def test_split_input_rejects_null_shard(L):
    vp = ctypes.c_void_p(0x10000)
    assert L.tp_rowwise_split_input_partial(None, tp.TP_ADALN_MOD, 8, vp, 64, vp, 64, 0, None) == tp.TP_ERR_ARG


def test_block_attention_and_merge_validation_without_device(L):
    vp = ctypes.c_void_p(0x10000)
    assert L.tp_attn_heads_block(None, 8, vp, 384, 8, vp, 384, vp, 128, vp, 1, None) == tp.TP_ERR_ARG
    a, b, c, d, o = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000   # never dereferenced

    def merge(o_parts=(a, b), lse_parts=(c, d), n=2, ldo_p=256, ld_l=2, T=0, heads=2, hd=128,
              out=o, ldo=256, dt=tp.TP_BF16, lse_out=None, ld_lo=0):
        OP = (ctypes.c_void_p * 2)(*o_parts)
        LP = (ctypes.c_void_p * 2)(*lse_parts)
        return L.tp_attn_merge(OP, LP, n, ldo_p, ld_l, T, heads, hd, out, ldo, dt, lse_out, ld_lo, None)

    assert merge() == tp.TP_OK                                  # tokens == 0: no-op
    assert merge(n=0) == tp.TP_ERR_ARG
    assert merge(n=17) == tp.TP_ERR_UNSUPPORTED
    assert merge(hd=6) == tp.TP_ERR_ARG                         # head_dim % 4
    assert merge(heads=0) == tp.TP_ERR_ARG
    assert merge(ld_l=1) == tp.TP_ERR_ARG                       # lse stride < heads
    assert merge(ldo_p=255) == tp.TP_ERR_ARG                    # < width / not 16-byte rows
    assert merge(o_parts=(a + 4, b)) == tp.TP_ERR_ARG           # misaligned
    assert merge(lse_parts=(0, d)) == tp.TP_ERR_ARG             # NULL
    assert merge(dt=9) == tp.TP_ERR_ARG
    assert merge(T=-1) == tp.TP_ERR_ARG
    assert merge(T=4, out=a) == tp.TP_ERR_ARG                   # output on top of a part
    assert "overlap" in tp.tp_last_error_detail()
    assert merge(T=4, lse_out=c, ld_lo=2) == tp.TP_ERR_ARG      # lse_out on top of a part


def test_split_attention_rejects_null_shard(L):
    vp = ctypes.c_void_p(0x10000)
    assert L.tp_attn_heads_split(None, 8, vp, 384, 2, vp, 128, 1024, vp, 1, 8, None) == tp.TP_ERR_ARG
    assert L.tp_attn_heads_block_split(None, 8, vp, 384, 8, vp, 384, 2, vp, 128, 1024, vp, 1, 8,
                                       None) == tp.TP_ERR_ARG


def test_ulysses_validation_without_device(L):
    a, b, o = 0x100000, 0x200000, 0x900000     # never dereferenced
    C = (ctypes.c_void_p * 2)(a, b)

    def s2h(degree=2, ld=3 * 4 * 128, n=0, heads=4, hd=128, blocks=3, rank=0, dt=tp.TP_BF16, out=o,
            ldo=3 * 2 * 128):
        return L.tp_ulysses_seq_to_heads(C, degree, ld, n, heads, hd, blocks, rank, dt, out, ldo, None)

    assert s2h() == tp.TP_OK                            # no tokens: no-op
    assert s2h(heads=3) == tp.TP_ERR_DIVISIBILITY       # degree does not divide the heads
    assert s2h(degree=0) == tp.TP_ERR_ARG
    assert s2h(degree=17) == tp.TP_ERR_UNSUPPORTED
    assert s2h(rank=2) == tp.TP_ERR_ARG
    assert s2h(blocks=4) == tp.TP_ERR_ARG
    assert s2h(hd=2) == tp.TP_ERR_UNSUPPORTED           # head block 2 heads x 2 bf16 = 8 bytes
    assert s2h(ldo=100) == tp.TP_ERR_ARG
    assert s2h(n=4, out=a) == tp.TP_ERR_ARG             # output on top of a chunk
    Pp = (ctypes.c_void_p * 2)(a, b)
    assert L.tp_ulysses_heads_to_seq(Pp, 2, 256, 0, 4, 128, 0, tp.TP_BF16, o, 512, None) == tp.TP_OK
    assert L.tp_ulysses_heads_to_seq(Pp, 2, 256, 0, 5, 128, 0, tp.TP_BF16, o, 640, None) == tp.TP_ERR_DIVISIBILITY


def _files(L, cfg, files, staging=1 << 20, ld_o=0, ld_down=0):
    f = binding.TpBlockWeightFiles()
    for k, v in files.items():
        setattr(f, k, binding.TpWeightFile(str(v[0]).encode(), v[1]))
    f.ld_o, f.ld_down = ld_o, ld_down
    out = ctypes.c_void_p(777)
    st = L.tp_block_shard_load(ctypes.byref(cfg), ctypes.byref(f), staging, ctypes.byref(out))
    return st, out.value


def test_load_validates_before_opening_any_file(L, tmp_path):
    missing = tmp_path / "does_not_exist.bin"
    attn = {k: (missing, 0) for k in ("w_q", "w_k", "w_v", "w_o")}
    # config errors win over the missing file: nothing is opened before the checks
    st, out = _files(L, tp.make_config(5, 0, 192, 24, 8, 0, tp.TP_BF16), attn)
    assert st == tp.TP_ERR_DIVISIBILITY and out is None
    st, out = _files(L, tp.make_config(2, 0, 32, 4, 8, 0, tp.TP_BF16), {"w_q": (missing, 0)})
    assert st == tp.TP_ERR_ARG and "missing" in tp.tp_last_error_detail()
    st, out = _files(L, tp.make_config(2, 0, 32, 4, 8, 0, tp.TP_BF16), attn, staging=1000)
    assert st == tp.TP_ERR_ARG and "staging" in tp.tp_last_error_detail()
    # a valid config whose file does not exist: TP_ERR_IO, before any device work
    st, out = _files(L, tp.make_config(2, 0, 32, 4, 8, 0, tp.TP_BF16), attn)
    assert st == tp.TP_ERR_IO and out is None and "cannot open" in tp.tp_last_error_detail()
    real = tmp_path / "w.bin"
    real.write_bytes(b"\0" * 64)
    st, out = _files(L, tp.make_config(2, 0, 32, 4, 8, 0, tp.TP_BF16),
                     {**{k: (real, 0) for k in ("w_q", "w_k", "w_v", "w_o")}, "w_q": (real, -2)})
    assert st == tp.TP_ERR_ARG and "offset" in tp.tp_last_error_detail()
    assert L.tp_block_shard_load(None, None, 1 << 20, None) == tp.TP_ERR_ARG
    assert "TP_ERR_IO" in tp.tp_status_string(tp.TP_ERR_IO)


def test_weight_files_struct_matches_the_header(tmp_path):
    src = tmp_path / "files.c"
    names = list(binding._WEIGHT_FIELDS) + ["ld_o", "ld_down"]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "tp_shard.h"', 'int main(void) {',
             'printf("%zu %zu\\n", sizeof(tp_weight_file), sizeof(tp_block_weight_files));']
    lines += [f'printf("%zu\\n", offsetof(tp_block_weight_files, {n}));' for n in names]
    lines += ['return 0; }']
    src.write_text("\n".join(lines))
    exe = tmp_path / "files"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [ctypes.sizeof(binding.TpWeightFile), ctypes.sizeof(binding.TpBlockWeightFiles)]
    want += [getattr(binding.TpBlockWeightFiles, n).offset for n in names]
    assert got == want

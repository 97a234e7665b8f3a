"""GPU parity of context-parallel attention against the float64 oracle
(Diffusers CP page, §Ring Attention): the block attention call (fp32
normalised output and log-sum-exp) on both attention kernels, ragged and
single-token blocks, and its key ranges split in one launch; the merge on
seeded partials (1..16 parts, bf16 and fp32 output, optional lse); and Ring
Attention simulated on one GPU -- every ring rank's steps (whole or as key
ranges) plus the merge -- against attention over the whole sequence, also at
the full 16384-token, 12-head rank shape on sampled rows.
Tolerances: outputs 2e-2 of max|ref| (bf16 operands, bf16 P); log-sum-exp
5e-3 absolute (the only rounding is the bf16 P summed in fp32, relative
2^-9 per term, so ln of the sum moves by at most ~2e-3)."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import tensor_dit_transformer_amd as tp
import tp_harness as H
import tp_inputs
from tp_inputs import Workload

pytestmark = pytest.mark.gpu
LSE_ATOL = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def attn_shard(heads_r, P=2):
    """A bf16 attention-only shard with heads_r local heads of 128."""
    H_ = heads_r * P
    w = Workload(f"attn_H{H_}_P{P}", 8, H_ * 128, H_, 128, 0, P, "bf16")
    inp = tp_inputs.make_inputs(w, seed=2)
    return H.create_shards(w, inp, ranks=(0,))[0]


def seeded_qkv(T, heads_r, seed, std=1.5):
    v, b = tp_inputs.random_matrix((T, 3 * heads_r * 128), seed=seed, std=std)
    return v.astype(np.float64), torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()


def qkv_parts(a, Dr):
    return a[:, :Dr], a[:, Dr:2 * Dr], a[:, 2 * Dr:]


@pytest.mark.parametrize("Tq,Tkv,heads_r", [(777, 333, 2), (1, 1, 2), (65, 4000, 3), (300, 64, 1),
                                           (8192, 1000, 6)])
def test_block_attention(Tq, Tkv, heads_r):
    s = attn_shard(heads_r)
    Dr = s.d_r
    qv, qd = seeded_qkv(Tq, heads_r, seed=40)
    kv, kd = seeded_qkv(Tkv, heads_r, seed=41)
    o = torch.empty((Tq, Dr), dtype=torch.float32, device="cuda")
    lse = torch.empty((Tq, heads_r), dtype=torch.float32, device="cuda")
    tp.tp_attn_heads_block(s, Tq, qd, Tkv, kd, o, lse)
    torch.cuda.synchronize()
    q = qkv_parts(qv, Dr)[0]
    _, k, v = qkv_parts(kv, Dr)
    rows = tp_inputs.sample_rows(Tq, 64, seed=5) if Tq > 2048 else np.arange(Tq)
    o_ref, l_ref = O.attention_block(q[rows], k, v, heads_r, 128)
    e_o = H.rel_err(H.as_f64(o[rows]), o_ref)
    e_l = float(np.max(np.abs(H.as_f64(lse[rows]) - l_ref)))
    say(f"block Tq={Tq} Tkv={Tkv} heads={heads_r}: o {e_o:.2e}  lse abs {e_l:.2e}")
    assert e_o <= H.TOL["bf16"] and e_l <= LSE_ATOL
    torch.cuda.synchronize()
    s.close()


@pytest.mark.parametrize("n,out_dtype,with_lse", [(1, "bf16", True), (2, "f32", True),
                                                  (5, "bf16", False), (16, "f32", True)])
def test_merge_on_seeded_partials(n, out_dtype, with_lse):
    T, heads, hd = 333, 3, 128
    o_parts = [tp_inputs.random_matrix((T, heads * hd), seed=50 + i, dtype="f32")[0] for i in range(n)]
    lse_parts = [3.0 * tp_inputs.random_matrix((T, heads), seed=80 + i, dtype="f32")[0] for i in range(n)]
    od = [torch.from_numpy(a).cuda() for a in o_parts]
    ld = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in lse_parts]
    dt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = torch.empty((T, heads * hd), dtype=dt, device="cuda")
    lse_out = torch.empty((T, heads), dtype=torch.float32, device="cuda") if with_lse else None
    tp.tp_attn_merge(od, ld, out, heads, hd, lse_out=lse_out)
    torch.cuda.synchronize()
    o_ref, l_ref = O.attention_merge(o_parts, lse_parts, hd)
    if out_dtype == "bf16":
        o_ref = O.to_bf16_rne(o_ref)
    e = H.rel_err(H.as_f64(out), o_ref)
    tol = 8e-3 if out_dtype == "bf16" else 1e-5
    say(f"merge n={n} {out_dtype}: o {e:.2e}")
    assert e <= tol
    if with_lse:
        assert float(np.max(np.abs(H.as_f64(lse_out) - l_ref))) <= 1e-5


def ring_on_one_gpu(s, qkv, T, R, splits=1):
    """Every ring rank c: step t attends its query chunk to K/V chunk
    (c - t) mod R -- with splits > 1 as that many key ranges in one launch --
    then merges its R * splits partials into its output chunk."""
    n, Dr, Hr = T // R, s.d_r, s.heads_r
    out = torch.empty((T, Dr), dtype=torch.bfloat16, device="cuda")
    o_parts = torch.empty((R, splits, n, Dr), dtype=torch.float32, device="cuda")
    l_parts = torch.empty((R, splits, n, Hr), dtype=torch.float32, device="cuda")
    for c in range(R):
        for t in range(R):
            j = (c - t) % R
            q, kv = qkv[c * n:(c + 1) * n], qkv[j * n:(j + 1) * n]
            if splits == 1:
                tp.tp_attn_heads_block(s, n, q, n, kv, o_parts[t, 0], l_parts[t, 0])
            else:
                tp.tp_attn_heads_block_split(s, n, q, n, kv, o_parts[t], l_parts[t])
        tp.tp_attn_merge(list(o_parts.flatten(0, 1)), list(l_parts.flatten(0, 1)),
                         out[c * n:(c + 1) * n], Hr, 128)
    return out


@pytest.mark.parametrize("T,heads_r,R,splits", [(4096, 2, 4, 1), (1200, 3, 3, 1), (2048, 2, 1, 1),
                                                (4096, 2, 4, 2), (1200, 3, 3, 4)])
def test_ring_attention_equals_attention(T, heads_r, R, splits):
    s = attn_shard(heads_r)
    qv, qd = seeded_qkv(T, heads_r, seed=60)
    out = ring_on_one_gpu(s, qd, T, R, splits)
    mono = torch.empty((T, s.d_r), dtype=torch.bfloat16, device="cuda")
    tp.tp_attn_heads(s, T, qd, mono)
    torch.cuda.synchronize()
    q, k, v = qkv_parts(qv, s.d_r)
    ref = O.to_bf16_rne(O.attention_heads(q, k, v, heads_r, 128))
    e = H.rel_err(H.as_f64(out), ref)
    e_m = H.rel_err(H.as_f64(out), H.as_f64(mono))
    say(f"ring T={T} heads={heads_r} R={R} splits={splits}: vs oracle {e:.2e}, vs one call {e_m:.2e}")
    assert e <= H.TOL["bf16"] and e_m <= H.TOL["bf16"]
    torch.cuda.synchronize()
    s.close()


@pytest.mark.parametrize("splits", [1, 2])
def test_ring_attention_full_rank_shape(splits):
    """16384 tokens, 12 local heads, ring of 4 (steps whole or as two key
    ranges): sampled rows of two heads."""
    T, heads_r, R = 16384, 12, 4
    s = attn_shard(heads_r, P=4)
    qv, qd = seeded_qkv(T, heads_r, seed=61)
    out = ring_on_one_gpu(s, qd, T, R, splits)
    torch.cuda.synchronize()
    rows = tp_inputs.sample_rows(T, 32, seed=7)
    Dr = s.d_r
    for j in (0, 11):
        c = slice(j * 128, (j + 1) * 128)
        ref = O.to_bf16_rne(O.attention_rows(qv[rows, c], qv[:, Dr + j * 128:Dr + (j + 1) * 128],
                                             qv[:, 2 * Dr + j * 128:2 * Dr + (j + 1) * 128], 1, 128))
        e = H.rel_err(H.as_f64(out[rows, c]), ref)
        say(f"ring T=16384 R=4 splits={splits} head {j}: {e:.2e}")
        assert e <= H.TOL["bf16"]
    s.close()


@pytest.mark.parametrize("T,heads_r,S", [(4608, 6, 2), (4608, 6, 4), (777, 2, 3), (5, 1, 5),
                                         (1000, 3, 16), (300, 2, 1)])
def test_single_launch_key_split_then_merge(T, heads_r, S):
    """Key ranges [floor(zT/S), floor((z+1)T/S)) in one launch: each part
    against the oracle's block attention over its keys, and the merge
    against attention over all keys and the one-call attention."""
    s = attn_shard(heads_r)
    Dr = s.d_r
    qv, qd = seeded_qkv(T, heads_r, seed=70)
    op = torch.empty((S, T, Dr), dtype=torch.float32, device="cuda")
    lp = torch.empty((S, T, heads_r), dtype=torch.float32, device="cuda")
    tp.tp_attn_heads_split(s, T, qd, op, lp)
    out = torch.empty((T, Dr), dtype=torch.bfloat16, device="cuda")
    tp.tp_attn_merge(list(op), list(lp), out, heads_r, 128)
    mono = torch.empty((T, Dr), dtype=torch.bfloat16, device="cuda")
    tp.tp_attn_heads(s, T, qd, mono)
    torch.cuda.synchronize()
    q, k, v = qkv_parts(qv, Dr)
    rows = tp_inputs.sample_rows(T, 48, seed=8)
    for z in range(S):
        a, b = (z * T) // S, ((z + 1) * T) // S
        o_ref, l_ref = O.attention_block(q[rows], k[a:b], v[a:b], heads_r, 128)
        assert H.rel_err(H.as_f64(op[z][rows]), o_ref) <= H.TOL["bf16"]
        assert float(np.max(np.abs(H.as_f64(lp[z][rows]) - l_ref))) <= LSE_ATOL
    ref = O.to_bf16_rne(O.attention_rows(q[rows], k, v, heads_r, 128))
    e = H.rel_err(H.as_f64(out[rows]), ref)
    e_m = H.rel_err(H.as_f64(out), H.as_f64(mono))
    say(f"split T={T} heads={heads_r} S={S}: merged vs oracle {e:.2e}, vs one call {e_m:.2e}")
    assert e <= H.TOL["bf16"] and e_m <= H.TOL["bf16"]
    if S == 1:
        assert torch.equal(out, mono)
    torch.cuda.synchronize()
    s.close()


@pytest.mark.parametrize("Tq,Tkv,heads_r,S", [(1152, 1152, 6, 2), (777, 333, 2, 3), (65, 4000, 3, 4),
                                              (8192, 1000, 6, 2), (300, 16, 1, 16), (40, 50, 2, 1)])
def test_block_key_split_parts(Tq, Tkv, heads_r, S):
    """Queries of one buffer against a key block of another, the block's
    keys cut into S ranges in one launch: each part against the oracle's
    block attention over its keys; one range is bitwise the block call."""
    s = attn_shard(heads_r)
    Dr = s.d_r
    qv, qd = seeded_qkv(Tq, heads_r, seed=90)
    kv, kd = seeded_qkv(Tkv, heads_r, seed=91)
    op = torch.empty((S, Tq, Dr), dtype=torch.float32, device="cuda")
    lp = torch.empty((S, Tq, heads_r), dtype=torch.float32, device="cuda")
    tp.tp_attn_heads_block_split(s, Tq, qd, Tkv, kd, op, lp)
    torch.cuda.synchronize()
    q = qkv_parts(qv, Dr)[0]
    _, k, v = qkv_parts(kv, Dr)
    rows = tp_inputs.sample_rows(Tq, 48, seed=9) if Tq > 512 else np.arange(Tq)
    for z in range(S):
        a, b = (z * Tkv) // S, ((z + 1) * Tkv) // S
        o_ref, l_ref = O.attention_block(q[rows], k[a:b], v[a:b], heads_r, 128)
        e_o = H.rel_err(H.as_f64(op[z][rows]), o_ref)
        e_l = float(np.max(np.abs(H.as_f64(lp[z][rows]) - l_ref)))
        assert e_o <= H.TOL["bf16"] and e_l <= LSE_ATOL, f"part {z}: o {e_o:.2e} lse {e_l:.2e}"
    say(f"block split Tq={Tq} Tkv={Tkv} heads={heads_r} S={S}: {S} parts within tolerance")
    if S == 1:
        o1 = torch.empty((Tq, Dr), dtype=torch.float32, device="cuda")
        l1 = torch.empty((Tq, heads_r), dtype=torch.float32, device="cuda")
        tp.tp_attn_heads_block(s, Tq, qd, Tkv, kd, o1, l1)
        torch.cuda.synchronize()
        assert torch.equal(o1, op[0]) and torch.equal(l1, lp[0])
    torch.cuda.synchronize()
    s.close()


def test_block_key_split_errors():
    """More key ranges than keys, more than 16 ranges, and overlapping parts
    are rejected before any launch; no queries is a no-op."""
    s = attn_shard(2)
    Dr = s.d_r
    _, qd = seeded_qkv(40, 2, seed=92)
    _, kd = seeded_qkv(3, 2, seed=93)

    def parts(S, T=40):
        return (torch.empty((S, T, Dr), dtype=torch.float32, device="cuda"),
                torch.empty((S, T, 2), dtype=torch.float32, device="cuda"))

    op, lp = parts(4)
    with pytest.raises(tp.TpError) as e:
        tp.tp_attn_heads_block_split(s, 40, qd, 3, kd, op, lp)      # 4 ranges over 3 keys
    assert e.value.status == tp.TP_ERR_ARG
    op, lp = parts(17)
    with pytest.raises(tp.TpError) as e:
        tp.tp_attn_heads_block_split(s, 40, qd, 3, kd, op, lp)
    assert e.value.status == tp.TP_ERR_UNSUPPORTED
    o_all = torch.empty((2 * 40 * Dr,), dtype=torch.float32, device="cuda")
    l_all = torch.empty((2 * 40 * 2,), dtype=torch.float32, device="cuda")
    short = o_all.as_strided((2, 40, Dr), (40 * Dr - 4, Dr, 1))    # part 1 starts inside part 0
    with pytest.raises(tp.TpError) as e:
        tp.tp_attn_heads_block_split(s, 40, qd, 3, kd, short, l_all.view(2, 40, 2))
    assert e.value.status == tp.TP_ERR_ARG
    op, lp = parts(5)
    tp.tp_attn_heads_block_split(s, 0, qd, 3, kd, op, lp)           # no queries: nothing to do,
                                                                     # even with 5 ranges over 3 keys
    torch.cuda.synchronize()
    s.close()


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("u,heads,blocks,n", [(2, 4, 3, 100), (4, 8, 1, 33), (3, 6, 3, 64), (1, 2, 3, 5)])
def test_ulysses_relayouts_are_exact(u, heads, blocks, n):
    """Both all-to-alls against the oracle's placements, bit for bit."""
    d = 128
    chunks_v, chunks_d = [], []
    for s in range(u):
        v, b = tp_inputs.random_matrix((n, blocks * heads * d), seed=90 + s)
        chunks_v.append(v)
        chunks_d.append(_dev_bf16(b))
    W = heads // u * d
    outs = []
    for r in range(u):
        out = torch.empty((u * n, blocks * W), dtype=torch.bfloat16, device="cuda")
        tp.tp_ulysses_seq_to_heads(chunks_d, heads, d, blocks, r, out)
        outs.append(out)
    torch.cuda.synchronize()
    for b in range(blocks):
        ref = O.ulysses_seq_to_heads([c[:, b * heads * d:(b + 1) * heads * d] for c in chunks_v], heads, d)
        for r in range(u):
            assert np.array_equal(H.as_f64(outs[r][:, b * W:(b + 1) * W]), ref[r])
    # back: the Q block of every rank's head view returns to the token chunks
    parts = [o[:, :W].contiguous() for o in outs]
    ref_back = O.ulysses_heads_to_seq([H.as_f64(p) for p in parts], heads, d)
    for s in range(u):
        back = torch.empty((n, heads * d), dtype=torch.bfloat16, device="cuda")
        tp.tp_ulysses_heads_to_seq(parts, heads, d, s, back)
        torch.cuda.synchronize()
        assert np.array_equal(H.as_f64(back), ref_back[s])
        assert np.array_equal(H.as_f64(back), chunks_v[s][:, :heads * d])


@pytest.mark.parametrize("u,T,heads", [(2, 1024, 4), (4, 4096, 8)])
def test_ulysses_attention_equals_attention(u, T, heads):
    """Token-chunked packed qkv -> first all-to-all -> each rank's attention
    over its H/u heads (tp_attn_heads on the re-laid-out packed buffer) ->
    second all-to-all, against attention over all heads."""
    d, n = 128, T // u
    qv, qb = tp_inputs.random_matrix((T, 3 * heads * d), seed=95, std=1.5)
    chunks = [_dev_bf16(qb[s * n:(s + 1) * n]) for s in range(u)]
    s_ = attn_shard(heads // u, P=u)
    W = heads // u * d
    o_heads = []
    for r in range(u):
        hv = torch.empty((T, 3 * W), dtype=torch.bfloat16, device="cuda")
        tp.tp_ulysses_seq_to_heads(chunks, heads, d, 3, r, hv)
        o = torch.empty((T, W), dtype=torch.bfloat16, device="cuda")
        tp.tp_attn_heads(s_, T, hv, o)
        o_heads.append(o)
    outs = []
    for s in range(u):
        back = torch.empty((n, heads * d), dtype=torch.bfloat16, device="cuda")
        tp.tp_ulysses_heads_to_seq(o_heads, heads, d, s, back)
        outs.append(back)
    torch.cuda.synchronize()
    q64 = qv.astype(np.float64)
    HD = heads * d
    rows = tp_inputs.sample_rows(T, 48, seed=9)
    ref = O.to_bf16_rne(O.attention_rows(q64[rows, :HD], q64[:, HD:2 * HD], q64[:, 2 * HD:], heads, d))
    got = torch.cat(outs)[rows]
    e = H.rel_err(H.as_f64(got), ref)
    say(f"ulysses u={u} T={T} heads={heads}: {e:.2e}")
    assert e <= H.TOL["bf16"]
    torch.cuda.synchronize()
    s_.close()

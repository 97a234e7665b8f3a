"""Benchmark of the tensor-parallel DiT block shard on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input:
for every simulated rank r = 0..P-1 of the full block (T=16384 tokens,
hidden 6144, 48 heads x 128, ffn 18432, tp_degree 4),
    fused colwise QKV + MLP-up (bias, GELU-tanh)   -> qkv_r, h_r
    attention over the rank's 12 heads              -> o_r
    packed rowwise out over [o_r | h_r]             -> fp32 partial_r
and then the partial reduce (+ rowwise biases) that stands in for the
boundary AllReduce.  Inputs and weights are resident in HBM before timing.

Prints one JSON line: value = algorithmic TFLOP/s of the step (GEMM
2*M*N*K + attention 4*T^2*d per head, all ranks) / step time; "roofline"
for the kernel with the largest share of step time, from HIP events around
each launch on the stream it runs on; "cpu_baseline" = the float64 oracle
timed on the host cores on a bounded sample (rank 0's shard of the same
block on the first 12288 tokens).

--workload single_swiglu_bf16_T16384_D6144_H48_F18432_P4 times the
single-stream variant of the same block instead: shards created from one
packed input projection (Q, K, V, gate, up; blocks [1, 1, 1, 3, 3]) and one
packed output projection over [inner_dim, mlp_hidden_dim], MLP activation
SwiGLU fused into the colwise epilogue.  Other workloads: the mid-size
shards (4608 tokens), the AdaLN modulation projection sharded
"rowwise_split_input" (adaln_mod_bf16_R8_D6144_N36864_P4), and
context-parallel attention over 4 simulated GPUs at the CP page's
benchmark size (cp_ring_bf16_T4608_H24_R4, cp_ulysses_bf16_T4608_H24_U4).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
HBM_PEAK_GBS = 8000.0
PCIE_PEAK_GBS = 64.0             # host link, PCIe 5.0 x16, one direction


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(name: str) -> str:
    p = os.path.join(ROOT, "tensor_dit_transformer_amd", "csrc", name)
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(kernel_key: str, source: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if absent or taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    e = t.get(kernel_key)
    if not e or e.get("source_sha") != kernel_source_hash(source):
        return None
    return e.get("bytes_per_launch")


class ClockSampler:
    """Samples the GPU's current shader clock (the '*' level of the DRM
    pp_dpm_sclk file, which holds the live frequency) every `period` seconds
    from a background thread while the timed steps run.  MI355X lowers its
    clock under sustained matrix-core load, so the held clock says how far
    the published 2.4 GHz peak is from what the chip ran at."""

    def __init__(self, period: float = 0.005):
        import glob
        import threading
        self.path = None
        for d in sorted(glob.glob("/sys/class/drm/card*/device")):
            try:
                if open(os.path.join(d, "vendor")).read().strip() == "0x1002" and \
                        os.path.exists(os.path.join(d, "pp_dpm_sclk")):
                    self.path = os.path.join(d, "pp_dpm_sclk")
                    break
            except OSError:
                continue
        self.period = period
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._loop, daemon=True)

    def _read(self):
        try:
            for line in open(self.path):
                if line.rstrip().endswith("*"):
                    return float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
        except (OSError, ValueError, IndexError):
            return None
        return None

    def _loop(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.path:
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        s = sorted(self.samples)
        return {"source": "pp_dpm_sclk (live shader clock) sampled during the timed steps",
                "median_mhz": s[len(s) // 2], "min_mhz": s[0], "max_mhz": s[-1],
                "samples": len(s)}


def cpu_baseline(w, tokens_sample: int = 12288):
    """The oracle, as it stands, on rank 0 of workload `w` for the first
    `tokens_sample` tokens (a shorter sequence of the same block)."""
    import numpy as np
    import oracle as O
    import tp_inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    if w.cp:
        T = min(1536, w.tokens)
        qv, _ = tp_inputs.cp_qkv(w, seed=0, tokens=T)
        HD = w.num_heads * w.head_dim
        q, k, v = qv[:, :HD], qv[:, HD:2 * HD], qv[:, 2 * HD:]
        t0 = time.perf_counter()
        if w.cp == "ring":
            O.ring_attention(q, k, v, w.num_heads, w.head_dim, w.cp_degree)
        else:
            O.ulysses_attention(q, k, v, w.num_heads, w.head_dim, w.cp_degree)
        dt = time.perf_counter() - t0
        flops = 4 * T * T * w.head_dim * w.num_heads
        return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                "sample": f"{w.cp} attention over {w.cp_degree} ranks of {w.name} on the first {T} "
                          f"tokens: {flops / 1e9:.1f} GFLOP fp64 in {dt:.2f} s",
                "seconds": round(dt, 2), "cpu_count": os.cpu_count()}
    tokens_sample = min(tokens_sample, w.tokens)
    inp = tp_inputs.make_inputs(w, seed=0, tokens=tokens_sample)
    t0 = time.perf_counter()
    if w.has_attn or w.has_mlp:
        O.rank_forward(inp["x"], inp.values, w.tp_degree, 0, w.num_heads, w.head_dim, bf16=True,
                       mlp_act=w.mlp_act)
    if w.has_mod:
        O.split_input_rank(inp["c"], inp["w_mod"], w.tp_degree, 0)
    dt = time.perf_counter() - t0
    T = tokens_sample
    flops = step_flops(w, T)
    what = f"the first {T} tokens" if T > 0 else f"its {w.mod_rows} conditioning rows"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"rank 0 of {w.tp_degree} of {w.name} on {what}: "
                      f"{flops / 1e9:.1f} GFLOP fp64 in {dt:.2f} s",
            "seconds": round(dt, 2), "cpu_count": os.cpu_count()}


def cpu_baseline_load(w, path):
    """The CPU way the TP page contrasts with: read the whole checkpoint into
    host memory, then slice rank 0's weights with the oracle's shard_weights."""
    import numpy as np
    import oracle as O
    D, Hh, d, F, P = w.hidden, w.num_heads, w.head_dim, w.ffn, w.tp_degree
    HD = Hh * d
    t0 = time.perf_counter()
    raw = np.fromfile(path, dtype=np.uint16)
    shapes = [("w_q", (HD, D)), ("w_k", (HD, D)), ("w_v", (HD, D)), ("w_o", (D, HD)),
              ("w_up", (F, D)), ("w_dn", (D, F))]
    wts, off = {}, 0
    for name, shp in shapes:
        n = shp[0] * shp[1]
        wts[name] = raw[off:off + n].reshape(shp)
        off += n
    wts.update(b_q=np.zeros(HD), b_k=np.zeros(HD), b_v=np.zeros(HD), b_up=np.zeros(F))
    sl = O.shard_weights(wts, P, 0, Hh, d)
    dt = time.perf_counter() - t0
    slice_bytes = raw.nbytes // P
    del raw, wts, sl
    return {"value": slice_bytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"rank 0 of {P}: whole {off * 2 / 1e6:.0f} MB checkpoint read into host memory, "
                      f"then sliced by the oracle (float64 slices), {dt:.2f} s",
            "seconds": round(dt, 2), "cpu_count": os.cpu_count()}


def step_kernels(w, T):
    """Kernels of one rank's pass, with algorithmic work per launch (FLOPs for
    the MFMA kernels) and their bound."""
    D, P, d = w.hidden, w.tp_degree, w.head_dim
    Dr = D // P if w.has_attn else 0
    Fr, Hr = w.ffn // P, w.num_heads // P
    U = 2 * Fr if w.mlp_act == "swiglu" else Fr      # colwise MLP-in rows
    kernels = {}
    if w.has_attn and w.has_mlp:
        kernels["colwise_qkv_up"] = ("gemm_bf16.hip", 2 * T * D * (3 * Dr + U), "mfma")
        kernels["attention"] = ("attn_fwd.hip", 4 * T * T * d * Hr, "mfma")
        kernels["rowwise_block_out"] = ("gemm_bf16.hip", 2 * T * (Dr + Fr) * D, "mfma")
    elif w.has_attn:
        kernels["colwise_qkv"] = ("gemm_bf16.hip", 2 * T * D * 3 * Dr, "mfma")
        kernels["attention"] = ("attn_fwd.hip", 4 * T * T * d * Hr, "mfma")
        kernels["rowwise_attn_out"] = ("gemm_bf16.hip", 2 * T * Dr * D, "mfma")
    elif w.has_mlp:
        kernels["colwise_mlp_up"] = ("gemm_bf16.hip", 2 * T * D * U, "mfma")
        kernels["rowwise_mlp_down"] = ("gemm_bf16.hip", 2 * T * Fr * D, "mfma")
    if w.has_mod:
        # few-row split-input partial: streams the weight slice; bytes =
        # weight slice + replicated input slice + fp32 partial written
        R, Kr, N = w.mod_rows, D // P, w.mod_out
        kernels["split_input_mod"] = ("skinny_bf16.hip", 2 * N * Kr + 2 * R * Kr + 4 * R * N, "hbm")
    return kernels


def step_text(w):
    parts = []
    if w.has_mod:
        parts.append(f"split-input modulation partial over {w.mod_rows} replicated rows")
    if w.has_attn and w.has_mlp:
        parts.append("fused colwise QKV+MLP-in, attention, packed rowwise out")
    elif w.has_attn:
        parts.append("colwise QKV, attention, rowwise attention out")
    elif w.has_mlp:
        parts.append("colwise MLP-in, rowwise MLP-down")
    return "per rank: " + "; ".join(parts) + "; then partial reduce"


def step_flops(w, T):
    """Algorithmic FLOPs of one rank's pass (GEMMs 2 M N K, attention 4 T^2 d
    per head, the modulation projection 2 R K_r N)."""
    f = sum(work for _src, work, bound in step_kernels(w, T).values() if bound == "mfma")
    if w.has_mod:
        f += 2 * w.mod_rows * (w.hidden // w.tp_degree) * w.mod_out
    return f


class Setup:
    """What one workload's step needs: `kernels` maps a kernel name to
    (source file, algorithmic work per launch, bound), `run(mark)` enqueues
    one step (each launch wrapped in mark(name, fn)), `flops` is the step's
    algorithmic FLOPs, `config` its description, `close()` frees it."""

    def __init__(self, kernels, run, flops, config, close):
        self.kernels, self.run, self.flops, self.config, self.close = kernels, run, flops, config, close


def setup_block(w):
    import torch
    import tensor_dit_transformer_amd as tp
    import tp_harness as H
    import tp_inputs

    T, D, P, d = w.tokens, w.hidden, w.tp_degree, w.head_dim
    inp = tp_inputs.make_inputs(w, seed=0)
    # a single-stream SwiGLU block comes as a packed checkpoint (fused input
    # and output projections)
    packed = w.mlp_act == "swiglu" and w.has_attn
    shards = H.create_shards(w, inp, packed=packed)
    x = H.to_device(inp, "x") if w.tokens > 0 else None
    biases = H.rowwise_biases(w, inp)
    c = H.to_device(inp, "c") if w.has_mod else None
    mod_bias = [H.f32_device(inp.values["b_mod"])] if w.has_mod else []
    del inp
    block = w.has_attn or w.has_mlp
    if block:
        partials = [torch.empty((T, D), dtype=torch.float32, device="cuda") for _ in range(P)]
        bufs = H.RankBuffers(shards[0], T, partial=partials[0])
        y = torch.empty((T, D), dtype=torch.float32, device="cuda")
    if w.has_mod:
        mod_parts = [torch.empty((w.mod_rows, w.mod_out), dtype=torch.float32, device="cuda")
                     for _ in range(P)]
        y_mod = torch.empty((w.mod_rows, w.mod_out), dtype=torch.float32, device="cuda")

    kernels = step_kernels(w, T)
    if block:
        reduce_bytes = (P + 1) * T * D * 4 + len(biases) * D * 4
        kernels["partial_reduce"] = ("partial_reduce.hip", reduce_bytes, "hbm")
    if block and bufs.splits > 1:
        S, Hr = bufs.splits, w.num_heads // P
        Dr = Hr * d
        kernels["attn_merge"] = ("attn_merge.hip", S * T * (Dr + Hr) * 4 + T * Dr * 2, "hbm")
    if w.has_mod:
        kernels["mod_reduce"] = ("partial_reduce.hip",
                                 (P + 1) * w.mod_rows * w.mod_out * 4 + w.mod_out * 4, "hbm")

    def run(mark):
        def attention(s):
            if bufs.splits > 1:
                mark("attention", lambda: tp.tp_attn_heads_split(s, T, bufs.qkv, bufs.o_parts,
                                                                 bufs.lse_parts))
                mark("attn_merge", lambda: tp.tp_attn_merge(list(bufs.o_parts), list(bufs.lse_parts),
                                                            bufs.o, s.heads_r, d))
            else:
                mark("attention", lambda: tp.tp_attn_heads(s, T, bufs.qkv, bufs.o))

        for r, s in enumerate(shards):
            if w.has_mod:
                mark("split_input_mod", lambda: tp.tp_rowwise_split_input_partial(
                    s, tp.TP_ADALN_MOD, w.mod_rows, c, mod_parts[r]))
            if not block:
                continue
            bufs.partial = partials[r]
            if w.has_attn and w.has_mlp:
                mark("colwise_qkv_up", lambda: tp.tp_colwise_qkv_up(s, T, x, bufs.qkv, bufs.h))
                attention(s)
                mark("rowwise_block_out", lambda: tp.tp_rowwise_linear_partial(
                    s, tp.TP_BLOCK_OUT, T, bufs.oh, bufs.partial))
            elif w.has_attn:
                mark("colwise_qkv", lambda: tp.tp_colwise_linear(s, tp.TP_QKV, T, x, bufs.qkv))
                attention(s)
                mark("rowwise_attn_out", lambda: tp.tp_rowwise_linear_partial(
                    s, tp.TP_ATTN_OUT, T, bufs.o, bufs.partial))
            else:
                mark("colwise_mlp_up", lambda: tp.tp_colwise_linear(s, tp.TP_MLP_UP, T, x, bufs.h))
                mark("rowwise_mlp_down", lambda: tp.tp_rowwise_linear_partial(
                    s, tp.TP_MLP_DOWN, T, bufs.h, bufs.partial))
        if block:
            mark("partial_reduce", lambda: tp.tp_partial_reduce(partials, biases, y))
        if w.has_mod:
            mark("mod_reduce", lambda: tp.tp_partial_reduce(mod_parts, mod_bias, y_mod))

    def close():
        torch.cuda.synchronize()
        for s in shards:
            s.close()

    config = {"workload": w.name, "tokens": T, "hidden": D, "num_heads": w.num_heads,
              "head_dim": d, "ffn": w.ffn, "tp_degree": P, "ranks_per_step": P,
              "mlp_act": w.mlp_act, "packed_checkpoint": packed, "step": step_text(w)}
    return Setup(kernels, run, step_flops(w, T) * P, config, close)


def setup_cp(w):
    """Context-parallel attention of all heads over cp_degree simulated GPUs:
    Ring (every rank's steps over the K/V chunks it is passed, then the merge)
    or Ulysses (first all-to-all, each rank's attention over its heads, second
    all-to-all)."""
    import numpy as np
    import torch
    import tensor_dit_transformer_amd as tp
    import tp_harness as H
    import tp_inputs

    T, Hh, d, R = w.tokens, w.num_heads, w.head_dim, w.cp_degree
    HD, n = Hh * d, w.tokens // w.cp_degree
    _, bits = tp_inputs.cp_qkv(w, seed=0)
    qkv = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    # an attention-capable shard handle with the heads one rank attends to
    P = 1 if w.cp == "ring" else R
    hw = tp_inputs.Workload("cp_heads", 8, HD, Hh, d, 0, P, "bf16")
    shard = H.create_shards(hw, tp_inputs.make_inputs(hw, seed=0), ranks=(0,))[0]
    kernels = {}
    if w.cp == "ring":
        # a step's chunks may be too short to fill the GPU: then each step
        # runs as S key ranges in one launch and the merge takes R * S parts
        S = key_splits = tp.tp_attn_split_hint(shard, n)
        o_parts = torch.empty((R, S, n, HD), dtype=torch.float32, device="cuda")
        l_parts = torch.empty((R, S, n, Hh), dtype=torch.float32, device="cuda")
        o_list, l_list = list(o_parts.flatten(0, 1)), list(l_parts.flatten(0, 1))
        out = torch.empty((T, HD), dtype=torch.bfloat16, device="cuda")
        kernels["attention_block"] = ("attn_fwd.hip", 4 * n * n * d * Hh, "mfma")
        kernels["attn_merge"] = ("attn_merge.hip", R * S * n * (HD + Hh) * 4 + n * HD * 2, "hbm")

        def step(t, q, kv):
            if S == 1:
                tp.tp_attn_heads_block(shard, n, q, n, kv, o_parts[t, 0], l_parts[t, 0])
            else:
                tp.tp_attn_heads_block_split(shard, n, q, n, kv, o_parts[t], l_parts[t])

        def run(mark):
            for c in range(R):
                for t in range(R):
                    j = (c - t) % R
                    mark("attention_block", lambda: step(t, qkv[c * n:(c + 1) * n],
                                                         qkv[j * n:(j + 1) * n]))
                mark("attn_merge", lambda: tp.tp_attn_merge(o_list, l_list, out[c * n:(c + 1) * n],
                                                            Hh, d))
    else:
        W = HD // R
        chunks = [qkv[s * n:(s + 1) * n] for s in range(R)]
        hv = torch.empty((T, 3 * W), dtype=torch.bfloat16, device="cuda")
        o_heads = [torch.empty((T, W), dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        back = [torch.empty((n, HD), dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        splits = key_splits = tp.tp_attn_split_hint(shard, T)
        if splits > 1:
            op = torch.empty((splits, T, W), dtype=torch.float32, device="cuda")
            lp = torch.empty((splits, T, Hh // R), dtype=torch.float32, device="cuda")
            kernels["attn_merge"] = ("attn_merge.hip", splits * T * (W + Hh // R) * 4 + T * W * 2, "hbm")
        kernels["ulysses_seq_to_heads"] = ("relayout.hip", 2 * T * 3 * W * 2, "hbm")
        kernels["attention"] = ("attn_fwd.hip", 4 * T * T * d * (Hh // R), "mfma")
        kernels["ulysses_heads_to_seq"] = ("relayout.hip", 2 * n * HD * 2, "hbm")

        def run(mark):
            for r in range(R):
                mark("ulysses_seq_to_heads", lambda: tp.tp_ulysses_seq_to_heads(chunks, Hh, d, 3, r, hv))
                if splits > 1:
                    mark("attention", lambda: tp.tp_attn_heads_split(shard, T, hv, op, lp))
                    mark("attn_merge", lambda: tp.tp_attn_merge(list(op), list(lp), o_heads[r],
                                                                Hh // R, d))
                else:
                    mark("attention", lambda: tp.tp_attn_heads(shard, T, hv, o_heads[r]))
            for s in range(R):
                mark("ulysses_heads_to_seq", lambda: tp.tp_ulysses_heads_to_seq(o_heads, Hh, d, s,
                                                                                back[s]))

    def close():
        torch.cuda.synchronize()
        shard.close()

    config = {"workload": w.name, "tokens": T, "num_heads": Hh, "head_dim": d, "cp": w.cp,
              "cp_degree": R, "ranks_per_step": R, "key_splits": key_splits,
              "step": f"{w.cp} attention of all {Hh} heads over {R} simulated GPUs"}
    return Setup(kernels, run, 4 * T * T * d * Hh, config, close)


def setup_load(w, tmpdir):
    """Shard-on-read loading: a raw checkpoint of the block's unsharded bf16
    weights (patterned values; loading does not look at them) is written once;
    a step creates every rank's shard from it with tp_block_shard_load (64 MiB
    of pinned staging) and frees it again.  Work = the slice bytes that reach
    the device; the file stays in the host page cache, so this is the
    host -> HBM path, not disk."""
    import numpy as np
    import torch
    import tensor_dit_transformer_amd as tp

    D, Hh, d, F, P = w.hidden, w.num_heads, w.head_dim, w.ffn, w.tp_degree
    HD = Hh * d
    sizes = [("w_q", HD * D), ("w_k", HD * D), ("w_v", HD * D), ("w_o", D * HD),
             ("w_up", F * D), ("w_down", D * F)]
    path = os.path.join(tmpdir, "block_checkpoint.bin")
    files, off = {}, 0
    pattern = (np.arange(8 << 20, dtype=np.uint16) & 0x3f7f).tobytes()
    with open(path, "wb") as f:
        for name, n in sizes:
            files[name] = (path, off)
            left = n * 2
            while left:
                k = min(left, len(pattern))
                f.write(pattern[:k])
                left -= k
            off += n * 2
    total = off
    cfgs = [tp.make_config(P, r, D, Hh, d, F, tp.TP_BF16) for r in range(P)]
    kernels = {"shard_load": ("shard.hip", total // P, "host")}

    def run(mark):
        for cfg in cfgs:
            mark("shard_load", lambda: tp.tp_block_shard_load(cfg, files, 64 << 20).close())

    config = {"workload": w.name, "hidden": D, "num_heads": Hh, "head_dim": d, "ffn": F,
              "tp_degree": P, "ranks_per_step": P, "checkpoint_bytes": total,
              "staging_bytes": 64 << 20,
              "step": "every rank loads its slices of a raw bf16 checkpoint (page cache warm)",
              "context": "the TP page's FLUX.2-dev (32B, bf16) loads in 12.5 s with 6.8 GB peak "
                         "CPU memory per rank at tp_degree 4 on 4x A10G when loading sharded, "
                         "vs 30.4 s / 64.1 GB loading whole then sharding"}
    return Setup(kernels, run, total, config, lambda: torch.cuda.synchronize())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="block_bf16_T16384_D6144_H48_F18432_P4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before warmup, run a plain 512 MiB device-to-device copy twice so a "
                         "counter run can scale FETCH_SIZE / WRITE_SIZE by a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the shard's ranks are "
              "simulated one after another on a single MI355X; there is no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import tp_inputs

    w = tp_inputs.WORKLOADS[args.workload]
    log(f"[bench] generating inputs for {w.name}")
    t0 = time.time()
    import tempfile
    tmp = tempfile.TemporaryDirectory()
    if w.name.startswith("load_"):
        st = setup_load(w, tmp.name)
    else:
        st = setup_cp(w) if w.cp else setup_block(w)
    kernels = st.kernels
    log(f"[bench] setup {time.time() - t0:.1f} s")

    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        src = torch.ones(128 * 1024 * 1024, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(ev=None):
        def mark(name, fn):
            if ev is None:
                fn()
                return
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ev.setdefault(name, []).append((a, b))

        st.run(mark)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    ev = {}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    with ClockSampler() as clock:
        g0.record(stream)
        for _ in range(args.steps):
            step(ev)
        g1.record(stream)
        torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gpu_ms = g0.elapsed_time(g1)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step")

    loading = w.name.startswith("load_")
    # a load step's work is bytes: value in GB/s
    value = st.flops / (ms_per_step * 1e-3) / (1e9 if loading else 1e12)

    per_kernel = {}
    for name, (src, work, bound) in kernels.items():
        times = [a.elapsed_time(b) for a, b in ev[name]]
        avg_ms = sum(times) / len(times)
        per_launch = work
        if bound == "mfma":
            ach = per_launch / (avg_ms * 1e-3) / 1e12
            per_kernel[name] = {"avg_ms": round(avg_ms, 4), "launches_per_step": len(times) // args.steps,
                                "tflops": round(ach, 1), "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                                "step_share": 0.0}
        else:
            ach = per_launch / (avg_ms * 1e-3) / 1e9
            peak = PCIE_PEAK_GBS if bound == "host" else HBM_PEAK_GBS
            per_kernel[name] = {"avg_ms": round(avg_ms, 4), "launches_per_step": len(times) // args.steps,
                                "gbs": round(ach, 1), "frac": round(ach / peak, 4),
                                "step_share": 0.0}
        per_kernel[name]["step_share"] = round(avg_ms * per_kernel[name]["launches_per_step"]
                                               / ms_per_step, 4)
        srt = sorted(times)
        per_kernel[name]["median_ms"] = round(srt[len(srt) // 2] if len(srt) % 2
                                              else 0.5 * (srt[len(srt) // 2 - 1] + srt[len(srt) // 2]), 4)
        per_kernel[name]["min_ms"] = round(srt[0], 4)
    dom = max(per_kernel, key=lambda n: per_kernel[n]["step_share"])
    src, work, bound = kernels[dom]
    k = per_kernel[dom]
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": k["tflops"], "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": k["frac"]}
    elif bound == "host":
        roof = {"bound": "pcie", "achieved": k["gbs"], "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                "frac": k["frac"]}
    else:
        roof = {"bound": "hbm", "achieved": k["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": k["frac"]}
    roof["kernel"] = dom
    roof["traffic"] = load_traffic(dom, src)
    clk = clock.summary()
    if clk and bound == "mfma":
        # the same rate against the peak at the clock the chip held
        clk["frac_at_held_clock"] = round(k["frac"] * 2400.0 / clk["median_mhz"], 4)

    st.close()

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle sample")
        cpu = (cpu_baseline_load(w, os.path.join(tmp.name, "block_checkpoint.bin")) if loading
               else cpu_baseline(w))
        log(f"[bench] oracle: {cpu['sample']}")

    out = {
        "metric": ("shard-on-read load throughput, GB/s of rank slices" if loading else
                   "TFLOP/s per TP-rank DiT block shard (bf16) + % of MI355X MFMA peak"),
        "value": round(value, 2),
        "unit": "GB/s" if loading else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) activations, N(0,0.02) weights, N(0,0.01) biases, bf16 RNE",
        "mfma_peak_frac": None if loading else round(value / MFMA_BF16_PEAK_TFLOPS, 4),
        "config": st.config,
        "roofline": roof,
        "clock": clk,
        "kernels": per_kernel,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

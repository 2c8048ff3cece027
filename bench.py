"""Benchmark: physical-frame state moments, forward + recompute backward, on one GPU.

One step = moments_fwd + moments_bwd over one batch of the workload (every
kernel of the path). Prints one JSON line (rank 0) with the throughput in
tokens/s (tokens = b * valid_len; all heads included), the roofline of the
dominant kernel measured live with HIP events on its stream, and the CPU
oracle's throughput on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3      # MI355X fp32 MFMA / vector
PEAK_HBM_GBS = 8000.0


def algorithmic(w, ell, l=None):
    """Algorithmic flops and HBM bytes per launch of each kernel, counted as the
    method's contractions over the causal triangle at chunk length l (the
    caller's chunk_len by default; per token-head: states c*p*r*(l+1), m2 and d_c
    2*p*r^2 each, d_W and <G, W> p*r*(l+1) each). Bytes count every input read
    once and every output written once; the fp32 carries are the implementation's
    own extra (p*r*4 per kernel chunk of ell tokens, written by the carry pass and
    read back)."""
    V = min(w.valid_len, w.s)
    th = w.b * V * w.h                         # token-heads
    p, r, c = w.p, w.r, w.c
    l = w.chunk_len if l is None else l
    e = 2 if w.dtype == "bf16" else 4
    states = c * p * r * (l + 1)
    gram = 2 * p * r * r
    dw = p * r * (l + 1)
    rw = w.rot_width
    tok_in = (c * p + c * r + 1 + rw) * e          # xhat, bhat, da, rot per token-head
    nk = -(-V // ell)
    carry_b = w.b * w.h * nk * p * r * 4          # one fp32 carry per kernel chunk
    small = w.b * w.h * (2 * p * r + r * r) * 4   # h0 in, m2/m1 out or d_m2/d_m1 in, d_h0 out
    fwd_b = th * tok_in + small
    bwd_b = 2 * th * tok_in + small + w.b * w.h * p * r * e
    return {
        "k_fwd": dict(flops=th * (states + gram), bytes=fwd_b + carry_b),
        "k_bwd": dict(flops=th * (states + gram + 2 * dw), bytes=bwd_b + 2 * carry_b),
        "k_carry": dict(flops=th * 2 * c * p * r, bytes=th * (c * p + c * r + 1) * e + carry_b),
        "k_scan": dict(flops=0, bytes=2 * carry_b),
        # one sequential walk per chain: inputs read once, carries written once
        "k_cscan": dict(flops=th * 2 * c * p * r, bytes=th * (c * p + c * r + 1) * e + carry_b),
        # its group forms: summaries read the inputs (all but each chain's last
        # group, counted whole here) and store almost nothing; the group walks
        # read the inputs and write every carry
        "k_cscan_sum": dict(flops=th * 2 * c * p * r, bytes=th * (c * p + c * r + 1) * e),
        "k_cscan_grp": dict(flops=th * 2 * c * p * r, bytes=th * (c * p + c * r + 1) * e + carry_b),
        "step": dict(flops=th * (2 * states + 2 * gram + 2 * dw), bytes=fwd_b + bwd_b),
    }


def source_digest():
    """Digest of the kernel sources: a stored traffic figure applies only to the
    build it was measured on."""
    import hashlib
    d = hashlib.sha256()
    src = os.path.join(ROOT, "mamba_ssm_chunkwise_amd", "csrc")
    for name in sorted(os.listdir(src)):
        if name.endswith((".h", ".hip")):
            with open(os.path.join(src, name), "rb") as f:
                d.update(name.encode() + b"\0" + f.read())
    return d.hexdigest()[:16]


def stored_traffic(kernel, workload):
    """HBM bytes per launch measured by rocprofv3 (FETCH_SIZE + WRITE_SIZE, scaled
    by a plain copy of known size), from profiles/<kernel>_<workload>.traffic.txt,
    or None when absent or measured on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_digest") != source_digest():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, t, seconds_hint=15.0):
    """The oracle (as it stands) on a bounded sample of the workload's own draw:
    the first k (b,h) chains of the tensors the GPU runs on, whole valid length,
    fwd + bwd in fp64 on all host cores, k a multiple of the thread count chosen
    for about seconds_hint of work; plus one chain on a single thread over a
    prefix of the sequence. Workload tokens/s = (chains * V / h) / time (a token
    of the workload carries h chains)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from oracle import oracle_bwd, oracle_fwd
    from oracle.oracle import default_threads
    from parity_util import sub_chains

    nt = default_threads()
    V = min(w.valid_len, w.s)

    def run(nch, T, threads):
        sub = sub_chains(t, list(range(nch)), w.h)
        a = {k: (None if v is None else v[:, :T].double().cpu().numpy() if k in ("xhat", "bhat", "da", "rot")
                 else v.double().cpu().numpy()) for k, v in sub.items()}
        t0 = time.perf_counter()
        oracle_fwd(a["xhat"], a["bhat"], a["da"], a["rot"], a["h0"], T, w.rot_kind, w.rope_dim,
                   nthreads=threads)
        oracle_bwd(a["xhat"], a["bhat"], a["da"], a["rot"], a["h0"], a["d_m2"], a["d_m1"], T, w.rot_kind,
                   w.rope_dim, nthreads=threads)
        return time.perf_counter() - t0
    T1 = min(V, 512)
    dt1 = run(1, T1, 1)                               # one chain, one thread, a prefix
    single = T1 / w.h / dt1
    per_round = dt1 * V / T1                          # about nt chains of V tokens on nt threads
    k = int(max(1, min(64, round(seconds_hint / max(per_round, 1e-3)))))
    nch = min(nt * k, w.b * w.h)
    dt = run(nch, V, nt)
    rate = nch * V / w.h / dt
    return {"value": rate, "unit": "tokens/s", "cores": nt, "kind": "oracle",
            "single_thread_value": single,
            "sample": f"the first {nch} (b,h) chains of the {w.name} draw, {V} tokens each, fwd+bwd fp64 on "
                      f"{nt} threads in {dt:.1f} s; single thread: 1 chain x {T1} tokens in {dt1:.2f} s; "
                      f"tokens/s = chains*tokens/h/time"}


def producer_leg(w, M, W, dev, reps=10):
    """Times the rotation-sequence producer (moments_rot_fwd) and its VJP
    (moments_rot_bwd) on the workload's increments, outside the timed step.
    Both are HBM-bound streams: the algorithmic bytes are one read of each input
    and one write of the output (2 and 3 tensors of rot's size); the kernels read
    their inputs twice (segment totals, then the walk), which the per-kernel
    figures show."""
    import torch
    if w.rot_kind == W.ROT_NONE:
        return None
    inc, d_rot = W.rotation_increments(w, dev)
    d = M.rot_desc(inc, w.rot_kind)
    rot = torch.empty_like(inc)
    d_inc = torch.empty_like(inc)
    size = inc.numel() * inc.element_size()
    out = {"shape": list(inc.shape), "dtype": w.dtype}
    for name, call, nbytes in (("fwd", lambda: M.moments_rot_fwd(d, inc, rot), 2 * size),
                               ("bwd", lambda: M.moments_rot_bwd(d, inc, d_rot, d_inc), 3 * size)):
        call()
        torch.cuda.synchronize()
        M.profile_reset()
        M.profile_enable(True)
        for _ in range(reps):
            call()
        torch.cuda.synchronize()
        M.profile_enable(False)
        prof = {k: v for k, v in M.profile_read().items() if k.startswith("k_rot") and v[0] > 0}
        ms = sum(tot for _, tot in prof.values()) / reps
        gbs = nbytes / (ms / 1e3) / 1e9
        out[name] = {"ms": round(ms, 4), "algorithmic_bytes": nbytes, "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "kernels_ms": {k: round(tot / max(n, 1), 4) for k, (n, tot) in sorted(prof.items())}}
    M.profile_reset()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="bf16_pairwise_b8_s8192")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--ragged", action="store_true",
                    help="per-sequence valid lengths (seeded, uniform in [V/4, V]); tokens = their sum")
    ap.add_argument("--saved-carry", action="store_true",
                    help="time the saved-carry variant: moments_fwd_save keeps the chunk-boundary states, "
                         "moments_bwd_saved reads them instead of running its carry pass")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed steps, run one plain device copy of 1 GiB (reads 1 GiB, writes "
                         "1 GiB) so a counter run can calibrate HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path shards over (b,h) chains by construction, see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import mamba_ssm_chunkwise_amd as M
    import workloads as W

    w = W.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = W.generate(w, device=dev)
    d = M.Desc(w.b, w.s, w.c, w.h, w.p, w.r, w.chunk_len, w.valid_len,
               M.BF16 if w.dtype == "bf16" else M.F32, w.rot_kind, w.rope_dim, w.quat_blocks)
    lens = None
    if args.ragged:
        gl = torch.Generator().manual_seed(w.seed + 31)
        V = min(w.valid_len, w.s)
        lens = torch.randint(max(V // 4, 1), V + 1, (w.b,), generator=gl, dtype=torch.int32)
        M.set_valid_lens(d, lens.to(dev))
    ws = torch.empty(max(M.moments_workspace_size(d, False), M.moments_workspace_size(d, True)),
                     dtype=torch.uint8, device=dev)
    m2 = torch.empty(w.b, w.h, w.r, w.r, dtype=torch.float32, device=dev)
    m1 = torch.empty(w.b, w.h, w.p, w.r, dtype=torch.float32, device=dev)
    grads = M.moments_bwd(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"], t["d_m2"], t["d_m1"],
                          workspace=ws)

    saved = (torch.empty(max(M.moments_saved_size(d), 1), dtype=torch.uint8, device=dev)
             if args.saved_carry else None)

    def step():
        if saved is None:
            M.moments_fwd(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"], m2=m2, m1=m1, workspace=ws)
            M.moments_bwd(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"], t["d_m2"], t["d_m1"],
                          out=grads, workspace=ws)
        else:
            M.moments_fwd_save(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"], m2=m2, m1=m1, saved=saved,
                               workspace=ws)
            M.moments_bwd_saved(d, t["xhat"], t["bhat"], t["da"], t["rot"], t["h0"], saved, t["d_m2"],
                                t["d_m1"], out=grads, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    M.profile_reset()
    M.profile_enable(True)
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    M.profile_enable(False)
    ms = e0.elapsed_time(e1) / args.steps
    prof = M.profile_read()
    V = min(w.valid_len, w.s)
    tokens = w.b * V if lens is None else int(lens.clamp(0, V).sum())
    value = tokens / (ms / 1e3)

    ell = M.kernel_chunk_len()
    alg = algorithmic(w, ell)
    alg_k = algorithmic(w, ell, l=ell)          # the same contractions at the kernels' chunk length
    # per-kernel names as the library reports them (the transposed bf16 kernels
    # report under the same names as the general ones)
    per_kernel = {k: (n, tot / max(n, 1)) for k, (n, tot) in prof.items() if n > 0}
    dom = max(per_kernel, key=lambda k: per_kernel[k][0] * per_kernel[k][1])
    avg_ms = per_kernel[dom][1]
    a = alg.get(dom, {"flops": 0, "bytes": 0})
    # the profiled kernel behind the library's name: the bf16 forward is the
    # lane-pair kernel, the bf16 backward the transposed one (c = 4 walks token pairs)
    kname = {"k_bwd": "k_bwdt", "k_fwd": "k_fwd4"}.get(dom, dom) if w.dtype == "bf16" and w.c != 3 else dom
    traffic = stored_traffic(kname, w.name)
    if a["flops"] > 0:
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        achieved = a["flops"] / (avg_ms / 1e3) / 1e12
        ak = alg_k[dom]["flops"] / (avg_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic, "kernel": kname,
                "avg_ms": round(avg_ms, 4),
                "count": f"method contractions over the causal triangle at the caller's chunk length l={w.chunk_len}",
                "at_kernel_chunk": {"l": ell, "flops": alg_k[dom]["flops"], "achieved": round(ak, 2),
                                    "frac": round(ak / peak, 4)}}
    else:
        achieved = a["bytes"] / (avg_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic, "kernel": kname,
                "avg_ms": round(avg_ms, 4)}
    # whole fwd+bwd step against its roofline time max(flops / MFMA peak, bytes / HBM peak)
    st = alg["step"]
    pk = (PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS) * 1e12
    t_roof = max(st["flops"] / pk, st["bytes"] / (PEAK_HBM_GBS * 1e9))
    stk = alg_k["step"]
    t_roof_k = max(stk["flops"] / pk, stk["bytes"] / (PEAK_HBM_GBS * 1e9))
    step_roof = {"flops": st["flops"], "bytes": st["bytes"], "roofline_ms": round(t_roof * 1e3, 3),
                 "frac": round(t_roof * 1e3 / ms, 4),
                 "at_kernel_chunk": {"l": ell, "flops": stk["flops"], "roofline_ms": round(t_roof_k * 1e3, 3),
                                     "frac": round(t_roof_k * 1e3 / ms, 4)}}
    for k, (n, avg) in sorted(per_kernel.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
        fl = alg.get(k, {}).get("flops", 0)
        by = alg.get(k, {}).get("bytes", 0)
        print(f"[bench] {k:12s} launches {n:4d} avg {avg:9.4f} ms  "
              f"{fl / (avg / 1e3) / 1e12 if fl else 0:8.1f} TFLOP/s  {by / (avg / 1e3) / 1e9:8.1f} GB/s",
              file=sys.stderr, flush=True)

    if args.copy_probe:
        src_t = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst_t = torch.empty_like(src_t)
        torch.cuda.synchronize()
        torch.add(src_t, 0.0, out=dst_t)   # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src_t, dst_t

    producer = producer_leg(w, M, W, dev)

    cpu = None
    if not args.no_cpu:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, t)

    out = {
        "metric": "moments fwd+bwd tokens/sec on 1 MI355X; % MFMA/HBM roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "b": w.b, "s": w.s, "valid_len": w.valid_len, "c": w.c, "h": w.h,
                   "p": w.p, "r": w.r, "chunk_len": w.chunk_len, "rot_kind": w.rot_kind,
                   "rope_dim": w.rope_dim, "quat_blocks": w.quat_blocks, "parallelism": "none",
                   "saved_carry": bool(args.saved_carry),
                   "valid_lens": None if lens is None else [int(x) for x in lens]},
        "roofline": roof,
        "step_roofline": step_roof,
        "cpu_baseline": cpu,
        "producer": producer,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

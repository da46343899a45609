"""Benchmark of the KDA mixer on one MI355X.

One step runs every entry point of the hot path once, each on its workload,
with all inputs already resident in HBM:
  prefill    : 1 sequence x 4096 tokens, 64 heads of 128, bf16, zero initial
               state, final fp32 state written, two-pass schedule with a
               caller-provided workspace (kda_prefill: intra_kernel + scan_kernel)
  decode     : 256 sequences x 1 token, 64 heads, fp32 state 256x64x128x128
               updated in place, bf16 tokens                  (kda_decode)
  short_conv : the same 4096-token q|k|v rows as a [4096, 24576] bf16 tensor,
               conv width 4                                   (kda_short_conv)
and, reported beside the step, the same decode with the state stored as bf16
(KDA_F_STATE_BF16), and one speculative decode step (verification of k = 5
drafted tokens plus one):
  spec_decode: 256 sequences x 6 tokens, 64 heads, fp32 state; each call first
               commits the previous call's accepted prefix (1 + Binomial(5, 0.8)
               tokens per sequence), then verifies 6 new tokens
                                         (kda_decode_multi with pending records)
  spec_commit: the same commit on its own, as at the end of a speculative
               run                                          (kda_decode_commit)
  gate_proj  : the gate and beta in-projections of the prefill's tokens
               (hidden 4096, rank 128, log-decay epilogue)  (kda_gate_beta_proj)
  state_copy : 128 rows of the decode pool (state + conv state) copied to
               128 others, as prefix snapshots             (kda_state_copy)
Every call is bracketed by HIP events on the stream it is launched on, after a
512 MiB scratch write that evicts L2 and the MALL (not timed); `value` is
prefill tokens per second per layer from the median prefill call time, decode
reports the state bandwidth (read + write of the fp32 state).

Prints ONE JSON line.  --gpus N > 1 is refused: the mixer runs on one GPU here.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix, published
METRIC = "KDA prefill tokens/s/layer (H=64,d=128) + decode state GB/s, 1 MI355X"


def _source_sha(name):
    path = os.path.join(ROOT, "gated_delta_rule_short_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def _traffic_from_profile(kernel_src, fname):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None when
    the summary is absent or was taken on a different version of the kernel source."""
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != _source_sha(kernel_src):
        return None
    return float(m_b.group(1))


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["all", "prefill", "decode", "decode_bf16_state", "short_conv",
                                       "spec_decode", "spec_commit", "gate_proj", "state_copy",
                                       "copy"],
                    default="all", help="run one entry point only (for profiler passes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: the KDA mixer is built and measured on one GPU; --gpus %d is not "
              "supported (the path would shard over heads, sequences or dv columns; only the "
              "one-GPU path is built)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import kda_inputs as KI
    import gated_delta_rule_short_amd as kda

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kda.load_library()
    stream = torch.cuda.current_stream(dev)

    # ---------------- inputs (resident in HBM before the timed region)
    P = KI.workload_inputs(1, device=dev)
    T, H = P["q"].shape[0], P["q"].shape[1]
    o = torch.empty_like(P["v"])
    st_out = torch.empty((1, H, 128, 128), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.prefill_workspace_bytes(T, H, 1), dtype=torch.uint8, device=dev)
    Dd = KI.workload_inputs(2, device=dev)
    N_dec = Dd["q"].shape[0]
    o_dec = torch.empty_like(Dd["v"])
    st16 = Dd["state"].to(torch.bfloat16)  # the same workload with 16-bit state storage
    cs16 = Dd["conv_state"].clone()
    o_dec16 = torch.empty_like(Dd["v"])
    X = torch.cat([P["q"].reshape(T, -1), P["k"].reshape(T, -1), P["v"].reshape(T, -1)], 1).contiguous()
    Y = torch.empty_like(X)
    cu1 = P["cu_seqlens"]
    Sp = KI.workload_inputs(5, device=dev)
    N_sp, T_sp = Sp["q"].shape[0], Sp["q"].shape[1]
    acc_sp = KI.make_accepted(N_sp, T_sp, seed=5, device=dev)
    rec_sp = [torch.empty((N_sp, H, T_sp, kda.UPDATE_FLOATS), dtype=torch.float32, device=dev)
              for _ in range(2)]
    o_sp = torch.empty_like(Sp["v"])
    sp_turn = [0]
    Gp = KI.make_gate_proj(T, H=H, device=dev)  # the prefill's 4096 tokens, hidden 4096
    g_out = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    b_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    g_ws = torch.empty(kda.gate_beta_workspace_bytes(T, H), dtype=torch.uint8, device=dev)
    # prefix snapshots: 128 pool rows of the decode workload's pool copied to 128 others
    n_cp = N_dec // 2
    cp_src = torch.arange(0, n_cp, dtype=torch.int32, device=dev)
    cp_dst = cp_src + n_cp
    copy_src = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev)
    copy_dst = torch.empty_like(copy_src)
    scratch = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev)

    def run_prefill():
        kda.kda_prefill(P["q"], P["k"], P["v"], P["gate"], P["beta"], P["conv_w"], cu_seqlens=cu1,
                        state_out=st_out, o=o, workspace=ws)

    def run_decode():
        kda.kda_decode(Dd["q"], Dd["k"], Dd["v"], Dd["gate"], Dd["beta"], Dd["conv_w"],
                       Dd["conv_state"], Dd["state"], o=o_dec)

    def run_spec():
        # records alternate between two buffers: this call commits the other one
        i = sp_turn[0]
        sp_turn[0] ^= 1
        kda.kda_decode_multi(Sp["q"], Sp["k"], Sp["v"], Sp["gate"], Sp["beta"], Sp["conv_w"],
                             Sp["conv_state"], Sp["state"], updates=rec_sp[i], o=o_sp,
                             pending_updates=rec_sp[i ^ 1], pending_accepted=acc_sp)

    def run_commit():
        kda.kda_decode_commit(rec_sp[0], acc_sp, Sp["conv_state"], Sp["state"])

    # the first verification has nothing to commit: it primes the pending records
    kda.kda_decode_multi(Sp["q"], Sp["k"], Sp["v"], Sp["gate"], Sp["beta"], Sp["conv_w"],
                         Sp["conv_state"], Sp["state"], updates=rec_sp[1], o=o_sp)

    def run_decode16():
        kda.kda_decode(Dd["q"], Dd["k"], Dd["v"], Dd["gate"], Dd["beta"], Dd["conv_w"], cs16, st16,
                       o=o_dec16)

    def run_gate_proj():
        kda.kda_gate_beta_proj(Gp["x"], Gp["w_a"], Gp["w_b"], Gp["w_beta"], gate=g_out, beta=b_out,
                               workspace=g_ws, log=True)

    def run_state_copy():
        kda.kda_state_copy(Dd["state"], cp_src, cp_dst, conv_pool=Dd["conv_state"])

    def run_conv():
        kda.kda_short_conv(X, P["conv_w"], cu_seqlens=cu1, y=Y)

    def run_copy():
        copy_dst.copy_(copy_src)

    ops = {"prefill": run_prefill, "decode": run_decode, "short_conv": run_conv,
           "decode_bf16_state": run_decode16, "spec_decode": run_spec, "spec_commit": run_commit,
           "gate_proj": run_gate_proj, "state_copy": run_state_copy, "copy": run_copy}
    step_names = ["short_conv", "prefill", "decode"]
    if args.only == "all":
        names = step_names + ["decode_bf16_state", "spec_decode", "spec_commit", "gate_proj",
                              "state_copy"]
    else:
        names = [args.only]

    for _ in range(args.warmup):
        for nm in names:
            ops[nm]()
    torch.cuda.synchronize()

    ev = {nm: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)] for nm in names}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for nm in names:
            a, b = ev[nm][s]
            if nm != "copy":
                scratch.fill_(s & 0xff)  # evict L2 and MALL before the timed call
            a.record(stream)
            ops[nm]()
            b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = {nm: sorted(a.elapsed_time(b) for a, b in ev[nm]) for nm in names}
    ms = {nm: times[nm][len(times[nm]) // 2] for nm in names}  # median
    ms_mean = {nm: sum(times[nm]) / len(times[nm]) for nm in names}
    ms_per_step = wall * 1e3 / args.steps

    if args.only != "all":
        print(json.dumps({"only": args.only, "ms_per_launch": ms[args.only],
                          "ms_mean": ms_mean[args.only], "steps": args.steps}), flush=True)
        return

    # ---------------- derived figures
    units = T * H                                   # token-heads per prefill launch
    pre_bytes = units * KI.bytes_per_token_head() + H * 128 * 128 * 4   # + final state
    pre_s = ms["prefill"] * 1e-3
    pre_flops = units * KI.prefill_flops_per_token_head()
    tok_per_s = T / pre_s                           # one layer = all 64 heads
    dec_state_bytes = 2 * N_dec * H * 128 * 128 * 4  # fp32 state read + written
    dec_other = N_dec * H * (KI.bytes_per_token_head() + 2 * 3 * 128 * 2)  # tokens + conv cache
    dec_s = ms["decode"] * 1e-3
    conv_bytes = 2 * X.numel() * X.element_size()
    # speculative step, per (sequence, head): state read and written back, the
    # pending records' alpha, k, u rows and the raw rows of the last <= 3 accepted
    # tokens, conv cache read and written, the 6 new tokens (q, k, v, gate, beta),
    # their outputs and their records
    acc_l = acc_sp.cpu().tolist()
    sp_bytes = 0
    for a_ in acc_l:
        a_ = max(0, min(T_sp, a_))
        per = 65536 + (65536 if a_ else 0) + a_ * 3 * 512 + min(a_, 3) * 3 * 512
        per += 3 * 384 * 2 * (2 if a_ else 1)
        per += T_sp * (4 * 128 * 2 + 2) + T_sp * 128 * 2 + T_sp * 6 * 512
        sp_bytes += per * H
    sp_s = ms["spec_decode"] * 1e-3
    sp_state_bytes = 2 * N_sp * H * 128 * 128 * 4
    # gate projections: x [T][4096] and the three weights in, gate [T][H*128] and beta out
    cp_bytes = 2 * n_cp * H * (128 * 128 * 4 + 9 * 128 * 2)  # state and conv rows, read + written
    hid_gp = Gp["x"].shape[1]
    gp_flops = 2 * T * hid_gp * (128 + H) + 2 * T * 128 * H * 128
    gp_bytes = 2 * (T * hid_gp + (128 + H) * hid_gp + H * 128 * 128 + T * H * 128 + T * H)
    traffic = _traffic_from_profile("kda_prefill_split.hip", "prefill_bf16_T4096_H64_pmc.md")
    dec_traffic = _traffic_from_profile("kda_decode.hip", "decode_bf16_N256_H64_pmc.md")

    result = {
        "metric": METRIC,
        "value": round(tok_per_s, 1),
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sum(ms[nm] for nm in step_names), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, distributions of the published workloads)",
        "config": {"workload": "prefill B=1 T=4096 H=64 d=128 bf16 (two-pass, 16-token "
                               "sub-chunks); decode N=256 H=64 fp32 state; short_conv T=4096 "
                               "C=24576", "global_batch": 1, "seq_len": T, "heads": H,
                   "head_dim": 128, "parallelism": "none (1 GPU)"},
        "wall_ms_per_step": round(ms_per_step, 4),
        "decode_state_GBps": round(dec_state_bytes / dec_s / 1e9, 1),
        "per_call_us": {nm: round(ms[nm] * 1e3, 2) for nm in names},
        "per_call_us_mean": {nm: round(ms_mean[nm] * 1e3, 2) for nm in names},
        "roofline": {
            "bound": "hbm",
            "achieved": round(pre_bytes / pre_s / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(pre_bytes / pre_s / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "kda_prefill = intra_kernel + scan_kernel<2> (one call, both launches)",
            "algorithmic_bytes_per_launch": pre_bytes,
            "mfma_util": round(pre_flops / pre_s / 1e12 / BF16_PEAK_TFLOPS, 4),
        },
        "roofline_decode": {
            "bound": "hbm",
            "achieved": round((dec_state_bytes + dec_other) / dec_s / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round((dec_state_bytes + dec_other) / dec_s / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": dec_traffic,
            "algorithmic_bytes_per_launch": dec_state_bytes + dec_other,
        },
        "short_conv_GBps": round(conv_bytes / (ms["short_conv"] * 1e-3) / 1e9, 1),
        "gate_proj": {
            "workload": "gate and beta in-projections of the prefill's 4096 tokens: hidden 4096, "
                        "rank 128, 64 heads x 128 gate channels, bf16, log-decay epilogue",
            "us_per_call": round(ms["gate_proj"] * 1e3, 2),
            "TFLOPs": round(gp_flops / (ms["gate_proj"] * 1e-3) / 1e12, 1),
            "GBps": round(gp_bytes / (ms["gate_proj"] * 1e-3) / 1e9, 1),
            "flops_per_call": gp_flops,
            "algorithmic_bytes_per_call": gp_bytes,
        },
        "state_copy": {
            "workload": "%d pool rows (fp32 state, 64 heads, and conv state) copied to %d other "
                        "rows of the decode workload's pool" % (n_cp, n_cp),
            "us_per_call": round(ms["state_copy"] * 1e3, 2),
            "GBps": round(cp_bytes / (ms["state_copy"] * 1e-3) / 1e9, 1),
            "roofline": {"bound": "hbm", "achieved": round(cp_bytes / (ms["state_copy"] * 1e-3) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(cp_bytes / (ms["state_copy"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": cp_bytes},
        },
        "decode_bf16_state": {
            "workload": "workload 2 with the state stored as bf16 (256 x 64 x 128 x 128, 512 MiB)",
            "us_per_call": round(ms["decode_bf16_state"] * 1e3, 2),
            "state_GBps": round(dec_state_bytes / 2 / (ms["decode_bf16_state"] * 1e-3) / 1e9, 1),
            "roofline": {
                "bound": "hbm",
                "achieved": round((dec_state_bytes / 2 + dec_other) / (ms["decode_bf16_state"] * 1e-3) / 1e9, 1),
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s",
                "frac": round((dec_state_bytes / 2 + dec_other) / (ms["decode_bf16_state"] * 1e-3) / 1e9
                              / HBM_PEAK_GBS, 4),
                "algorithmic_bytes_per_launch": dec_state_bytes // 2 + dec_other,
            },
        },
        "spec_decode": {
            "workload": "256 sequences x 6 tokens (k=5 drafts + 1), H=64, bf16 tokens, fp32 "
                        "state; fused commit of the previous step's accepted prefix",
            "us_per_call": round(ms["spec_decode"] * 1e3, 2),
            "commit_us_per_call": round(ms["spec_commit"] * 1e3, 2),
            "verified_tokens_per_s": round(N_sp * T_sp / sp_s, 1),
            "accepted_tokens_per_s": round(sum(max(0, min(T_sp, a_)) for a_ in acc_l) / sp_s, 1),
            "mean_accepted": round(sum(acc_l) / len(acc_l), 3),
            "state_GBps": round(sp_state_bytes / sp_s / 1e9, 1),
            "roofline": {
                "bound": "hbm",
                "achieved": round(sp_bytes / sp_s / 1e9, 1),
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s",
                "frac": round(sp_bytes / sp_s / 1e9 / HBM_PEAK_GBS, 4),
                "traffic": _traffic_from_profile("kda_decode.hip",
                                                 "spec_decode_bf16_N256_T6_H64_pmc.md"),
                "algorithmic_bytes_per_launch": sp_bytes,
            },
        },
    }

    if not args.no_cpu_baseline:
        import oracle  # the CPU baseline leg: the fp64 oracle as it stands
        threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
        host = {k_: (v_.cpu() if torch.is_tensor(v_) else v_) for k_, v_ in P.items()}
        runs = []
        t_all = time.perf_counter()
        while len(runs) < 3 or (time.perf_counter() - t_all < 5.0 and len(runs) < 50):
            t0 = time.perf_counter()
            oracle.prefill(host["q"], host["k"], host["v"], host["gate"], host["beta"],
                           host["conv_w"], host["cu_seqlens"], nthreads=threads)
            runs.append(time.perf_counter() - t0)
        cpu_s = sorted(runs)[len(runs) // 2]
        result["cpu_baseline"] = {
            "value": round(T / cpu_s, 1), "unit": "tokens/s/layer",
            "cores": min(threads, H), "kind": "oracle",
            "sample": "the full prefill workload (1 x 4096 tokens x 64 heads), fp64 token-by-token "
                      "oracle, OpenMP over heads; median of %d runs, %.3f s each" % (len(runs), cpu_s),
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

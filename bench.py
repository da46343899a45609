"""Benchmark of the KDA mixer on one MI355X.

One step runs every row of the hot path once, each on its workload, with all
inputs already resident in HBM:
  prefill    : 16 packed sequences of 512..16,384 tokens (137,314 in all), 64
               heads of 128, bf16, fp32 initial and final states, the automatic
               schedule (1024 (sequence, head) pairs, above the 384 from which the
               automatic choice is the fused schedule:
               kda_prefill -> fused_kernel, one workgroup per pair)
  decode     : 256 sequences x 1 token, 64 heads, fp32 state 256x64x128x128
               updated in place, bf16 tokens                  (kda_decode)
  short_conv : the prefill's q|k|v rows as one [137,314, 24,576] bf16 tensor,
               conv width 4                                   (kda_short_conv)
`value` is the prefill's tokens per second per layer (all 64 heads).  Reported
beside the step, each with its own roofline: the prefill of 1 x 4096 tokens and
of 1 x 65,536 tokens with decays near the bound; the same decode with bf16
state storage; a speculative decode step (k = 5 drafts + 1, fused commit of the
previous accepted prefix) and the commit alone; the gate and beta
in-projections; pool-row copies; and the HBM ceiling measured with the
calibration kernels (decode's state stream without its arithmetic, a copy).
Every call is bracketed by HIP events on the stream it is launched on, after a
512 MiB scratch write that evicts L2 and the MALL (not timed); figures use the
median call time.

Prints ONE JSON line.  --gpus N > 1 is refused: the mixer runs on one GPU here.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix, published
METRIC = "KDA prefill tokens/s/layer (H=64,d=128) + decode state GB/s, 1 MI355X"
PREFILL = {4: "prefill_varlen", 1: "prefill_T4096", 3: "prefill_T65536"}
PROFILE_OF = {  # committed rocprofv3 counter summaries holding HBM bytes per launch
    "prefill_varlen": ("kda_prefill_split.hip", "prefill_varlen_N16_H64.md"),
    "prefill_T4096": ("kda_prefill_split.hip", "prefill_T4096_H64.md"),
    "prefill_T65536": ("kda_prefill_split.hip", "prefill_T65536_H64.md"),
    "decode": ("kda_decode.hip", "decode_N256_H64.md"),
    "decode_bf16_state": ("kda_decode.hip", "decode_bf16_state_N256_H64.md"),
    "spec_decode": ("kda_decode.hip", "spec_decode_N256_T6_H64.md"),
    "short_conv": ("kda_conv.hip", "short_conv_T137314_C24576.md"),
    "state_copy": ("kda_pool.hip", "state_copy_128rows_H64.md"),
    "gate_proj": ("kda_gate_proj.hip", "gate_proj_T4096_hid4096_H64.md"),
}
OPS = ["prefill_varlen", "prefill_T4096", "prefill_T65536", "decode", "short_conv",
       "decode_bf16_state", "spec_decode", "spec_commit", "gate_proj", "state_copy",
       "calib_state_rmw", "calib_copy", "calib_fill"]


def _source_sha(name):
    """Hash of a kernel source's code: comments removed and whitespace runs folded,
    so that an edit of a comment leaves the summaries of its kernels in force."""
    path = os.path.join(ROOT, "gated_delta_rule_short_amd", "csrc", name)
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def _profile_field(key, field):
    """A number from a committed rocprofv3 summary, or None when the summary is
    absent or was taken on different code (comments and layout aside)."""
    src, fname = PROFILE_OF[key]
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    m = re.search(r"%s:\s*([0-9.eE+-]+)" % re.escape(field), text)
    if not m_sha or not m or m_sha.group(1) != _source_sha(src):
        return None
    return float(m.group(1))


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["all"] + OPS, default="all",
                    help="time one entry point only (for profiler passes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def roofline(bytes_, seconds, traffic=None, **extra):
    achieved = bytes_ / seconds / 1e9
    r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
         "algorithmic_bytes_per_launch": int(bytes_)}
    if traffic is not None:
        # counted bytes over the measured time: a rate above the peak means the
        # summary does not describe this run, so it is not reported as traffic
        rate = traffic / seconds / 1e9
        r["traffic_GBps"] = round(rate, 1)
        if rate > HBM_PEAK_GBS:
            r["traffic"] = None
            r["traffic_note"] = "counted bytes / time exceed the HBM peak: summary not used"
    r.update(extra)
    return r


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
    want = set(OPS) if args.only == "all" else {args.only}

    # ---------------- inputs (resident in HBM before the timed region)
    pre = {}
    for idx, key in PREFILL.items():
        if key not in want and not (key == "prefill_varlen" and "short_conv" in want):
            continue
        P = KI.workload_inputs(idx, device=dev)
        T, H = P["q"].shape[0], P["q"].shape[1]
        N = len(P["lengths"])
        P["o"] = torch.empty_like(P["v"])
        P["st_out"] = torch.empty((N, H, 128, 128), dtype=torch.float32, device=dev)
        P["cu_host"] = P["cu_seqlens"].cpu()
        ws_bytes = kda.prefill_workspace_bytes(T, H, N)
        P["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        P["T"], P["H"], P["N"], P["idx"] = T, H, N, idx
        pre[key] = P

    def prefill_op(P):
        def run():
            kda.kda_prefill(P["q"], P["k"], P["v"], P["gate"], P["beta"], P["conv_w"],
                            cu_seqlens=P["cu_seqlens"], cu_seqlens_host=P["cu_host"],
                            state_in=P["state_in"], state_out=P["st_out"], o=P["o"],
                            workspace=P["ws"])
        return run

    ops = {key: prefill_op(P) for key, P in pre.items()}
    H = 64
    if want & {"decode", "decode_bf16_state", "state_copy"}:
        Dd = KI.workload_inputs(2, device=dev)
        N_dec = Dd["q"].shape[0]
        o_dec = torch.empty_like(Dd["v"])
        ops["decode"] = lambda: kda.kda_decode(Dd["q"], Dd["k"], Dd["v"], Dd["gate"], Dd["beta"],
                                               Dd["conv_w"], Dd["conv_state"], Dd["state"], o=o_dec)
        if "decode_bf16_state" in want:
            st16 = Dd["state"].to(torch.bfloat16)  # the same workload with 16-bit state storage
            cs16 = Dd["conv_state"].clone()
            o_dec16 = torch.empty_like(Dd["v"])
            ops["decode_bf16_state"] = lambda: kda.kda_decode(
                Dd["q"], Dd["k"], Dd["v"], Dd["gate"], Dd["beta"], Dd["conv_w"], cs16, st16,
                o=o_dec16)
        # prefix snapshots: 128 pool rows of the decode workload's pool copied to 128 others
        n_cp = N_dec // 2
        cp_src = torch.arange(0, n_cp, dtype=torch.int32, device=dev)
        cp_dst = cp_src + n_cp
        ops["state_copy"] = lambda: kda.kda_state_copy(Dd["state"], cp_src, cp_dst,
                                                       conv_pool=Dd["conv_state"])
    if "short_conv" in want:
        Pv = pre["prefill_varlen"]
        Tv = Pv["T"]
        X = torch.cat([Pv["q"].reshape(Tv, -1), Pv["k"].reshape(Tv, -1), Pv["v"].reshape(Tv, -1)],
                      1).contiguous()
        Y = torch.empty_like(X)
        ops["short_conv"] = lambda: kda.kda_short_conv(X, Pv["conv_w"], cu_seqlens=Pv["cu_seqlens"],
                                                       cu_seqlens_host=Pv["cu_host"], y=Y)
    if want & {"spec_decode", "spec_commit"}:
        Sp = KI.workload_inputs(5, device=dev)
        N_sp, T_sp = Sp["q"].shape[0], Sp["q"].shape[1]
        acc_sp = KI.make_accepted(N_sp, T_sp, seed=5, device=dev)
        rec_sp = [torch.empty((N_sp, H, T_sp, kda.UPDATE_FLOATS), dtype=torch.float32, device=dev)
                  for _ in range(2)]
        o_sp = torch.empty_like(Sp["v"])
        sp_turn = [0]

        def run_spec():
            # records alternate between two buffers: this call commits the other one
            i = sp_turn[0]
            sp_turn[0] ^= 1
            kda.kda_decode_multi(Sp["q"], Sp["k"], Sp["v"], Sp["gate"], Sp["beta"], Sp["conv_w"],
                                 Sp["conv_state"], Sp["state"], updates=rec_sp[i], o=o_sp,
                                 pending_updates=rec_sp[i ^ 1], pending_accepted=acc_sp)

        # the first verification has nothing to commit: it primes the pending records
        kda.kda_decode_multi(Sp["q"], Sp["k"], Sp["v"], Sp["gate"], Sp["beta"], Sp["conv_w"],
                             Sp["conv_state"], Sp["state"], updates=rec_sp[1], o=o_sp)
        ops["spec_decode"] = run_spec
        ops["spec_commit"] = lambda: kda.kda_decode_commit(rec_sp[0], acc_sp, Sp["conv_state"],
                                                           Sp["state"])
    if "gate_proj" in want:
        Tg = 4096
        Gp = KI.make_gate_proj(Tg, H=H, device=dev)  # 4096 tokens, hidden 4096
        g_out = torch.empty((Tg, H, 128), dtype=torch.bfloat16, device=dev)
        b_out = torch.empty((Tg, H), dtype=torch.bfloat16, device=dev)
        g_ws = torch.empty(kda.gate_beta_workspace_bytes(Tg, H), dtype=torch.uint8, device=dev)
        ops["gate_proj"] = lambda: kda.kda_gate_beta_proj(Gp["x"], Gp["w_a"], Gp["w_b"],
                                                          Gp["w_beta"], gate=g_out, beta=b_out,
                                                          workspace=g_ws, log=True)
    GiB = 2 ** 30
    if want & {"calib_state_rmw", "calib_copy", "calib_fill"}:
        kda.load_calib_library()
        c_state = torch.zeros((GiB // (128 * 128 * 4), 128, 128), dtype=torch.float32, device=dev)
        c_src = torch.zeros(GiB // 4, dtype=torch.float32, device=dev)
        c_dst = torch.empty_like(c_src)
        ops["calib_state_rmw"] = lambda: kda.calib_state_rmw(c_state, 1.0)
        ops["calib_copy"] = lambda: kda.calib_copy(c_dst, c_src)
        ops["calib_fill"] = lambda: kda.calib_fill(c_dst, 1.0)
    scratch = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev)

    step_names = ["prefill_varlen", "decode", "short_conv"]
    names = [nm for nm in OPS if nm in want]

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
            scratch.fill_(s & 0xff)  # evict L2 and MALL before the timed call
            a.record(stream)
            ops[nm]()
            b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = {nm: sorted(a.elapsed_time(b) for a, b in ev[nm]) for nm in names}
    ms = {nm: times[nm][len(times[nm]) // 2] for nm in names}  # median
    ms_mean = {nm: sum(times[nm]) / len(times[nm]) for nm in names}

    if args.only != "all":
        print(json.dumps({"only": args.only, "ms_per_launch": ms[args.only],
                          "ms_mean": ms_mean[args.only], "steps": args.steps}), flush=True)
        return

    # ---------------- derived figures
    bpth = KI.bytes_per_token_head()
    fpth = KI.prefill_flops_per_token_head()
    prefill_out = {}
    for key, P in pre.items():
        units = P["T"] * P["H"]
        st_bytes = P["N"] * P["H"] * 128 * 128 * 4
        byts = units * bpth + st_bytes * (2 if P["state_in"] is not None else 1)
        sec = ms[key] * 1e-3
        prefill_out[key] = {
            "workload": KI.WORKLOADS[P["idx"]].name,
            "tokens": P["T"], "sequences": P["N"],
            "tokens_per_s_per_layer": round(P["T"] / sec, 1),
            "us_per_call": round(ms[key] * 1e3, 2),
            "roofline": roofline(byts, sec, _profile_field(key, "hbm_bytes_per_launch"),
                                 kernel=("kda_prefill, fused schedule (fused_kernel)"
                                         if P["N"] * P["H"] >= kda.FUSED_MIN_PAIRS else
                                         "kda_prefill, two-pass schedule (intra_kernel, then scan_kernel "
                                         "or scan_wide_kernel, per workspace window)"),
                                 mfma_algorithmic_frac=round(units * fpth / sec / 1e12 /
                                                             BF16_PEAK_TFLOPS, 4),
                                 mfma_busy_frac=_profile_field(key, "mfma_busy_frac"),
                                 valu_busy_frac=_profile_field(key, "valu_busy_frac")),
        }
    Pv = pre["prefill_varlen"]
    dec_state_bytes = 2 * N_dec * H * 128 * 128 * 4
    dec_other = N_dec * H * (bpth + 2 * 3 * 3 * 128 * 2)  # tokens + q|k|v conv cache read and written
    dec_s = ms["decode"] * 1e-3
    conv_bytes = 2 * X.numel() * X.element_size()
    acc_l = acc_sp.cpu().tolist()
    sp_bytes = 0
    for a_ in acc_l:
        # per (sequence, head): state read and written back, the pending records'
        # alpha, k, u rows and the raw rows of the last <= 3 accepted tokens, conv
        # cache read and written, the 6 new tokens, their outputs and their records
        a_ = max(0, min(T_sp, a_))
        per = 65536 + (65536 if a_ else 0) + a_ * 3 * 512 + min(a_, 3) * 3 * 512
        per += 3 * 384 * 2 * (2 if a_ else 1)
        per += T_sp * (4 * 128 * 2 + 2) + T_sp * 128 * 2 + T_sp * 6 * 512
        sp_bytes += per * H
    sp_s = ms["spec_decode"] * 1e-3
    cp_bytes = 2 * n_cp * H * (128 * 128 * 4 + 9 * 128 * 2)
    hid_gp = Gp["x"].shape[1]
    gp_flops = 2 * Tg * hid_gp * (128 + H) + 2 * Tg * 128 * H * 128
    gp_bytes = 2 * (Tg * hid_gp + (128 + H) * hid_gp + H * 128 * 128 + Tg * H * 128 + Tg * H)
    ceil_rmw = 2 * GiB / (ms["calib_state_rmw"] * 1e-3) / 1e9
    ceil_copy = 2 * GiB / (ms["calib_copy"] * 1e-3) / 1e9
    ceil_fill = GiB / (ms["calib_fill"] * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": prefill_out["prefill_varlen"]["tokens_per_s_per_layer"],
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
        "config": {"workload": "prefill of 16 packed sequences, lengths U{512..16384} "
                               "(137,314 tokens), H=64, d=128, bf16, fp32 states in and out; "
                               "decode N=256 H=64 fp32 state; short_conv over the prefill's "
                               "q|k|v rows", "global_batch": Pv["N"], "seq_len": Pv["T"],
                   "heads": H, "head_dim": 128, "parallelism": "none (1 GPU)"},
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "roofline": prefill_out["prefill_varlen"]["roofline"],
        "prefill": prefill_out,
        "decode_state_GBps": round(dec_state_bytes / dec_s / 1e9, 1),
        "roofline_decode": roofline(dec_state_bytes + dec_other, dec_s,
                                    _profile_field("decode", "hbm_bytes_per_launch"),
                                    frac_of_measured_ceiling=round(
                                        (dec_state_bytes + dec_other) / dec_s / 1e9 / ceil_rmw, 4)),
        "hbm_ceiling_GBps": {
            "state_rmw_1GiB": round(ceil_rmw, 1), "copy_1GiB": round(ceil_copy, 1),
            "fill_1GiB": round(ceil_fill, 1),
            "note": "calibration kernels of libkda_calib.so: decode's state stream (read and "
                    "write in place, same mapping, no arithmetic), a streaming copy, a fill"},
        "per_call_us": {nm: round(ms[nm] * 1e3, 2) for nm in names},
        "per_call_us_mean": {nm: round(ms_mean[nm] * 1e3, 2) for nm in names},
        "short_conv": {"us_per_call": round(ms["short_conv"] * 1e3, 2),
                       "roofline": roofline(conv_bytes, ms["short_conv"] * 1e-3,
                                            _profile_field("short_conv", "hbm_bytes_per_launch"))},
        "gate_proj": {
            "workload": "gate and beta in-projections of 4096 tokens: hidden 4096, rank 128, "
                        "64 heads x 128 gate channels, bf16, log-decay epilogue",
            "us_per_call": round(ms["gate_proj"] * 1e3, 2),
            "TFLOPs": round(gp_flops / (ms["gate_proj"] * 1e-3) / 1e12, 1),
            "roofline": roofline(gp_bytes, ms["gate_proj"] * 1e-3,
                                 _profile_field("gate_proj", "hbm_bytes_per_launch"), flops_per_call=gp_flops),
        },
        "state_copy": {
            "workload": "%d pool rows (fp32 state, 64 heads, and conv state) copied to %d other "
                        "rows of the decode workload's pool" % (n_cp, n_cp),
            "us_per_call": round(ms["state_copy"] * 1e3, 2),
            "roofline": roofline(cp_bytes, ms["state_copy"] * 1e-3,
                                 _profile_field("state_copy", "hbm_bytes_per_launch")),
        },
        "decode_bf16_state": {
            "workload": "the decode workload with the state stored as bf16 (512 MiB)",
            "us_per_call": round(ms["decode_bf16_state"] * 1e3, 2),
            "roofline": roofline(dec_state_bytes // 2 + dec_other, ms["decode_bf16_state"] * 1e-3,
                                 _profile_field("decode_bf16_state", "hbm_bytes_per_launch")),
        },
        "spec_decode": {
            "workload": "256 sequences x 6 tokens (k=5 drafts + 1), H=64, bf16 tokens, fp32 "
                        "state; fused commit of the previous step's accepted prefix",
            "us_per_call": round(ms["spec_decode"] * 1e3, 2),
            "commit_us_per_call": round(ms["spec_commit"] * 1e3, 2),
            "verified_tokens_per_s": round(N_sp * T_sp / sp_s, 1),
            "accepted_tokens_per_s": round(sum(max(0, min(T_sp, a_)) for a_ in acc_l) / sp_s, 1),
            "mean_accepted": round(sum(acc_l) / len(acc_l), 3),
            "roofline": roofline(sp_bytes, sp_s, _profile_field("spec_decode", "hbm_bytes_per_launch")),
        },
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(pre["prefill_varlen"], Dd, torch)
    print(json.dumps(result), flush=True)


def cpu_baseline(P, Dd, torch):
    """The fp64 oracle as it stands, on bounded samples of the prefill and decode
    workloads, OpenMP over (sequence, head) on the host's threads."""
    import oracle  # the CPU baseline leg: the fp64 oracle as it stands
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    H = P["H"]
    heads = list(range(16))  # 16 of the 64 heads, every sequence
    sub = {k_: P[k_][:, heads].cpu() for k_ in ("q", "k", "v", "gate", "beta")}
    sub["state_in"] = P["state_in"][:, heads].cpu()
    # conv weight rows of those heads, in q, k, v order
    w = torch.cat([P["conv_w"][part * H * 128 + h * 128: part * H * 128 + (h + 1) * 128]
                   for part in range(3) for h in heads], 0).cpu()
    cu = P["cu_host"]
    runs = []
    t_all = time.perf_counter()
    while len(runs) < 2 or (time.perf_counter() - t_all < 12.0 and len(runs) < 20):
        t0 = time.perf_counter()
        oracle.prefill(sub["q"], sub["k"], sub["v"], sub["gate"], sub["beta"], w, cu,
                       state_in=sub["state_in"], nthreads=threads)
        runs.append(time.perf_counter() - t0)
    pre_s = sorted(runs)[len(runs) // 2] * H / len(heads)  # all 64 heads of one layer
    # decode: 64 of the 256 sequences, all heads
    ns = 64
    d = {k_: Dd[k_][:ns].cpu() for k_ in ("q", "k", "v", "gate", "beta", "conv_state", "state")}
    druns = []
    t_all = time.perf_counter()
    while len(druns) < 2 or (time.perf_counter() - t_all < 4.0 and len(druns) < 20):
        t0 = time.perf_counter()
        oracle.decode(d["q"], d["k"], d["v"], d["gate"], d["beta"], Dd["conv_w"].cpu(),
                      d["conv_state"], d["state"], nthreads=threads)
        druns.append(time.perf_counter() - t0)
    dec_s = sorted(druns)[len(druns) // 2]
    return {
        "value": round(P["T"] / pre_s, 1), "unit": "tokens/s/layer",
        "cores": threads, "cpu": _cpu_model(), "kind": "oracle",
        "sample": "prefill: the 16-sequence workload (137,314 tokens) on 16 of its 64 heads, "
                  "fp64 token-by-token oracle, median of %d runs of %.2f s, scaled to 64 heads"
                  % (len(runs), sorted(runs)[len(runs) // 2]),
        "decode_state_GBps": round(2 * ns * H * 128 * 128 * 4 / dec_s / 1e9, 3),
        "decode_sample": "64 of the 256 decode sequences, all 64 heads (fp32 state read and "
                         "written), median of %d runs of %.3f s" % (len(druns), dec_s),
    }


if __name__ == "__main__":
    main()

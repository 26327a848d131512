"""Benchmark of the rollout-guided FP4 fake-quant hot path on one MI355X.

One step = one pass of the whole path over one batch of a workload.  For each
tensor of the workload (default: the batched MoE step, routed-expert
activations 128 experts x 1024 tokens x 4096 hidden, Student-t(3), plus one
KV layer, K and V 65536 tokens x 8 heads x 128, in one [2, T, H, D] buffer
with one global scale each; bf16, rollout copies with relative noise 0.01,
k = 2 guidance bits):

  rollout   amax(Y) + RTN quantise + guidance (k): the one-pass kernel (one
            read of Y) when one global-scale group fits on chip (one launch
            per block of groups that fits), else amax(Y) then the quantise
            kernel (--rollout picks either); full-code pack (k = 4)
  training  guided fake-quant (k) -> full-code fake-quant -> plain QAT:
            amax(X) + RTN fake-quant with own scales (one-pass kernel when a
            group fits on chip, else the two kernels)

`value` is the whole step's algorithmic bytes per second (GB/s) over K timed
steps, replayed from a HIP graph (`value_is` says so in the output).
Algorithmic bytes: every operation of the step reads its inputs once and
writes its outputs once (16.875 B per element at k = 2); a separate amax pass
re-reads its input and is not counted there, only on its own per-kernel line.
`roofline` is the guided fake-quant kernel (the metric's subject) on the
workload's first tensor (one launch of k_fakequant_guided<k, one group>),
against the 8 TB/s HBM peak, its launch duration timed with HIP events on the
stream it runs on over K back-to-back launches; `guided_fakequant` gives the
same for every tensor of the workload; `kernels` gives it for every step
kernel; `mismatch` holds the train/rollout code-mismatch rates;
`cpu_baseline` is the CPU oracle on a bounded sample of the same step (a
slice of every tensor, in proportion to its size).

    python bench.py [--steps K] [--warmup W] [--workload 1..5] [--k 1|2] [--no-cpu]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = 5
# HBM counter summary of the roofline kernel, per default-workload launch
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_fakequant_guided_k2_moe_act_128x1024x4096.txt")
KERNEL_SRC = os.path.join(ROOT, "precision_numerics_block_amd", "csrc", "trace_quant.hip")

STEP = ["rollout", "guidance_pack_full", "fakequant_guided", "fakequant_fullcode", "qat_rtn_own"]
# per-kernel lines: the step's launches, and both paths of each fused pair on their own
KERNELS = STEP + ["rollout_onepass", "amax_rollout", "quant_rollout", "rtn_onepass", "amax_training",
                  "fakequant_rtn_own", "fakequant_ste_grad"]
ROOF = "fakequant_guided@0"            # the roofline line: the guided kernel on the first tensor alone


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD, choices=[1, 2, 3, 4, 5])
    p.add_argument("--k", type=int, default=2, choices=[1, 2, 3], help="guidance bits of the compact stream")
    p.add_argument("--no-variants", action="store_true",
                   help="skip the other guidance widths', the MXFP4 variant's and the FP4 weight kernel lines")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--no-transport", action="store_true", help="skip the guidance-transport measurements")
    p.add_argument("--eager", action="store_true", help="launch the step eagerly instead of replaying a graph")
    p.add_argument("--separate-kv", action="store_true",
                   help="K and V as two tensors (G = 1 each) instead of one [2, T, H, D] buffer with G = 2")
    p.add_argument("--rollout", choices=["auto", "onepass", "twopass"], default="auto",
                   help="rollout and plain-QAT paths: auto = one-pass for tensors that fit on chip")
    p.add_argument("--cpu-elems", type=int, default=1 << 25, help="oracle sample size (elements)")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="also run a plain copy of this size (for counter calibration)")
    return p.parse_args()


def bytes_per_elem(k):
    """Algorithmic bytes per element of each kernel line (read once, write once)."""
    gbits = k / 8.0
    rollout = 2.0 + 0.5 + 1 / 16 + (1 / 16 + gbits)         # read y; codes, scales, guidance
    return {
        "rollout": rollout,
        "rollout_onepass": rollout,
        "amax_rollout": 2.0,
        "quant_rollout": rollout,
        "guidance_pack_full": (0.5 + 1 / 16) + (1 / 16 + 0.5),
        "fakequant_guided": 2.0 + (1 / 16 + gbits) + 2.0,
        "fakequant_fullcode": 2.0 + (1 / 16 + 0.5) + 2.0,
        "amax_training": 2.0,
        "fakequant_rtn_own": 2.0 + 2.0,
        "qat_rtn_own": 2.0 + 2.0,
        "rtn_onepass": 2.0 + 2.0,
        "fakequant_ste_grad": 2.0 + 1 / 16 + 2.0 + 2.0,        # x, scales, gy in; gx out (bf16)
    }


def step_bytes_per_elem(k):
    """Algorithmic bytes per element of the whole step: each operation reads
    its inputs once and writes its outputs once (the amax passes, which
    re-read an input, are not algorithmic)."""
    b = bytes_per_elem(k)
    return sum(b[nm] for nm in STEP if not nm.startswith("amax"))


def load_traffic():
    """HBM bytes per launch of the guided kernel from the committed counter
    summary, or None when the kernel source changed since it was taken."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    kv = {}
    for line in open(PROFILE_TRAFFIC):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    src = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if kv.get("kernel_source_sha256") != src:
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(pairs, names, n_sample, k):
    """The CPU oracle on a bounded sample of the workload: the first elements
    of every tensor's X and Y, in proportion to the tensor's size (each slice
    one global-scale group), through the whole step; single-threaded, then
    on all host threads of one GPU's share."""
    import numpy as np
    import torch

    import oracle

    ns = [X.numel() for X, _ in pairs]
    take = [max(16, n_sample * n // sum(ns) // 16 * 16) for n in ns]
    h = lambda t, m: t.reshape(-1)[:m].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)  # noqa
    samples = [(h(X, m), h(Y, m)) for (X, Y), m in zip(pairs, take)]
    n = sum(take)

    def step_one(Xh, Yh, gy, gx):
        codes, scales, gd = oracle.quant_rollout(Yh, gy, k)
        gd4 = oracle.guidance_pack(codes, scales, Yh.size, 4)
        oracle.fakequant_guided(Xh, gy, gd, k, codes=False)
        oracle.fakequant_fullcode(Xh, gy, gd4, codes=False)
        oracle.fakequant_rtn(Xh, gx, codes=False)

    t0 = time.perf_counter()
    gs = []
    for Xh, Yh in samples:
        gy, _ = oracle.amax(Yh)
        gx, _ = oracle.amax(Xh)
        step_one(Xh, Yh, gy, gx)
        gs.append((gy, gx))
    dt = time.perf_counter() - t0
    step_bytes = step_bytes_per_elem(k) * n
    what = ", ".join(f"{m} of {nm}" for nm, m in zip(names, take))
    out = {"value": round(step_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"first elements of each tensor's X and Y ({what}; {n} in all), whole step, "
                     f"{dt:.1f} s single-threaded C"}
    # The same oracle on all host cores of one GPU's share: each slice cut
    # into contiguous pieces (whole blocks), one thread per piece (ctypes
    # releases the GIL).  A slice's global scale is the largest of its
    # pieces' scales (the division by 2688 rounds monotonically); given it,
    # blocks are independent.
    from concurrent.futures import ThreadPoolExecutor

    T = min(16, os.cpu_count() or 1)
    pieces = []
    for si, (Xh, Yh) in enumerate(samples):
        cut = [(Xh.size // 16) * i // T * 16 for i in range(T + 1)]
        pieces += [(si, Xh[a:b], Yh[a:b]) for a, b in zip(cut[:-1], cut[1:]) if b > a]
    with ThreadPoolExecutor(max_workers=T) as ex:
        t0 = time.perf_counter()
        gy_p = list(ex.map(lambda p_: oracle.amax(p_[2])[0], pieces))
        gx_p = list(ex.map(lambda p_: oracle.amax(p_[1])[0], pieces))
        gy_s = [np.max(np.stack([g for p_, g in zip(pieces, gy_p) if p_[0] == si]), axis=0)
                for si in range(len(samples))]
        gx_s = [np.max(np.stack([g for p_, g in zip(pieces, gx_p) if p_[0] == si]), axis=0)
                for si in range(len(samples))]
        list(ex.map(lambda p_: step_one(p_[1], p_[2], gy_s[p_[0]], gx_s[p_[0]]), pieces))
        dt_t = time.perf_counter() - t0
    for (gy, gx), gy2, gx2 in zip(gs, gy_s, gx_s):
        assert np.array_equal(gy, gy2) and np.array_equal(gx, gx2)
    model = ""
    try:
        model = next(ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name"))
    except (OSError, StopIteration):
        pass
    out["all_cores"] = {"value": round(step_bytes / dt_t / 1e9, 4), "unit": "GB/s", "cores": T,
                        "sample": f"the same sample in {len(pieces)} pieces, one thread each, {dt_t:.2f} s"}
    out["host"] = {"nproc": os.cpu_count(), "cpu_model": model}
    return out


def variant_stats(tq, sets, bufs, ns, Gs, K, k_main):
    """The other guidance widths (k = 1, 2, 3 besides the step's): rollout
    quantise + guidance emit and guided fake-quant, per-kernel burst timing
    and the guided mismatch against the rollout codes."""
    import torch

    out = {}
    n_total = sum(ns)
    for k in (1, 2, 3):
        if k == k_main:
            continue
        gds = [[torch.empty(tq.guidance_bytes(n, k), dtype=torch.uint8, device=b[0]["codes"].device)
                for n in ns] for b in bufs]
        lines = {}
        for nm in ("quant_rollout", "fakequant_guided"):
            def launch(i):
                for (X, Y), b, gd, G in zip(sets[i % 2], bufs[i % 2], gds[i % 2], Gs):
                    if nm == "quant_rollout":
                        tq.quant_rollout(Y, b["g"], k, G, guidance=gd, codes=b["codes"], scales=b["scales"])
                    else:
                        tq.fakequant_guided(X, b["g"], gd, k, G, out=b["y_g"])
            for i in range(2):
                launch(i)
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(K):
                launch(i)
            e.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(e) / K
            bpe = (2.0 + 0.5 + 1 / 16 + 1 / 16 + k / 8) if nm == "quant_rollout" else (2.0 + 1 / 16 + k / 8 + 2.0)
            gbs = bpe * n_total / (ms * 1e-3) / 1e9
            lines[nm] = {"us": round(ms * 1e3, 2), "GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
        # mismatch of the guided choice against the rollout's codes (set 0)
        bad = tot = 0
        for (X, Y), b, gd, G in zip(sets[0], bufs[0], gds[0], Gs):
            tq.amax(Y, G, out=b["g"])
            tq.quant_rollout(Y, b["g"], k, G, guidance=gd, codes=b["codes"], scales=b["scales"])
            _, c = tq.fakequant_guided(X, b["g"], gd, k, G, codes_out=True)
            d = c ^ b["codes"]                              # two nibbles (elements) per byte
            bad += int(((d & 15) != 0).sum().item() + ((d >> 4) != 0).sum().item())
            tot += 2 * b["codes"].numel()
        lines["guidance_bits_per_element"] = round(8 * tq.guidance_bytes(ns[0], k) / ns[0], 4)
        lines["mismatch_guided"] = round(bad / tot, 6)
        out[f"k{k}"] = lines
    return out


def weight_stats(tq, K):
    """FP4 weight quantisation (trace_quant_weight) on 64 x 1024 x 2048 bf16
    expert weights, one global scale per expert matrix: per-kernel burst
    timing of its amax and its RTN quantiser (no guidance), the whole call,
    and the one-pass rollout without guidance, which gives the same results.
    Two weight buffers alternate (as the step's input sets do), so no call
    finds its input in the last-level cache; each line is the best of three
    loops of K calls after 20 untimed ones.  Algorithmic bytes read the
    weights once: 2 + 0.5 + 1/16 B per element."""
    import torch
    from precision_numerics_block_amd import synth

    dev = "cuda:0"
    Ws = [synth.make_weights(synth.WEIGHT_SHAPE, dev).reshape(-1)]
    Ws.append(Ws[0].view(synth.WEIGHT_SHAPE).roll(1, 0).reshape(-1).contiguous())
    E = synth.WEIGHT_SHAPE[0]
    n = Ws[0].numel()
    g = torch.empty(E, dtype=torch.float32, device=dev)
    codes = torch.empty(n // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(n // 16, dtype=torch.uint8, device=dev)
    work = torch.zeros(max(tq.onepass_work_bytes(E), 256), dtype=torch.uint8, device=dev)
    b = 2.0 + 0.5 + 1 / 16
    runs = {"weight_amax": (2.0, lambda W: tq.amax(W, E, out=g)),
            "weight_quant": (b, lambda W: tq.quant_rollout(W, g, 2, E, guidance=False, codes=codes, scales=scales)),
            "quant_weight": (b, lambda W: tq.quant_weight(W, E, g=g, codes=codes, scales=scales)),
            # the same results from one read of the weights: every matrix fits on chip, so the one-pass
            # rollout without guidance runs one launch per block of matrices
            "quant_weight_onepass": (b, lambda W: tq.quant_rollout_onepass(W, 2, E, g=g, guidance=False,
                                                                           codes=codes, scales=scales, work=work))}
    out = {"workload": f"expert weights {'x'.join(map(str, synth.WEIGHT_SHAPE))} bf16, G={E} (one per matrix), "
                       "two buffers alternating"}
    for nm, (bpe, fn) in runs.items():
        for i in range(20):
            fn(Ws[i % 2])
        torch.cuda.synchronize()
        best = None
        for _ in range(3):
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(K):
                fn(Ws[i % 2])
            e.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(e) / K
            best = ms if best is None else min(best, ms)
        gbs = bpe * n / (best * 1e-3) / 1e9
        out[nm] = {"us": round(best * 1e3, 2), "GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
    del Ws
    return out


def per_expert_stats(tq, sets, bufs, names_shapes, K, k):
    """The activation tensor with one global scale per expert (G = experts,
    the reported variant of the global-scale grouping): every expert fits on
    chip, so the one-pass entry points read it once, one launch per block of
    experts that fits; against amax + the streaming kernel.  Per-kernel burst
    timing over K launches on alternating input sets."""
    import torch

    name, shape = names_shapes[0]
    E = shape[0]
    n = sets[0][0][0].numel()
    dev = sets[0][0][0].device
    g = torch.empty(E, dtype=torch.float32, device=dev)
    work = torch.zeros(tq.onepass_work_bytes(E), dtype=torch.uint8, device=dev)
    st = torch.zeros(4, dtype=torch.int32, device=dev)
    rb = 2.0 + 0.5 + 1 / 16 + (1 / 16 + k / 8)

    def run(nm, i):
        (X, Y), b = sets[i % 2][0], bufs[i % 2][0]
        if nm == "rollout_onepass":
            tq.quant_rollout_onepass(Y, k, E, g=g, guidance=b["gd"], codes=b["codes"], scales=b["scales"],
                                     work=work, status=st)
        elif nm == "rollout_two_kernel":
            tq.amax(Y, E, out=g)
            tq.quant_rollout(Y, g, k, E, guidance=b["gd"], codes=b["codes"], scales=b["scales"])
        elif nm == "qat_rtn_onepass":
            tq.fakequant_rtn_onepass(X, E, g=g, out=b["y_r"], work=work, status=st)
        else:
            tq.amax(X, E, out=g)
            tq.fakequant_rtn(X, g, None, E, out=b["y_r"])

    out = {"tensor": f"{name} {'x'.join(map(str, shape))}, G={E} (one global scale per expert)"}
    for nm, bpe in (("rollout_onepass", rb), ("rollout_two_kernel", rb), ("qat_rtn_onepass", 4.0),
                    ("qat_rtn_two_kernel", 4.0)):
        for i in range(4):
            run(nm, i)
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(K):
            run(nm, i)
        e.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(e) / K
        gbs = bpe * n / (ms * 1e-3) / 1e9
        out[nm] = {"us": round(ms * 1e3, 2), "GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
    if int(st[0].item()) != 0:
        raise RuntimeError(f"per-expert one-pass status {int(st[0].item())}")
    out["onepass_speedup"] = {"rollout": round(out["rollout_two_kernel"]["us"] / out["rollout_onepass"]["us"], 3),
                              "qat_rtn": round(out["qat_rtn_two_kernel"]["us"] / out["qat_rtn_onepass"]["us"], 3)}
    return out


def mx_stats(tq, sets, ns, K, k):
    """MXFP4 variant (32-element blocks, E8M0 scales): rollout quantise +
    guidance, guided fake-quant and own-scale RTN, per-kernel burst timing
    over the workload's tensors, and train/rollout code mismatch."""
    import torch

    dev = sets[0][0][0].device
    n_total = sum(ns)
    bufs = [[dict(codes=torch.empty(n // 2, dtype=torch.uint8, device=dev),
                  scales=torch.empty(n // 32, dtype=torch.uint8, device=dev),
                  gd=torch.empty(tq.mx_guidance_bytes(n, k), dtype=torch.uint8, device=dev),
                  y=torch.empty(n, dtype=torch.bfloat16, device=dev)) for n in ns] for _ in range(2)]
    bpe = {"mx_quant_rollout": 2.0 + 0.5 + 1 / 32 + (1 / 32 + k / 8),
           "mx_fakequant_guided": 2.0 + (1 / 32 + k / 8) + 2.0,
           "mx_fakequant_rtn_own": 2.0 + 2.0}

    def launch(nm, i):
        for (X, Y), b in zip(sets[i % 2], bufs[i % 2]):
            if nm == "mx_quant_rollout":
                tq.mx_quant_rollout(Y.reshape(-1), k, guidance=b["gd"], codes=b["codes"], scales=b["scales"])
            elif nm == "mx_fakequant_guided":
                tq.mx_fakequant_guided(X.reshape(-1), b["gd"], k, out=b["y"])
            else:
                tq.mx_fakequant_rtn(X.reshape(-1), None, out=b["y"])

    out = {}
    for nm in bpe:
        for i in range(2):
            launch(nm, i)
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(K):
            launch(nm, i)
        e.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(e) / K
        gbs = bpe[nm] * n_total / (ms * 1e-3) / 1e9
        out[nm] = {"us": round(ms * 1e3, 2), "GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
    launch("mx_quant_rollout", 0)
    bad_g = bad_r = tot = 0
    for (X, Y), b in zip(sets[0], bufs[0]):
        _, cg = tq.mx_fakequant_guided(X.reshape(-1), b["gd"], k, codes_out=True)
        _, cr, _ = tq.mx_fakequant_rtn(X.reshape(-1), b["scales"], codes_out=True)
        for c, acc in ((cg, "g"), (cr, "r")):
            d = c ^ b["codes"]
            m = int(((d & 15) != 0).sum().item() + ((d >> 4) != 0).sum().item())
            if acc == "g":
                bad_g += m
            else:
                bad_r += m
        tot += 2 * b["codes"].numel()
    out["mismatch"] = {"rtn_shared_scale": round(bad_r / tot, 6), f"guided_k{k}": round(bad_g / tot, 6)}
    return out


def mismatch_stats(tq, pairs, bufs, k, Gs):
    """Element-level code mismatch between the training side and the rollout
    codes, summed over the workload's tensors."""
    import torch

    def signed(c):
        c = c.to(torch.int32)
        lo, hi = c & 15, c >> 4
        nib = torch.stack([lo, hi], 1).reshape(-1)
        mag = nib & 7
        return torch.where((nib & 8) != 0, -mag, mag)

    tot = {"rtn_shared_scale": 0, "guided": 0, "full_code": 0, "rtn_own_scale_value": 0}
    hist = torch.zeros(8, dtype=torch.int64, device=pairs[0][0].device)
    n_all = 0
    for (X, Y), b, G in zip(pairs, bufs, Gs):
        r = signed(b["codes"])
        _, c_rtn, _ = tq.fakequant_rtn(X, b["g"], b["scales"], G, codes_out=True)
        _, c_gd = tq.fakequant_guided(X, b["g"], b["gd"], k, G, codes_out=True)
        _, c_fc = tq.fakequant_fullcode(X, b["g"], b["gd4"], G, codes_out=True)
        y_own, _, _ = tq.fakequant_rtn(X, b["gx"], None, G)
        y_roll, _, _ = tq.fakequant_rtn(Y, b["g"], b["scales"], G)   # the rollout's dequantised values
        for name, c in (("rtn_shared_scale", c_rtn), ("guided", c_gd), ("full_code", c_fc)):
            d = signed(c) - r
            tot[name] += int((d != 0).sum().item())
            if name == "rtn_shared_scale":
                ad = d.abs()
                hist += torch.bincount(ad[ad > 0], minlength=8)[:8]
        tot["rtn_own_scale_value"] += int((y_own.float() != y_roll.float()).sum().item())
        n_all += r.numel()
    out = {("guided_k%d" % k if nm == "guided" else nm): round(v / n_all, 6) for nm, v in tot.items()}
    out["rtn_abs_index_step_hist"] = {str(i): int(v) for i, v in enumerate(hist.tolist()) if i and v}
    return out


def transport_stats(tq, graphs, sets, bufs, ns, Gs, K, k):
    """Guidance transport ("TRACE Core Concept": the guidance travels GPU ->
    CPU memory -> disk -> CPU -> GPU): per-stage rates for the compact (k)
    and the full-code stream of the first tensor, and the step time when
    each step's stream is copied to pinned host memory after the step."""
    import tempfile

    import torch

    out = {}
    n, G = ns[0], Gs[0]
    for label, kk, key in ((f"compact_k{k}", k, "gd"), ("full_k4", 4, "gd4")):
        b = bufs[0][0]
        rec = torch.empty(tq.record_bytes(n, kk, G), dtype=torch.uint8, pin_memory=True)
        gd2 = torch.empty_like(b[key])
        g2 = torch.empty_like(b["g"])
        reps = 10
        for _ in range(3):                               # first touch of the pinned pages
            tq.record_to_host(b[key], b["g"], n, kk, G, out=rec)
            tq.record_from_host(rec, gd2, g2)
        torch.cuda.synchronize()
        tq.record_seal(rec)
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record()
        for _ in range(reps):
            tq.record_to_host(b[key], b["g"], n, kk, G, out=rec)
        e1.record()
        for _ in range(reps):
            tq.record_from_host(rec, gd2, g2)
        e2.record()
        torch.cuda.synchronize()
        d2h = e0.elapsed_time(e1) / reps * 1e-3
        h2d = e1.elapsed_time(e2) / reps * 1e-3
        t = time.perf_counter()
        tq.record_seal(rec)
        t_seal = time.perf_counter() - t
        with tempfile.TemporaryDirectory() as d:
            path = os.path.join(d, "guidance.trg")
            back = torch.empty(rec.numel(), dtype=torch.uint8, pin_memory=True)
            tq.record_write(path, rec)
            tq.record_read(path, rec.numel(), out=back)      # warm: page cache and pinned pages
            t = time.perf_counter()
            tq.record_write(path, rec)
            t_w = time.perf_counter() - t
            t = time.perf_counter()
            back = tq.record_read(path, rec.numel(), out=back)
            t_r = time.perf_counter() - t
            t = time.perf_counter()
            ok = tq.record_check(back) == (n, kk, G)
            t_chk = time.perf_counter() - t
        nb = rec.numel()
        out[label] = {"record_bytes": nb, "bits_per_element": round(8 * nb / n, 4),
                      "d2h_GBps": round(nb / d2h / 1e9, 2), "h2d_GBps": round(nb / h2d / 1e9, 2),
                      "seal_GBps": round(nb / t_seal / 1e9, 2), "file_write_GBps": round(nb / t_w / 1e9, 2),
                      "file_read_GBps": round(nb / t_r / 1e9, 2), "check_GBps": round(nb / t_chk / 1e9, 2),
                      "round_trip_ok": bool(ok and torch.equal(gd2, b[key]))}

    if not graphs:
        return out

    # Each step's stream is copied right after the step on the same stream.
    # On this runtime a device-to-host copy into pinned memory runs as a blit
    # kernel on the compute units, and the one-pass kernels need every compute
    # unit at once, so a copy on a side stream cannot overlap the step; it
    # only delays a one-pass launch.  The serial form gives the cost per step.
    def run(key, kk):
        recs = [torch.empty(tq.record_bytes(n, kk, G), dtype=torch.uint8, pin_memory=True) for _ in range(2)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(2 * K):                          # first K steps warm the pinned pages
            if i == K:
                torch.cuda.synchronize()
                t0 = time.perf_counter()
            graphs[i % 2].replay()
            if key:
                b = bufs[i % 2][0]
                tq.record_to_host(b[key], b["g"], n, kk, G, out=recs[i % 2])
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / K

    base = run(None, k)
    out["step_ms"] = round(base, 4)
    out[f"step_ms_with_d2h_compact_k{k}"] = round(run("gd", k), 4)
    out["step_ms_with_d2h_full_k4"] = round(run("gd4", 4), 4)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the path has no multi-GPU leg: "
              "each 16-element block is independent and shards need at most one max-reduction of the "
              "global scale.", file=sys.stderr)
        sys.exit(2)
    import torch

    from precision_numerics_block_amd import synth, trace_quant as tq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    k = args.k
    W = synth.WORKLOADS[args.workload]
    specs = synth.tensor_specs(args.workload)
    # two input sets per tensor (the second rolled along the leading dim):
    # consecutive steps alternate, so no step finds its inputs in the 256 MB
    # last-level cache
    pairs = [synth.make_pair(args.workload, pos, shape, dev) for pos, (_, shape) in enumerate(specs)]
    Gs = [1] * len(pairs)
    names_shapes = [(nm, tuple(shape)) for nm, shape in specs]
    if not args.separate_kv and [nm for nm, _ in specs][-2:] == ["k", "v"]:
        # K and V of a layer in one [2, T, H, D] buffer, one global-scale group
        # each (G = 2): every kernel runs once over both, scales stay per tensor
        (K, Ky), (V, Vy) = pairs[-2:]
        pairs = pairs[:-2] + [(torch.stack([K, V]), torch.stack([Ky, Vy]))]
        Gs = Gs[:-2] + [2]
        names_shapes = names_shapes[:-2] + [("kv", (2,) + tuple(K.shape))]
        del K, Ky, V, Vy
    rd = lambda t: 1 if t.dim() == 4 else 0        # roll tokens / experts, never K against V  # noqa: E731
    sets = [pairs, [(X.roll(1, rd(X)).contiguous(), Y.roll(1, rd(Y)).contiguous()) for X, Y in pairs]]
    ns = [X.numel() for X, _ in pairs]
    n_total = sum(ns)
    shapes = [X.shape for X, _ in pairs]

    def make_bufs(shape, n, G):
        return dict(
            g=torch.empty(G, dtype=torch.float32, device=dev),
            gx=torch.empty(G, dtype=torch.float32, device=dev),
            codes=torch.empty(n // 2, dtype=torch.uint8, device=dev),
            scales=torch.empty(n // 16, dtype=torch.uint8, device=dev),
            gd=torch.empty(tq.guidance_bytes(n, k), dtype=torch.uint8, device=dev),
            gd4=torch.empty(tq.guidance_bytes(n, 4), dtype=torch.uint8, device=dev),
            y_g=torch.empty(shape, dtype=torch.bfloat16, device=dev),
            y_f=torch.empty(shape, dtype=torch.bfloat16, device=dev),
            y_r=torch.empty(shape, dtype=torch.bfloat16, device=dev),
            work=torch.zeros(max(tq.onepass_work_bytes(G), 256), dtype=torch.uint8, device=dev),
            work2=torch.zeros(max(tq.onepass_work_bytes(G), 256), dtype=torch.uint8, device=dev),
            st=torch.zeros(4, dtype=torch.int32, device=dev),
        )

    bufs = [[make_bufs(shape, n, G) for shape, n, G in zip(shapes, ns, Gs)] for _ in range(2)]
    # rollout path per tensor: one-pass when one group (in whole tiles of 8192
    # elements) fits on chip; the library runs one launch per block of whole
    # groups that fits when the tensor as a whole does not
    cap = tq.onepass_capacity()
    fits = [-(-(n // G) // 8192) * 8192 <= cap for n, G in zip(ns, Gs)]
    onepass = [args.rollout == "onepass" or (args.rollout == "auto" and f) for f in fits]

    def qat_rtn(X, b, G, one):
        if one:
            tq.fakequant_rtn_onepass(X, G, g=b["gx"], out=b["y_r"], work=b["work2"], status=b["st"])
        else:
            tq.amax(X, G, out=b["gx"])
            tq.fakequant_rtn(X, b["gx"], None, G, out=b["y_r"])

    def rollout(Y, b, G, one):
        if one:
            tq.quant_rollout_onepass(Y, k, G, g=b["g"], guidance=b["gd"], codes=b["codes"], scales=b["scales"],
                                     work=b["work"], status=b["st"])
        else:
            tq.amax(Y, G, out=b["g"])
            tq.quant_rollout(Y, b["g"], k, G, guidance=b["gd"], codes=b["codes"], scales=b["scales"])

    def launch(nm, i):
        """Kernel `nm` once on every tensor of input set i % 2 (`nm@t`: on
        tensor t alone)."""
        nm, _, only = nm.partition("@")
        for t, ((X, Y), b, n, G, one) in enumerate(zip(sets[i % 2], bufs[i % 2], ns, Gs, onepass)):
            if only and t != int(only):
                continue
            if nm == "rollout":
                rollout(Y, b, G, one)
            elif nm == "rollout_onepass":
                rollout(Y, b, G, True)
            elif nm == "qat_rtn_own":
                qat_rtn(X, b, G, one)
            elif nm == "rtn_onepass":
                qat_rtn(X, b, G, True)
            elif nm == "amax_rollout":
                tq.amax(Y, G, out=b["g"])
            elif nm == "quant_rollout":
                tq.quant_rollout(Y, b["g"], k, G, guidance=b["gd"], codes=b["codes"], scales=b["scales"])
            elif nm == "guidance_pack_full":
                tq.guidance_pack(b["codes"], b["scales"], n, 4, out=b["gd4"])
            elif nm == "fakequant_guided":
                tq.fakequant_guided(X, b["g"], b["gd"], k, G, out=b["y_g"])
            elif nm == "fakequant_fullcode":
                tq.fakequant_fullcode(X, b["g"], b["gd4"], G, out=b["y_f"])
            elif nm == "amax_training":
                tq.amax(X, G, out=b["gx"])
            elif nm == "fakequant_ste_grad":            # the guided leg's backward, gy = its output
                tq.fakequant_ste_grad(X, b["g"], b["gd"], b["y_g"], G, out=b["y_f"])
            else:
                tq.fakequant_rtn(X, b["gx"], None, G, out=b["y_r"])

    # One stream: running the independent plain-QAT chain (amax(X) -> RTN) on
    # a second stream was measured slower (two HBM-bound chains interfere).
    def step(i):
        for nm in STEP:
            launch(nm, i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The step is captured once per input set into a HIP graph (kernel
    # launches only, no memset/memcpy nodes) and replayed; eager launching is
    # timed too, for reference.
    graphs = []
    if not args.eager:
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            for i in range(2):
                gph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gph, stream=s_cap):
                    step(i)
                graphs.append(gph)
        torch.cuda.current_stream().wait_stream(s_cap)
        for i in range(2 * args.warmup):
            graphs[i % 2].replay()
        torch.cuda.synchronize()

    def run_steps(K, use_graph):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for i in range(K):
            if use_graph:
                graphs[i % 2].replay()
            else:
                step(i)
        e1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) * 1e3 / K, e0.elapsed_time(e1) / K

    # timed region 1: K whole steps (the headline value)
    K = args.steps
    ms_eager, gpu_ms_eager = run_steps(K, False)
    if graphs:
        ms_step, gpu_ms_step = run_steps(K, True)
    else:
        ms_step, gpu_ms_step = ms_eager, gpu_ms_eager
    # spread: five more loops of K steps each, after the headline region
    loops = sorted(run_steps(K, bool(graphs))[0] for _ in range(5))

    # timed region 2: per-kernel launch durations, K back-to-back launches of
    # each kernel on alternating input sets, HIP events on the launch stream
    # (a single launch between two events would also count the event's own
    # dispatch and release, ~2-4 us)
    per = {}
    guided_each = [f"fakequant_guided@{t}" for t in range(len(pairs))] if len(pairs) > 1 else [ROOF]
    floor_each = [f"{nm}@{t}" for t, one in enumerate(onepass) if one
                  for nm in ("rollout_onepass", "rtn_onepass", "amax_rollout")]
    for nm in KERNELS + guided_each + floor_each:
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(K):
            launch(nm, i)
        b_.record()
        torch.cuda.synchronize()
        per[nm] = a.elapsed_time(b_) / K                   # ms per launch of every tensor

    bpe = bytes_per_elem(k)
    step_bytes = step_bytes_per_elem(k) * n_total
    value = step_bytes / (ms_step * 1e-3) / 1e9
    g_ms = per[ROOF]                                    # the first tensor's guided launch
    g_bytes = bpe["fakequant_guided"] * ns[0]
    achieved = g_bytes / (g_ms * 1e-3) / 1e9
    guided = {}
    for t, nm in enumerate(guided_each):
        gb = bpe["fakequant_guided"] * ns[t]
        guided[f"{names_shapes[t][0]} {'x'.join(map(str, names_shapes[t][1]))} G={Gs[t]}"] = {
            "us": round(per[nm] * 1e3, 2), "GBps": round(gb / (per[nm] * 1e-3) / 1e9, 1),
            "frac_of_peak": round(gb / (per[nm] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    gall = bpe["fakequant_guided"] * n_total / (per["fakequant_guided"] * 1e-3) / 1e9
    guided["all tensors"] = {"us": round(per["fakequant_guided"] * 1e3, 2), "GBps": round(gall, 1),
                             "frac_of_peak": round(gall / HBM_PEAK_GBS, 4)}
    kernels = {nm: {"us": round(per[nm] * 1e3, 2),
                    "GBps": round(bpe[nm] * n_total / (per[nm] * 1e-3) / 1e9, 1),
                    "frac_of_peak": round(bpe[nm] * n_total / (per[nm] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
               for nm in KERNELS}

    # Floor of the one-pass kernels per tensor that runs them: the input read
    # once (the amax kernel on the same tensor: a read of it and little else)
    # plus the outputs written once (a write-only fill of the same number of
    # bytes, torch's fill kernel), one after the other, since no block can be
    # written before the whole group has been read.
    def fill_us(nbytes):
        bufw = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(2)]
        for i in range(4):
            bufw[i % 2].fill_(i)
        torch.cuda.synchronize()
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(K):
            bufw[i % 2].fill_(i & 255)
        e.record()
        torch.cuda.synchronize()
        return a.elapsed_time(e) / K * 1e3

    floors = {}
    for t, one in enumerate(onepass):
        if not one:
            continue
        n_t = ns[t]
        rd = per[f"amax_rollout@{t}"] * 1e3
        lines = {}
        for nm, out_b, bpe_nm in (("rollout_onepass", n_t * (0.5 + 1 / 16 + 1 / 16 + k / 8), "rollout_onepass"),
                                  ("rtn_onepass", 2 * n_t, "rtn_onepass")):
            wr = fill_us(int(out_b))
            us = per[f"{nm}@{t}"] * 1e3
            alg = bpe[bpe_nm] * n_t
            lines[nm] = {"us": round(us, 2), "frac_of_peak": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "read_floor_us": round(rd, 2), "write_floor_us": round(wr, 2),
                         "floor_us": round(rd + wr, 2),
                         "floor_frac_of_peak": round(alg / ((rd + wr) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "kernel_over_floor": round(us / (rd + wr), 3)}
        floors[f"{names_shapes[t][0]} {'x'.join(map(str, names_shapes[t][1]))} G={Gs[t]}"] = lines

    if args.calib_copy_mib:
        m = args.calib_copy_mib << 20
        src = torch.empty(m, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # Same-run reference: torch's device copy of a 256 MiB buffer (the
    # runtime's blit kernel), 2 bytes moved per byte copied.
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dsts = [torch.empty_like(src) for _ in range(2)]
    for i in range(3):
        dsts[i % 2].copy_(src)
    torch.cuda.synchronize()
    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(20):
        dsts[i % 2].copy_(src)
    e.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() / (a.elapsed_time(e) / 20 * 1e-3) / 1e9
    del src, dsts

    bad = [int(b["st"][0].item()) for bs in bufs for b in bs if int(b["st"][0].item()) != 0]
    if bad:                                      # e.g. a one-pass launch whose workgroups were not all resident
        raise RuntimeError(f"device status words report {bad} ({tq.lib.trace_status_str(bad[0]).decode()})")
    variants = None if args.no_variants else variant_stats(tq, sets, bufs, ns, Gs, min(K, 20), k)
    mx = None if args.no_variants else mx_stats(tq, sets, ns, min(K, 20), k)
    weights = None if args.no_variants else weight_stats(tq, min(K, 20))
    experts = None
    if not args.no_variants and names_shapes[0][0] == "act":
        experts = per_expert_stats(tq, sets, bufs, names_shapes, min(K, 20), k)
    step(0)
    mism = mismatch_stats(tq, sets[0], bufs[0], k, Gs)
    torch.cuda.synchronize()
    transport = None if args.no_transport else transport_stats(tq, graphs, sets, bufs, ns, Gs, min(K, 20), k)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(pairs, [nm for nm, _ in names_shapes], min(args.cpu_elems, n_total), k)

    default = args.workload == DEFAULT_WORKLOAD and k == 2
    dist = {"normal_outliers": "N(0,1), 0.5% x20", "student_t4": "Student-t nu=4",
            "kv": "LogNormal(0,0.5) per-channel scale x N(0,1)", "kv_outliers": "as KV plus 1% token rows x10",
            "moe_step": "activations Student-t nu=3 + KV"}[W.dist]
    out = {
        "metric": "guided FP4 fake-quant GB/s and % of HBM peak on 1 MI355X; mismatch rate",
        "value": round(value, 1),
        "unit": "GB/s",
        "value_is": f"whole rollout+training step: {step_bytes_per_elem(k)} algorithmic B/element x "
                    f"{n_total} elements / ms_per_step (the guided kernel alone: roofline, guided_fakequant)",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "gpu_ms_per_step": round(gpu_ms_step, 4),
        "launch": "hip graph replay" if graphs else "eager",
        "ms_per_step_eager": round(ms_eager, 4),
        "ms_per_step_5_loops": {"median": round(loops[2], 4), "min": round(loops[0], 4), "max": round(loops[-1], 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "io_dtypes": {"inputs": "bf16", "outputs": "u8 (FP4 E2M1 codes, E4M3 scales, guidance bits), bf16 "
                                                  "fake-quant values", "arithmetic": "f32 (scale chain, RTN)"},
        "data": "synthetic",
        "config": {"workload": f"{W.name} bf16 ({dist}, rollout relative noise {W.rel_noise}), k={k} "
                               f"guidance, G={max(Gs)}, whole rollout+training step",
                   "tensors": [f"{nm} {'x'.join(map(str, sh))} G={G} "
                               f"rollout+qat={'one-pass' if one else 'two-kernel'}"
                               for (nm, sh), G, one in zip(names_shapes, Gs, onepass)],
                   "onepass_capacity_elements": cap,
                   "elements": n_total, "k": k, "G": max(Gs), "step_bytes": int(step_bytes)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic() if default else None,
                     "kernel": f"k_fakequant_guided<{k},{'true' if Gs[0] == 1 else 'false'},false> "
                               f"(trace_fakequant_guided, k={k}, bf16 out) on {names_shapes[0][0]} "
                               f"{'x'.join(map(str, names_shapes[0][1]))}",
                     "algorithmic_bytes_per_launch": int(g_bytes), "avg_launch_us": round(g_ms * 1e3, 2)},
        "guided_fakequant": guided,
        "onepass_floor": floors,
        "copy_reference": {"GBps": round(copy_gbs, 1), "frac_of_peak": round(copy_gbs / HBM_PEAK_GBS, 4),
                           "what": "torch copy_ of a 256 MiB buffer on the same GPU in the same run (runtime blit "
                                   "kernel), read + write bytes"},
        "elements_per_s": {"step": float(f"{n_total / (ms_step * 1e-3):.4g}"),
                           "fakequant_guided": float(f"{n_total / (per['fakequant_guided'] * 1e-3):.4g}")},
        "cpu_baseline": cpu,
        "mismatch": mism,
        "kernels": kernels,
        "guidance_widths": variants,
        "mxfp4": mx,
        "fp4_weight": weights,
        "per_expert_scales": experts,
        "transport": transport,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()

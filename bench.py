"""Throughput of the fused attention forward and the paged decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras]
    python bench.py --only {fwd,fwd_causal,fwd_4k,fwd_gqa,fwd_fp8,bwd,prefill_paged,prefill_paged_short,decode,copy,fwd_sweep} [--steps K]

One step is one pass of the whole hot path over its synthetic batch:
  * fa_fwd on B=1 H=8 N=16384 d=128 bf16 Q/K/V, non-causal (the headline workload), then
  * fa_paged_decode on 64 sequences x 1 query token, Hq=32 Hkv=8 d=128 bf16, 16-token blocks
    shuffled through a pool, lengths uniform in [512, 32768].
W untimed steps, then K timed steps between device synchronisations.  Each call is also
bracketed by HIP events on the stream it is launched on, so every kernel's own average
duration is known.  ``value`` is the forward's TFLOP/s (4*B*H*N^2*d / average forward time);
the decode's GB/s (algorithmic bytes / average decode time) is reported beside it.  Inputs are
resident in device memory before the timed region starts.

Prints ONE JSON line.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (% MFMA peak) at N=16384,d=128; decode GB/s (% HBM)"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def _profiled_traffic(kernel):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/traffic.json), or None when
    any source of the kernel has changed since the counters were taken."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    with open(PROFILE_TRAFFIC) as f:
        entry = json.load(f).get(kernel)
    if not entry:
        return None
    h = hashlib.sha256()
    for src in entry["sources"]:  # the kernel's file and the headers it is built from
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return entry["hbm_bytes_per_launch"] if h.hexdigest()[:16] == entry["sources_sha256_16"] else None


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _time_calls(torch, fn, iters, warmup=3, warm_s=0.3):
    """Average ms of fn() over iters calls, HIP events on the current stream, after untimed
    calls for at least `warmup` calls and `warm_s` seconds: after an idle spell (the CPU
    baseline leg) the engine clock takes about 20 calls of a 0.5 ms kernel to ramp back up, and
    a fixed small warm-up count measured the ramp (0.59 against 0.47 ms for the causal 16K
    forward)."""
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < warm_s:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    evs = [_events(torch) for _ in range(iters)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / iters


class ClockSampler:
    """Samples the GPU's engine (gfx) clock and socket power with amdsmi from a background
    thread while the main thread keeps the GPU busy (it waits in device synchronisations
    meanwhile).  The published peaks assume the maximum clock; the clock held under load is
    recorded beside the throughput.  The GPU's metrics refresh about once a second, so the
    window must last a few seconds.  Reports None with the reason if amdsmi cannot read the
    device."""

    def __init__(self, torch, period_s=0.1):
        import threading
        self.samples, self.power, self.error, self.max_mhz = [], [], None, None
        self._stop = threading.Event()
        self._period = period_s
        self._handle = None
        try:
            import amdsmi
            self._smi = amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if len(handles) == 1:
                self._handle = handles[0]
            else:  # match the torch device by PCI bus
                bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
                for h in handles:
                    if bus is not None and int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == bus:
                        self._handle = h
            if self._handle is None:
                raise RuntimeError(f"cannot tell which of {len(handles)} devices is cuda:0")
            info = amdsmi.amdsmi_get_clock_info(self._handle, amdsmi.AmdSmiClkType.GFX)
            self.max_mhz = info.get("max_clk")
        except Exception as e:  # noqa: BLE001 -- reported in the JSON, never fatal
            self.error = f"{type(e).__name__}: {e}"
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._handle)
        per_xcd = [x for x in (m.get("current_gfxclks") or []) if isinstance(x, (int, float))]
        clk = sum(per_xcd) / len(per_xcd) if per_xcd else m.get("current_gfxclk")
        pw = m.get("current_socket_power")
        return (clk if isinstance(clk, (int, float)) else None,
                pw if isinstance(pw, (int, float)) else None)

    def _run(self):
        while not self._stop.is_set():
            try:
                clk, pw = self._read()
                if clk is not None:
                    self.samples.append(float(clk))
                if pw is not None:
                    self.power.append(float(pw))
            except Exception as e:  # noqa: BLE001
                self.error = f"{type(e).__name__}: {e}"
                return
            time.sleep(self._period)

    def __enter__(self):
        if self._handle is not None:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()
        return False

    def report(self, what):
        if not self.samples:
            return {"mhz_median": None, "samples": 0,
                    "note": self.error or "no clock sample during the window"}
        s = sorted(self.samples)
        pw = sorted(self.power)
        return {"mhz_median": round(s[len(s) // 2], 1), "mhz_min": round(s[0], 1),
                "mhz_max": round(s[-1], 1), "samples": len(s), "max_engine_mhz": self.max_mhz,
                "socket_power_w_median": round(pw[len(pw) // 2], 1) if pw else None,
                "source": f"amdsmi gpu metrics every 0.1 s (gfx clock, mean over the XCDs) {what}"}


def clock_under_load(torch, fn, seconds=2.5):
    """Engine clock while fn() runs back to back for about `seconds`."""
    with ClockSampler(torch) as clock:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(20):
                fn()
            torch.cuda.synchronize()
    return clock


def _err(got, ref):
    import numpy as np
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref))) if ref.size else 0.0


def cpu_baseline(prefill_inputs, w, gpu, budget_s=10.0):
    """The fp64 oracle on a bounded sample of the forward workload: successive blocks of R query
    rows (head 0 first) against all N keys, until about budget_s seconds of CPU work.

    ``gpu`` holds host copies of the outputs the timed GPU calls produced (the forward's o and
    lse, the small workloads', the decode's); every oracle result computed here is also compared
    with them, so the returned ``parity`` reports the max-abs error of each workload on exactly
    the rows the baseline timed.  Returns (baseline, parity)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention_ref

    q, k, v, _ = prefill_inputs(w["B"], w["H"], w["Hkv"], w["N"], w["d"], "bf16", seed=w["seed"])
    qf = q.float().numpy().astype(np.float64)
    kf = k.float().numpy().astype(np.float64)
    vf = v.float().numpy().astype(np.float64)
    R = 2048
    N, d = w["N"], w["d"]
    done, elapsed = 0, 0.0
    eo = el = 0.0
    for h in range(w["H"]):
        for r0 in range(0, N, R):
            t0 = time.perf_counter()
            ro, rl = attention_ref(qf[:, h:h + 1], kf[:, h:h + 1], vf[:, h:h + 1], 1 / math.sqrt(d),
                                   rows=list(range(r0, r0 + R)))
            elapsed += time.perf_counter() - t0
            eo = max(eo, _err(gpu["fwd"][0][:, h:h + 1, r0:r0 + R], ro))
            el = max(el, _err(gpu["fwd"][1][:, h:h + 1, r0:r0 + R], rl))
            done += 1
            if elapsed >= budget_s:
                break
        if elapsed >= budget_s:
            break
    flops = 4.0 * done * R * N * d
    threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    small, small_parity = oracle_small_workloads(prefill_inputs, gpu)
    parity = {"prefill_16k": {"rows": done * R, "o_max_abs": eo, "lse_max_abs": el,
                              "tol_o": 2e-2, "tol_lse": 1e-3}}
    parity.update(small_parity)
    parity["paged_decode"] = decode_parity(gpu["decode"])
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"fp64 three-pass oracle on {done} blocks of {R} query rows (head-major, "
                  f"head 0 first) x {N} keys, d={d}, {elapsed:.1f} s; flops counted as 4*rows*N*d "
                  f"like the GPU figure",
        "small_workloads": small,
    }, parity


def decode_parity(dec, every=4):
    """Oracle of every `every`-th sequence of the decode workload against the GPU's output."""
    import numpy as np

    from oracle import paged_decode_ref

    dq, kc, vc, table, lens, o, lse = dec
    kcf, vcf = kc.float().numpy(), vc.float().numpy()
    eo = el = 0.0
    seqs = list(range(0, dq.shape[0], every))
    for b in seqs:
        ro, rl = paged_decode_ref(dq[b:b + 1].float().numpy().astype(np.float64), kcf, vcf,
                                  table[b:b + 1].numpy(), [int(lens[b])], 1 / math.sqrt(dq.shape[2]))
        eo = max(eo, _err(o[b:b + 1], ro))
        el = max(el, _err(lse[b:b + 1], rl))
    return {"sequences": len(seqs), "o_max_abs": eo, "lse_max_abs": el, "tol_o": 2e-2,
            "tol_lse": 1e-3}


def oracle_small_workloads(prefill_inputs, gpu, repeats=3):
    """The fp64 oracle over the two small workloads in full (single-head fp32 N=256 d=64, and
    B=1 H=8 N=4096 d=128), on one thread and on all host cores: median wall seconds of
    `repeats` runs, input generation excluded.  Also returns the max-abs error of the GPU's
    outputs for them (every row)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from io_aware_attention_02_amd.inputs import WORKLOADS
    from oracle import attention_ref

    all_threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    res = {"cpu": _cpu_model(), "all_threads": int(all_threads)}
    parity = {}
    for name in ("single_head_fp32", "prefill_4k"):
        w = WORKLOADS[name]
        q, k, v, _ = prefill_inputs(w["B"], w["H"], w["Hkv"], w["N"], w["d"], w["dtype"],
                                    seed=w["seed"])
        qf, kf, vf = (t.float().numpy().astype(np.float64) for t in (q, k, v))
        for label, limit in (("1_thread", 1), ("all_threads", all_threads)):
            times = []
            with threadpool_limits(limits=limit):
                for _ in range(repeats):
                    t0 = time.perf_counter()
                    ro, rl = attention_ref(qf, kf, vf, 1 / math.sqrt(w["d"]))
                    times.append(time.perf_counter() - t0)
            res[f"{name}_{label}_s"] = round(sorted(times)[len(times) // 2], 4)
        go, gl = gpu[name]
        parity[name] = {"rows": int(ro.shape[2]), "o_max_abs": _err(go, ro),
                        "lse_max_abs": _err(gl, rl),
                        "tol_o": 1e-5 if w["dtype"] == "f32" else 2e-2, "tol_lse": 1e-3}
    return res, parity


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def only(args, torch, dev, wf, wd):
    """One kernel alone, W untimed + K timed calls: the command the profiles are taken with."""
    from io_aware_attention_02_amd import fa_fwd, fa_paged_decode
    from io_aware_attention_02_amd.inputs import paged_decode_inputs, prefill_inputs

    if args.only in ("fwd", "fwd_causal"):
        q, k, v, _ = prefill_inputs(wf["B"], wf["H"], wf["Hkv"], wf["N"], wf["d"], "bf16",
                                    seed=wf["seed"])
        q, k, v = q.to(dev), k.to(dev), v.to(dev)
        o = torch.empty_like(q)
        lse = torch.empty((wf["B"], wf["H"], wf["N"]), dtype=torch.float32, device=dev)
        causal = args.only == "fwd_causal"
        fn = lambda: fa_fwd(q, k, v, o, lse, causal=causal)  # noqa: E731
        what = f"fa_fwd B=1 H=8 N=16384 d=128 bf16 causal={causal}"
    elif args.only == "fwd_4k":
        from io_aware_attention_02_amd.inputs import WORKLOADS
        w2 = WORKLOADS["prefill_4k"]
        q, k, v, _ = prefill_inputs(w2["B"], w2["H"], w2["Hkv"], w2["N"], w2["d"], "bf16",
                                    seed=w2["seed"])
        q, k, v = q.to(dev), k.to(dev), v.to(dev)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        fn = lambda: fa_fwd(q, k, v, o, lse)  # noqa: E731
        what = "fa_fwd B=1 H=8 N=4096 d=128 bf16 non-causal"
    elif args.only == "fwd_gqa":
        from io_aware_attention_02_amd.inputs import WORKLOADS
        w4 = WORKLOADS["gqa_varlen_8k"]
        q, k, v, lens = prefill_inputs(w4["B"], w4["H"], w4["Hkv"], w4["N"], w4["d"], "bf16",
                                       seed=w4["seed"], len_lo=w4["len_lo"], len_hi=w4["len_hi"])
        what = (f"fa_fwd B=4 Hq=32 Hkv=8 N=8192 d=128 bf16 causal, seq_lens={lens.tolist()}")
        q, k, v, lens = q.to(dev), k.to(dev), v.to(dev), lens.to(dev)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        fn = lambda: fa_fwd(q, k, v, o, lse, causal=True, seq_lens=lens)  # noqa: E731
    elif args.only == "fwd_fp8":
        from io_aware_attention_02_amd import fa_fwd_fp8
        from io_aware_attention_02_amd.inputs import WORKLOADS, fp8_inputs
        w8 = WORKLOADS["fp8_16k"]
        q8, k8, v8, sc8, _ = fp8_inputs(w8["B"], w8["H"], w8["Hkv"], w8["N"], w8["d"], seed=w8["seed"])
        q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)
        o8 = torch.empty(q8.shape, dtype=torch.bfloat16, device=dev)
        l8 = torch.empty(q8.shape[:3], dtype=torch.float32, device=dev)
        fn = lambda: fa_fwd_fp8(q8, k8, v8, *sc8, o=o8, lse=l8)  # noqa: E731
        what = "fa_fwd_fp8 B=1 H=8 N=16384 d=128 e4m3 non-causal"
    elif args.only == "bwd":
        from io_aware_attention_02_amd import fa_bwd
        from io_aware_attention_02_amd.inputs import output_gradient
        q, k, v, _ = prefill_inputs(wf["B"], wf["H"], wf["Hkv"], wf["N"], wf["d"], "bf16",
                                    seed=wf["seed"])
        q, k, v = q.to(dev), k.to(dev), v.to(dev)
        dout = output_gradient(wf["B"], wf["H"], wf["N"], wf["d"], seed=wf["seed"]).to(dev)
        o, lse = fa_fwd(q, k, v)
        gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        fn = lambda: fa_bwd(q, k, v, o, lse, dout, gq, gk, gv)  # noqa: E731
        what = "fa_bwd B=1 H=8 N=16384 d=128 bf16 non-causal"
    elif args.only in ("prefill_paged", "prefill_paged_short"):
        from io_aware_attention_02_amd import fa_paged_prefill, fa_paged_prefill_workspace_bytes
        from io_aware_attention_02_amd.inputs import WORKLOADS, paged_prefill_inputs
        w5 = WORKLOADS["paged_prefill"]
        ts = paged_prefill_inputs(w5["S"], w5["Hq"], w5["Hkv"], w5["d"], w5["max_q"],
                                  w5["block_size"], w5["len_lo"], w5["len_hi"], seed=w5["seed"])
        pq, pkc, pvc, ptb, psl, pql = (t.to(dev) for t in ts)
        pws = torch.empty(fa_paged_prefill_workspace_bytes(w5["S"], w5["max_q"], w5["Hq"], w5["Hkv"],
                                                           w5["d"], ptb.shape[1]),
                          dtype=torch.uint8, device=dev)
        if args.only == "prefill_paged_short":  # the same contexts, chunks cut to 128 tokens
            pql = torch.clamp(pql, max=128)
        fn = lambda: fa_paged_prefill(pq, pkc, pvc, ptb, psl, pql, workspace=pws)  # noqa: E731
        what = ("fa_paged_prefill 16 seqs, chunks <= " + ("128" if args.only.endswith("short") else "1024")
                + " of contexts U[1024,32768], Hq=32 Hkv=8")
    elif args.only == "decode":
        dq, kc, vc, table, lens = paged_decode_inputs(wd["S"], wd["Hq"], wd["Hkv"], wd["d"],
                                                      wd["block_size"], wd["len_lo"], wd["len_hi"],
                                                      seed=wd["seed"])
        dq, kc, vc, table, lens = dq.to(dev), kc.to(dev), vc.to(dev), table.to(dev), lens.to(dev)
        do = torch.empty_like(dq)
        fn = lambda: fa_paged_decode(dq, kc, vc, table, lens, do)  # noqa: E731
        what = "fa_paged_decode 64 seqs Hq=32 Hkv=8 d=128 lens U[512,32768]"
    else:
        n = 1 << 29  # 512 Mi bf16 elements: 1 GiB read + 1 GiB written per copy
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        fn = lambda: dst.copy_(src)  # noqa: E731
        what = "device copy of 1 GiB (bf16), the byte-counter calibration"
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    ms = _time_calls(torch, fn, args.steps, warmup=0, warm_s=0.0)
    print(json.dumps({"only": args.only, "what": what, "calls": args.steps, "ms_per_call": round(ms, 4)}),
          flush=True)


def sweep(args, torch, dev):
    """fa_fwd over sequence lengths, B=1 H=8 d=128 bf16, both masks: one JSON line per case
    (kernel configuration as the launcher picks it), then the engine clock under the largest."""
    from io_aware_attention_02_amd import accounting as acc
    from io_aware_attention_02_amd import fa_fwd
    from io_aware_attention_02_amd.inputs import prefill_inputs

    B, H, d = 1, 8, 128
    fn = None
    for N in (1024, 2048, 4096, 8192, 16384, 32768, 65536):
        q, k, v, _ = prefill_inputs(B, H, H, N, d, "bf16", seed=7)
        q, k, v = q.to(dev), k.to(dev), v.to(dev)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        for causal in (False, True):
            fn = lambda: fa_fwd(q, k, v, o, lse, causal=causal)  # noqa: E731
            ms = _time_calls(torch, fn, args.steps, warmup=args.warmup, warm_s=0.3)
            f = acc.attention_flops(B, H, N, d, causal=causal)
            print(json.dumps({"only": "fwd_sweep", "B": B, "H": H, "N": N, "d": d, "causal": causal,
                              "ms_per_call": round(ms, 4), "TFLOP/s": round(f / ms / 1e9, 1),
                              "frac": round(f / ms / 1e9 / acc.MI355X_BF16_DENSE_TFLOPS, 4)}),
                  flush=True)
    clock = clock_under_load(torch, fn)
    print(json.dumps({"only": "fwd_sweep", "engine_clock": clock.report(
        "over 2.5 s of the last case (N=65536, causal)")}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--only", choices=["fwd", "fwd_causal", "fwd_4k", "fwd_gqa", "fwd_fp8", "bwd",
                                       "prefill_paged", "prefill_paged_short", "decode", "copy",
                                       "fwd_sweep"],
                    default=None,
                    help="time one kernel alone (profiler runs); prints a short JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "prefill shards by heads and decode by sequences with no exchange, so the "
              "per-GPU kernel at its share is what one GPU shows.", file=sys.stderr)
        sys.exit(2)

    import torch

    from io_aware_attention_02_amd import fa_fwd, fa_paged_decode, fa_paged_decode_workspace_bytes
    from io_aware_attention_02_amd import accounting as acc
    from io_aware_attention_02_amd.inputs import WORKLOADS, paged_decode_inputs, prefill_inputs

    dev = torch.device("cuda:0")
    wf = WORKLOADS["prefill_16k"]
    wd = WORKLOADS["paged_decode"]
    if args.only == "fwd_sweep":
        sweep(args, torch, dev)
        return
    if args.only is not None:
        only(args, torch, dev, wf, wd)
        return

    q, k, v, _ = prefill_inputs(wf["B"], wf["H"], wf["Hkv"], wf["N"], wf["d"], "bf16", seed=wf["seed"])
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((wf["B"], wf["H"], wf["N"]), dtype=torch.float32, device=dev)

    dq, kc, vc, table, lens = paged_decode_inputs(wd["S"], wd["Hq"], wd["Hkv"], wd["d"],
                                                  wd["block_size"], wd["len_lo"], wd["len_hi"],
                                                  seed=wd["seed"])
    lens_host = lens.tolist()
    dq, kc, vc, table, lens = dq.to(dev), kc.to(dev), vc.to(dev), table.to(dev), lens.to(dev)
    do = torch.empty_like(dq)
    dlse = torch.empty((wd["S"], wd["Hq"]), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, fa_paged_decode_workspace_bytes(wd["S"], wd["Hq"], wd["d"],
                                                             table.shape[1], wd["block_size"])),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def prefill():
        fa_fwd(q, k, v, o, lse, causal=False)

    def decode():
        fa_paged_decode(dq, kc, vc, table, lens, do, dlse, workspace=ws)

    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()

    K = args.steps
    ev = [(_events(torch), _events(torch)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for (pa, pb), (da, db) in ev:
        pa.record()
        prefill()
        pb.record()
        da.record()
        decode()
        db.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_pre = sum(a.elapsed_time(b) for (a, b), _ in ev) / K      # ms
    t_dec = sum(a.elapsed_time(b) for _, (a, b) in ev) / K      # ms

    # Host copies of what the timed calls computed (the extras below reuse these buffers), for
    # the parity report of the cpu_baseline leg.
    timed_out = None
    if not args.no_cpu_baseline:
        timed_out = {"fwd": (o.float().cpu().numpy(), lse.cpu().numpy()),
                     "decode": (dq.cpu(), kc.cpu(), vc.cpu(), table.cpu(), lens_host,
                                do.float().cpu().numpy(), dlse.cpu().numpy())}

    # The metrics the clock is read from refresh about once a second, longer than the timed
    # steps, so the clock is taken over a window of the same forward right after them.
    clock = clock_under_load(torch, prefill)

    flops = acc.attention_flops(wf["B"], wf["H"], wf["N"], wf["d"], causal=False)
    tflops = flops / (t_pre * 1e-3) / 1e12
    dbytes = acc.decode_bytes(lens_host, wd["Hq"], wd["Hkv"], wd["d"], wd["block_size"])
    gbps = dbytes / (t_dec * 1e-3) / 1e9

    traffic = _profiled_traffic("fwd")
    dec_traffic = _profiled_traffic("decode")

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "fa_fwd B=1 H=8 N=16384 d=128 bf16 non-causal; then fa_paged_decode "
                        "64 seqs x 1 token, Hq=32 Hkv=8 d=128 bf16, 16-token blocks, "
                        "lengths U[512,32768]",
            "global_batch": wf["B"],
            "seq_len": wf["N"],
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": acc.MI355X_BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / acc.MI355X_BF16_DENSE_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "fwd_bf16_kernel",
            "ms_per_launch": round(t_pre, 4),
            "flops_per_launch": flops,
        },
        "engine_clock": clock.report("over 2.5 s of the same forward right after the timed "
                                     "steps"),
        "decode": {
            "value": round(gbps, 1),
            "unit": "GB/s",
            "ms_per_call": round(t_dec, 4),
            "roofline": {
                "bound": "hbm",
                "achieved": round(gbps, 1),
                "peak": acc.MI355X_HBM_GBPS,
                "unit": "GB/s",
                "frac": round(gbps / acc.MI355X_HBM_GBPS, 4),
                "traffic": dec_traffic,
                "bytes_per_call": dbytes,
            },
        },
    }

    # The part holds its clock below the published peak's under this load (power limit); the
    # same rate as a fraction of the peak scaled to the median clock it held.
    ec = out["engine_clock"]
    if ec.get("mhz_median"):
        ec["frac_of_peak_at_median_clock"] = round(
            tflops / (acc.MI355X_BF16_DENSE_TFLOPS * ec["mhz_median"] / acc.MI355X_PEAK_MHZ), 4)

    if not args.no_extras:
        extras = {}
        wc = WORKLOADS["prefill_16k_causal"]
        t = _time_calls(torch, lambda: fa_fwd(q, k, v, o, lse, causal=True), 10)
        f = acc.attention_flops(wc["B"], wc["H"], wc["N"], wc["d"], causal=True)
        extras["prefill_16k_causal"] = {"ms": round(t, 4), "TFLOP/s": round(f / t / 1e9, 2)}
        w2 = WORKLOADS["prefill_4k"]
        q2, k2, v2, _ = prefill_inputs(w2["B"], w2["H"], w2["Hkv"], w2["N"], w2["d"], "bf16", seed=w2["seed"])
        q2, k2, v2 = q2.to(dev), k2.to(dev), v2.to(dev)
        t = _time_calls(torch, lambda: fa_fwd(q2, k2, v2, causal=False), 20)
        f = acc.attention_flops(w2["B"], w2["H"], w2["N"], w2["d"])
        extras["prefill_4k"] = {"ms": round(t, 4), "TFLOP/s": round(f / t / 1e9, 2)}
        w4 = WORKLOADS["gqa_varlen_8k"]
        q4, k4, v4, l4 = prefill_inputs(w4["B"], w4["H"], w4["Hkv"], w4["N"], w4["d"], "bf16",
                                        seed=w4["seed"], len_lo=w4["len_lo"], len_hi=w4["len_hi"])
        lh = l4.tolist()
        q4, k4, v4, l4 = q4.to(dev), k4.to(dev), v4.to(dev), l4.to(dev)
        t = _time_calls(torch, lambda: fa_fwd(q4, k4, v4, causal=True, seq_lens=l4), 10)
        f = acc.attention_flops(w4["B"], w4["H"], w4["N"], w4["d"], causal=True, seq_lens=lh)
        extras["gqa_varlen_8k_causal"] = {"ms": round(t, 4), "TFLOP/s": round(f / t / 1e9, 2),
                                          "seq_lens": lh}
        # Decode on the literal reading of its pool: 4096 physical blocks (256 MiB of K and V)
        # whose ids every sequence draws with replacement.  The pool fits the caches, so reads
        # are mostly cache hits: reported apart, never against the HBM peak.
        sq, skc, svc, stb, ssl = paged_decode_inputs(wd["S"], wd["Hq"], wd["Hkv"], wd["d"],
                                                     wd["block_size"], wd["len_lo"], wd["len_hi"],
                                                     seed=wd["seed"], pool_blocks=4096)
        sbytes = acc.decode_bytes(ssl.tolist(), wd["Hq"], wd["Hkv"], wd["d"], wd["block_size"])
        sq, skc, svc, stb, ssl = (t.to(dev) for t in (sq, skc, svc, stb, ssl))
        so_, sl_ = torch.empty_like(sq), torch.empty((wd["S"], wd["Hq"]), dtype=torch.float32,
                                                     device=dev)
        t = _time_calls(torch, lambda: fa_paged_decode(sq, skc, svc, stb, ssl, so_, sl_,
                                                       workspace=ws), 20, warmup=5)
        extras["decode_shared_pool_4096"] = {
            "ms": round(t, 4), "GB/s": round(sbytes / t / 1e6, 1), "bytes_per_call": sbytes,
            "cache_resident": True,
            "note": "block ids drawn with replacement from a 4096-block pool (256 MiB of K+V); "
                    "the bytes are the same algorithmic count as the decode line, mostly served "
                    "from L2/MALL, so this is not an HBM figure"}
        del skc, svc
        # The standard unfused forward (S and P through device memory) on the 4K and 16K
        # inputs: the baseline the pages compare fused attention against.
        from io_aware_attention_02_amd import fa_fwd_unfused, fa_fwd_unfused_workspace_bytes
        for name, (qq, kk, vv, ww, t_fused) in (
                ("unfused_4k", (q2, k2, v2, w2, extras["prefill_4k"]["ms"])),
                ("unfused_16k", (q, k, v, wf, t_pre))):
            wsu = torch.empty(fa_fwd_unfused_workspace_bytes(ww["B"], ww["H"], ww["N"]),
                              dtype=torch.uint8, device=dev)
            ou = torch.empty_like(qq)
            lu = torch.empty(qq.shape[:3], dtype=torch.float32, device=dev)
            t = _time_calls(torch, lambda: fa_fwd_unfused(qq, kk, vv, ou, lu, workspace=wsu), 5)
            f = acc.attention_flops(ww["B"], ww["H"], ww["N"], ww["d"])
            extras[name] = {"ms": round(t, 4), "TFLOP/s": round(f / t / 1e9, 2),
                            "fused_speedup": round(t / t_fused, 2)}
            del wsu
        # Chunked prefill against the paged cache (16 sequences, chunks of up to 1024 tokens),
        # then the same contexts with every chunk cut to at most 128 tokens (short chunks against
        # long contexts: the key loops are split over several workgroups and merged).
        from io_aware_attention_02_amd import fa_paged_prefill, fa_paged_prefill_workspace_bytes
        from io_aware_attention_02_amd.inputs import paged_prefill_inputs
        w5 = WORKLOADS["paged_prefill"]
        pq, pkc, pvc, ptb, psl, pql = paged_prefill_inputs(
            w5["S"], w5["Hq"], w5["Hkv"], w5["d"], w5["max_q"], w5["block_size"], w5["len_lo"],
            w5["len_hi"], seed=w5["seed"])
        f = acc.paged_prefill_flops(psl.tolist(), pql.tolist(), w5["Hq"], w5["d"])
        pq, pkc, pvc, ptb, psl, pql = (t.to(dev) for t in (pq, pkc, pvc, ptb, psl, pql))
        po = torch.empty_like(pq)
        pl = torch.empty(pq.shape[:3], dtype=torch.float32, device=dev)
        pws = torch.empty(fa_paged_prefill_workspace_bytes(w5["S"], w5["max_q"], w5["Hq"], w5["Hkv"],
                                                           w5["d"], ptb.shape[1]),
                          dtype=torch.uint8, device=dev)
        t = _time_calls(torch, lambda: fa_paged_prefill(pq, pkc, pvc, ptb, psl, pql, po, pl,
                                                        workspace=pws), 10)
        extras["paged_prefill"] = {"ms": round(t, 4), "TFLOP/s": round(f / t / 1e9, 2)}
        pql128 = torch.clamp(pql, max=128)
        f128 = acc.paged_prefill_flops(psl.tolist(), pql128.tolist(), w5["Hq"], w5["d"])
        t = _time_calls(torch, lambda: fa_paged_prefill(pq, pkc, pvc, ptb, psl, pql128, po, pl,
                                                        workspace=pws), 10)
        extras["paged_prefill_chunks_le_128"] = {"ms": round(t, 4),
                                                 "TFLOP/s": round(f128 / t / 1e9, 2)}
        del pkc, pvc, pws
        # Backward (recompute from the forward's LSE) on the headline inputs, both masks.
        from io_aware_attention_02_amd import fa_bwd, fa_bwd_workspace_bytes
        from io_aware_attention_02_amd.inputs import output_gradient
        dout = output_gradient(wf["B"], wf["H"], wf["N"], wf["d"], seed=wf["seed"]).to(dev)
        wsb = torch.empty(fa_bwd_workspace_bytes(wf["B"], wf["H"], wf["N"]), dtype=torch.uint8,
                          device=dev)
        gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        for causal, name in ((False, "backward_16k"), (True, "backward_16k_causal")):
            ob, lb = fa_fwd(q, k, v, causal=causal)
            t = _time_calls(torch, lambda: fa_bwd(q, k, v, ob, lb, dout, gq, gk, gv, causal=causal,
                                                  workspace=wsb), 10)
            f = acc.attention_bwd_flops(wf["B"], wf["H"], wf["N"], wf["d"], causal=causal)
            extras[name] = {"ms": round(t, 4), "TFLOP/s": round(f / t / 1e9, 2)}
        # FP8 forward (e4m3 Q, K, V with per-tensor scales) on the 16K shapes, both masks.
        from io_aware_attention_02_amd import fa_fwd_fp8
        from io_aware_attention_02_amd.inputs import fp8_inputs
        w8 = WORKLOADS["fp8_16k"]
        q8, k8, v8, sc8, _ = fp8_inputs(w8["B"], w8["H"], w8["Hkv"], w8["N"], w8["d"], seed=w8["seed"])
        q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)
        o8 = torch.empty(q8.shape, dtype=torch.bfloat16, device=dev)
        l8 = torch.empty(q8.shape[:3], dtype=torch.float32, device=dev)
        for causal, name in ((False, "fp8_16k"), (True, "fp8_16k_causal")):
            t = _time_calls(torch, lambda: fa_fwd_fp8(q8, k8, v8, *sc8, o=o8, lse=l8, causal=causal), 20,
                            warmup=20)
            f = acc.attention_flops(w8["B"], w8["H"], w8["N"], w8["d"], causal=causal)
            extras[name] = {"ms": round(t, 4), "TFLOP/s": round(f / t / 1e9, 2),
                            "frac_of_fp8_peak": round(f / t / 1e9 / acc.MI355X_FP8_DENSE_TFLOPS, 4)}
        del q8, k8, v8
        out["extras"] = extras

    if not args.no_cpu_baseline:
        gpu = dict(timed_out)
        for name in ("single_head_fp32", "prefill_4k"):
            ws_ = WORKLOADS[name]
            qs, ks, vs, _ = prefill_inputs(ws_["B"], ws_["H"], ws_["Hkv"], ws_["N"], ws_["d"],
                                           ws_["dtype"], seed=ws_["seed"])
            os_, ls_ = fa_fwd(qs.to(dev), ks.to(dev), vs.to(dev))
            gpu[name] = (os_.float().cpu().numpy(), ls_.cpu().numpy())
        out["cpu_baseline"], out["parity"] = cpu_baseline(prefill_inputs, wf, gpu)
    else:
        out["cpu_baseline"] = None

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Throughput benchmark: exact attention forward + backward on one MI355X.

One step is one pass of the whole path over one batch: fa_fwd (O, LSE), then
fa_bwd as its two launches, called apart (fa_bwd_dq_ws: the dQ sweep over
query blocks, which also forms D = rowsum(dO o O); fa_bwd_dkdv_ws: the dK/dV
sweep over key blocks). The workload is the Llama-2-7B-shaped causal attention layer
(batch 16, 32 heads, N = 2048, d = 128, bf16; rotary Q/K, dO ~ N(0, 0.01)),
with inputs resident in device memory before the timed region.

FLOPs follow the pages' accounting: forward 4*B*H*N^2*d, backward
10*B*H*N^2*d (the recompute of S included), halved under the causal mask.
The dQ sweep recomputes S and dP a second time; those products are not
counted (of the backward's 10, the dK/dV sweep is credited with 8 -- S, dP,
dV, dK -- and the dQ sweep with 2 -- the dS K product).

Prints ONE JSON line. Besides the required keys it carries:
  roofline      the dominant kernel (the backward sweep with the longer
                duration) against the bf16 dense MFMA peak, its duration
                measured with HIP events on the launch stream inside the
                timed region; HBM traffic from the committed rocprofv3 counter
                summary when it was taken on the current kernel source, else
                null;
  cpu_baseline  the fp64 oracle timed on host cores on a sample of the same
                workload (also used as a parity spot-check of the timed run);
  sweep         forward and forward+backward TFLOPS for bf16 d = 128 at
                N = 2048, 4096, 8192 (B*N = 16384 tokens, 16 heads), causal
                and not, and for the workloads B4 H32 N2048 d128 bf16 and
                B1 H16 N8192 d64 fp16 causal.
  small         the two small workloads, launch-latency-bound: B1 H1 N256 d64
                fp32 (forward only, against the fp32 MFMA peak) and B2 H8
                N1024 d64 bf16; medians in microseconds and as TFLOPS (part
                of the sweep leg).
  splitkv       fa_fwd against fa_fwd_splitkv (the library's split choice) on
                grids with fewer query blocks than the chip has workgroup
                slots, and the merge kernel's HBM rate.
  kvcache       fa_fwd_kvcache: decoding (one new query per slice over an
                8192-key cache; HBM-bound, reported in GB/s of K and V read)
                and chunked prefill (512 new queries over 8192 keys).
  gpu_clock     graphics clock (mean over the XCDs) and socket power sampled
                with amdsmi (in-process) while the main workload runs (settle, timed and
                forward-only launches, after the first 0.8 s), and the dense
                bf16 MFMA rate at that clock.
  kernels       each kernel of the step: mean launch time (HIP events), the
                flops it executes and those the pages' count credits to it,
                and both rates as TFLOP/s and as a fraction of the peak.
"""
import argparse
import hashlib
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOPS (fwd; fwd+bwd) bf16 d=128 N=2k–8k, % of MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA (published)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "c5_traffic.json")


def _src_hash(path):
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(kernel, workload):
    """Per-launch HBM bytes of a kernel from the committed counter summary, or
    None if absent, taken on another workload, or taken on other source of
    that kernel (every file listed for it must hash the same)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("workload") != workload:
            return None
        k = t["kernels"][kernel]
        if any(_src_hash(p) != h for p, h in k["sources"].items()):
            return None
        return k["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        return None


def _inputs(w, torch, dev):
    import attn_inputs as ai
    inp = ai.make_inputs(w)
    return {k: v.to(dev) for k, v in inp.items()}, inp


def _step_fns(fa, torch, w, d):
    B, H, N, D = w.B, w.H, w.N, w.d
    o = torch.empty_like(d["q"])
    lse = torch.empty((B, H, N), dtype=torch.float32, device=d["q"].device)
    dq, dk, dv = (torch.empty_like(d["q"]) for _ in range(3))
    L = fa.lib()
    code = {torch.float32: fa.F32, torch.bfloat16: fa.BF16, torch.float16: fa.F16}[d["q"].dtype]
    ws_bytes = L.fa_bwd_workspace_bytes(code, B, H, N, D) if w.backward else 0
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=d["q"].device)
    P = lambda t: t.data_ptr()
    st = torch.cuda.current_stream().cuda_stream
    c = int(w.causal)

    def ck(rc):
        if rc != 0:
            raise fa.FAError("bench", rc)

    def fwd():
        ck(L.fa_fwd(code, B, H, N, D, P(d["q"]), P(d["k"]), P(d["v"]), w.scale, c, P(o),
                    P(lse), st))

    # fa_bwd as its two launches, one ABI call each so that each can be
    # timed (the same kernels, arguments and results as one fa_bwd call): the
    # dQ sweep, which also forms D = rowsum(dO o O) and LSE * log2(e) into the
    # workspace, then the dK/dV sweep, which reads them.
    def dqs():
        ck(L.fa_bwd_dq_ws(code, B, H, N, D, P(d["q"]), P(d["k"]), P(d["v"]), P(o), P(d["do"]),
                          P(lse), w.scale, c, P(dq), P(ws), ws_bytes, st))

    def dkdv():
        ck(L.fa_bwd_dkdv_ws(code, B, H, N, D, P(d["q"]), P(d["k"]), P(d["v"]), P(d["do"]),
                            w.scale, c, P(dk), P(dv), P(ws), ws_bytes, st))

    fns = (fwd, dqs, dkdv) if w.backward else (fwd,)
    return fns, {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


class ClockSampler:
    """Samples the GPU's graphics clocks (mean over the XCDs) and socket power
    in a background thread, through the amdsmi library loaded in this process
    (sysfs reads through the kernel driver: no HIP call, no child process).
    Samples from the first `skip_s` seconds are dropped: the clock is still
    climbing from idle then. It does not start under a profiler's preloaded
    library (reported as an error in the result instead)."""

    TOOL = "amdsmi (in-process): gpu_metrics current_gfxclks, current_socket_power"

    def __init__(self, period_s=0.2, skip_s=0.8):
        self.period_s, self.skip_s = period_s, skip_s
        self.samples, self.error = [], None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._smi, self._handle = None, None

    @staticmethod
    def profiler_present():
        pre = os.environ.get("LD_PRELOAD", "")
        return "rocprof" in pre or any(k.startswith(("ROCPROF", "ROCP_")) for k in os.environ)

    @staticmethod
    def _num(x):
        return x if isinstance(x, (int, float)) and not isinstance(x, bool) else None

    def _open(self):
        import amdsmi
        amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
        handles = amdsmi.amdsmi_get_processor_handles()
        if not handles:
            raise RuntimeError("amdsmi sees no GPU")
        handle = handles[0]
        if len(handles) > 1:
            # Several GPUs visible to amdsmi: take the one torch runs on, by
            # PCI bus.
            import torch
            pr = torch.cuda.get_device_properties(torch.cuda.current_device())
            bus = getattr(pr, "pci_bus_id", None)
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)   # "dddd:bb:dd.f"
                if bus is not None and int(bdf.split(":")[1], 16) == bus:
                    handle = h
                    break
        self._smi, self._handle = amdsmi, handle

    def _sample(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._handle)
        clks = [c for c in (self._num(v) for v in (m.get("current_gfxclks") or []))
                if c is not None and 0 < c < 10000]
        if not clks and self._num(m.get("current_gfxclk")):
            clks = [m["current_gfxclk"]]
        pw = self._num(m.get("current_socket_power"))
        if pw is None or pw >= 0xFFFF:
            pw = self._num(m.get("average_socket_power"))
        return (sum(clks) / len(clks) if clks else None,
                pw if pw is not None and pw < 0xFFFF else None)

    def _run(self):
        t0 = time.perf_counter()
        try:
            self._open()
            while not self._stop.is_set():
                clk, pw = self._sample()
                if time.perf_counter() - t0 >= self.skip_s and clk is not None:
                    self.samples.append((clk, pw))
                self._stop.wait(self.period_s)
        except Exception as e:  # no amdsmi, no permission, or fields it lacks
            self.error = "%s: %s" % (type(e).__name__, e)
        finally:
            if self._smi is not None:
                try:
                    self._smi.amdsmi_shut_down()
                except Exception:
                    pass

    def start(self):
        if self.profiler_present():
            self.error = "not sampled under a profiler"
            return
        self._thread.start()

    def stop(self):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join(timeout=10)
        if not self.samples:
            return {"samples": 0, "error": self.error or "no sample"}
        clk = sorted(c for c, _ in self.samples)
        pw = sorted(p for _, p in self.samples if p is not None)
        med = clk[len(clk) // 2]
        # 256 CUs x 4 SIMDs x 1024 bf16 flops per clock.
        return {"gfx_mhz": round(med, 1), "gfx_mhz_min": round(clk[0], 1),
                "gfx_mhz_max": round(clk[-1], 1),
                "socket_power_w": pw[len(pw) // 2] if pw else None,
                "samples": len(clk), "tool": self.TOOL,
                "mfma_bf16_tflops_at_clock": round(256 * 4 * 1024 * med * 1e6 / 1e12, 1)}


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def time_workload(fa, torch, w, steps, warmup, per_kernel=True, settle_s=0.0, sampler=None,
                  fwd_runs=50):
    """Times one workload. Returns a dict: ms_step (mean over the `steps` timed
    steps, one event pair around all of them), ms_step_median (median of the
    per-step times), ms_fwd and ms_fwd_median (forward alone, `fwd_runs`
    launches), kern (mean per-kernel times of the steps, or None), outs (the
    outputs of a last clean step) and host (the host inputs).

    After the `warmup` steps, further untimed steps run until `settle_s`
    seconds have passed since the first one: the GPU clock climbs from its
    idle level over a fraction of a second under this load, and the timed
    steps should see the clock a sustained run gets."""
    d, host = _inputs(w, torch, "cuda")
    fns, outs = _step_fns(fa, torch, w, d)
    if sampler is not None:
        sampler.start()
    t_start = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t_start < settle_s:
        for f in fns:
            f()
        done += 1
        if done >= warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    names = ("fwd", "bwd_dq", "bwd_dkdv")[:len(fns)]
    # Events between the launches of every step (they sit on the same stream
    # and add no work); the step time is first event to last.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
          for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for s in range(steps):
        for i, f in enumerate(fns):
            ev[s][i].record()
            f()
        ev[s][-1].record()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    ms_step_median = _median([ev[s][0].elapsed_time(ev[s][-1]) for s in range(steps)])
    kern = None
    if per_kernel:
        kern = {n: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) / steps
                for i, n in enumerate(names)}
    # forward alone
    fe = [torch.cuda.Event(enable_timing=True) for _ in range(fwd_runs + 1)]
    for r in range(fwd_runs):
        fe[r].record()
        fns[0]()
    fe[-1].record()
    torch.cuda.synchronize()
    ms_fwd = fe[0].elapsed_time(fe[-1]) / fwd_runs
    ms_fwd_median = _median([fe[r].elapsed_time(fe[r + 1]) for r in range(fwd_runs)])
    # one clean step so the outputs correspond to the inputs
    for f in fns:
        f()
    torch.cuda.synchronize()
    # Stopped only now: joining the thread can take a sample's time, and an
    # idle GPU lowers its clock before the forward-only launches above.
    if sampler is not None:
        sampler.clock = sampler.stop()
    return {"ms_step": ms_step, "ms_step_median": ms_step_median, "ms_fwd": ms_fwd,
            "ms_fwd_median": ms_fwd_median, "kern": kern, "outs": outs, "host": host}


def slice_errors(outs, b, h, o_ref, lse_ref, g):
    """Errors of the timed run's outputs on one slice against the oracle."""
    import numpy as np

    def a(t):
        return t[b, h].detach().cpu().double().numpy()

    def rel(x, ref):
        return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))

    return {"o_max_abs": float(np.abs(a(outs["o"]) - o_ref).max()),
            "o_rel_l2": rel(a(outs["o"]), o_ref),
            "lse_max_abs": float(np.abs(a(outs["lse"]) - lse_ref).max()),
            "dq_rel_l2": rel(a(outs["dq"]), g["dq"]),
            "dk_rel_l2": rel(a(outs["dk"]), g["dk"]),
            "dv_rel_l2": rel(a(outs["dv"]), g["dv"])}


def cpu_baseline(w, host, outs, min_seconds=10.0, max_slices=256):
    """The fp64 oracle on whole (batch, head) slices of the same workload,
    until min_seconds of work; also compares those slices with the GPU run."""
    import oracle
    t_total, n, errs = 0.0, 0, []
    slices = [(b, h) for b in (0, w.B - 1) for h in (0, w.H - 1)]
    slices += [(b, h) for b in range(w.B) for h in range(w.H) if (b, h) not in slices]
    for b, h in slices[:max_slices]:
        q, k, v, do = (host[x][b, h].double().numpy() for x in ("q", "k", "v", "do"))
        t = time.perf_counter()
        o_ref, lse_ref = oracle.attention_fwd(q, k, v, w.scale, w.causal)
        g = oracle.attention_bwd(q, k, v, do, w.scale, w.causal)
        t_total += time.perf_counter() - t
        n += 1
        errs.append(slice_errors(outs, b, h, o_ref, lse_ref, g))
        if t_total >= min_seconds:
            break
    flops = n * (w.fwd_flops() + w.bwd_flops()) / (w.B * w.H)
    worst = {k: max(e[k] for e in errs) for k in errs[0]}
    return {"value": flops / t_total / 1e12, "unit": "TFLOPS", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%d of %d (batch, head) slices of the workload, fwd+bwd in fp64 "
                      "(%.1f s)" % (n, w.B * w.H, t_total)}, worst


# Whole (batch, head) slices of each workload the oracle is timed on: every
# slice of the small ones, a sample of the large ones (about 1-3 s each).
ORACLE_SLICES = {"c1": 1, "c2": 16, "c3": 4, "c4": 1, "c5": 8}


def oracle_by_config(have=None):
    """The fp64 oracle timed per workload on the host's cores (as many OpenMP
    threads as it runs with), forward and, where the workload has one,
    backward, on ORACLE_SLICES[name] whole slices; the whole workload's time
    is that mean per slice times B*H (every slice has the same shape and
    work). GFLOP/s use the pages' count (4 N^2 d forward, 10 N^2 d backward,
    halved under the mask). Then c1 and c2 once more on one thread: the
    per-core figure. `have`: host inputs already drawn, by workload name."""
    import attn_inputs as ai
    import oracle
    have = have or {}
    threads = oracle.num_threads()

    def run(w, host, n):
        t = 0.0
        for i in range(n):
            b, h = divmod(i * max(1, (w.B * w.H) // n), w.H)
            q, k, v = (host[x][b, h].double().numpy() for x in ("q", "k", "v"))
            t0 = time.perf_counter()
            oracle.attention_fwd(q, k, v, w.scale, w.causal)
            if w.backward:
                oracle.attention_bwd(q, k, v, host["do"][b, h].double().numpy(), w.scale,
                                     w.causal)
            t += time.perf_counter() - t0
        return t

    out = []
    for name, n in ORACLE_SLICES.items():
        w = ai.WORKLOADS[name]
        host = have.get(name) or ai.make_inputs(w, with_do=w.backward)
        per_slice = w.fwd_flops() / (w.B * w.H)
        if w.backward:
            per_slice += w.bwd_flops() / (w.B * w.H)
        t = run(w, host, n)
        rec = {"workload": name, "pass": "fwd+bwd" if w.backward else "fwd",
               "threads": threads, "slices_timed": n, "slices": w.B * w.H,
               "seconds_timed": round(t, 3),
               "seconds_whole_workload": round(t / n * w.B * w.H, 2),
               "gflops": round(per_slice * n / t / 1e9, 2)}
        if name in ("c1", "c2"):
            oracle.set_num_threads(1)
            try:
                n1 = 1 if name == "c1" else 2
                t1 = run(w, host, n1)
            finally:
                oracle.set_num_threads(threads)
            rec["one_thread"] = {"slices_timed": n1, "seconds_timed": round(t1, 3),
                                 "gflops": round(per_slice * n1 / t1 / 1e9, 3)}
        out.append(rec)
        print("# oracle %s: %d of %d slices in %.2f s on %d threads (%.2f GFLOP/s)%s" %
              (name, n, w.B * w.H, t, threads, rec["gflops"],
               "; one thread %.3f GFLOP/s" % rec["one_thread"]["gflops"]
               if "one_thread" in rec else ""), file=sys.stderr, flush=True)
        del host
    return out


def _time_ms(torch, fn, iters, settle_s):
    t_start = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    while time.perf_counter() - t_start < settle_s:
        fn()
        torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def splitkv_report(fa, torch, settle_s):
    """Forward with and without key splits where the plain grid under-fills
    the chip; the merge kernel timed alone on the same partial results."""
    import attn_inputs as ai
    L = fa.lib()
    out = []
    cases = [ai.WORKLOADS["c2"],
             ai.custom("b1-h4-n8192", 1, 4, 8192, 128, "bf16", False, seed=42),
             ai.custom("b1-h4-n8192-causal", 1, 4, 8192, 128, "bf16", True, seed=42)]
    for w in cases:
        d = {k: v.cuda() for k, v in ai.make_inputs(w, with_do=False).items()}
        B, H, N, D = w.B, w.H, w.N, w.d
        code = {torch.bfloat16: fa.BF16, torch.float16: fa.F16}[d["q"].dtype]
        parts = fa.fwd_splitkv_parts(B, H, N, 0, w.causal)
        nbytes = fa.fwd_splitkv_workspace_bytes(d["q"].dtype, B, H, N, D, 0, w.causal)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        o = torch.empty_like(d["q"])
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        st = torch.cuda.current_stream().cuda_stream
        P = lambda t: t.data_ptr()

        def plain():
            L.fa_fwd(code, B, H, N, D, P(d["q"]), P(d["k"]), P(d["v"]), w.scale,
                     int(w.causal), P(o), P(lse), st)

        def split():
            L.fa_fwd_splitkv(code, B, H, N, D, P(d["q"]), P(d["k"]), P(d["v"]), w.scale,
                             int(w.causal), 0, P(o), P(lse), P(ws), nbytes, st)

        rows = B * H * N
        obytes = -(-parts * rows * D * 4 // 256) * 256

        def merge():
            L.fa_lse_merge(code, parts, rows, D, P(ws), P(ws) + obytes, P(o), P(lse), st)

        ms_plain = _time_ms(torch, plain, 20, settle_s)
        ms_split = _time_ms(torch, split, 20, settle_s)
        ms_merge = _time_ms(torch, merge, 20, 0.0)
        merge_bytes = parts * rows * (4 * D + 4) + rows * (2 * D + 4)
        out.append({"workload": w.name, "B": B, "H": H, "N": N, "d": D, "causal": w.causal,
                    "parts": parts, "fwd_tflops": round(w.fwd_flops() / ms_plain / 1e9, 1),
                    "splitkv_tflops": round(w.fwd_flops() / ms_split / 1e9, 1),
                    "ms_fwd": round(ms_plain, 4), "ms_splitkv": round(ms_split, 4),
                    "merge_ms": round(ms_merge, 4),
                    "merge_gbs": round(merge_bytes / ms_merge / 1e6, 1)})
        print("# splitkv %s parts %d: fwd %.3f ms, split %.3f ms (merge %.3f ms, %.0f GB/s)" %
              (w.name, parts, ms_plain, ms_split, ms_merge, merge_bytes / ms_merge / 1e6),
              file=sys.stderr, flush=True)
    return out


def kvcache_report(fa, torch, settle_s):
    """Attention of Nq new queries over an Nk-key cache."""
    out = []
    for name, B, H, Nq, Nk, causal in (("decode-b16-h32-nk8192", 16, 32, 1, 8192, True),
                                       ("decode-b1-h32-nk32768", 1, 32, 1, 32768, True),
                                       ("prefill-b1-h32-nq512-nk8192", 1, 32, 512, 8192, True)):
        d = 128
        g = torch.Generator().manual_seed(42)
        q, k, v = (torch.randn(B, H, n, d, generator=g).to(torch.bfloat16).cuda()
                   for n in (Nq, Nk, Nk))
        parts = fa.fwd_kvcache_parts(B, H, Nq, Nk, 0, causal)
        ws = torch.empty(fa.fwd_kvcache_workspace_bytes(torch.bfloat16, B, H, Nq, Nk, d, 0,
                                                        causal),
                         dtype=torch.uint8, device="cuda")
        ms = _time_ms(torch, lambda: fa.fwd_kvcache(q, k, v, d ** -0.5, causal, 0, ws), 20,
                      settle_s)
        kv_bytes = 2 * B * H * Nk * d * 2
        vis = Nq * Nk - (Nq * (Nq - 1)) // 2 if causal else Nq * Nk   # visible (q, k) pairs
        flops = 4.0 * B * H * vis * d
        out.append({"workload": name, "B": B, "H": H, "Nq": Nq, "Nk": Nk, "d": d,
                    "causal": causal, "parts": parts, "ms": round(ms, 4),
                    "kv_gbs": round(kv_bytes / ms / 1e6, 1), "tflops": round(flops / ms / 1e9, 1)})
        print("# kvcache %s parts %d: %.4f ms, %.0f GB/s of K/V, %.1f TFLOPS" %
              (name, parts, ms, kv_bytes / ms / 1e6, flops / ms / 1e9), file=sys.stderr,
              flush=True)
    return out


def std_report(fa, torch, settle_s):
    """Standard attention that stores S and P (the pages' baseline) against
    the tiled path on the same inputs: time and the device memory of the
    N x N arrays (S fp32 and P in the forward, dS in the backward) against
    the tiled path's only per-row extras (LSE and D, fp32)."""
    import attn_inputs as ai
    L = fa.lib()
    out = []
    for w in (ai.WORKLOADS["c5"], ai.WORKLOADS["perf-2k"], ai.WORKLOADS["perf-8k"]):
        d = {k: v.cuda() for k, v in ai.make_inputs(w).items()}
        B, H, N, D = w.B, w.H, w.N, w.d
        dt = d["q"].dtype
        code = {torch.bfloat16: fa.BF16, torch.float16: fa.F16}[dt]
        P_ = lambda t: t.data_ptr()
        st = torch.cuda.current_stream().cuda_stream
        o, lse = torch.empty_like(d["q"]), torch.empty((B, H, N), dtype=torch.float32,
                                                       device="cuda")
        dq, dk, dv = (torch.empty_like(d["q"]) for _ in range(3))
        pbytes = fa.std_p_bytes(dt, B, H, N, D)
        fws = fa.std_fwd_workspace_bytes(dt, B, H, N, D)
        bws = fa.std_bwd_workspace_bytes(dt, B, H, N, D)
        Pm = torch.empty(pbytes, dtype=torch.uint8, device="cuda")
        ws = torch.empty(max(fws, bws), dtype=torch.uint8, device="cuda")
        gws = torch.empty(fa.bwd_workspace_bytes(dt, B, H, N, D), dtype=torch.uint8,
                          device="cuda")

        def ck(rc):
            if rc != 0:
                raise RuntimeError("library call failed: %d" % rc)

        def std_f():
            ck(L.fa_std_fwd(code, B, H, N, D, P_(d["q"]), P_(d["k"]), P_(d["v"]), w.scale,
                            int(w.causal), P_(o), P_(lse), P_(Pm), P_(ws), fws, st))

        def std_fb():
            std_f()
            ck(L.fa_std_bwd(code, B, H, N, D, P_(d["q"]), P_(d["k"]), P_(d["v"]), P_(o),
                            P_(d["do"]), P_(Pm), w.scale, P_(dq), P_(dk), P_(dv), P_(ws), bws,
                            st))

        def fl_f():
            ck(L.fa_fwd(code, B, H, N, D, P_(d["q"]), P_(d["k"]), P_(d["v"]), w.scale,
                        int(w.causal), P_(o), P_(lse), st))

        def fl_fb():
            fl_f()
            ck(L.fa_bwd(code, B, H, N, D, P_(d["q"]), P_(d["k"]), P_(d["v"]), P_(o),
                        P_(d["do"]), P_(lse), w.scale, int(w.causal), P_(dq), P_(dk), P_(dv),
                        P_(gws), gws.numel(), st))

        ms = {name: _time_ms(torch, fn, 5, settle_s)
              for name, fn in (("std_fwd", std_f), ("std_fwdbwd", std_fb), ("fwd", fl_f),
                               ("fwdbwd", fl_fb))}
        flops = w.fwd_flops(), w.fwd_flops() + w.bwd_flops()
        nxn = fws + pbytes + bws - fa.bwd_workspace_bytes(dt, B, H, N, D)
        rec = {"workload": w.name, "B": B, "H": H, "N": N, "d": D, "causal": w.causal,
               "std_fwd_ms": round(ms["std_fwd"], 3), "std_fwdbwd_ms": round(ms["std_fwdbwd"], 3),
               "fwd_ms": round(ms["fwd"], 3), "fwdbwd_ms": round(ms["fwdbwd"], 3),
               "std_fwd_tflops": round(flops[0] / ms["std_fwd"] / 1e9, 1),
               "std_fwdbwd_tflops": round(flops[1] / ms["std_fwdbwd"] / 1e9, 1),
               "fwd_speedup": round(ms["std_fwd"] / ms["fwd"], 2),
               "fwdbwd_speedup": round(ms["std_fwdbwd"] / ms["fwdbwd"], 2),
               "nxn_gib": round(nxn / 2 ** 30, 2),
               "tiled_extra_mib": round(2 * B * H * N * 4 / 2 ** 20, 2)}
        out.append(rec)
        print("# std %s: stored-P fwd %.3f ms, fwd+bwd %.3f ms; tiled %.3f / %.3f ms; N x N "
              "arrays %.2f GiB" % (w.name, ms["std_fwd"], ms["std_fwdbwd"], ms["fwd"],
                                   ms["fwdbwd"], nxn / 2 ** 30), file=sys.stderr, flush=True)
        del Pm, ws, gws, d
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle", type=float, default=2.0,
                    help="seconds of untimed steps (at least --warmup of them) before timing")
    ap.add_argument("--workload", default="c5")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline leg")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-splitkv", action="store_true")
    ap.add_argument("--no-kvcache", action="store_true")
    ap.add_argument("--no-std", action="store_true",
                    help="skip the stored-P standard-attention comparison")
    ap.add_argument("--no-clock", action="store_true",
                    help="do not sample the clock and power (the sampler also stays off "
                         "by itself under a profiler's preloaded library)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (scales the HBM "
                         "byte counters read under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path. "
              "(Every (batch, head) slice is independent, so several GPUs would each "
              "run the one-GPU kernels on their share of slices.) Run with --gpus 1.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import attn_inputs as ai
    import exact_attention_34_amd as fa
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "dispatches": 5}), flush=True)
        return
    fa.lib()

    w = ai.WORKLOADS[args.workload]
    sampler = None if args.no_clock else ClockSampler()
    tw = time_workload(fa, torch, w, args.steps, args.warmup, settle_s=args.settle,
                       sampler=sampler)
    ms_step, ms_fwd, kern, outs, host = (tw["ms_step"], tw["ms_fwd"], tw["kern"], tw["outs"],
                                         tw["host"])
    clock = sampler.clock if sampler is not None else {"samples": 0, "error": "--no-clock"}
    flops_step = w.fwd_flops() + w.bwd_flops()
    value = flops_step / (ms_step * 1e-3) / 1e12
    fwd_tflops = w.fwd_flops() / (ms_fwd * 1e-3) / 1e12

    # Algorithmic flops per launch of each backward sweep (see the header).
    sweeps = {"bwd_dkdv": ("bwd_dkdv64_kernel" if w.d == 64 else "bwd_dkdv_kernel",
                           0.8 * w.bwd_flops()),
              "bwd_dq": ("bwd_dq_kernel", 0.2 * w.bwd_flops())}
    dom = max(sweeps, key=lambda k: kern[k])
    kname, kflops = sweeps[dom]
    achieved = kflops / (kern[dom] * 1e-3) / 1e12
    roofline = {"kernel": kname, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": _traffic(kname, w.name),
                "ms_per_launch": round(kern[dom], 4),
                "flops_per_launch": kflops}
    bwd_ms = kern["bwd_dkdv"] + kern["bwd_dq"]
    # Executed MFMA work per launch: forward S and P V (4 N^2 d), dK/dV sweep
    # S, dP, dV, dK (8 N^2 d), dQ sweep S, dP, dQ (6 N^2 d); halved when
    # causal. Credited work is the pages' count (4 and 10 N^2 d), the
    # backward split 8 : 2 as above.
    unit = w.fwd_flops() / 4
    per = {"fwd": (4 * unit, w.fwd_flops()), "bwd_dq": (6 * unit, 0.2 * w.bwd_flops()),
           "bwd_dkdv": (8 * unit, 0.8 * w.bwd_flops())}
    kernels = {}
    for k, (ex, cr) in per.items():
        t = kern[k] * 1e-3
        kernels[k] = {"ms": round(kern[k], 4),
                      "executed_tflops": round(ex / t / 1e12, 1),
                      "credited_tflops": round(cr / t / 1e12, 1),
                      "executed_frac": round(ex / t / 1e12 / PEAK_BF16_TFLOPS, 4),
                      "credited_frac": round(cr / t / 1e12 / PEAK_BF16_TFLOPS, 4)}

    out = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOPS", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "settle_s": args.settle, "ms_per_step": round(ms_step, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if w.dtype == "bf16" else w.dtype,
           "data": "synthetic (seeded N(0,1) inputs, rotary Q/K, dO ~ N(0,0.01))",
           "config": {"workload": "%s: %s" % (w.name, w.note), "B": w.B, "H": w.H, "N": w.N,
                      "d": w.d, "causal": w.causal, "global_batch": w.B, "seq_len": w.N,
                      "parallelism": "none (1 GPU)"},
           "fwd_tflops": round(fwd_tflops, 2),
           "bwd_tflops": round(w.bwd_flops() / (bwd_ms * 1e-3) / 1e12, 2),
           "median": {"fwd_tflops": round(w.fwd_flops() / tw["ms_fwd_median"] / 1e9, 2),
                      "fwdbwd_tflops": round(flops_step / tw["ms_step_median"] / 1e9, 2),
                      "fwd_runs": 50, "fwdbwd_runs": args.steps,
                      "ms_fwd": round(tw["ms_fwd_median"], 4),
                      "ms_fwdbwd": round(tw["ms_step_median"], 4)},
           "fwd_frac_of_peak": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
           "fwdbwd_frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
           "kernel_ms": {k: round(v, 4) for k, v in kern.items()},
           "kernels": kernels,
           "roofline": roofline,
           "gpu_clock": clock}
    if clock.get("mfma_bf16_tflops_at_clock"):
        roofline["frac_of_peak_at_measured_clock"] = round(
            achieved / clock["mfma_bf16_tflops_at_clock"], 4)

    if not args.no_sweep:
        sweep = []
        for name in ("perf-2k", "perf-4k", "perf-8k", "perf-2k-causal", "perf-4k-causal",
                     "perf-8k-causal", "c3", "c4"):
            ws = ai.WORKLOADS[name]
            r = time_workload(fa, torch, ws, 20, 3, per_kernel=False,
                              settle_s=min(args.settle, 1.0))
            # Median of 20 fwd+bwd steps and of 50 forward launches.
            s_ms, f_ms = r["ms_step_median"], r["ms_fwd_median"]
            del r
            tf = (ws.fwd_flops() + ws.bwd_flops()) / (s_ms * 1e-3) / 1e12
            ff = ws.fwd_flops() / (f_ms * 1e-3) / 1e12
            sweep.append({"workload": name, "B": ws.B, "H": ws.H, "N": ws.N, "d": ws.d,
                          "dtype": ws.dtype, "causal": ws.causal, "fwd_tflops": round(ff, 1),
                          "fwdbwd_tflops": round(tf, 1),
                          "fwd_frac": round(ff / PEAK_BF16_TFLOPS, 4),
                          "fwdbwd_frac": round(tf / PEAK_BF16_TFLOPS, 4)})
            print("# sweep %s fwd %.1f TFLOPS fwd+bwd %.1f TFLOPS" % (name, ff, tf),
                  file=sys.stderr, flush=True)
        out["sweep"] = sweep
        # The two small workloads: c1, the fp32 forward (the shape of the
        # essay's test harness), and c2. One or a few workgroups per launch:
        # launch latency dominates, so these are latencies, not throughput.
        small = []
        for name in ("c1", "c2"):
            ws = ai.WORKLOADS[name]
            r = time_workload(fa, torch, ws, 20, 3, per_kernel=False, settle_s=0.2)
            f_ms = r["ms_fwd_median"]
            peak = PEAK_F32_TFLOPS if ws.dtype == "f32" else PEAK_BF16_TFLOPS
            ff = ws.fwd_flops() / (f_ms * 1e-3) / 1e12
            rec = {"workload": name, "B": ws.B, "H": ws.H, "N": ws.N, "d": ws.d,
                   "dtype": ws.dtype, "causal": ws.causal, "fwd_us": round(f_ms * 1e3, 2),
                   "fwd_tflops": round(ff, 2), "fwd_frac": round(ff / peak, 4), "peak": peak}
            if ws.backward:
                s_ms = r["ms_step_median"]
                tf = (ws.fwd_flops() + ws.bwd_flops()) / (s_ms * 1e-3) / 1e12
                rec.update(fwdbwd_us=round(s_ms * 1e3, 2), fwdbwd_tflops=round(tf, 2),
                           fwdbwd_frac=round(tf / peak, 4))
            del r
            small.append(rec)
            print("# small %s fwd %.1f us" % (name, rec["fwd_us"]), file=sys.stderr, flush=True)
        out["small"] = small
    if not args.no_splitkv:
        out["splitkv"] = splitkv_report(fa, torch, min(args.settle, 0.5))
    if not args.no_kvcache:
        out["kvcache"] = kvcache_report(fa, torch, min(args.settle, 0.5))
    if not args.no_std:
        out["standard"] = std_report(fa, torch, min(args.settle, 0.5))
    # The oracle runs last: its OpenMP threads (and their spinning after the
    # parallel regions) would otherwise compete with the launching thread.
    if not args.no_cpu:
        cb, worst = cpu_baseline(w, host, outs)
        out["cpu_baseline"] = cb
        out["parity_spot_check"] = worst
        out["oracle_by_config"] = oracle_by_config({w.name: host})
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

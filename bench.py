#!/usr/bin/env python3
"""Benchmark of the MoE layer's routed-expert hot path on one MI355X.

Prints ONE JSON line.  A "step" is one pass of the whole path (route, group,
expert FFN, combine) over one batch of synthetic input, for every layer of the
workload.  Default workload: the 48-layer decode step (T = 4 tokens, H = 2048,
I = 512, E = 512 + 1 shared, top-10, Zipf s = 1.0 routing, block-FP4 experts,
every (layer, expert) resident in an HBM slot pool).  Inputs for every timed
step are generated on the device before timing starts.

Extra objects on the line:
  roofline      the dominant kernel, the expert FFN's gate/up stage (one
                launch of moe_expert_ffn_stages with stages = 1 per layer):
                algorithmic bytes (decode, HBM-bound: the gate and up codes,
                scales and global scales of every distinct expert touched) or
                flops (prefill, MFMA-bound: 4 H I per row) per launch, divided
                by its mean duration from HIP events on its stream, against the
                MI355X spec peak (HBM 8.0 TB/s; dense bf16 MFMA 2.5 PFLOP/s).
                The down stage is reported beside it.  "traffic" is the HBM
                bytes per launch measured with rocprofv3 counters and recorded
                in profiles/ (null unless it was measured on this kernel source).
                With --ffn one-launch the dominant kernel is the one launch of
                moe_expert_ffn_combine (both stages and the combine), against
                both stages' expert bytes.
  prefill8192,  (default workload only) the 8192-token prefill layer and the
  decode43x64   43-layer decode over 64 steps, measured in the same run:
                tokens/s and their own roofline; for decode43x64 also the p50
                and p90 of the 64 step times and the expert-weight GB/s of a
                step.  --no-extra skips them.
  probes        (default workload only) measured peaks beside the spec ones:
                the stream-read probe's best HBM read rate and the dense MFMA
                rate of back-to-back bf16, fp8 x fp4 and fp8 MFMAs.
  cpu_baseline  the CPU oracle (oracle/, fp64 numpy) on a bounded sample of
                the same workload, scaled to tokens/s: on every host core this
                process may use (cores), and on one thread (one_thread).

The streamed workload adds "h2d" (the copy rate and the overlap fraction of
copy and compute) and "serial" (the same layers with one slot, each copy then
its compute on one stream: the reference without the second buffer).

--probes runs only the probes.  --copy-calibration BYTES runs only a plain device copy of BYTES bytes five
times (the reference kernel that scales the FETCH_SIZE / WRITE_SIZE counters).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; decode expert-weight GB/s & prefill TFLOP/s vs peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0   # dense fp8 MFMA: the rate of the scaled FP8 x FP4 instruction


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="decode48",
                    help="tiny | decode48 | decode43x64 | prefill8192 | streamed4x4096 | cached48x64 | prefill8192_mx | "
                         "decode48_mx "
                         "(default decode48)")
    ap.add_argument("--eager", action="store_true", help="launch every call eagerly instead of HIP graphs")
    ap.add_argument("--ffn", default="routed-dc", choices=("layer", "routed", "routed-dc", "one-launch", "split"),
                    help="decode windows: the routing in one launch with the FFN's first step (moe_route_group_ffn: "
                         "inside the gate/up launch; moe_route_group_ffn_mx: with MXFP8(x); stages 1, then the down "
                         "stage and moe_combine (routed) or both in one call, moe_expert_ffn_down_combine "
                         "(routed-dc, the default; MX keeps routed); where the window allows, else split), FFN and combine in "
                         "one launch (moe_expert_ffn_combine) or one launch per FFN stage plus the combine's "
                         "(moe_expert_ffn_stages 1, 2; moe_combine)")
    ap.add_argument("--policy", default="lru", choices=("lru", "hotcold"),
                    help="cached workloads: lru (fill every miss; the layer's outputs) or hotcold (measure the "
                         "hot/cold swap policy over the routing)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=10.0,
                    help="oracle seconds per timing (it is timed twice: all host cores, then one thread)")
    ap.add_argument("--no-extra", action="store_true",
                    help="decode48: skip the prefill8192 and decode43x64 measurements added to its line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES")
    ap.add_argument("--probes", action="store_true",
                    help="run only the HBM-read and MFMA-loop probes and print their line")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_gateup_%s_traffic.txt")
LAYER_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "layer_dec_%s_traffic.txt")
CSRC = os.path.join(ROOT, "moe_expert_ffn_top_amd", "csrc")


def ffn_kernel(cfg):
    """(kernel name, source file) of the FFN path the library takes for these
    shapes: the grouped GEMM when groups average >= 16 rows (T k >= 16 E),
    else the weight-streaming kernel."""
    if cfg.fmt == "mx" and cfg.T * cfg.k >= 16 * cfg.E:
        return "k_ffn_mx", os.path.join(CSRC, "ffn_mx.hip")
    if cfg.T * cfg.k >= 16 * cfg.E:
        return "k_ffn_gemm", os.path.join(CSRC, "ffn_gemm.hip")
    return "k_ffn_dec", os.path.join(CSRC, "ffn_dec.hip")


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch already loaded (same
    SONAME, so the same runtime instance), for kernel-bracketing launches."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = []

    def new(self):
        e = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(e))
        assert rc == 0, "hipEventCreate failed (%d)" % rc
        self.handles.append(e.value)
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        assert rc == 0, "hipEventElapsedTime failed (%d)" % rc
        return float(ms.value)

    def close(self):
        for e in self.handles:
            self.hip.hipEventDestroy(e)
        self.handles = []


def source_hash(path):
    """sha256[:16] of a kernel source followed by the library headers it
    includes (#include "x.hpp", recursively, each once), so a change to any
    code compiled into the kernel changes the hash."""
    h, seen = hashlib.sha256(), set()

    def add(f):
        if f in seen:
            return
        seen.add(f)
        with open(f, "rb") as fh:
            data = fh.read()
        h.update(data)
        for line in data.decode("utf-8", "replace").splitlines():
            line = line.strip()
            if line.startswith('#include "'):
                inc = os.path.join(os.path.dirname(f), line.split('"')[1])
                if os.path.exists(inc):
                    add(inc)

    add(path)
    return h.hexdigest()[:16]


def kernel_source_hash(cfg):
    return source_hash(ffn_kernel(cfg)[1])


def recorded_traffic(cfg, layer=False):
    """HBM bytes per launch of the dominant kernel (the gate/up launch, or with
    layer the one-launch layer) from the counter summary in profiles/, if it
    was taken on the current kernel source; else None."""
    path = (LAYER_TRAFFIC_FILE if layer else TRAFFIC_FILE) % cfg.name
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash(cfg):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Workload:
    """Device-resident inputs of every step to be run, plus one set of layer buffers."""

    def __init__(self, cfg, n_steps, B, DevGen, ffn="split"):
        import torch
        from moe_expert_ffn_top_amd.layer import LayerBuffers
        from synth import zipf_logits

        self.cfg = cfg
        self.ffn_mode = ffn
        self.dims = B.Dims(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.L)
        self.mx = cfg.fmt == "mx"
        self.layout = B.moe_blob_layout_init_mx(cfg.H, cfg.I) if self.mx else B.moe_blob_layout_init(cfg.H, cfg.I)
        dev = DevGen()
        E1, L = cfg.E1, cfg.L
        self.n_slots = L * E1
        self.slot_table = torch.arange(self.n_slots, dtype=torch.int32, device="cuda").view(L, E1).contiguous()
        self.pool_bytes = self.n_slots * self.layout.slot_stride
        log("allocating %.2f GB expert pool (%d slots x %d B)" % (self.pool_bytes / 1e9, self.n_slots,
                                                                 self.layout.slot_stride))
        self.pool = torch.zeros(self.pool_bytes, dtype=torch.uint8, device="cuda")
        t0 = time.time()
        (dev.pool_mx if self.mx else dev.pool)(cfg, 0, L, self.slot_table.data_ptr(), self.n_slots, self.layout,
                                               self.pool.data_ptr())
        torch.cuda.synchronize()
        log("pool generated on device in %.1f s" % (time.time() - t0))
        # per-step inputs: steps cycle through the workload's own steps
        self.n_inputs = min(n_steps, max(cfg.steps, 1)) if cfg.router == "zipf" else min(n_steps, 4)
        self.x = torch.empty((self.n_inputs, L, cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
        for s in range(self.n_inputs):
            for l in range(L):
                dev.x(cfg, l, s, self.x[s, l].data_ptr())
        self.wsg = torch.empty((L, cfg.H), dtype=torch.float32, device="cuda")
        for l in range(L):
            dev.w_shared_gate(cfg, l, self.wsg[l].data_ptr())
        if cfg.router == "matrix":
            self.wr = torch.empty((L, cfg.H, cfg.E), dtype=torch.float32, device="cuda")
            for l in range(L):
                dev.w_router(cfg, l, self.wr[l].data_ptr())
            self.logits = None
        else:
            self.wr = None
            lg = np.stack([np.stack([zipf_logits(cfg, l, s) for l in range(L)]) for s in range(self.n_inputs)])
            self.logits = torch.from_numpy(lg).cuda()
        torch.cuda.synchronize()
        self.buf = LayerBuffers.allocate(self.dims, mx=self.mx)

    def ffn(self, x, stages=3, ev_start=None, ev_stop=None, stream=None):
        """The expert FFN of the current layer (the blob format's entry point)."""
        from moe_expert_ffn_top_amd import binding as B
        d, buf = self.dims, self.buf
        if self.mx:
            B.moe_expert_ffn_mx(d, x, self.pool, self.pool_bytes, self.layout, buf.offsets, buf.perm,
                                buf.group_slot, buf.h, buf.y_rows, buf.status, buf.ws, buf.mx_ws, stages,
                                ev_start, ev_stop, stream=stream)
        else:
            B.moe_expert_ffn_stages(d, x, self.pool, self.pool_bytes, self.layout, buf.offsets, buf.perm,
                                    buf.group_slot, buf.h, buf.y_rows, buf.status, buf.ws, stages, ev_start,
                                    ev_stop, stream=stream)

    def input_index(self, step):
        return step % self.n_inputs

    @property
    def one_launch(self):
        """NVFP4 decode windows: the FFN and the combine run through
        moe_expert_ffn_combine, one launch per layer."""
        return not self.mx and self.cfg.T * self.cfg.k < 16 * self.cfg.E and self.ffn_mode == "one-launch"

    @property
    def layer_launch(self):
        """NVFP4 decode windows with drawn logits, --ffn layer: route, group,
        both FFN stages and the combine through moe_route_group_ffn_combine,
        one launch per layer."""
        return (not self.mx and self.wr is None and self.ffn_mode == "layer" and routed_shape(self.cfg)
                and self.cfg.k <= 16)

    @property
    def routed(self):
        """Decode windows with drawn logits whose routing runs in one launch with
        the FFN's first step: moe_route_group_ffn (NVFP4: route, group and
        gate/up together) or moe_route_group_ffn_mx (MX: route, group and
        MXFP8(x) together), then the rest of the FFN and the combine."""
        return self.wr is None and self.ffn_mode in ("routed", "routed-dc", "layer") and routed_shape(self.cfg)

    @property
    def down_combine(self):
        """routed-dc: the down stage and the combine through moe_expert_ffn_down_combine."""
        return not self.mx and self.ffn_mode == "routed-dc"

    def ffn_combine(self, x, ev_start=None, ev_stop=None, stream=None):
        from moe_expert_ffn_top_amd import binding as B
        d, buf = self.dims, self.buf
        B.moe_expert_ffn_combine(d, x, self.pool, self.pool_bytes, self.layout, buf.offsets, buf.perm,
                                 buf.group_slot, buf.inv_perm, buf.w, buf.sigma, buf.h, buf.y_rows, buf.y,
                                 buf.status, buf.ws, ev_start, ev_stop, stream=stream)

    def run_step(self, step, stream=None, ffn_events=None, hip_events=None):
        """Enqueue every layer of one step.  With ffn_events (a list) the FFN
        launches carry HIP events that the device records at the kernel's own
        start and end: on the one-launch path one pair around the FFN +
        combine launch, otherwise one pair per stage; per layer (events,
        offsets) is appended."""
        from moe_expert_ffn_top_amd import binding as B

        s = self.input_index(step)
        d, buf = self.dims, self.buf
        for l in range(self.cfg.L):
            x = self.x[s, l]
            wr = self.wr[l] if self.wr is not None else None
            lg_in = None if self.wr is not None else self.logits[s, l]
            lg_out = buf.logits if self.wr is not None else None
            if self.layer_launch:
                ev = [hip_events.new() for _ in range(2)] if ffn_events is not None else [None, None]
                B.moe_route_group_ffn_combine(d, l, x, None, lg_in, self.wsg[l], None, buf.ids, buf.w, buf.sigma,
                                              self.slot_table, self.n_slots, buf.offsets, buf.perm, buf.inv_perm,
                                              buf.group_slot, self.pool, self.pool_bytes, self.layout, buf.h,
                                              buf.y_rows, buf.y, buf.status, buf.ws, ev[0], ev[1], stream=stream)
                if ffn_events is not None:
                    ffn_events.append((ev, buf.offsets.clone()))
                continue
            if self.routed:
                ev = [hip_events.new() for _ in range(4)] if ffn_events is not None else [None] * 4
                if self.mx:
                    B.moe_route_group_ffn_mx(d, l, x, wr, lg_in, self.wsg[l], lg_out, buf.ids, buf.w, buf.sigma,
                                             self.slot_table, self.n_slots, buf.offsets, buf.perm, buf.inv_perm,
                                             buf.group_slot, self.pool, self.pool_bytes, self.layout, buf.h,
                                             buf.y_rows, buf.status, buf.ws, buf.mx_ws, 1, ev[0], ev[1],
                                             stream=stream)
                else:
                    B.moe_route_group_ffn(d, l, x, wr, lg_in, self.wsg[l], lg_out, buf.ids, buf.w, buf.sigma,
                                          self.slot_table, self.n_slots, buf.offsets, buf.perm, buf.inv_perm,
                                          buf.group_slot, self.pool, self.pool_bytes, self.layout, buf.h,
                                          buf.y_rows, buf.status, buf.ws, 1, ev[0], ev[1], stream=stream)
                if self.down_combine:
                    # the down stage and the combine in one call (one launch on decode windows)
                    B.moe_expert_ffn_down_combine(d, x, self.pool, self.pool_bytes, self.layout, buf.offsets,
                                                  buf.perm, buf.group_slot, buf.inv_perm, buf.w, buf.sigma, buf.h,
                                                  buf.y_rows, buf.y, buf.status, buf.ws, ev[2], ev[3],
                                                  stream=stream)
                    if ffn_events is not None:
                        ffn_events.append((ev, buf.offsets.clone()))
                    continue
                self.ffn(x, 2, ev[2], ev[3], stream=stream)
                if ffn_events is not None:
                    ffn_events.append((ev, buf.offsets.clone()))
                B.moe_combine(d, buf.y_rows, buf.inv_perm, buf.w, buf.sigma, buf.y, stream)
                continue
            B.moe_route_group(d, l, x, wr, lg_in, self.wsg[l], lg_out, buf.ids, buf.w, buf.sigma, self.slot_table,
                              self.n_slots, buf.offsets, buf.perm, buf.inv_perm, buf.group_slot, buf.status, buf.ws,
                              stream=stream)
            if self.one_launch:
                ev = [hip_events.new() for _ in range(2)] if ffn_events is not None else [None, None]
                self.ffn_combine(x, ev[0], ev[1], stream=stream)
                if ffn_events is not None:
                    ffn_events.append((ev, buf.offsets.clone()))
                continue
            if ffn_events is None:
                if self.ffn_mode in ("split", "routed", "routed-dc", "layer") and not self.mx:
                    for st in (1, 2):
                        self.ffn(x, st, stream=stream)
                else:
                    self.ffn(x, stream=stream)
            else:
                ev = [hip_events.new() for _ in range(4)]
                for st in (1, 2):
                    self.ffn(x, st, ev[2 * st - 2], ev[2 * st - 1], stream=stream)
                ffn_events.append((ev, buf.offsets.clone()))
            B.moe_combine(d, buf.y_rows, buf.inv_perm, buf.w, buf.sigma, buf.y, stream)


def expert_work(cfg, offsets_list):
    """Algorithmic work of each FFN stage per launch, from the group offsets:
    bytes of the distinct experts touched (routed groups with rows, plus the
    shared expert) and flops per row.
      gate/up: codes 2 I H / 2, scales 2 I H / 16, two fp32 globals; 4 H I flops
      down:    codes H I / 2,   scales H I / 16,   one fp32 global;  2 H I flops
    MX blobs: scales per 32 values (2 I H / 32, H I / 32), no globals.
    Returns arrays (gu_bytes, dn_bytes, gu_flops, dn_flops)."""
    H, I = cfg.H, cfg.I
    gu_b, dn_b, gu_f, dn_f = [], [], [], []
    for off in offsets_list:
        o = off.cpu().numpy()
        active = int(np.count_nonzero(np.diff(o[:cfg.E + 1]))) + 1
        rows = int(o[cfg.E]) + cfg.T
        if cfg.fmt == "mx":
            gu_b.append(active * (I * H + I * H // 16))
            dn_b.append(active * (H * I // 2 + H * I // 32))
        else:
            gu_b.append(active * (I * H + I * H // 8 + 8))
            dn_b.append(active * (H * I // 2 + H * I // 16 + 4))
        gu_f.append(4.0 * H * I * rows)
        dn_f.append(2.0 * H * I * rows)
    return tuple(np.array(v, dtype=np.float64) for v in (gu_b, dn_b, gu_f, dn_f))


def cpu_baseline(cfg, seconds, threads=1):
    """Time the oracle (fp64 numpy, BLAS on `threads` threads) on a bounded
    sample of the workload: whole layers of step 0 for decode (all T tokens),
    a token sample for prefill; scaled to tokens/s of the full step."""
    from threadpoolctl import threadpool_limits

    from oracle import moe_oracle as O
    from synth import HostGen, zipf_logits

    gen = HostGen()
    mx = cfg.fmt == "mx"
    olay = O.mx_blob_layout(cfg.H, cfg.I) if mx else O.blob_layout(cfg.H, cfg.I)
    make_blob = gen.expert_blob_mx if mx else gen.expert_blob
    done_layers, t_oracle = 0, 0.0
    sample = ""
    with threadpool_limits(limits=threads):
        if cfg.T <= 64:
            for l in range(cfg.L):
                x = gen.x(cfg, l, 0)
                wsg = gen.w_shared_gate(cfg, l)
                kw = dict(w_router=gen.w_router(cfg, l)) if cfg.router == "matrix" else dict(
                    logits=zipf_logits(cfg, l, 0))
                lg = O.router_logits(O.bf16_bits_to_f64(x), kw["w_router"]) if "w_router" in kw else kw["logits"]
                need = set(O.topk(lg, cfg.k).reshape(-1).tolist()) | {cfg.E}
                blobs = {e: make_blob(cfg, l, e, olay) for e in need}   # generation is not timed
                t0 = time.perf_counter()
                O.moe_layer(x, lambda e: blobs[e], cfg.H, cfg.I, cfg.E, cfg.k, wsg, fmt=cfg.fmt, **kw)
                t_oracle += time.perf_counter() - t0
                done_layers += 1
                if t_oracle >= seconds:
                    break
            value = cfg.T / (t_oracle / done_layers * cfg.L)
            sample = "%d of %d layers of decode step 0 (all %d tokens each), oracle time %.1f s, scaled to the " \
                     "full %d-layer step" % (done_layers, cfg.L, cfg.T, t_oracle, cfg.L)
        else:
            l = 0
            x = gen.x(cfg, l, 0)
            wsg = gen.w_shared_gate(cfg, l)
            wr = gen.w_router(cfg, l) if cfg.router == "matrix" else None
            lgz = None if wr is not None else zipf_logits(cfg, l, 0)
            ntok = 16 if cfg.H * cfg.I <= 2048 * 512 else 4
            blob_cache = {}

            def blob(e):
                if e not in blob_cache:
                    blob_cache[e] = make_blob(cfg, l, e, olay)
                return blob_cache[e]
            lg = O.router_logits(O.bf16_bits_to_f64(x), wr) if wr is not None else lgz
            toks = list(range(ntok))
            for e in set(O.topk(lg[toks], cfg.k).reshape(-1).tolist()) | {cfg.E}:
                blob(e)
            t0 = time.perf_counter()
            O.moe_layer(x, blob, cfg.H, cfg.I, cfg.E, cfg.k, wsg, w_router=wr, logits=lgz, tokens=toks, fmt=cfg.fmt)
            t_oracle = time.perf_counter() - t0
            value = ntok / t_oracle
            sample = "layer 0, routing and grouping of all %d tokens plus expert FFN and combine of %d sampled " \
                     "tokens; oracle time %.1f s; rate = sampled tokens / time" % (cfg.T, ntok, t_oracle)
    return {"value": value, "unit": "tokens/s", "cores": threads, "kind": "oracle", "sample": sample}


def cpu_baselines(cfg, seconds):
    """The oracle timed on every host core this process may use, then on one
    thread; both core counts are stated."""
    cores = len(os.sched_getaffinity(0))
    log("timing the CPU oracle on a bounded sample (%d threads, then 1)" % cores)
    cpu = cpu_baseline(cfg, seconds, cores)
    one = cpu_baseline(cfg, seconds, 1)
    cpu["one_thread"] = {"value": one["value"], "cores": 1, "sample": one["sample"]}
    return cpu


PCIE_GEN5_X16_GBS = 64.0   # the host link's published rate per direction


def host_device_pointer(host_ptr):
    """The device-readable address of page-locked host memory (hipHostGetDevicePointer)."""
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_uint]
    out = ctypes.c_void_p()
    rc = hip.hipHostGetDevicePointer(ctypes.byref(out), ctypes.c_void_p(host_ptr), 0)
    assert rc == 0 and out.value, "hipHostGetDevicePointer failed (%d)" % rc
    return out.value


def run_cached(cfg, args, B, DevGen):
    """Decode through a device cache of expert blobs (partial residency).  Every
    (layer, expert) blob sits in page-locked host memory; the pool holds
    cache_frac of them.  Per layer: route, the residency update (LRU over
    (layer, expert)), the fill of the misses from host memory, group, FFN and
    combine, all captured in the step graphs.  Reports tokens/s and, from one
    more eager pass with HIP events, the hit rate, the blobs filled per step,
    the fill kernel's rate over the host link and the residency kernel's time."""
    import torch
    from moe_expert_ffn_top_amd.layer import LayerBuffers

    K, W = args.steps, args.warmup
    n_meas = min(K, 4)
    wl = Workload(cfg, W + K + n_meas, B, DevGen)   # the measured eager steps continue the sequence
    log("copying %.2f GB of blobs to page-locked host memory" % (wl.pool_bytes / 1e9))
    host = torch.empty(wl.pool_bytes, dtype=torch.uint8, pin_memory=True)
    host.copy_(wl.pool)
    torch.cuda.synchronize()
    del wl.pool
    torch.cuda.empty_cache()
    hptr = host_device_pointer(host.data_ptr())
    L, E1, d, lay = cfg.L, cfg.E1, wl.dims, wl.layout
    S = max(1, int(round(cfg.cache_frac * wl.n_slots)))
    pool = torch.zeros(S * lay.slot_stride, dtype=torch.uint8, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    table = torch.full((L, E1), -1, **i32)
    owner, last, clock = torch.full((S,), -1, **i32), torch.full((S,), -1, **i32), torch.zeros(1, **i32)
    fills, n_fill = torch.zeros((L, E1, 2), **i32), torch.zeros(L, **i32)
    buf = LayerBuffers.allocate(d)
    log("cache of %d of %d blobs (%.2f GB)" % (S, wl.n_slots, pool.numel() / 1e9))

    def run_step(step, ev=None):
        s = wl.input_index(step)
        for l in range(L):
            x = wl.x[s, l]
            B.moe_route(d, x, None, wl.logits[s, l], wl.wsg[l], None, buf.ids, buf.w, buf.sigma)
            if ev is not None:
                ev.append([torch.cuda.Event(enable_timing=True) for _ in range(3)])
                ev[-1][0].record()
            B.moe_residency_update(d, l, buf.ids, table, owner, last, S, clock, fills[l], n_fill[l:l + 1],
                                   buf.status)
            if ev is not None:
                ev[-1][1].record()
            B.moe_residency_fill(d, lay, hptr, pool, pool.numel(), S, fills[l], n_fill[l:l + 1])
            if ev is not None:
                ev[-1][2].record()
            B.moe_group(d, l, buf.ids, table, S, buf.offsets, buf.perm, buf.inv_perm, buf.group_slot, buf.status,
                        buf.ws)
            B.moe_expert_ffn(d, x, pool, pool.numel(), lay, buf.offsets, buf.perm, buf.group_slot, buf.h,
                             buf.y_rows, buf.status, buf.ws)
            B.moe_combine(d, buf.y_rows, buf.inv_perm, buf.w, buf.sigma, buf.y)

    graphs = []
    if not args.eager:
        log("capturing %d step graphs" % wl.n_inputs)
        for s in range(wl.n_inputs):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_step(s)
            graphs.append(g)
        torch.cuda.synchronize()
        # capture ran nothing: the cache starts cold at the first warm-up step

    def step(i):
        if graphs:
            graphs[wl.input_index(i)].replay()
        else:
            run_step(i)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    assert int(buf.status.item()) == 0, "device status %d after warmup" % int(buf.status.item())
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(K):
        step(W + i)
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / K
    tokens_per_s = cfg.T / (ms_per_step / 1e3)
    log("%.3f ms/step, %.1f tokens/s" % (ms_per_step, tokens_per_s))

    # eager steps with events: residency kernel time, fill time and bytes, hit rate
    res_ms, fill_ms, n_filled, n_needed = [], [], 0, 0
    for i in range(n_meas):
        ev = []
        run_step(W + K + i, ev)
        torch.cuda.synchronize()
        res_ms += [a.elapsed_time(b) for a, b, _ in ev]
        fill_ms += [b.elapsed_time(c) for _, b, c in ev]
        n_filled += int(n_fill.sum().item())
        s = wl.input_index(W + K + i)
        from synth import zipf_logits
        for l in range(L):
            ids = np.argsort(-zipf_logits(cfg, l, s), axis=1, kind="stable")[:, :cfg.k]
            n_needed += len(np.unique(ids)) + 1
    fill_bytes = n_filled * lay.blob_bytes
    fill_s = sum(fill_ms) * 1e-3
    fill_gbs = fill_bytes / fill_s / 1e9 if fill_s > 0 else 0.0
    residency = {"cache_slots": S, "blobs": wl.n_slots, "hit_rate": 1.0 - n_filled / max(1, n_needed),
                 "blobs_filled_per_step": n_filled / n_meas, "fill_gb_per_s": fill_gbs,
                 "fill_us_per_layer": float(np.mean(fill_ms) * 1e3),
                 "residency_update_us_per_layer": float(np.mean(res_ms) * 1e3)}
    log("residency: %s" % residency)
    roof = {"bound": "pcie", "achieved": fill_gbs, "peak": PCIE_GEN5_X16_GBS, "unit": "GB/s",
            "frac": fill_gbs / PCIE_GEN5_X16_GBS, "traffic": None,
            "kernel": "k_fill (moe_residency_fill), blob bytes filled / fill time",
            "peak_note": "host link: PCIe 5.0 x16 published rate per direction"}
    line = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded; random block-FP4 weights, bf16 activations)",
        "config": {"workload": cfg.name, "T": cfg.T, "layers": cfg.L, "H": cfg.H, "I": cfg.I, "E": cfg.E,
                   "k": cfg.k, "shared_experts": 1, "routing": "zipf s=%g, hot set moves every %d steps"
                   % (cfg.zipf_s, cfg.epoch_len), "cache_frac": cfg.cache_frac, "graphs": not args.eager,
                   "parallelism": "single GPU"},
        "roofline": roof, "residency": residency, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def run_hotcold(cfg, args, B, DevGen):
    """The hot/cold swap policy over the cached workload's routing (it measures
    the policy, not the layer: without a second place to compute misses, the
    experts out of the cache are not computed).  The cache starts with each
    layer's shared expert and its lowest-index experts.  Every step, each
    layer routes, groups and adds its routing counts to the heat; after the
    step one swap round runs (heat and table to the host, plan, plan to the
    device, apply, decay 0.7).  Reports the share of routed (layer, expert)
    uses whose expert was resident, swaps per round, the apply rate over the
    host link and the host planning time."""
    import torch
    from moe_expert_ffn_top_amd.layer import LayerBuffers

    K, W = args.steps, args.warmup
    wl = Workload(cfg, W + K, B, DevGen)
    log("copying %.2f GB of blobs to page-locked host memory" % (wl.pool_bytes / 1e9))
    host = torch.empty(wl.pool_bytes, dtype=torch.uint8, pin_memory=True)
    host.copy_(wl.pool)
    torch.cuda.synchronize()
    hptr = host_device_pointer(host.data_ptr())
    L, E, E1, d, lay = cfg.L, cfg.E, cfg.E1, wl.dims, wl.layout
    stride = lay.slot_stride
    S = max(L, int(round(cfg.cache_frac * wl.n_slots)))
    per = S // L
    table = np.full((L, E1), -1, np.int32)
    n = 0
    for l in range(L):
        for e in [E] + list(range(per - 1)):
            table[l, e] = n
            n += 1
    pool = torch.zeros(S * stride, dtype=torch.uint8, device="cuda")
    src = wl.pool.view(wl.n_slots, stride)
    for l in range(L):
        keys = [l * E1 + e for e in range(E1) if table[l, e] >= 0]
        slots = [int(table[l, e]) for e in range(E1) if table[l, e] >= 0]
        pool.view(S, stride)[torch.tensor(slots, device="cuda")] = src[torch.tensor(keys, device="cuda")]
    torch.cuda.synchronize()
    del wl.pool, src
    torch.cuda.empty_cache()
    t_dev = torch.from_numpy(table).cuda()
    heat = torch.zeros((L, E), dtype=torch.float32, device="cuda")
    buf = LayerBuffers.allocate(d)
    scratch = torch.zeros((96, 2), dtype=torch.int32, device="cuda")
    nsc = torch.zeros(1, dtype=torch.int32, device="cuda")
    log("cache of %d of %d blobs (%.2f GB), %d per layer at start" % (S, wl.n_slots, pool.numel() / 1e9, per))
    uses = hits = 0
    swaps, plan_ms, apply_ms = [], [], []
    for step in range(W + K):
        s = wl.input_index(step)
        for l in range(L):
            B.moe_route(d, wl.x[s, l], None, wl.logits[s, l], wl.wsg[l], None, buf.ids, buf.w, buf.sigma)
            B.moe_group(d, l, buf.ids, t_dev, S, buf.offsets, buf.perm, buf.inv_perm, buf.group_slot, buf.status,
                        buf.ws)
            B.moe_heat_update(d, l, buf.offsets, heat)
            if step >= W:
                ids = buf.ids.cpu().numpy()
                uses += ids.size
                hits += int((t_dev[l].cpu().numpy()[ids] >= 0).sum())
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        plan = B.moe_swap_plan(d, heat.cpu().numpy(), t_dev.cpu().numpy())
        t1 = time.perf_counter()
        if len(plan):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            p_dev = torch.from_numpy(plan).cuda()
            a.record()
            B.moe_swap_apply(d, lay, hptr, pool, pool.numel(), S, t_dev, p_dev, len(plan), scratch, nsc)
            b.record()
            torch.cuda.synchronize()
            if step >= W:
                apply_ms.append(a.elapsed_time(b))
        B.moe_heat_decay(d, heat, 0.7)
        if step >= W:
            swaps.append(len(plan))
            plan_ms.append((t1 - t0) * 1e3)
    moved = sum(swaps) * lay.blob_bytes
    apply_gbs = moved / (sum(apply_ms) * 1e-3) / 1e9 if apply_ms else 0.0
    pol = {"cache_slots": S, "blobs": wl.n_slots, "resident_share_of_routed_uses": hits / max(1, uses),
           "swaps_per_round": float(np.mean(swaps)), "apply_gb_per_s": apply_gbs,
           "apply_ms_per_round": float(np.mean(apply_ms)) if apply_ms else 0.0,
           "plan_ms_per_round": float(np.mean(plan_ms)), "round": "one per decode step, after all layers",
           "threshold": 1.5, "max_swaps": 96, "decay": 0.7}
    log("hot/cold: %s" % pol)
    line = {
        "metric": "hot/cold swap policy: share of routed (layer, expert) uses resident", "value": pol[
            "resident_share_of_routed_uses"], "unit": "fraction", "n_gpus": 1, "steps": K, "warmup": W,
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic (seeded; Zipf routing with a moving hot set)",
        "config": {"workload": cfg.name, "policy": "hotcold", "T": cfg.T, "layers": cfg.L, "E": cfg.E, "k": cfg.k,
                   "cache_frac": cfg.cache_frac, "parallelism": "single GPU"},
        "roofline": {"bound": "pcie", "achieved": apply_gbs, "peak": PCIE_GEN5_X16_GBS, "unit": "GB/s",
                     "frac": apply_gbs / PCIE_GEN5_X16_GBS, "traffic": None,
                     "kernel": "moe_swap_apply (k_fill of the round's swaps)"},
        "hotcold": pol,
    }
    print(json.dumps(line), flush=True)


def run_staged(cfg, args, B, DevGen):
    """The streamed workload: every layer's expert blobs sit in page-locked host
    memory and go through the two-slot device ring (copy stream) while the
    previous layer computes (compute stream).  A step is the whole L-layer
    stack.  Reports tokens/s, the H2D rate and the overlap fraction
    sum_l |compute_l n copy_(l+1)| / sum_l compute_l, beside the FFN roofline
    measured on a staged slot."""
    import torch
    from moe_expert_ffn_top_amd.staged import StagedLayers

    K, W = args.steps, args.warmup
    wl = Workload(cfg, 1, B, DevGen)
    log("copying %.2f GB of blobs to page-locked host memory" % (wl.pool_bytes / 1e9))
    host = torch.empty(wl.pool_bytes, dtype=torch.uint8, pin_memory=True)
    host.copy_(wl.pool)
    torch.cuda.synchronize()
    del wl.pool
    torch.cuda.empty_cache()
    copy_s, comp_s = torch.cuda.Stream(), torch.cuda.Stream()
    st = StagedLayers(wl.dims, wl.layout, host, cfg.L, copy_s, comp_s)

    def step(events=None):
        with torch.cuda.stream(comp_s):
            st.run(lambda l: wl.x[0, l], lambda l: wl.wsg[l], lambda l: wl.logits[0, l], layer_events=events)

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    assert int(st.buf.status.item()) == 0, "device status after warmup"
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / K
    tokens_per_s = cfg.T / (ms_per_step / 1e3)
    log("%.2f ms/step, %.1f tokens/s" % (ms_per_step, tokens_per_s))

    # the serial reference: one slot, copy then compute on one stream
    def serial_step():
        with torch.cuda.stream(comp_s):
            st.run_serial(lambda l: wl.x[0, l], lambda l: wl.wsg[l], lambda l: wl.logits[0, l])

    serial_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        serial_step()
    torch.cuda.synchronize()
    serial_ms = (time.perf_counter() - t0) * 1e3 / K
    serial = {"ms_per_step": serial_ms, "tokens_per_s": cfg.T / (serial_ms / 1e3),
              "ring_speedup": serial_ms / ms_per_step,
              "loss_without_second_buffer": ms_per_step / serial_ms - 1.0}
    log("serial (no ring): %s" % serial)

    # copy and compute intervals of one more step, on a common time base
    ev = []
    step(ev)
    torch.cuda.synchronize()
    ref = ev[0][0]
    iv = [tuple(ref.elapsed_time(e) for e in quad) for quad in ev]   # (copy0, copy1, comp0, comp1) per layer
    layer_gb = st.layer_bytes / 1e9
    copy_ms = np.array([c1 - c0 for c0, c1, _, _ in iv])
    comp_ms = np.array([k1 - k0 for _, _, k0, k1 in iv])
    inter = sum(max(0.0, min(iv[l][3], iv[l + 1][1]) - max(iv[l][2], iv[l + 1][0])) for l in range(len(iv) - 1))
    overlap = inter / max(1e-9, comp_ms[:-1].sum()) if len(iv) > 1 else 0.0
    h2d = {"layer_bytes": st.layer_bytes, "gb_per_s": float(layer_gb / (copy_ms.mean() * 1e-3)),
           "copy_ms_per_layer": float(copy_ms.mean()), "compute_ms_per_layer": float(comp_ms.mean()),
           "overlap_fraction": float(overlap)}
    log("h2d: %s" % h2d)

    # FFN roofline on a staged slot: stage layer 0, group it, time the two stages
    hev = HipEvents()
    d, buf = wl.dims, st.buf
    gu_ms, dn_ms, offs = [], [], []
    with torch.cuda.stream(comp_s):
        slot = B.moe_stage_h2d(st.ring, host.data_ptr(), st.layer_bytes)
        B.moe_ring_acquire(st.ring, slot, comp_s)
        pool = st.slots[slot]
        x = wl.x[0, 0]
        for rep in range(3):
            B.moe_route(d, x, None, wl.logits[0, 0], wl.wsg[0], None, buf.ids, buf.w, buf.sigma, comp_s)
            B.moe_group(d, 0, buf.ids, st.slot_table, cfg.E1, buf.offsets, buf.perm, buf.inv_perm, buf.group_slot,
                        buf.status, buf.ws, stream=comp_s)
            e = [hev.new() for _ in range(4)]
            for stg in (1, 2):
                B.moe_expert_ffn_stages(d, x, pool, st.layer_bytes, wl.layout, buf.offsets, buf.perm,
                                        buf.group_slot, buf.h, buf.y_rows, buf.status, buf.ws, stg, e[2 * stg - 2],
                                        e[2 * stg - 1], stream=comp_s)
            offs.append(buf.offsets.clone())
            comp_s.synchronize()
            gu_ms.append(hev.elapsed_ms(e[0], e[1]))
            dn_ms.append(hev.elapsed_ms(e[2], e[3]))
        B.moe_ring_release(st.ring, slot, comp_s)
    torch.cuda.synchronize()
    hev.close()
    st.close()
    gu_ms, dn_ms = np.array(gu_ms), np.array(dn_ms)
    gu_b, dn_b, gu_f, dn_f = expert_work(cfg, offs)
    achieved = float(gu_f.mean() / (gu_ms.mean() * 1e-3) / 1e12)
    roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved / BF16_PEAK_TFLOPS, "traffic": None,
            "kernel": "%s gate/up (moe_expert_ffn_stages, stages=1) on a staged slot" % ffn_kernel(cfg)[0],
            "launch_us": float(gu_ms.mean() * 1e3), "flops_per_launch": float(gu_f.mean()),
            "down": {"launch_us": float(dn_ms.mean() * 1e3), "flops_per_launch": float(dn_f.mean()),
                     "achieved": float(dn_f.mean() / (dn_ms.mean() * 1e-3) / 1e12)},
            "kernel_source_sha256_16": kernel_source_hash(cfg)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baselines(cfg, args.cpu_baseline_seconds)
    line = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded; random block-FP4 weights, bf16 activations)",
        "config": {"workload": cfg.name, "T": cfg.T, "layers": cfg.L, "H": cfg.H, "I": cfg.I, "E": cfg.E,
                   "k": cfg.k, "shared_experts": 1, "routing": "zipf s=%g" % cfg.zipf_s,
                   "staging": "pinned host blobs through a two-slot device ring", "graphs": False,
                   "parallelism": "single GPU"},
        "roofline": roof, "h2d": h2d, "serial": serial, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def measure_probes(B):
    """Measured peaks beside the spec ones: the best HBM read rate of the
    stream-read probe over launch shapes, and the dense MFMA rate of
    back-to-back bf16, fp8 x fp4 and fp8 MFMAs (moe_probe_*)."""
    import torch
    n = 8 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1 << 20, dtype=torch.float32, device="cuda")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    read = {}
    for grid in (1024, 2048, 4096, 8192):
        ms = timed(lambda: B.moe_probe_hbm_read(buf, n, grid, sink), 5)
        read[grid] = n / (ms * 1e-3) / 1e9
    best = max(read, key=read.get)
    out = {"hbm_read_gb_s": read[best], "hbm_read_grid": best, "hbm_read_bytes": n,
           "hbm_read_frac_of_spec": read[best] / HBM_PEAK_GBS}
    del buf
    iters = 4000
    for kind, name, flop, spec in ((0, "mfma_bf16", 32768, BF16_PEAK_TFLOPS), (1, "mfma_f8f4", 65536, FP8_PEAK_TFLOPS),
                                   (2, "mfma_f8", 65536, FP8_PEAK_TFLOPS)):
        best_t = 0.0
        for grid in (1024, 2048):
            ms = timed(lambda: B.moe_probe_mfma(kind, grid, iters, sink), 3)
            best_t = max(best_t, grid * 4 * iters * 4 * flop / (ms * 1e-3) / 1e12)
        out[name + "_tflops"] = best_t
        out[name + "_frac_of_spec"] = best_t / spec
    out["kernel_source_sha256_16"] = source_hash(os.path.join(CSRC, "probes.hip"))
    log("probes: %s" % out)
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build runs the MoE layer on a single MI355X and has no "
              "multi-GPU path (requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied %d bytes five times" % n)
        return
    from moe_expert_ffn_top_amd import binding as B
    from synth import DevGen, config_by_name

    if args.probes:
        print(json.dumps({"probes": measure_probes(B)}), flush=True)
        return
    cfg = config_by_name(args.config)
    if cfg.staged:
        run_staged(cfg, args, B, DevGen)
        return
    if cfg.cache_frac > 0:
        (run_hotcold if args.policy == "hotcold" else run_cached)(cfg, args, B, DevGen)
        return
    K, W = args.steps, args.warmup
    res = measure_workload(cfg, args, B, DevGen, K, W, ffn=args.ffn)
    extra = {}
    if cfg.name == "decode48" and not args.no_extra:
        # the other headline configurations, measured in the same run
        torch.cuda.empty_cache()
        pf = measure_workload(config_by_name("prefill8192"), args, B, DevGen, 10, 3, ffn=args.ffn)
        extra["prefill8192"] = summarize(pf)
        torch.cuda.empty_cache()
        dc = measure_workload(config_by_name("decode43x64"), args, B, DevGen, 64, 3, ffn=args.ffn, per_step=True)
        extra["decode43x64"] = summarize(dc)
        torch.cuda.empty_cache()
        extra["probes"] = measure_probes(B)
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baselines(cfg, args.cpu_baseline_seconds)

    line = {
        "metric": METRIC, "value": res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("mxfp8 x mxfp4" if cfg.T * cfg.k >= 16 * cfg.E else "bf16 (mxfp8 x mxfp4 values)")
        if cfg.fmt == "mx" else "bf16",
        "data": "synthetic (seeded; random MXFP4 weights, bf16 activations quantised to MXFP8)" if cfg.fmt == "mx"
        else "synthetic (seeded; random block-FP4 weights, bf16 activations)",
        "config": res["config"],
        "roofline": res["roof"], "cpu_baseline": cpu,
    }
    line.update(extra)
    print(json.dumps(line), flush=True)


def routed_shape(cfg):
    """The shapes whose routing moe_route_group_ffn(_mx) runs in one launch with
    the FFN's first step: weight streaming (T k < 16 E), T <= 16, T k <= 256,
    E <= 1024."""
    return cfg.T * cfg.k < 16 * cfg.E and cfg.T <= 16 and cfg.T * cfg.k <= 256 and cfg.E <= 1024


def ffn_label(cfg, ffn):
    """The FFN path a workload runs (Workload's choice, from the shapes)."""
    if cfg.T * cfg.k >= 16 * cfg.E:
        return "grouped GEMM"
    if ffn in ("routed", "routed-dc", "layer") and not (cfg.router == "zipf" and routed_shape(cfg)):
        return "split"
    if ffn == "layer" and (cfg.fmt == "mx" or cfg.k > 16):
        return "routed"
    if ffn == "routed-dc" and cfg.fmt == "mx":
        return "routed"
    return ffn


def workload_config(cfg, args, ffn):
    return {"workload": cfg.name, "T": cfg.T, "layers": cfg.L, "H": cfg.H, "I": cfg.I, "E": cfg.E,
            "k": cfg.k, "shared_experts": 1,
            "routing": ("zipf s=%g" % cfg.zipf_s) if cfg.router == "zipf" else "router matrix",
            "graphs": not args.eager, "ffn": ffn_label(cfg, ffn),
            "parallelism": "single GPU"}


def summarize(res):
    """The sub-object of an extra configuration on the bench line."""
    out = {"tokens_per_s": res["tokens_per_s"], "ms_per_step": res["ms_per_step"], "steps": res["steps"],
           "config": res["config"], "roofline": res["roof"]}
    if "step_ms" in res:
        v = np.array(res["step_ms"])
        out["step_ms_p50"] = float(np.percentile(v, 50))
        out["step_ms_p90"] = float(np.percentile(v, 90))
        out["expert_gb_per_step"] = res["expert_bytes_per_step"] / 1e9
        out["expert_gb_per_s"] = res["expert_bytes_per_step"] / (out["step_ms_p50"] * 1e-3) / 1e9
        out["expert_frac_of_hbm_peak"] = out["expert_gb_per_s"] / HBM_PEAK_GBS
    return out


def measure_workload(cfg, args, B, DevGen, K, W, ffn="split", per_step=False):
    """Time K steps of a workload (after W warm-up steps) with every step's
    inputs resident in HBM, each step one captured HIP graph (unless --eager);
    then the roofline of its dominant kernel from HIP events around its
    launches on their stream.  per_step: also each step's own time (HIP events
    around each replay) and the expert-weight bytes a step reads."""
    import torch
    wl = Workload(cfg, W + K, B, DevGen, ffn=ffn)
    graphs = []
    if not args.eager:
        log("%s: capturing %d step graphs" % (cfg.name, min(W + K, wl.n_inputs)))
        for s in range(min(W + K, wl.n_inputs)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                wl.run_step(s)
            graphs.append(g)
        torch.cuda.synchronize()

    def step(i):
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            wl.run_step(i)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    status = int(wl.buf.status.item())
    assert status == 0, "device status %d after warmup" % status
    res = {"steps": K, "config": workload_config(cfg, args, ffn)}
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if per_step:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        t0.record()
        for i in range(K):
            ev[i][0].record()
            step(W + i)
            ev[i][1].record()
        t1.record()
        torch.cuda.synchronize()
        res["step_ms"] = [a.elapsed_time(b) for a, b in ev]
    else:
        t0.record()
        for i in range(K):
            step(W + i)
        t1.record()
        torch.cuda.synchronize()
    res["ms_per_step"] = t0.elapsed_time(t1) / K
    res["tokens_per_s"] = cfg.T / (res["ms_per_step"] / 1e3)
    log("%s: %.4f ms/step, %.1f tokens/s" % (cfg.name, res["ms_per_step"], res["tokens_per_s"]))

    # roofline of the dominant kernel: HIP events around its launches on their stream
    events = []
    hev = HipEvents()
    for i in range(min(K, 8)):
        wl.run_step(W + i, ffn_events=events, hip_events=hev)
    torch.cuda.synchronize()
    if wl.one_launch or wl.layer_launch:
        fu_ms = np.array([hev.elapsed_ms(ev[0], ev[1]) for ev, _ in events])
    else:
        gu_ms = np.array([hev.elapsed_ms(ev[0], ev[1]) for ev, _ in events])
        dn_ms = np.array([hev.elapsed_ms(ev[2], ev[3]) for ev, _ in events])
    hev.close()
    gu_b, dn_b, gu_f, dn_f = expert_work(cfg, [o for _, o in events])
    decode = cfg.T * cfg.k < 16 * cfg.E
    if per_step:
        # expert-weight bytes of a whole step: every layer's distinct experts
        offs = []
        for i in range(min(K, 4)):
            lay_ev = []
            hev2 = HipEvents()
            wl.run_step(W + i, ffn_events=lay_ev, hip_events=hev2)
            torch.cuda.synchronize()
            hev2.close()
            g2, d2, _, _ = expert_work(cfg, [o for _, o in lay_ev])
            offs.append(float(g2.sum() + d2.sum()))
        res["expert_bytes_per_step"] = float(np.mean(offs))
    if wl.one_launch or wl.layer_launch:
        # the dominant kernel: gate/up, down and combine (and, for the layer
        # launch, the routing) in one launch; its algorithmic bytes are the
        # expert weights it streams (both stages)
        fu_b = gu_b + dn_b
        achieved = float(fu_b.mean() / (fu_ms.mean() * 1e-3) / 1e9)
        kname = ("k_layer_dec (moe_route_group_ffn_combine: route, group, gate/up, down and combine in one launch)"
                 if wl.layer_launch else
                 "k_ffn_dec_fused (moe_expert_ffn_combine: gate/up, down and combine in one launch)")
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(cfg, layer=wl.layer_launch),
                "kernel": kname,
                "launch_us": float(fu_ms.mean() * 1e3), "bytes_per_launch": float(fu_b.mean()),
                "bytes": "expert-weight bytes of the distinct experts touched: gate/up %.0f + down %.0f" % (
                    gu_b.mean(), dn_b.mean())}
    elif decode:
        achieved = float(gu_b.mean() / (gu_ms.mean() * 1e-3) / 1e9)
        if wl.routed and cfg.fmt == "mx":
            kname = "%s gate/up (moe_route_group_ffn_mx, stages=1: x quantised in the route + group launch)" % (
                ffn_kernel(cfg)[0])
        elif wl.routed:
            kname = "%s gate/up with the routing in its launch (moe_route_group_ffn, stages=1)" % ffn_kernel(cfg)[0]
        else:
            kname = "%s gate/up (%s, stages=1)" % (
                ffn_kernel(cfg)[0], "moe_expert_ffn_mx" if cfg.fmt == "mx" else "moe_expert_ffn_stages")
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(cfg),
                "kernel": kname,
                "launch_us": float(gu_ms.mean() * 1e3), "bytes_per_launch": float(gu_b.mean()),
                "down": {"launch_us": float(dn_ms.mean() * 1e3), "bytes_per_launch": float(dn_b.mean()),
                         "achieved": float(dn_b.mean() / (dn_ms.mean() * 1e-3) / 1e9)}}
        if wl.down_combine:
            roof["down"]["kernel"] = ("k_down_comb (moe_expert_ffn_down_combine: the down stage and the combine in "
                                      "one launch; launch_us includes the combine)")
    else:
        achieved = float(gu_f.mean() / (gu_ms.mean() * 1e-3) / 1e12)
        peak = FP8_PEAK_TFLOPS if cfg.fmt == "mx" else BF16_PEAK_TFLOPS
        entry = "moe_expert_ffn_mx" if cfg.fmt == "mx" else "moe_expert_ffn_stages"
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": None,
                "kernel": "%s gate/up (%s, stages=1)" % (ffn_kernel(cfg)[0], entry),
                "launch_us": float(gu_ms.mean() * 1e3), "flops_per_launch": float(gu_f.mean()),
                "down": {"launch_us": float(dn_ms.mean() * 1e3), "flops_per_launch": float(dn_f.mean()),
                         "achieved": float(dn_f.mean() / (dn_ms.mean() * 1e-3) / 1e12)}}
    roof["kernel_source_sha256_16"] = kernel_source_hash(cfg)
    log("%s roofline: %s" % (cfg.name, roof))
    res["roof"] = roof
    del graphs, wl
    return res


if __name__ == "__main__":
    main()

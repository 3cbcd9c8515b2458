#!/usr/bin/env python3
"""Benchmark of the DiffQKV decode hot path on one MI355X.

One step = one decode step of the workload: the newest K/V row of every
sequence is appended to the caches and attended together with the earlier
rows (the path's store, split and combine steps; the append is fused into the
split kernel, so a step is two kernels).  Inputs are seeded synthetic
caches, resident in HBM before timing starts.  Each step attends a different
replica of the caches (standing for successive layers) so that the replicas
together exceed the 256 MB Infinity Cache several times over and the timing
reflects HBM, not the last-level cache.

The timed steps are captured once in a HIP graph and replayed (the launch
rate from Python would otherwise bound the step).  The roofline's kernel
duration comes from a graph of that kernel alone, timed the same way.  HBM
traffic per launch is read from the committed rocprofv3 counter summary in
profiles/ when that summary was taken from the current kernel source.

Prints one JSON line.  ``value`` is the algorithmic HBM bytes of a step
(sum over sequences of ctx_len * (n_k d_k + n_v d_v) * element size, plus q,
out and the appended rows) divided by the measured step time.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode µs/step & achieved HBM GB/s (% of peak) at 32k/64k ctx, 1 MI355X"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode32k_asym")
    p.add_argument("--twin", default=None,
                   help="symmetric workload timed for the speedup (default: by workload)")
    p.add_argument("--no-twin", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--chunk", type=int, default=0, help="decode chunk rows (0 = auto)")
    p.add_argument("--eager", action="store_true", help="time eager launches, no graph")
    p.add_argument("--selective-k", type=int, default=100,
                   help="top_k of the selective-V decode leg (0 = skip it)")
    p.add_argument("--page-rows", type=int, default=64,
                   help="page size of the paged-cache leg (0 = skip it)")
    p.add_argument("--no-compat", action="store_true",
                   help="skip the kv_group_sharing leg")
    p.add_argument("--no-augq", action="store_true", help="skip the augmented-Q leg")
    p.add_argument("--no-workloads", action="store_true",
                   help="skip the other decode workloads (64k x 4 at d_k 64 / 128 and "
                        "symmetric, the ragged batch, the tiny fp32 case)")
    p.add_argument("--no-ket", action="store_true",
                   help="skip the KET replica (SIGMA-1.5B vs standard GQA, prefixes 2k-32k)")
    p.add_argument("--kernel-only", action="store_true",
                   help="only run steps (for profilers); skip twin, prefill, CPU baseline")
    p.add_argument("--ket", action="store_true",
                   help="only run the kernel-execution-time comparison of the pages' SIGMA-1.5B "
                        "and standard GQA attention shapes at prefixes 2k-32k and exit")
    p.add_argument("--only-augq", action="store_true",
                   help="only run the augmented-Q leg (1, 16 and 2048 tokens) and exit")
    p.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                   help="only run a plain device copy of BYTES bytes three times (calibrates "
                        "the HBM byte counters of a profiler) and exit")
    return p.parse_args()


def kv_elements_per_token(n_k: int, d_k: int, n_v: int, d_v: int) -> int:
    """Cache elements one token adds: n_k*d_k + n_v*d_v (the per-token factor
    of the KV-cache cost model, Eq. (1) of the Pith review page)."""
    return n_k * d_k + n_v * d_v


TWINS = {"decode32k_asym": "decode32k_sym", "decode64k_dk64": "decode64k_sym",
         "decode64k_dk128": "decode64k_sym"}

# Decode workloads measured beside the headline one in the default run (each
# is also a full-size parity case of the GPU tests).
OTHER_WORKLOADS = ("decode64k_dk64", "decode64k_dk128", "decode64k_sym", "ragged16",
                   "tiny_f32")


# ----------------------------------------------------------------- device side

class DecodeBench:
    """Device buffers and raw C-ABI argument tuples for one decode workload."""

    def __init__(self, name: str, chunk: int = 0):
        import numpy as np
        import torch

        import asymmetric_head_kv_amd as dq
        import synth

        self.torch, self.dq = torch, dq
        self.lib = dq.load()
        self.name = name
        wl = synth.workload(name)
        append_lens = name == "ragged16"
        case = synth.make_case(**wl)
        self.case = case
        B, n_q, n_k, n_v, d_k, d_v = (case.batch, case.n_q, case.n_k, case.n_v,
                                      case.d_k, case.d_v)
        self.shape = (n_q, n_k, n_v, d_k, d_v)
        self.B, self.l_cap = B, case.l_cap
        esize = 2 if case.dtype == "bf16" else 4
        self.esize = esize
        self.dtype_code = dq.BF16 if case.dtype == "bf16" else dq.F32
        if append_lens:   # cache holds ctx_len rows; append one, attend ctx_len + 1
            pos = np.asarray(case.ctx_len, dtype=np.int64)
            ctx = pos + 1
        else:             # the newest of ctx_len rows is (re)written by the append
            ctx = np.asarray(case.ctx_len, dtype=np.int64)
            pos = ctx - 1
        self.ctx = ctx
        self.max_ctx = int(ctx.max())
        k_new, v_new = synth.new_rows(wl["seed"], dtype=case.dtype, batch=B, t_new=1, n_k=n_k,
                                      n_v=n_v, d_k=d_k, d_v=d_v)
        dev = "cuda"

        def up(a):
            if case.dtype == "bf16":
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                    torch.bfloat16).to(dev)
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        self.q = up(case.q)
        k0, v0 = up(case.k_cache), up(case.v_cache)
        self.k_new, self.v_new = up(k_new), up(v_new)
        self.pos = torch.from_numpy(pos.astype(np.int32)).to(dev)
        self.ctx_t = torch.from_numpy(ctx.astype(np.int32)).to(dev)
        beta = kv_elements_per_token(n_k, d_k, n_v, d_v) * esize
        self.cache_bytes_attended = int(ctx.sum()) * beta
        self.alg_bytes_split = self.cache_bytes_attended + B * n_q * d_k * esize
        self.alg_bytes_step = (self.alg_bytes_split + B * n_q * d_v * esize
                               + B * beta)  # + out + appended rows
        footprint = (k0.numel() + v0.numel()) * esize
        self.replicas = max(2, min(16, math.ceil(4 * MALL_BYTES / max(1, footprint))))
        self.caches = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(self.replicas - 1)]
        self.out = torch.empty((B, n_q, d_v), dtype=self.q.dtype, device=dev)
        self.lse = torch.empty((B, n_q), dtype=torch.float32, device=dev)
        self.chunk = chunk
        self.ws_bytes = dq.decode_workspace_bytes(*self.shape, B, self.max_ctx, chunk)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.S = chunk or dq.decode_chunk(*self.shape, B, self.max_ctx)
        self.flops = 2 * n_q * (d_k + d_v) * int(ctx.sum())

    def _stream(self):
        return self.torch.cuda.current_stream().cuda_stream

    def append(self, r):
        """Standalone kv_append of the step's new rows (not part of a step)."""
        k, v = self.caches[r]
        st = self.lib.kv_append(*self.shape, self.dtype_code, self.B, 1, self.l_cap,
                                self.k_new.data_ptr(), self.v_new.data_ptr(),
                                self.pos.data_ptr(), k.data_ptr(), v.data_ptr(),
                                self._stream())
        assert st == 0, st

    def split(self, r):
        """Split kernel with the fused append of the newest row."""
        k, v = self.caches[r]
        st = self.lib.diffqkv_decode_split(
            *self.shape, self.dtype_code, self.B, self.l_cap, self.max_ctx, self.case.scale,
            self.q.data_ptr(), self.k_new.data_ptr(), self.v_new.data_ptr(), k.data_ptr(),
            v.data_ptr(), self.ctx_t.data_ptr(), self.chunk, self.ws.data_ptr(),
            self.ws_bytes, self._stream())
        assert st == 0, st

    def combine(self):
        st = self.lib.diffqkv_decode_combine(
            *self.shape, self.dtype_code, self.B, self.l_cap, self.max_ctx,
            self.ctx_t.data_ptr(), self.out.data_ptr(), self.lse.data_ptr(), self.chunk,
            self.ws.data_ptr(), self.ws_bytes, self._stream())
        assert st == 0, st

    def setup_selective(self, top_k: int):
        """Buffers of a selective-V decode step (diffqkv_decode_selective)."""
        torch, dq = self.torch, self.dq
        self.top_k = top_k
        self.sel_ws_bytes = dq.selective_workspace_bytes(*self.shape, self.B, self.max_ctx, top_k)
        self.sel_ws = torch.empty(self.sel_ws_bytes, dtype=torch.uint8, device="cuda")
        self.sel_out = torch.empty_like(self.out)
        n_q, n_k, n_v, d_k, d_v = self.shape
        kk = sum(min(top_k, int(L)) for L in self.ctx)
        self.sel_alg_bytes = (int(self.ctx.sum()) * n_k * d_k * self.esize   # all of K
                              + n_q * kk * d_v * self.esize                   # chosen V rows
                              + self.B * n_q * (d_k + d_v) * self.esize      # q, out
                              + self.B * (n_k * d_k + n_v * d_v) * self.esize)  # appended rows
        self.sel_ws_traffic = 2 * n_q * int(self.ctx.sum()) * 4   # logits written, re-read

    def setup_paged(self, page_rows: int, seed: int = 0):
        """Paged copies of every cache replica: each sequence's blocks of
        page_rows rows go to pages in a seeded random order."""
        torch = self.torch
        P = page_rows
        B, cap = self.B, self.l_cap
        nblk = -(-cap // P)
        g = torch.Generator().manual_seed(seed)
        perm = torch.randperm(B * nblk, generator=g)
        inv = torch.empty_like(perm)
        inv[perm] = torch.arange(B * nblk)
        self.page_rows, self.max_blocks, self.num_pages = P, nblk, B * nblk
        self.block_table = inv.view(B, nblk).to(torch.int32).to("cuda")

        def to_pages(c):
            b_, h, _, d = c.shape
            x = torch.zeros((b_, h, nblk * P, d), dtype=c.dtype, device="cuda")
            x[:, :, :cap] = c
            x = x.view(b_, h, nblk, P, d).permute(0, 2, 1, 3, 4).reshape(b_ * nblk, h, P, d)
            return x[perm.to("cuda")].contiguous()

        self.pages = [(to_pages(k), to_pages(v)) for k, v in self.caches]

    def paged_step(self, r):
        """The decode step (fused append + split + combine) over paged caches."""
        kp, vp = self.pages[r]
        st = self.lib.diffqkv_decode_paged(
            *self.shape, self.dtype_code, self.B, self.page_rows, self.num_pages,
            self.max_blocks, self.max_ctx, self.case.scale, self.q.data_ptr(),
            self.k_new.data_ptr(), self.v_new.data_ptr(), kp.data_ptr(), vp.data_ptr(),
            self.block_table.data_ptr(), self.ctx_t.data_ptr(), self.out.data_ptr(),
            self.lse.data_ptr(), self.chunk, self.ws.data_ptr(), self.ws_bytes, self._stream())
        assert st == 0, st

    def paged_selective_step(self, r):
        """The selective-V step (fused append, logits, top-k, V gather) over
        paged caches (after setup_selective and setup_paged)."""
        kp, vp = self.pages[r]
        st = self.lib.diffqkv_decode_selective_paged(
            *self.shape, self.dtype_code, self.B, self.page_rows, self.num_pages,
            self.max_blocks, self.max_ctx, self.case.scale, self.top_k, self.q.data_ptr(),
            self.k_new.data_ptr(), self.v_new.data_ptr(), kp.data_ptr(), vp.data_ptr(),
            self.block_table.data_ptr(), self.ctx_t.data_ptr(), self.sel_out.data_ptr(),
            self.lse.data_ptr(), None, self.sel_ws.data_ptr(), self.sel_ws_bytes, self._stream())
        assert st == 0, st

    def setup_compat(self):
        """kv_group_sharing copies of every replica (n_h = max(n_k, n_v) heads
        on both sides) and the time of one expansion."""
        torch, dq = self.torch, self.dq
        self.compat = []
        for k, v in self.caches:
            self.compat.append(dq.kv_group_sharing(k, v, n_q=self.shape[0]))
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        k, v = self.caches[0]
        t0.record()
        for _ in range(5):
            dq.kv_group_sharing(k, v, n_q=self.shape[0])
        t1.record()
        torch.cuda.synchronize()
        self.compat_expand_ms = t0.elapsed_time(t1) / 5
        n_q, n_k, n_v, d_k, d_v = self.shape
        n_h = max(n_k, n_v)
        self.compat_shape = (n_q, n_h, n_h, d_k, d_v)
        self.compat_ws_bytes = dq.decode_workspace_bytes(*self.compat_shape, self.B,
                                                         self.max_ctx, self.chunk)
        self.compat_ws = torch.empty(self.compat_ws_bytes, dtype=torch.uint8, device="cuda")
        kn = self.k_new.view(self.B, n_k, d_k)
        idx = torch.tensor([h * n_k // n_h for h in range(n_h)], device="cuda")
        self.compat_k_new = kn[:, idx].contiguous()
        vn = self.v_new.view(self.B, n_v, d_v)
        idx = torch.tensor([h * n_v // n_h for h in range(n_h)], device="cuda")
        self.compat_v_new = vn[:, idx].contiguous()

    def compat_step(self, r):
        """The decode step on the kv_group_sharing layout."""
        k, v = self.compat[r]
        st = self.lib.diffqkv_decode_append(
            *self.compat_shape, self.dtype_code, self.B, self.l_cap, self.max_ctx,
            self.case.scale, self.q.data_ptr(), self.compat_k_new.data_ptr(),
            self.compat_v_new.data_ptr(), k.data_ptr(), v.data_ptr(), self.ctx_t.data_ptr(),
            self.out.data_ptr(), self.lse.data_ptr(), self.chunk, self.compat_ws.data_ptr(),
            self.compat_ws_bytes, self._stream())
        assert st == 0, st

    def selective_step(self, r):
        """One decode step with selective V: append, logits, top-k, gather."""
        k, v = self.caches[r]
        st = self.lib.diffqkv_decode_selective(
            *self.shape, self.dtype_code, self.B, self.l_cap, self.max_ctx, self.case.scale,
            self.top_k, self.q.data_ptr(), self.k_new.data_ptr(), self.v_new.data_ptr(),
            k.data_ptr(), v.data_ptr(), self.ctx_t.data_ptr(), self.sel_out.data_ptr(),
            self.lse.data_ptr(), None, self.sel_ws.data_ptr(), self.sel_ws_bytes, self._stream())
        assert st == 0, st

    def step(self, r):
        """One decode step: append + attend + merge (diffqkv_decode_append)."""
        k, v = self.caches[r]
        st = self.lib.diffqkv_decode_append(
            *self.shape, self.dtype_code, self.B, self.l_cap, self.max_ctx, self.case.scale,
            self.q.data_ptr(), self.k_new.data_ptr(), self.v_new.data_ptr(), k.data_ptr(),
            v.data_ptr(), self.ctx_t.data_ptr(), self.out.data_ptr(), self.lse.data_ptr(),
            self.chunk, self.ws.data_ptr(), self.ws_bytes, self._stream())
        assert st == 0, st

    # -- timing -------------------------------------------------------------

    def time_steps(self, steps: int, warmup: int, eager: bool = False, fn=None):
        """Average ms per step over exactly `steps` steps (graph replay)."""
        torch = self.torch
        R = self.replicas
        fn = fn or self.step
        for w in range(warmup):
            fn(w % R)
        torch.cuda.synchronize()
        graphs = {}
        if not eager:
            try:
                for n in {R, steps % R} - {0}:
                    graphs[n] = self._graph(fn, n)
                for g in graphs.values():  # warm replays
                    g.replay()
                torch.cuda.synchronize()
            except Exception as e:  # fall back to eager timing
                log(f"graph capture failed ({e}); timing eager launches")
                graphs = {}
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        if graphs:
            for _ in range(steps // R):
                graphs[R].replay()
            if steps % R:
                graphs[steps % R].replay()
        else:
            for s in range(steps):
                fn(s % R)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        # Spread: each replay of R steps timed alone (untimed above), per-step
        # median and 10th / 90th percentiles.
        self.step_pct_us = None
        if graphs and R in graphs:
            n = max(10, min(100, steps // R))
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
            ev[0].record()
            for k in range(n):
                graphs[R].replay()
                ev[k + 1].record()
            torch.cuda.synchronize()
            per = sorted(ev[k].elapsed_time(ev[k + 1]) * 1e3 / R for k in range(n))
            pick = lambda f: round(per[min(n - 1, int(f * (n - 1) + 0.5))], 2)
            self.step_pct_us = {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9),
                                "replays": n, "steps_per_replay": R}
        return ms, bool(graphs)

    def _graph(self, fn, n):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(0)
        torch.cuda.current_stream().wait_stream(s)
        with torch.cuda.graph(g):
            for r in range(n):
                fn(r)
        return g

    def time_kernels(self, steps: int):
        """Average duration (ms) of the split kernel and of the combine kernel,
        each timed alone: a graph of back-to-back launches of that kernel
        (cycling over the cache replicas, at least 16 launches so that a replay
        outlasts its submission from the host), replayed between two events
        on the launch stream."""
        torch = self.torch
        R = max(16, self.replicas)
        out = []
        for fn in (lambda r: self.split(r % self.replicas), lambda r: self.combine()):
            g = self._graph(fn, R)
            g.replay()
            torch.cuda.synchronize()
            reps = max(1, steps // R)
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(reps):
                g.replay()
            t1.record()
            torch.cuda.synchronize()
            out.append(t0.elapsed_time(t1) / (reps * R))
        return out

    def free(self):
        self.caches = None
        self.torch.cuda.empty_cache()


PMC_SUMMARY = os.path.join(ROOT, "profiles", "decode_split_kernel_{}_pmc.txt")
KERNEL_SOURCES = ("asymmetric_head_kv_amd/csrc/decode.hip",
                  "asymmetric_head_kv_amd/csrc/device_common.h")


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def pmc_traffic(workload: str):
    """HBM bytes per split launch from the committed counter summary, or
    None when there is none or it was taken from other kernel sources."""
    path = PMC_SUMMARY.format(workload)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def decode_record(name: str, steps: int, warmup: int, chunk: int = 0,
                  selective_k: int = 0) -> dict:
    """Step time (split with the fused append + combine, graph replay over
    cache replicas) and the split kernel alone, for one decode workload; with
    selective_k > 0 also the selective-V step on the same caches."""
    bn = DecodeBench(name, chunk)
    ms, graphed = bn.time_steps(steps, warmup)
    spread = bn.step_pct_us
    split_ms, comb_ms = bn.time_kernels(steps)
    sel = None
    if selective_k > 0:
        bn.setup_selective(selective_k)
        ms_sel, _ = bn.time_steps(steps, warmup, fn=bn.selective_step)
        sel = {"top_k": selective_k, "us_per_step": round(ms_sel * 1e3, 2),
               "alg_bytes_per_step": bn.sel_alg_bytes,
               "GBps": round(bn.sel_alg_bytes / (ms_sel * 1e-3) / 1e9, 1),
               "speedup_over_full_decode": round(ms / ms_sel, 3)}
    n_q, n_k, n_v, d_k, d_v = bn.shape
    gbs = bn.alg_bytes_step / (ms * 1e-3) / 1e9
    split_gbs = bn.alg_bytes_split / (split_ms * 1e-3) / 1e9
    rec = {"us_per_step": round(ms * 1e3, 2), "GBps": round(gbs, 1),
           "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
           "us_per_step_spread": spread,
           "alg_bytes_per_step": bn.alg_bytes_step,
           "split_us": round(split_ms * 1e3, 2), "combine_us": round(comb_ms * 1e3, 2),
           "split_GBps": round(split_gbs, 1),
           "split_frac_of_hbm_peak": round(split_gbs / HBM_PEAK_GBS, 4),
           "split_alg_bytes_per_launch": bn.alg_bytes_split,
           "split_traffic": pmc_traffic(name),
           "dtype": bn.case.dtype,
           "shape": {"batch": bn.B, "max_ctx": bn.max_ctx, "ctx_sum": int(bn.ctx.sum()),
                     "n_q": n_q, "n_k": n_k, "n_v": n_v, "d_k": d_k, "d_v": d_v},
           "chunk_rows": bn.S, "cache_replicas": bn.replicas,
           "timing": "hip graph replay" if graphed else "eager launches"}
    if sel is not None:
        rec["selective_v"] = sel
    bn.free()
    del bn
    return rec


def ket_replica(steps: int):
    """Split- and combine-kernel times (each timed alone, graph replay) and
    their sum, for SIGMA-1.5B vs the standard GQA shape, with the relative
    improvement (STD - SIGMA) / STD the pages report per prefix length."""
    import synth
    rows = []
    for prefix in synth.KET_PREFIXES:
        t = {}
        for model in ("sigma", "std"):
            bn = DecodeBench(f"ket_{model}_{prefix}")
            split_ms, comb_ms = bn.time_kernels(steps)
            t[model] = (split_ms * 1e3, comb_ms * 1e3)
            bn.free()
            del bn
        rel = [(t["std"][k] - t["sigma"][k]) / t["std"][k] for k in (0, 1)]
        tot_s, tot_g = sum(t["sigma"]), sum(t["std"])
        rows.append({"prefix": prefix,
                     "sigma_us": {"split": round(t["sigma"][0], 2), "combine": round(t["sigma"][1], 2)},
                     "std_us": {"split": round(t["std"][0], 2), "combine": round(t["std"][1], 2)},
                     "improvement_pct": {"split": round(100 * rel[0], 2),
                                         "combine": round(100 * rel[1], 2),
                                         "total": round(100 * (tot_g - tot_s) / tot_g, 2)}})
        log(json.dumps(rows[-1]))
    return rows


def prefill_bench(steps: int = 10):
    import numpy as np
    import torch

    import asymmetric_head_kv_amd as dq
    import synth

    case = synth.make_case(**synth.workload("prefill2k_on_30k"))
    dev = "cuda"

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = up(case.q), up(case.k_cache), up(case.v_cache)
    ctx = torch.from_numpy(case.ctx_len.astype(np.int32)).to(dev)
    out = torch.empty((case.batch, case.t_new, case.n_q, case.d_v), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(16, dq.prefill_workspace_bytes(case.n_q, case.n_k, case.n_v, case.d_k,
                                                        case.d_v, case.batch, case.t_new)),
                     dtype=torch.uint8, device=dev)
    for _ in range(2):
        dq.prefill(q, k, v, ctx, out=out, workspace=ws)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        dq.prefill(q, k, v, ctx, out=out, workspace=ws)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    L, T = int(case.ctx_len[0]), case.t_new
    pairs = sum(L - T + r + 1 for r in range(T))
    flops = pairs * case.n_q * 2 * (case.d_k + case.d_v)
    tflops = flops / (ms * 1e-3) / 1e12
    rec = {"workload": "prefill2k_on_30k", "us_per_call": round(ms * 1e3, 2),
           "algorithmic_gflop": round(flops / 1e9, 2), "tflops": round(tflops, 1),
           "bound": "mfma", "peak_tflops": BF16_PEAK_TFLOPS,
           "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}
    # The same call over a paged cache: 64-row pages in a seeded random order.
    P = 64
    nblk = -(-case.l_cap // P)
    perm = torch.randperm(nblk, generator=torch.Generator().manual_seed(0)).to(dev)

    def to_pages(c):
        h, d = c.shape[1], c.shape[3]
        x = torch.zeros((h, nblk * P, d), dtype=c.dtype, device=dev)
        x[:, :case.l_cap] = c[0]
        pg = torch.empty((nblk, h, P, d), dtype=c.dtype, device=dev)
        pg[perm] = x.view(h, nblk, P, d).permute(1, 0, 2, 3)
        return pg

    kp, vp = to_pages(k), to_pages(v)
    table = perm.to(torch.int32).view(1, nblk)
    for _ in range(2):
        dq.prefill_paged(q, kp, vp, table, ctx, out=out, workspace=ws)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(steps):
        dq.prefill_paged(q, kp, vp, table, ctx, out=out, workspace=ws)
    t1.record()
    torch.cuda.synchronize()
    ms_p = t0.elapsed_time(t1) / steps
    rec["paged"] = {"page_rows": P, "us_per_call": round(ms_p * 1e3, 2),
                    "time_over_contiguous": round(ms_p / ms, 3)}
    return rec


def augq_bench(steps: int = 200):
    """The augmented-Q projection at the SIGMA-1.5B shape for 1 and 16 decode
    tokens (weight streaming; per-layer weight replicas so the timing is HBM,
    not the Infinity Cache) and for 2048 prefill tokens (matrix cores)."""
    import numpy as np
    import torch

    import asymmetric_head_kv_amd as dq
    import synth

    sh = synth.AUGQ_SIGMA15B
    d_m, d_i, d_out = sh["d_m"], sh["d_i"], sh["d_out"]
    case = synth.make_augq(7, M=2048, **sh)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to("cuda")

    w = [dq.augq_pack(up(x)) for x in (case.w_gate, case.w_up, case.w_down)]
    wbytes = sum(x.numel() for x in w) * 2
    R = max(2, math.ceil(4 * MALL_BYTES / wbytes))
    reps = [w] + [[x.clone() for x in w] for _ in range(R - 1)]
    h_all = up(case.h)
    lib = dq.load()
    out = {"shape": {"d_m": d_m, "d_i": d_i, "d_out": d_out}, "weight_bytes": wbytes,
           "weight_replicas": R}
    for M in (1, 16, 2048):
        h = h_all[:M].contiguous()
        q = torch.empty((M, d_out), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(max(16, M * d_i * 2), dtype=torch.uint8, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream

        def call(r):
            wg, wu, wd = reps[r]
            st = lib.augq_forward(M, d_m, d_i, d_out, h.data_ptr(), wg.data_ptr(), wu.data_ptr(),
                                  wd.data_ptr(), q.data_ptr(), ws.data_ptr(),
                                  ws.numel(), torch.cuda.current_stream().cuda_stream)
            assert st == 0, st

        for r in range(R):
            call(r)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            call(0)
        torch.cuda.current_stream().wait_stream(s)
        with torch.cuda.graph(g):
            for r in range(R):
                call(r)
        g.replay()
        torch.cuda.synchronize()
        n = max(1, (steps if M < 2048 else 20) // R)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(n):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) / (n * R) * 1e3
        flops = 2 * M * (2 * d_m * d_i + d_i * d_out)
        byts = wbytes + 2 * M * (d_m + 2 * d_i + d_out)
        out[f"M{M}"] = {"us": round(us, 2), "GBps": round(byts / us / 1e3, 1),
                        "frac_hbm": round(byts / us / 1e3 / HBM_PEAK_GBS, 4),
                        "tflops": round(flops / us / 1e6, 1),
                        "frac_mfma": round(flops / us / 1e6 / BF16_PEAK_TFLOPS, 4)}
        log(f"augq M={M}: {us:.2f} us")
        del g
    # Reference at 2048 tokens: torch's bf16 GEMMs (hipBLASLt) on the same
    # shapes, gate and up as one n = 2 d_i product, then the down product
    # (the gating's elementwise step left out), timed on the same box.
    h = h_all.contiguous()
    wgu = torch.cat([up(case.w_gate), up(case.w_up)]).t()        # [d_m, 2 d_i]
    wd = up(case.w_down).t()                                      # [d_i, d_out]
    a_in = torch.randn(2048, d_i, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        g_ = h @ wgu
        q_ = a_in @ wd
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(20):
        torch.matmul(h, wgu, out=g_)
        torch.matmul(a_in, wd, out=q_)
    t1.record()
    torch.cuda.synchronize()
    ref_us = t0.elapsed_time(t1) / 20 * 1e3
    out["M2048"]["torch_gemms_us"] = round(ref_us, 2)
    out["M2048"]["time_over_torch_gemms"] = round(out["M2048"]["us"] / ref_us, 3)
    log(f"augq M=2048 torch GEMMs: {ref_us:.2f} us")
    return out


def hbm_copy_gbs(nbytes: int = 2 << 30, reps: int = 10):
    """Practical HBM ceiling: a large device-to-device copy (read + write)."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        b.copy_(a)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


def bf16_gemm_tflops(n: int = 8192, reps: int = 20):
    """Practical dense-matrix-core rate on this machine: torch's bf16 GEMM
    (hipBLASLt) on n x n x n with every CU busy, for comparison with the
    prefill's own rate (both run under the same board power limit)."""
    import torch
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    c = a @ b
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del a, b, c
    torch.cuda.empty_cache()
    return 2.0 * n ** 3 / (ms * 1e-3) / 1e12


def _cpu_threads() -> int:
    """Worker threads for the oracle: the host's CPUs, at most 16 (one GPU's
    share of a host)."""
    return max(1, min(16, os.cpu_count() or 1))


def _oracle_units(name: str):
    """The workload as independent oracle calls: one (sequence, query head)
    decode per unit, or one prefill row (all query heads) per unit.  Returns
    (units, algorithmic bytes or flops of the whole step, unit name, metric
    unit)."""
    import numpy as np

    import oracle
    import synth
    case = synth.make_case(**synth.workload(name))
    # Widened once to float64 (exact), so each call reads its rows as they
    # are instead of converting them again.
    q, k, v = (x.astype(np.float64) for x in case.widened())
    ctx = np.asarray(case.ctx_len)
    esize = 2 if case.dtype == "bf16" else 4
    if case.t_new:
        T = case.t_new
        rows = list(range(T))
        units = [lambda r=r: oracle.prefill(q, k, v, ctx, case.scale, rows=[(0, r)])
                 for r in rows]
        pairs = sum(int(ctx[0]) - T + r + 1 for r in rows)
        work = pairs * case.n_q * 2 * (case.d_k + case.d_v)
        return units, work, "prefill row (all query heads)", "GFLOP/s"
    units = []
    for b in range(case.batch):
        L = int(ctx[b])
        for i in range(case.n_q):
            g = oracle.group_sharing_index(i, case.n_q, case.n_k)
            hv = oracle.group_sharing_index(i, case.n_q, case.n_v)
            units.append(lambda b=b, i=i, g=g, hv=hv, L=L: oracle.attend_one(
                q[b, i], k[b, g, :L], v[b, hv, :L], case.scale))
    work = int(ctx.sum()) * kv_elements_per_token(case.n_k, case.d_k, case.n_v, case.d_v) * esize
    return units, work, "(sequence, query head) decode", "GB/s"


def cpu_baseline_one(name: str, seconds: float, threads: int) -> dict:
    """The fp64 oracle, unchanged, on a bounded sample of one workload: its
    independent units (evenly spread over the step) run on `threads` host
    threads until about `seconds` have passed; the full step's time is the
    unit count over the measured unit rate."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    units, work, unit_name, unit = _oracle_units(name)
    n = len(units)
    # Units in a strided order, so a partial sample spreads over the step
    # (prefill rows grow with their position); whole passes repeat while
    # time is left.
    stride = max(1, n // 16)
    order = [u for r in range(stride) for u in range(r, n, stride)]
    done = 0
    t0 = time.perf_counter()
    # One BLAS thread per worker: the workers are the parallelism.
    with threadpool_limits(1), ThreadPoolExecutor(max_workers=threads) as ex:
        while True:
            batch = [units[order[(done + j) % n]] for j in range(threads)]
            list(ex.map(lambda f: f(), batch))
            done += len(batch)
            if time.perf_counter() - t0 >= seconds:
                break
    el = time.perf_counter() - t0
    step_s = el * n / done
    scale = 1e9
    rec = {"value": round(work / step_s / scale, 3), "unit": unit,
           "us_per_step": round(step_s * 1e6, 1),
           "sample": f"{done} unit calls ({unit_name}; {n} per step) in {el:.1f} s"}
    return rec


def cpu_baseline(name: str, seconds: float, per_config_seconds: float = 2.5,
                 configs=()) -> dict:
    """The fp64 oracle on the host cores: the headline workload, and a
    bounded sample of every other configuration."""
    threads = _cpu_threads()
    main = cpu_baseline_one(name, seconds, threads)
    out = {"value": main["value"], "unit": main["unit"], "cores": threads,
           "host_cpus": os.cpu_count(), "kind": "oracle",
           "us_per_step": main["us_per_step"],
           "sample": f"{name}: {main['sample']}, on {threads} threads (fp64 numpy oracle; "
                     f"step time = units / measured unit rate)"}
    per = {}
    for cfg in configs:
        try:
            per[cfg] = cpu_baseline_one(cfg, per_config_seconds, threads)
        except Exception as e:  # a baseline, never the product: report and go on
            per[cfg] = {"error": str(e)}
        log(f"cpu baseline {cfg}: {per[cfg]}")
    if per:
        out["per_config"] = per
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path "
              "is not sharded across GPUs.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        a = torch.ones(args.copy_probe // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": a.numel() * 4, "copies": 3}))
        return

    if args.only_augq:
        print(json.dumps({"augq": augq_bench(args.steps)}), flush=True)
        return
    if args.ket:
        print(json.dumps({"ket_replica": ket_replica(args.steps),
                          "note": "batch 1, one query token, bf16; kernel times from graphs "
                                  "of back-to-back launches over cache replicas"}), flush=True)
        return
    if args.workload.startswith("prefill"):
        # Prefill alone (for profilers): the decode metric is not measured.
        log(f"workload {args.workload}: prefill only")
        print(json.dumps({"prefill": prefill_bench(args.steps)}), flush=True)
        return
    log(f"workload {args.workload}: building inputs")
    bench = DecodeBench(args.workload, args.chunk)
    log(f"replicas {bench.replicas}, chunk {bench.S} rows, workspace {bench.ws_bytes} B")
    ms, graphed = bench.time_steps(args.steps, args.warmup, args.eager)
    log(f"step {ms * 1e3:.2f} us ({'graph' if graphed else 'eager'})")
    k_ms = bench.time_kernels(args.steps)
    log("kernels (us): split %.2f combine %.2f" % tuple(x * 1e3 for x in k_ms))
    traffic = pmc_traffic(args.workload)
    split_gbs = bench.alg_bytes_split / (k_ms[0] * 1e-3) / 1e9
    value = bench.alg_bytes_step / (ms * 1e-3) / 1e9
    n_q, n_k, n_v, d_k, d_v = bench.shape
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2), "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "us_per_step_spread": bench.step_pct_us,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": bench.case.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "batch": bench.B, "max_ctx": bench.max_ctx,
                   "n_q": n_q, "n_k": n_k, "n_v": n_v, "d_k": d_k, "d_v": d_v,
                   "chunk_rows": bench.S, "cache_replicas": bench.replicas,
                   "timing": "hip graph replay" if graphed else "eager launches",
                   "step": "split with fused kv_append (1 row/seq) + combine"},
        "roofline": {"bound": "hbm", "kernel": "decode_split_kernel",
                     "achieved": round(split_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(split_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, scaled)",
                     "alg_bytes_per_launch": bench.alg_bytes_split,
                     "avg_launch_us": round(k_ms[0] * 1e3, 2)},
        "kernels_us": {"split_with_append": round(k_ms[0] * 1e3, 2),
                       "combine": round(k_ms[1] * 1e3, 2)},
        "kernel_source_sha256": kernel_source_hash(),
    }
    if args.selective_k > 0:
        bench.setup_selective(args.selective_k)
        ms_sel, _ = bench.time_steps(args.steps, args.warmup, args.eager, bench.selective_step)
        log(f"selective-V step (top_k {args.selective_k}) {ms_sel * 1e3:.2f} us")
        result["selective_v"] = {
            "top_k": args.selective_k, "us_per_step": round(ms_sel * 1e3, 2),
            "alg_bytes_per_step": bench.sel_alg_bytes,
            "GBps": round(bench.sel_alg_bytes / (ms_sel * 1e-3) / 1e9, 1),
            "workspace_bytes_per_step": bench.sel_ws_traffic,
            "speedup_over_full_decode": round(ms / ms_sel, 3),
            "step": "fused kv_append + logits + per-range top-k + final top-k and V gather"}
    if args.page_rows > 0 and not args.kernel_only:
        bench.setup_paged(args.page_rows)
        ms_pg, _ = bench.time_steps(args.steps, args.warmup, args.eager, bench.paged_step)
        log(f"paged step (page rows {args.page_rows}) {ms_pg * 1e3:.2f} us")
        result["paged"] = {"page_rows": args.page_rows, "us_per_step": round(ms_pg * 1e3, 2),
                           "GBps": round(bench.alg_bytes_step / (ms_pg * 1e-3) / 1e9, 1),
                           "time_over_contiguous": round(ms_pg / ms, 3),
                           "pages": "each sequence's blocks in a seeded random page order"}
        if args.selective_k > 0:
            ms_ps, _ = bench.time_steps(args.steps, args.warmup, args.eager,
                                        bench.paged_selective_step)
            log(f"paged selective-V step {ms_ps * 1e3:.2f} us")
            result["paged"]["selective_us_per_step"] = round(ms_ps * 1e3, 2)
            result["paged"]["selective_time_over_contiguous"] = round(ms_ps / ms_sel, 3)
        bench.pages = None
    n_q_, n_k_, n_v_, d_k_, d_v_ = bench.shape
    if not args.no_compat and not args.kernel_only and n_k_ != n_v_:
        bench.setup_compat()
        ms_cp, _ = bench.time_steps(args.steps, args.warmup, args.eager, bench.compat_step)
        n_h = max(n_k_, n_v_)
        ratio = kv_elements_per_token(n_h, d_k_, n_h, d_v_) / kv_elements_per_token(
            n_k_, d_k_, n_v_, d_v_)
        log(f"kv_group_sharing step {ms_cp * 1e3:.2f} us")
        result["kv_group_sharing"] = {
            "heads": [n_q_, n_h, n_h], "us_per_step": round(ms_cp * 1e3, 2),
            "time_over_native": round(ms_cp / ms, 3), "cache_bytes_ratio": round(ratio, 3),
            "expand_us_once": round(bench.compat_expand_ms * 1e3, 1)}
        bench.compat = None
    sym_name = None if args.no_twin else (args.twin or TWINS.get(args.workload))
    asym_bytes = bench.alg_bytes_step
    bench.free()
    del bench
    if not args.kernel_only:
        if sym_name:
            log(f"symmetric twin {sym_name}")
            tw = DecodeBench(sym_name, args.chunk)
            ms_t, _ = tw.time_steps(args.steps, args.warmup, args.eager)
            result["symmetric_twin"] = {
                "workload": sym_name, "us_per_step": round(ms_t * 1e3, 2),
                "GBps": round(tw.alg_bytes_step / (ms_t * 1e-3) / 1e9, 1),
                "speedup_asym_over_sym": round(ms_t / ms, 3),
                "byte_ratio_bound": round(tw.alg_bytes_step / asym_bytes, 3)}
            tw.free()
            del tw
        try:
            result["hbm_copy_GBps"] = round(hbm_copy_gbs(), 1)
        except Exception as e:
            log(f"copy bandwidth probe failed: {e}")
        if not args.no_prefill:
            log("prefill 2048 on 30720")
            result["prefill"] = prefill_bench()
            g = bf16_gemm_tflops()
            result["prefill"]["bf16_gemm_8192_tflops"] = round(g, 1)
            result["prefill"]["frac_of_gemm"] = round(result["prefill"]["tflops"] / g, 4)
        if not args.no_augq:
            log("augmented Q")
            result["augq"] = augq_bench()
        if not args.no_workloads:
            recs = {}
            for name in OTHER_WORKLOADS:
                if name == args.workload:
                    continue
                log(f"workload {name}")
                recs[name] = decode_record(name, args.steps, args.warmup, args.chunk,
                                           args.selective_k)
                log(f"  step {recs[name]['us_per_step']} us, split {recs[name]['split_us']} us")
            sym = recs.get("decode64k_sym")
            for name in ("decode64k_dk64", "decode64k_dk128"):
                if sym and name in recs:
                    r = recs[name]
                    r["speedup_over_decode64k_sym"] = round(sym["us_per_step"] / r["us_per_step"], 3)
                    r["byte_ratio_bound"] = round(sym["alg_bytes_per_step"] / r["alg_bytes_per_step"], 3)
            result["workloads"] = recs
        if not args.no_ket:
            log("KET replica")
            result["ket_replica"] = ket_replica(args.steps)
        if not args.no_cpu_baseline:
            log("cpu baseline (oracle)")
            cfgs = [c for c in ("tiny_f32", "decode32k_sym", "ragged16", "decode64k_dk64",
                                "decode64k_dk128", "decode64k_sym", "prefill2k_on_30k")
                    if c != args.workload]
            result["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds,
                                                  configs=cfgs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

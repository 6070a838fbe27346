"""Per-stage timing from the engine's in-kernel trace records.

A monolithic persistent kernel hides per-operator time from kernel-level
profilers (SemiAnalysis TileRT page, challenges section). The engine
therefore records, for every stage and workgroup, when the workgroup entered
the stage, when its dependency wait ended and when it signalled completion
(wall clock, 100 MHz), plus marks inside the stage: input staged, weights
consumed, epilogue done (0 where a stage has no such point). This module turns those records into per-stage spans,
work and wait times and the idle fraction of the step.
"""
from __future__ import annotations

import numpy as np

WALLCLOCK_HZ = 100e6


def summarize(trace: np.ndarray, plan: list, hz: float = WALLCLOCK_HZ) -> dict:
    """trace: int64 [n_stages, n_workgroups, 8] of one step; plan: describe_plan() list."""
    t = trace.astype(np.float64)
    enter, ready, done = t[:, :, 0], t[:, :, 1], t[:, :, 2]
    t0 = enter.min()
    us = 1e6 / hz
    rows = []
    prev_end = t0
    for s, st in enumerate(plan):
        start, end = enter[s].min(), done[s].max()
        work = (done[s] - ready[s]) * us
        wait = (ready[s] - enter[s]) * us
        span = (end - prev_end) * us  # critical-path increment of this stage
        rows.append({
            "stage": s, "type": st["type"], "layer": st["layer"], "weight_bytes": st["weight_bytes"],
            "end_us": (end - t0) * us, "span_us": span, "work_us_mean": float(work.mean()),
            "work_us_max": float(work.max()), "wait_us_mean": float(wait.mean()),
            "GBps": st["weight_bytes"] / max(span, 1e-3) / 1e3 if st["weight_bytes"] else 0.0,
        })
        prev_end = max(prev_end, end)
    total = (done.max() - t0) * us
    busy = ((done - ready) * us).sum()
    G = trace.shape[1]
    return {"total_us": total, "idle_frac": 1.0 - busy / (total * G), "stages": rows}


def by_type(summary: dict) -> dict:
    agg = {}
    for r in summary["stages"]:
        a = agg.setdefault(r["type"], {"span_us": 0.0, "weight_bytes": 0, "count": 0})
        a["span_us"] += r["span_us"]
        a["weight_bytes"] += r["weight_bytes"]
        a["count"] += 1
    for a in agg.values():
        a["GBps"] = a["weight_bytes"] / max(a["span_us"], 1e-3) / 1e3
    return agg


def format_table(summary: dict) -> str:
    lines = [f"step {summary['total_us']:.1f} us, idle fraction {summary['idle_frac']:.3f}",
             f"{'type':>10} {'count':>5} {'span_us':>9} {'MB':>9} {'GB/s':>7}"]
    for k, a in sorted(by_type(summary).items(), key=lambda kv: -kv[1]["span_us"]):
        lines.append(f"{k:>10} {a['count']:>5} {a['span_us']:>9.1f} {a['weight_bytes'] / 1e6:>9.1f} {a['GBps']:>7.0f}")
    return "\n".join(lines)


def phases(trace: np.ndarray, plan: list, hz: float = WALLCLOCK_HZ) -> list:
    """Per-stage breakdown of one step from the 8-word records: mean and max
    over workgroups of setup (stage entered -> dependency wait entered: plan
    reads, address set-up, early weight loads), wait (-> dependency
    satisfied), stage (-> input staged), stream (-> weights consumed), epi (->
    epilogue done), ack (-> signalled) and gap (signalled -> the next stage
    entered). Phases a stage does not mark are None."""
    t = trace.astype(np.float64) * (1e6 / hz)
    enter, ready, done = t[:, :, 0], t[:, :, 1], t[:, :, 2]
    entry = t[:, :, 7]
    m0, m1, m2 = t[:, :, 4], t[:, :, 5], t[:, :, 6]
    has = (trace[:, :, 4] != 0) & (trace[:, :, 5] != 0) & (trace[:, :, 6] != 0)
    t0 = enter.min()
    out = []
    prev_end = t0
    for s, st in enumerate(plan):
        def mm(v, sel=None):
            v = v if sel is None else v[sel]
            return None if v.size == 0 else (float(v.mean()), float(v.max()))
        h = has[s]
        row = {"stage": s, "type": st["type"], "layer": st["layer"],
               "span_us": float(done[s].max() - prev_end), "start_us": float(enter[s].min() - t0),
               "setup": mm(enter[s] - entry[s]), "wait": mm(ready[s] - enter[s]),
               "stage_in": mm(m0[s] - ready[s], h), "stream": mm(m1[s] - m0[s], h),
               "epi": mm(m2[s] - m1[s], h), "ack": mm(done[s] - m2[s], h),
               "gap": mm(entry[s + 1] - done[s]) if s + 1 < len(plan) else None}
        out.append(row)
        prev_end = max(prev_end, done[s].max())
    return out


def format_phases(rows: list) -> str:
    def f(v):
        return f"{'-':>11}" if v is None else f"{v[0]:5.1f}[{v[1]:4.1f}]"
    lines = ["per stage, mean[max] over workgroups (us): setup = stage entered -> dependency wait entered, wait = "
             "-> dependency satisfied, stage = -> input staged, stream = -> weights consumed, epi = -> epilogue "
             "done, ack = -> signalled, gap = -> next stage entered",
             f"{'st':>3} {'type':>9} {'L':>2} {'span':>6} {'start':>7} {'setup':>11} {'wait':>11} {'stage':>11} "
             f"{'stream':>11} {'epi':>11} {'ack':>11} {'gap':>11}"]
    for r in rows:
        lines.append(f"{r['stage']:>3} {r['type']:>9} {r['layer']:>2} {r['span_us']:>6.1f} {r['start_us']:>7.1f} "
                     f"{f(r['setup'])} {f(r['wait'])} {f(r['stage_in'])} {f(r['stream'])} {f(r['epi'])} "
                     f"{f(r['ack'])} {f(r['gap'])}")
    return "\n".join(lines)

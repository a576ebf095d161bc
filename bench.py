"""Throughput of the DFlash drafter hot path on one MI355X.

One step is one speculative round of the Qwen3-8B-shaped drafter (hidden 4096,
5 draft layers, 32/8 heads of 128, SwiGLU 12288, vocab 151936, block 16) at a
2048-token context:
  draft_block  - embed [anchor, 15 x mask], 5 layers, LM head + argmax;
  verify       - greedy, against planted target logits (tau ~ min(Geom(0.25), 16));
  append       - fuse the tau accepted rows' 5 target hidden states, inject their
                 K/V at positions 2048.., then trim the cache back to 2048 so every
                 step drafts at the same context length.
The headline loop is device-resident: the cache length, tau and the anchor stay
in device memory, the append takes the first tau of the round's 16 fused rows
on the device, and nothing is read back between rounds. The same rounds are
also timed as two captured HIP graphs per round (draft; verify + append +
trim) and as a host-driven loop (tau read back to size the append); the
dominant kernel's launches are timed inside the host-driven loop with HIP
events on the handle's stream. Inputs are resident in HBM before timing
starts.

Prints one JSON line (rank 0) with the metric, the roofline of the dominant
kernel and the CPU oracle timed on a bounded sample on the host.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft-block forward µs & blocks/s (block 16, ctx 2048); % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
STAGE_BITS = {"gate_up": 4, "lm_head": 6, "fuse_context": 7, "inject_kv": 8}
# the kernel behind each timed stage, and the source file it is built from
STAGE_KERNEL = {"lm_head": ("stream_gemm<...EpiLM>", "skinny.hip"),
                "gate_up": ("stream_gemm<...EpiSwiglu> + stream_finish", "skinny.hip")}
CSRC = os.path.join(ROOT, "block_diffusion_drafter_layer_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def _sha256(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def counter_traffic(stage, workload):
    """HBM bytes per launch of the stage's kernel from the committed rocprofv3
    counter summary (FETCH_SIZE + WRITE_SIZE scaled by a plain copy's), or
    None when there is none or the kernel source changed since it was taken."""
    path = os.path.join(PROFILES, f"pmc_traffic_{stage}_{workload}.txt")
    if stage not in STAGE_KERNEL or not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    src = os.path.join(CSRC, STAGE_KERNEL[stage][1])
    if fields.get("source_sha256") != _sha256(src) or "traffic_bytes_per_launch" not in fields:
        return None
    return int(float(fields["traffic_bytes_per_launch"]))


def _kernel_rows(db):
    import sqlite3
    c = sqlite3.connect(db)
    return c.execute("select name, count(*), sum(end-start), avg(end-start), min(end-start), "
                     "max(end-start) from kernels group by name order by sum(end-start) desc").fetchall()


def summarize_trace(db, out, cmd):
    """Text summary of a rocprofv3 --kernel-trace --stats database."""
    import re
    rows = _kernel_rows(db)
    tot = sum(r[2] for r in rows)
    with open(out, "w") as f:
        f.write(f"# rocprofv3 kernel trace summary\n# command: {cmd}\n")
        f.write(f"# {'kernel':<78s} {'calls':>6s} {'total_us':>10s} {'avg_us':>9s} {'min_us':>9s} "
                f"{'max_us':>9s} {'%':>6s}\n")
        for n, cnt, sm, av, mn, mx in rows:
            short = re.sub(r"\(.*", "", n.replace("(anonymous namespace)::", ""))[:78]
            f.write(f"{short:<80s} {cnt:6d} {sm / 1e3:10.1f} {av / 1e3:9.2f} {mn / 1e3:9.2f} "
                    f"{mx / 1e3:9.2f} {100 * sm / tot:6.2f}\n")


def _pmc(db, counter, pattern):
    import re
    import sqlite3
    c = sqlite3.connect(db)
    rows = c.execute("select name, counter_value from pmc_events where counter_name = ?",
                     (counter,)).fetchall()
    vals = [v for n, v in rows if re.search(pattern, n)]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def summarize_pmc(fetch_db, write_db, copy_fetch_db, copy_write_db, pattern, source, out, cmds,
                  copy_bytes=1 << 30):
    """HBM traffic per dispatch of the kernels matching `pattern`: FETCH_SIZE
    and WRITE_SIZE (KiB) scaled by what they read for a plain device copy of
    copy_bytes read + copy_bytes written."""
    copy_pat = r"copy_bytes"
    cf, _ = _pmc(copy_fetch_db, "FETCH_SIZE", copy_pat)
    cw, _ = _pmc(copy_write_db, "WRITE_SIZE", copy_pat)
    kf, nf = _pmc(fetch_db, "FETCH_SIZE", pattern)
    kw, nw = _pmc(write_db, "WRITE_SIZE", pattern)
    fs = copy_bytes / (cf * 1024.0)
    ws = copy_bytes / (cw * 1024.0)
    traffic = kf * 1024.0 * fs + kw * 1024.0 * ws
    with open(out, "w") as f:
        f.write("# HBM traffic per dispatch from rocprofv3 counters\n")
        for c in cmds:
            f.write(f"# command: {c}\n")
        f.write(f"kernel_pattern: {pattern}\n")
        f.write(f"fetch_size_kib_per_dispatch: {kf:.1f} (n={nf})\n")
        f.write(f"write_size_kib_per_dispatch: {kw:.1f} (n={nw})\n")
        f.write(f"copy_fetch_size_kib: {cf:.1f}\ncopy_write_size_kib: {cw:.1f}\n")
        f.write(f"fetch_scale: {fs:.4f}\nwrite_scale: {ws:.4f}\n")
        f.write(f"traffic_bytes_per_launch: {traffic:.0f}\n")
        f.write(f"source: {os.path.relpath(source, ROOT)}\nsource_sha256: {_sha256(source)}\n")


def _pmc_all(db, pattern):
    """{counter: (mean per dispatch, dispatches)} of the kernels matching
    pattern. A counter arrives as one row per hardware instance (XCC, shader
    engine); per dispatch they are summed, except GRBM_GUI_ACTIVE (active
    cycles, the same clock on every instance), of which the maximum is taken."""
    import re
    import sqlite3
    c = sqlite3.connect(db)
    rows = c.execute("select dispatch_id, name, counter_name, counter_value from pmc_events").fetchall()
    per = {}
    for did, n, cn, v in rows:
        if re.search(pattern, n):
            key = (did, cn)
            if cn == "GRBM_GUI_ACTIVE":
                per[key] = max(per.get(key, 0.0), v)
            else:
                per[key] = per.get(key, 0.0) + v
    acc = {}
    for (did, cn), v in per.items():
        acc.setdefault(cn, []).append(v)
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def summarize_mfma(counts_db, util_db, trace_db, out, cmds, kernels):
    """MFMA utilisation of the context GEMMs from counter runs: per dispatch,
    SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 = bf16 MFMA FLOPs executed,
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE, and rocprofv3's derived
    MfmaUtil (busy cycles over active cycles x SIMDs); the average duration of
    the same kernels from a kernel-trace run of the same command gives the
    FLOP rate against the 2.5 PFLOP/s bf16 peak."""
    import re
    import sqlite3
    tr = sqlite3.connect(trace_db).execute(
        "select name, avg(end-start), count(*) from kernels group by name").fetchall()
    with open(out, "w") as f:
        f.write("# MFMA utilisation of the context GEMMs from rocprofv3 counters\n")
        for c in cmds:
            f.write(f"# command: {c}\n")
        f.write("# per dispatch means; flops_counter = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512;\n"
                "# tflops_counter = flops_counter / avg_us (trace run); frac = / 2500 TFLOP/s\n")
        for label, pattern, alg_flops in kernels:
            cnt = _pmc_all(counts_db, pattern)
            ut = _pmc_all(util_db, pattern)
            durs = [(av, n) for name, av, n in tr if re.search(pattern, name)]
            avg_ns = sum(a * n for a, n in durs) / max(1, sum(n for _, n in durs))
            mops = cnt.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", (0.0, 0))[0]
            fl = mops * 512.0
            f.write(f"\n[{label}] kernel_pattern: {pattern}\n")
            for k in sorted(cnt):
                f.write(f"  {k}: {cnt[k][0]:.6g} (n={cnt[k][1]})\n")
            for k in sorted(ut):
                f.write(f"  {k}: {ut[k][0]:.6g} (n={ut[k][1]})\n")
            f.write(f"  avg_us (trace): {avg_ns / 1e3:.2f}\n")
            busy = cnt.get("SQ_VALU_MFMA_BUSY_CYCLES", (0.0, 0))[0]
            act = cnt.get("GRBM_GUI_ACTIVE", (0.0, 0))[0]
            if act:
                f.write(f"  mfma_busy_frac = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 1024 SIMDs): "
                        f"{busy / (act * 1024):.4f}\n")
                if avg_ns:
                    f.write(f"  clock_GHz = GRBM_GUI_ACTIVE / avg duration: {act / avg_ns:.3f}\n")
            f.write(f"  flops_counter: {fl:.6g}  flops_algorithmic: {alg_flops:.6g}  "
                    f"ratio: {fl / alg_flops:.4f}\n")
            if avg_ns:
                tf = fl / (avg_ns * 1e-9) / 1e12
                f.write(f"  tflops_counter: {tf:.1f}  frac_of_peak_counter: {tf / MFMA_BF16_PEAK_TFLOPS:.4f}\n")
                ta = alg_flops / (avg_ns * 1e-9) / 1e12
                f.write(f"  tflops_timed_algorithmic: {ta:.1f}  frac_of_peak_timed: {ta / MFMA_BF16_PEAK_TFLOPS:.4f}\n")


def summarize_traffic(fetch_db, write_db, copy_fetch_db, copy_write_db, out, cmds,
                      copy_bytes=1 << 30):
    """HBM traffic per dispatch of every library kernel: FETCH_SIZE and
    WRITE_SIZE (KiB) scaled by what they read for the plain device copy of
    copy_bytes read + copy_bytes written."""
    import re
    import sqlite3
    cf, _ = _pmc(copy_fetch_db, "FETCH_SIZE", r"copy_bytes")
    cw, _ = _pmc(copy_write_db, "WRITE_SIZE", r"copy_bytes")
    fs, ws = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)

    def per_kernel(db, counter):
        rows = sqlite3.connect(db).execute(
            "select name, counter_value from pmc_events where counter_name = ?", (counter,)).fetchall()
        acc = {}
        for n, v in rows:
            if "dfl::" in n and "copy_bytes" not in n:
                k = re.sub(r"\(.*", "", n.replace("(anonymous namespace)::", ""))
                k = re.sub(r"^void ", "", k)
                acc.setdefault(k, []).append(v)
        return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}

    fk, wk = per_kernel(fetch_db, "FETCH_SIZE"), per_kernel(write_db, "WRITE_SIZE")
    with open(out, "w") as f:
        f.write("# HBM traffic per dispatch of the library's kernels, from rocprofv3 counters\n"
                "# (FETCH_SIZE and WRITE_SIZE in KiB per dispatch, scaled by what the same counters read\n"
                "#  for the library's plain device copy of 1 GiB read + 1 GiB written)\n")
        for c in cmds:
            f.write(f"# command: {c}\n")
        f.write(f"fetch_scale: {fs:.4f}\nwrite_scale: {ws:.4f}\n")
        f.write(f"# {'kernel':<70s} {'dispatches':>10s} {'fetch_MB':>9s} {'write_MB':>9s}\n")
        for k in sorted(fk, key=lambda k: -fk[k][0]):
            fmb = fk[k][0] * 1024.0 * fs / 1e6
            wmb = wk.get(k, (0.0, 0))[0] * 1024.0 * ws / 1e6
            f.write(f"{k[:70]:<72s} {fk[k][1]:10d} {fmb:9.2f} {wmb:9.2f}\n")


def stage_bytes(dc, M):
    """Algorithmic HBM bytes of one launch per stage (weights + activations)."""
    D, F, V = dc.hidden, dc.ffn, dc.vocab
    qd, kvd = dc.q_dim, dc.kv_dim
    g = dc.block_size - 1
    return {
        "gate_up": 2 * F * D * 2 + M * D * 2 * 2 + M * F * 2 * 2,
        "lm_head": V * D * 2 + g * D * 2 * 2,
        "qkv": (qd + 2 * kvd) * D * 2,
        "o_proj": D * qd * 2,
        "down_proj": D * F * 2,
    }


def draft_block_bytes(dc, ctx):
    D, F, V, L = dc.hidden, dc.ffn, dc.vocab, dc.n_layers
    qd, kvd = dc.q_dim, dc.kv_dim
    per_layer = ((qd + 2 * kvd) * D + D * qd + 2 * F * D + D * F) * 2
    kv = L * 2 * (ctx + dc.block_size) * kvd * 2
    return L * per_layer + V * D * 2 + kv


def _ev_time(fn, reps, torch):
    """Median, p10 and p90 of fn() over reps runs, in microseconds (HIP events)."""
    import numpy as np
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    return (float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90)))


def _fill_context(kv, dc, S, seq, synth):
    """Seeded synthetic context K/V rows [S, Hkv, hd] straight into the cache."""
    for i in range(dc.n_layers):
        k, v = synth.gen.make_context_kv(dc, i, S, device=kv.buf.device, seq=seq)
        kv.k_view(i)[:, :S, :] = k.transpose(0, 1)
        kv.v_view(i)[:, :, :S] = v.permute(1, 2, 0)
    kv.kv.len = S


def roof(nbytes, flops):
    """Time at the binding MI355X roof (8 TB/s, 2.5 PFLOP/s bf16), us, and its name."""
    t_hbm, t_mfma = nbytes / (HBM_PEAK_GBS * 1e3), flops / (MFMA_BF16_PEAK_TFLOPS * 1e6)
    return (t_hbm, "hbm") if t_hbm >= t_mfma else (t_mfma, "mfma")


def draft_flops(dc, rows, ctx_total):
    D, F, V, L = dc.hidden, dc.ffn, dc.vocab, dc.n_layers
    qd, kvd = dc.q_dim, dc.kv_dim
    per_layer = (qd + 2 * kvd) * D + D * qd + 2 * F * D + D * F
    g = dc.block_size - 1
    attn = 4.0 * dc.n_heads * dc.head_dim * dc.block_size * ctx_total  # QK^T and PV
    return 2.0 * rows * L * per_layer + 2.0 * (rows // dc.block_size) * g * V * D + L * attn


def wl_d2048(reps, torch, synth, B, Drafter, config_from, dev):
    """The D=2048 block-8 drafter: draft, prefill fuse/inject, p/q verify."""
    dc = synth.CONFIGS[4]
    w = synth.make_weights(dc, device=dev)
    d = Drafter(config_from(dc), w, max_seqs=1, max_tokens=dc.ctx_len, device=dev)
    kv = d.new_kv(dc.ctx_len + 64)
    feats = synth.make_feats(dc, dc.ctx_len, device=dev)
    fu = _ev_time(lambda: d.fuse_context(feats), 3, torch)
    ctx = d.fuse_context(feats)
    inj = _ev_time(lambda: d.inject_kv(kv, ctx, 0), 3, torch)
    anchors = torch.from_numpy(synth.make_anchor(dc)).to(dev)
    blk = torch.empty(1, dc.block_size, dtype=torch.int32, device=dev)
    for _ in range(3):
        d.draft_block([kv], anchors, block_out=blk)
    dr = _ev_time(lambda: d.draft_block([kv], anchors, block_out=blk), reps, torch)
    tl = synth.make_target_logits(dc, dc.block_size, device=dev).unsqueeze(0).contiguous()
    dlog = synth.make_target_logits(dc, dc.block_size - 1, device=dev, draft=True).unsqueeze(0).contiguous()
    tau, bonus = torch.empty(1, dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.int32, device=dev)
    vq = _ev_time(lambda: d.verify(blk, tl, dlog, temperature=1.0, seed=0, tau=tau, bonus=bonus), reps, torch)
    T = dc.ctx_len
    t_roof, bound = roof(draft_block_bytes(dc, T), draft_flops(dc, dc.block_size, T + dc.block_size))
    f_fl = 2.0 * T * dc.n_feat * dc.hidden * dc.hidden
    i_fl = 2.0 * T * dc.hidden * 2 * dc.kv_dim * dc.n_layers
    out = {
        "draft_block_us": round(dr[0], 1), "draft_block_us_p10_p90": [round(dr[1], 1), round(dr[2], 1)],
        "blocks_per_s": round(1e6 / dr[0], 1), "draft_roofline": {"bound": bound, "frac": round(t_roof / dr[0], 4)},
        "prefill_fuse_us": round(fu[0], 1), "prefill_fuse_mfma_frac": round(f_fl / (fu[0] * 1e6) / MFMA_BF16_PEAK_TFLOPS, 4),
        "prefill_inject_us": round(inj[0], 1),
        "prefill_inject_mfma_frac": round(i_fl / (inj[0] * 1e6) / MFMA_BF16_PEAK_TFLOPS, 4),
        "pq_verify_us": round(vq[0], 1)}
    d.close()
    del w, d, kv, feats, ctx, tl, dlog
    torch.cuda.empty_cache()
    return dc.name, out


def wl_32seq(reps, torch, synth, B, Drafter, config_from, dev, w=None):
    """32 sequences, ragged contexts uniform in [512, 4096], one draft call."""
    import numpy as np
    dc = synth.CONFIGS[3]
    w = synth.make_weights(dc, device=dev) if w is None else w
    n = dc.n_seqs
    lens = [int(x) for x in synth.gen.ragged_lengths(n)]
    d = Drafter(config_from(dc), w, max_seqs=n, max_tokens=n * dc.block_size, device=dev)
    kvs = []
    for s_, S in enumerate(lens):
        kv = d.new_kv(S + 64)
        _fill_context(kv, dc, S, s_, synth)
        kvs.append(kv)
    anchors = torch.from_numpy(synth.make_anchor(dc, n=n)).to(dev)
    blk = torch.empty(n, dc.block_size, dtype=torch.int32, device=dev)
    for _ in range(2):
        d.draft_block(kvs, anchors, block_out=blk)
    dr = _ev_time(lambda: d.draft_block(kvs, anchors, block_out=blk), max(3, reps // 3), torch)
    kv_bytes = sum(dc.n_layers * 2 * (S + dc.block_size) * dc.kv_dim * 2 for S in lens)
    nbytes = draft_block_bytes(dc, 0) + kv_bytes
    t_roof, bound = roof(nbytes, draft_flops(dc, n * dc.block_size, sum(lens) + n * dc.block_size))
    out = {"draft_block_us": round(dr[0], 1),
           "draft_block_us_p10_p90": [round(dr[1], 1), round(dr[2], 1)],
           "blocks_per_s": round(n * 1e6 / dr[0], 1),
           "draft_roofline": {"bound": bound, "frac": round(t_roof / dr[0], 4)},
           "context_lengths": "32 uniform in [512, 4096], mean %d" % int(np.mean(lens))}
    d.close()
    del d, kvs
    torch.cuda.empty_cache()
    return dc.name, out, w


def wl_ctx8192(reps, torch, synth, B, Drafter, config_from, dev, w=None):
    """The 8192-token context: prefill fuse, then 4 host-driven rounds of
    draft, verify, trim and append."""
    import numpy as np
    dc = synth.CONFIGS[2]
    # the timing does not depend on the values: the Qwen-shaped weights of
    # another workload serve when given
    w2 = synth.make_weights(dc, device=dev) if w is None else w
    S0, Bs = dc.ctx_len, dc.block_size
    d = Drafter(config_from(dc), w2, max_seqs=1, max_tokens=S0, device=dev)
    kv = d.new_kv(S0 + Bs * (dc.rounds + 1))
    feats = synth.make_feats(dc, S0, device=dev)
    fu = _ev_time(lambda: d.fuse_context(feats), 2, torch)
    ctx = d.fuse_context(feats)
    d.inject_kv(kv, ctx, 0)
    anchors = torch.from_numpy(synth.make_anchor(dc)).to(dev)
    blk = torch.empty(1, Bs, dtype=torch.int32, device=dev)
    taus = synth.planted_taus(dc, dc.rounds)
    rounds_us, drafts_us = [], []
    for r in range(dc.rounds):
        S = kv.len
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        lg = synth.make_target_logits(dc, Bs, round_index=10 + r)
        app = synth.make_feats(dc, Bs, round_index=20 + r, device=dev)
        torch.cuda.synchronize()
        e[0].record()
        d.draft_block([kv], anchors, block_out=blk)
        e[1].record()
        torch.cuda.synchronize()
        synth.plant_agreement(lg, blk[0].cpu().numpy(), int(taus[r]) - 1)
        lgd = lg.unsqueeze(0).to(dev)
        torch.cuda.synchronize()
        e[2].record()
        t_, b_ = d.verify(blk, lgd)
        tau = int(t_.item())
        d.kv_trim(kv, S)
        d.inject_kv(kv, d.fuse_context([f[:tau] for f in app]), S)
        e3 = torch.cuda.Event(enable_timing=True)
        e3.record()
        torch.cuda.synchronize()
        drafts_us.append(e[0].elapsed_time(e[1]) * 1e3)
        rounds_us.append(e[0].elapsed_time(e[1]) * 1e3 + e[2].elapsed_time(e3) * 1e3)
        anchors = b_.to(torch.int32)
    t_roof, bound = roof(draft_block_bytes(dc, S0 + Bs), draft_flops(dc, Bs, S0 + 2 * Bs))
    out = {"prefill_fuse_us_T8192": round(fu[0], 1),
           "prefill_fuse_mfma_frac": round(2.0 * S0 * dc.n_feat * dc.hidden ** 2 / (fu[0] * 1e6)
                                           / MFMA_BF16_PEAK_TFLOPS, 4),
           "round_us": [round(x, 1) for x in rounds_us],
           "draft_block_us": [round(x, 1) for x in drafts_us],
           "draft_roofline": {"bound": bound, "frac": round(t_roof / float(np.median(drafts_us)), 4)},
           "final_context": kv.len}
    d.close()
    del d, kv
    torch.cuda.empty_cache()
    return dc.name, out


def other_workloads(reps, torch, synth, B, Drafter, config_from, dev):
    """The other workloads' timed units (one GPU): the 32-sequence ragged
    batch (one draft call, 512 rows), the D=2048 block-8 drafter (draft,
    prefill fuse/inject, p/q verify) and the 8192-token context over 4
    trim/append rounds. Each against its binding roof."""
    out = {}
    name, r = wl_d2048(reps, torch, synth, B, Drafter, config_from, dev)
    out[name] = r
    name, r, w = wl_32seq(reps, torch, synth, B, Drafter, config_from, dev)
    out[name] = r
    name, r = wl_ctx8192(reps, torch, synth, B, Drafter, config_from, dev, w=w)
    out[name] = r
    return out


def prefill_only(torch, synth, Drafter, config_from, dev, reps=3):
    """Only the context GEMMs: fuse and inject of a 2048-token context at the
    Qwen shape (for hardware-counter runs)."""
    out = {}
    for dc in (synth.CONFIGS[1],):
        w = synth.make_weights(dc, device=dev)
        d = Drafter(config_from(dc), w, max_seqs=1, max_tokens=dc.ctx_len, device=dev)
        kv = d.new_kv(dc.ctx_len + 64)
        feats = synth.make_feats(dc, dc.ctx_len, device=dev)
        ctx = d.fuse_context(feats)
        fu = _ev_time(lambda: d.fuse_context(feats, out=ctx), reps, torch)
        inj = _ev_time(lambda: d.inject_kv(kv, ctx, 0), reps, torch)
        T = dc.ctx_len
        f_fl = 2.0 * T * dc.n_feat * dc.hidden * dc.hidden
        i_fl = 2.0 * T * dc.hidden * 2 * dc.kv_dim * dc.n_layers
        out[dc.name] = {"fuse_us": round(fu[0], 1), "fuse_flops": f_fl,
                        "fuse_mfma_frac": round(f_fl / (fu[0] * 1e6) / MFMA_BF16_PEAK_TFLOPS, 4),
                        "inject_us": round(inj[0], 1), "inject_flops": i_fl,
                        "inject_mfma_frac": round(i_fl / (inj[0] * 1e6) / MFMA_BF16_PEAK_TFLOPS, 4)}
        d.close()
        del w, d, kv, feats, ctx
        torch.cuda.empty_cache()
    return out


def cpu_baseline(dc, w, feats_np, ctx_cache_fn, planted, budget_s=30.0):
    """One speculative round of the oracle on host cores: draft forward at the
    2048-token context, greedy verify, fuse + inject of the accepted rows."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    f = lambda t: t.float().cpu().numpy()  # noqa: E731
    wn = {k: f(v) for k, v in w.items() if k != "layers"}
    wn["layers"] = [{k: f(v) for k, v in lw.items()} for lw in w["layers"]]
    cache = ctx_cache_fn(wn)
    anchor, logits, tau_rows = planted
    t0 = time.perf_counter()
    rounds = 0
    while True:
        out = O.draft_block(dc, wn, [cache], [anchor])
        block = np.concatenate([[anchor], out["draft"][0]])
        tau, _ = O.verify_greedy(block, logits)
        H = O.fuse_context([x[:tau] for x in feats_np], wn["w_c"], wn["ctx_norm"], dc.rms_eps)
        S = cache.len
        O.cache_inject(cache, H, wn["layers"], dc, S)
        cache.trim(S)
        rounds += 1
        el = time.perf_counter() - t0
        if el > budget_s or (rounds >= 3 and el > budget_s / 3):
            break
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": rounds / el, "unit": "blocks/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": model,
            "oracle": "numpy fp64 (matrix products by the BLAS numpy links, on the threads above)",
            "sample": f"{rounds} full speculative round(s) of the numpy fp64 oracle at the "
                      f"same workload (draft forward at ctx {cache.len}, greedy verify, "
                      f"fuse+inject of the accepted rows), {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="time only the headline workload")
    ap.add_argument("--profile-all", action="store_true",
                    help="also time every stage once after the timed region")
    ap.add_argument("--copy-reference", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates HBM byte counters)")
    ap.add_argument("--only", choices=["d2048_b8_ctx2048_pq", "qwen3_8b_shape_b16_32seq_ragged",
                                       "qwen3_8b_shape_b16_ctx8192_4rounds", "prefill"],
                    help="time only this workload (or only the context GEMMs) and print its "
                         "figures; for profiler runs")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("DB", "OUT", "CMD"),
                    help="write a text summary of a rocprofv3 kernel-trace database")
    ap.add_argument("--summarize-mfma", nargs=5, metavar=("COUNTS_DB", "UTIL_DB", "TRACE_DB", "OUT", "CMDS"),
                    help="write the MFMA utilisation summary of the context GEMMs of a "
                         "--only prefill run (CMDS: the commands joined by ' ;; ')")
    ap.add_argument("--summarize-traffic", nargs=6,
                    metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB", "COPY_WRITE_DB", "OUT", "CMDS"),
                    help="write the per-kernel HBM traffic summary of four counter runs")
    ap.add_argument("--summarize-pmc", nargs=8,
                    metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB", "COPY_WRITE_DB", "PATTERN",
                             "SOURCE", "OUT", "CMDS"),
                    help="write the HBM traffic summary of a kernel from four counter runs "
                         "(CMDS: the four commands joined by ' ;; ')")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_traffic:
        a = args.summarize_traffic
        summarize_traffic(a[0], a[1], a[2], a[3], a[4], a[5].split(" ;; "))
        return
    if args.summarize_mfma:
        a = args.summarize_mfma
        f_fl = 2.0 * 2048 * 5 * 4096 * 4096
        i_fl = 2.0 * 2048 * 4096 * 2 * 1024 * 5
        ks = [("fuse, qwen3_8b_shape_b16_ctx2048 (T=2048, K=5D=20480, N=4096)",
               r"ctx_gemm<256, dfl::EpiFuse>", f_fl),
              ("inject, qwen3_8b_shape_b16_ctx2048 (T=2048, K=4096, N=5 layers x 2048)",
               r"ctx_gemm<320, dfl::EpiInject>", i_fl)]
        summarize_mfma(a[0], a[1], a[2], a[3], a[4].split(" ;; "), ks)
        return
    if args.summarize_pmc:
        a = args.summarize_pmc
        summarize_pmc(a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7].split(" ;; "))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library "
              "has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from block_diffusion_drafter_layer_amd import binding as B
    from block_diffusion_drafter_layer_amd.drafter import Drafter, config_from

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_reference:
        # 1 GiB read and 1 GiB written per copy, by the library's reference
        # copy (the weight streams' request shape)
        from block_diffusion_drafter_layer_amd import binding as Bc
        n = 1 << 30
        src = torch.ones(n // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        st = torch.cuda.current_stream().cuda_stream
        for _ in range(3):
            Bc.dflash_copy_bytes(dst.data_ptr(), src.data_ptr(), n, st)
        torch.cuda.synchronize()
        assert bool(torch.equal(dst, src))
        print(json.dumps({"copy_reference_bytes_read": n, "copy_reference_bytes_written": n,
                          "copies": 3}), flush=True)
        return
    if args.only:
        print(f"[bench] only {args.only}", file=sys.stderr, flush=True)
        if args.only == "prefill":
            res = prefill_only(torch, synth, Drafter, config_from, dev)
        elif args.only == "d2048_b8_ctx2048_pq":
            res = dict([wl_d2048(args.steps, torch, synth, B, Drafter, config_from, dev)])
        elif args.only == "qwen3_8b_shape_b16_32seq_ragged":
            name, r, _ = wl_32seq(args.steps, torch, synth, B, Drafter, config_from, dev)
            res = {name: r}
        else:
            res = dict([wl_ctx8192(args.steps, torch, synth, B, Drafter, config_from, dev)])
        print(json.dumps({"only": args.only, **res}), flush=True)
        return
    dc = synth.CONFIGS[1]
    S0, Bsz = dc.ctx_len, dc.block_size
    print(f"[bench] workload {dc.name}: generating weights", file=sys.stderr, flush=True)
    w = synth.make_weights(dc, device=dev)
    d = Drafter(config_from(dc), w, max_seqs=1, max_tokens=S0, device=dev)
    kv = d.new_kv(S0 + 64)

    # prefill: fuse + inject the 2048-token context (timed separately)
    feats = synth.make_feats(dc, S0, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for _ in range(2):
        kv.kv.len = 0
        ev[0].record()
        ctx = d.fuse_context(feats)
        ev[1].record()
        d.inject_kv(kv, ctx, 0)
        ev[2].record()
    torch.cuda.synchronize()
    fuse_us = ev[0].elapsed_time(ev[1]) * 1e3
    inject_us = ev[1].elapsed_time(ev[2]) * 1e3
    assert kv.len == S0

    anchors = torch.from_numpy(synth.make_anchor(dc)).to(dev)
    block, _, _ = d.draft_block([kv], anchors)
    torch.cuda.synchronize()
    blk = block.cpu().numpy()[0]
    taus = synth.planted_taus(dc, 64)
    n_plant = 16
    planted = []
    for j in range(n_plant):
        lg = synth.make_target_logits(dc, Bsz, round_index=j, device=dev)
        synth.plant_agreement(lg, blk, int(taus[j]) - 1)
        planted.append(lg.unsqueeze(0).contiguous())
    app_feats = [synth.make_feats(dc, Bsz, round_index=100 + j, device=dev) for j in range(n_plant)]
    app_ctx = torch.empty(Bsz, dc.hidden, dtype=torch.bfloat16, device=dev)
    tau_t = torch.empty(1, dtype=torch.int32, device=dev)
    bonus_t = torch.empty(1, dtype=torch.int32, device=dev)
    blk_out = torch.empty(1, Bsz, dtype=torch.int32, device=dev)

    def step(j):
        d.draft_block([kv], anchors, block_out=blk_out)
        d.verify(blk_out, planted[j % n_plant], tau=tau_t, bonus=bonus_t)
        tau = int(tau_t.item())
        f = [x[:tau] for x in app_feats[j % n_plant]]
        B.dflash_fuse_context(d.h, [x.data_ptr() for x in f], f[0].stride(0), tau, app_ctx.data_ptr())
        d.inject_kv(kv, app_ctx[:tau], S0)
        d.kv_trim(kv, S0)
        return tau

    for j in range(args.warmup):
        step(j)
    torch.cuda.synchronize()

    # the dominant kernel: the LM-head GEMM (one launch of ~1.25 GB of weights
    # per step; the next largest, the gate/up GEMM, streams 5 x 0.2 GB), timed
    # on the handle's stream by the library's own events around that launch
    mask = 1 << STAGE_BITS["lm_head"]
    B.dflash_profile_enable(d.h, mask, 8 * (args.steps + 1))
    dstart = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    dend = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    tau_sum = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        dstart[j].record()
        d.draft_block([kv], anchors, block_out=blk_out)
        dend[j].record()
        d.verify(blk_out, planted[j % n_plant], tau=tau_t, bonus=bonus_t)
        tau = int(tau_t.item())
        f = [x[:tau] for x in app_feats[j % n_plant]]
        B.dflash_fuse_context(d.h, [x.data_ptr() for x in f], f[0].stride(0), tau, app_ctx.data_ptr())
        d.inject_kv(kv, app_ctx[:tau], S0)
        d.kv_trim(kv, S0)
        tau_sum += tau
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    recs = B.dflash_profile_read(d.h, 8 * (args.steps + 1))
    B.dflash_profile_enable(d.h, 0, 0)
    draft_us = float(np.median([a.elapsed_time(b) for a, b in zip(dstart, dend)])) * 1e3

    per_stage = {}
    for name, ms in recs:
        per_stage.setdefault(name, []).append(ms)
    sb = stage_bytes(dc, Bsz)
    tot = {k: sum(v) for k, v in per_stage.items()}
    dom = max(tot, key=tot.get)
    avg_ms = float(np.mean(per_stage[dom]))
    achieved = sb[dom] / (avg_ms * 1e-3) / 1e9

    stages_all = None
    if args.profile_all:
        B.dflash_profile_enable(d.h, (1 << len(B.STAGES)) - 1, 256)
        for j in range(3):
            step(j)
        torch.cuda.synchronize()
        recs = B.dflash_profile_read(d.h, 256)
        B.dflash_profile_enable(d.h, 0, 0)
        acc = {}
        for name, ms in recs:
            acc.setdefault(name, []).append(ms * 1e3)
        stages_all = {k: round(float(np.sum(v)) / 3, 2) for k, v in acc.items()}

    host_loop = {"blocks_per_s": round(args.steps / elapsed, 2),
                 "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
                 "draft_block_us": round(draft_us, 1), "mean_tau": round(tau_sum / args.steps, 3)}

    # device-resident rounds: the draft reads the device length; the rest
    # verifies against planted logits j, appends the first tau fused rows at
    # the device length, trims the length back to the context and adds tau to
    # a device counter. Timed launched directly, then as captured graphs (one
    # for the draft, one per planted-logits set for the rest).
    len_dev = torch.full((1,), S0, dtype=torch.int32, device=dev)
    tau_acc = torch.zeros(1, dtype=torch.int64, device=dev)

    def dev_rest(j):
        d.verify(blk_out, planted[j], tau=tau_t, bonus=bonus_t)
        d.append_dev([kv], len_dev, tau_t, app_feats[j], Bsz)
        d.kv_trim_dev(len_dev, S0)
        tau_acc.add_(tau_t)

    def timed_rounds(draft, rest):
        for j in range(args.warmup):
            draft()
            rest(j % n_plant)
        torch.cuda.synchronize()
        tau_acc.zero_()
        ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for j in range(args.steps):
            ev0[j].record()
            draft()
            ev1[j].record()
            rest(j % n_plant)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        dt = int(tau_acc.item())
        # every round did its work: the planted agreement lengths come back
        assert dt == sum(int(taus[j % n_plant]) for j in range(args.steps)), dt
        assert int(len_dev.item()) == S0 and kv.len == S0
        dts = [a.elapsed_time(b) * 1e3 for a, b in zip(ev0, ev1)]
        timed_rounds.spread = (float(np.percentile(dts, 10)), float(np.percentile(dts, 90)))
        return el, dt, float(np.median(dts))

    # device-resident rounds launched directly
    el_e, tau_e, draft_e = timed_rounds(lambda: d.draft_block_dev([kv], len_dev, anchors, blk_out), dev_rest)
    draft_spread = timed_rounds.spread
    eager_loop = {"blocks_per_s": round(args.steps / el_e, 2), "ms_per_step": round(el_e * 1e3 / args.steps, 4),
                  "draft_block_us": round(draft_e, 1)}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g_draft = torch.cuda.CUDAGraph()
    g_rest = [torch.cuda.CUDAGraph() for _ in range(n_plant)]
    with torch.cuda.stream(side):
        B.dflash_set_stream(d.h, side.cuda_stream)
        with torch.cuda.graph(g_draft, stream=side):
            d.draft_block_dev([kv], len_dev, anchors, blk_out)
        for j in range(n_plant):
            with torch.cuda.graph(g_rest[j], stream=side):
                dev_rest(j)
    # back on the default stream (outside the side-stream context, where the
    # current stream is the default one again)
    B.dflash_set_stream(d.h, torch.cuda.current_stream().cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    el_g, _, draft_g = timed_rounds(g_draft.replay, lambda j: g_rest[j].replay())
    graph_loop = {"blocks_per_s": round(args.steps / el_g, 2), "ms_per_step": round(el_g * 1e3 / args.steps, 4),
                  "draft_block_us": round(draft_g, 1)}
    # the headline: device-resident rounds launched directly
    assert tau_e == tau_sum, (tau_e, tau_sum)
    elapsed, dev_tau, draft_us = el_e, tau_e, draft_e

    # the achieved peak of a plain device copy (the library's reference copy,
    # 1 GiB read + 1 GiB written), reported beside the 8 TB/s figure
    nb = 1 << 30
    src = torch.ones(nb // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    cst = torch.cuda.current_stream().cuda_stream
    B.dflash_copy_bytes(dst.data_ptr(), src.data_ptr(), nb, cst)
    cp = _ev_time(lambda: B.dflash_copy_bytes(dst.data_ptr(), src.data_ptr(), nb, cst), 5, torch)
    copy_gbs = 2.0 * nb / (cp[0] * 1e3)

    # the read ceiling of the weight streams' access pattern (the library's
    # read reference, nothing computed) on the LM head's weights, each time
    # after 1 GiB of other data was read (so the memory-side cache holds none
    # of it)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    lm = w["lm_head"]
    lm_bytes = lm.numel() * 2 // (128 * 1024) * (128 * 1024)

    def flush():
        B.dflash_read_bytes(src.data_ptr(), nb, sink.data_ptr(), cst)

    rd = []
    for _ in range(5):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        B.dflash_read_bytes(lm.data_ptr(), lm_bytes, sink.data_ptr(), cst)
        e1.record()
        torch.cuda.synchronize()
        rd.append(e0.elapsed_time(e1) * 1e3)
    read_gbs = lm_bytes / (float(np.median(rd)) * 1e3)

    # the draft with a cold memory-side cache: 1 GiB of other data read
    # before each timed draft
    cold = []
    for j in range(max(5, args.steps // 2)):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        d.draft_block_dev([kv], len_dev, anchors, blk_out)
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1) * 1e3)
    draft_cold = (float(np.median(cold)), float(np.percentile(cold, 10)), float(np.percentile(cold, 90)))
    del src, dst

    # DFlash 2 candidate selector on the headline block (top-16, rank 256):
    # the greedy walk, and the sampled walk (T = 1) followed by p/q
    # verification on the candidate sets
    sel = synth.make_selector(dc, device=dev)
    d.set_selector(sel["hidden_proj"], sel["pred_codebook"], sel["succ_codebook"], 16)
    s_hid = torch.empty(dc.n_layers, Bsz, dc.hidden, dtype=torch.float32, device=dev)
    s_lg = torch.empty(1, Bsz - 1, dc.vocab, dtype=torch.float32, device=dev)
    s_blk = torch.empty(1, Bsz, dtype=torch.int32, device=dev)
    d.draft_block_dev([kv], len_dev, anchors, s_blk, hidden=s_hid, logits=s_lg)
    s_last = s_hid[dc.n_layers - 1]
    s_cand = torch.empty(1, Bsz - 1, 16, dtype=torch.int32, device=dev)
    s_q = torch.empty(1, Bsz - 1, 16, dtype=torch.float32, device=dev)
    s_tl = torch.cat([s_lg[0] * 3.0, planted[0][0, -1:]]).unsqueeze(0).contiguous()
    sel_g = _ev_time(lambda: d.select_block(s_blk, s_last, s_lg, anchors), args.steps, torch)
    sel_s = _ev_time(lambda: d.select_block(s_blk, s_last, s_lg, anchors, 1.0, 1, 0, s_cand, s_q),
                     args.steps, torch)
    ver_c = _ev_time(lambda: d.verify_candidates(s_blk, s_tl, s_cand, s_q, 1.0, 2, 0), args.steps, torch)
    B.dflash_set_selector(d.h, None)
    # the selector's reads: the drafted rows' logits, the hidden projection,
    # the last layer's rows and two codes per candidate pair row
    sel_bytes = ((Bsz - 1) * dc.vocab * 4 + 256 * dc.hidden * 2 + (Bsz - 1) * dc.hidden * 4
                 + (Bsz - 1) * 2 * 16 * 256 * 2)
    selector = {"select_greedy_us": round(sel_g[0], 1), "select_sampled_us": round(sel_s[0], 1),
                "verify_candidates_us": round(ver_c[0], 1), "top_k": 16, "rank": 256,
                "select_hbm_frac": round(sel_bytes / (sel_g[0] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "select_over_draft": round(sel_g[0] / draft_e, 4)}

    # DFlash 2 dynamic two-tap conv on the headline block's rows (16 channels
    # per group): the prepare call (projection + conv) and the finish call;
    # a layer holds two instances, each with both calls
    cv = synth.make_conv(dc, 1, Bsz, 16, device=dev)
    c_y, c_corr = d.conv_prepare(cv["x"], cv["prev"], cv["base"], cv["proj"], Bsz)
    c_y2 = d.conv_finish(cv["z"], cv["zprev"], cv["base"], c_corr, Bsz)
    cp_args = (d.h, 1, Bsz, 16, cv["base"].data_ptr(), cv["proj"].data_ptr(), cv["x"].data_ptr(),
               cv["prev"].data_ptr(), c_y.data_ptr(), c_corr.data_ptr())
    cf_args = (d.h, 1, Bsz, 16, cv["base"].data_ptr(), cv["z"].data_ptr(), cv["zprev"].data_ptr(),
               c_corr.data_ptr(), c_y2.data_ptr())
    # 20 calls back to back per timed interval: the device time of a call,
    # not the host's call overhead
    def _rep(fn, n=20):
        def run():
            for _ in range(n):
                fn()
        return run
    cp_t = [t / 20 for t in _ev_time(_rep(lambda: B.dflash_conv_prepare(*cp_args)), args.steps, torch)]
    cf_t = [t / 20 for t in _ev_time(_rep(lambda: B.dflash_conv_finish(*cf_args)), args.steps, torch)]
    n_grp = dc.hidden // 16
    # algorithmic bytes: the projection and base read once, the rows read and
    # written once, the corrections written (prepare) or read (finish)
    rows_b = Bsz * dc.hidden * 4
    conv_p_bytes = 4 * n_grp * dc.hidden * 2 + 4 * dc.hidden * 2 + 2 * rows_b + dc.hidden * 4 + Bsz * 2 * n_grp * 4
    conv = {"prepare_us": round(cp_t[0], 1), "finish_us": round(cf_t[0], 1), "group_size": 16,
            "prepare_hbm_frac": round(conv_p_bytes / (cp_t[0] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "per_draft_over_draft": round(2 * dc.n_layers * (cp_t[0] + cf_t[0]) / draft_e, 4)}
    del cv, c_y, c_y2, c_corr
    # the draft with the convs inside every layer (two instances, both calls)
    cl = synth.make_conv_layers(dc, 16, device=dev)
    d.set_conv(cl)
    for _ in range(3):
        d.draft_block_dev([kv], len_dev, anchors, blk_out)
    dct = _ev_time(lambda: d.draft_block_dev([kv], len_dev, anchors, blk_out), args.steps, torch)
    d.set_conv(None)
    conv["draft_with_convs_us"] = round(dct[0], 1)
    conv["draft_with_convs_over_draft"] = round(dct[0] / draft_e - 1.0, 4)
    del cl

    ms_per_step = elapsed * 1e3 / args.steps
    value = args.steps / elapsed
    dbytes = draft_block_bytes(dc, S0)
    fuse_flops = 2.0 * S0 * dc.n_feat * dc.hidden * dc.hidden
    inject_flops = 2.0 * S0 * dc.hidden * 2 * dc.kv_dim * dc.n_layers
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": dc.name, "block_size": Bsz, "ctx_len": S0, "n_seqs": 1,
                   "hidden": dc.hidden, "draft_layers": dc.n_layers, "vocab": dc.vocab,
                   "step": "draft_block + greedy verify + fuse/inject of accepted rows + trim",
                   "loop": "device-resident, launched directly (no host read-back)"},
        "roofline": {"bound": "hbm", "kernel": f"{dom}: {STAGE_KERNEL.get(dom, (dom,))[0]}",
                     "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic(dom, dc.name), "avg_launch_us": round(avg_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": sb[dom]},
        "draft_block_us": round(draft_us, 1),
        "draft_block_us_p10_p90": [round(draft_spread[0], 1), round(draft_spread[1], 1)],
        "draft_block_hbm_frac": round(dbytes / (draft_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "draft_block_copy_frac": round(dbytes / (draft_us * 1e-6) / 1e9 / copy_gbs, 4),
        "copy_peak_GBs": round(copy_gbs, 1),
        "read_ceiling_GBs": round(read_gbs, 1),
        "draft_block_read_ceiling_frac": round(dbytes / (draft_us * 1e-6) / 1e9 / read_gbs, 4),
        "draft_block_cold_us": round(draft_cold[0], 1),
        "draft_block_cold_us_p10_p90": [round(draft_cold[1], 1), round(draft_cold[2], 1)],
        "draft_block_cold_hbm_frac": round(dbytes / (draft_cold[0] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        # the pages' per-token latency L = (T_draft + T_verify) / tau, with
        # this path's side only: the target's verify forward is not part of it
        "round_us_per_accepted_token": round(ms_per_step * 1e3 / max(dev_tau / args.steps, 1e-9), 1),
        "mean_tau": round(dev_tau / args.steps, 3),
        "host_loop": host_loop,
        "graph_loop": graph_loop,
        "prefill_fuse_us": round(fuse_us, 1),
        "prefill_fuse_mfma_frac": round(fuse_flops / (fuse_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "prefill_inject_us": round(inject_us, 1),
        "prefill_inject_mfma_frac": round(inject_flops / (inject_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "selector": selector,
        "dynamic_conv": conv,
    }
    if stages_all:
        result["stage_us_per_step"] = stages_all

    if not args.no_other_workloads:
        print("[bench] other workloads", file=sys.stderr, flush=True)
        result["other_workloads"] = other_workloads(args.steps, torch, synth, B, Drafter, config_from, dev)

    if not args.no_cpu_baseline:
        import oracle as O
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        feats_np = [x.float().cpu().numpy() for x in app_feats[0]]

        def ctx_cache(wn):
            # the timed sample does not depend on the context values: seeded
            # synthetic K/V rows stand in for the prefilled cache
            c = O.DraftCache(dc.n_layers)
            for i in range(dc.n_layers):
                k, v = synth.gen.make_context_kv(dc, i, S0)
                c.append(i, k.double().numpy(), v.double().numpy(), 0)
            return c

        result["cpu_baseline"] = cpu_baseline(
            dc, w, feats_np, ctx_cache,
            (int(blk[0]), planted[0][0].cpu().numpy(), None))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

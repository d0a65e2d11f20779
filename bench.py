"""Throughput of the layer-wise, spatially sharded VAE decode on one MI355X.

One step = one band decode (vaep_decode_bands) of the 1024x1024 bf16 preset:
latent 1x16x128x128 split into 4 uneven latent row bands (31/33/32/32), every
layer of the decoder on every band, output 1x3x1024x1024.  Latent, weights and
workspace are resident in HBM before timing starts.

Prints ONE JSON line.  `value` is decoded Mpixel/s from a plain timed region
(W warmup + K timed decodes between stream synchronisations).  A second region
of K decodes brackets every kernel launch with HIP events on the decode stream
(vaep_profile_begin/_end) to give each kernel's average duration, from which
the roofline fractions are computed with algorithmic flops / bytes per launch.
Each timed decode is also bracketed by its own pair of events, which gives
the median per-decode time beside the mean.  The CPU baseline times the
oracle's decode of the same workload (the 1024^2 preset itself) on the host
cores.  `shard_axes` times the same latent decoded on column bands of the same
sizes (vaep_decode_sharded, width axis) and with the per-request `auto` axis
policy; `tiled_baseline` times the overlap-blending tile decode
(vaep_decode_tiled) and reports its distance from the band decode and its
row-seam diagnostic.  `norm_fold` times the decode with the GroupNorm apply folded into
the latent-resolution resnet convs' operand load (vaep_model_set_norm_fold) beside
the separate apply pass.  `other_configs` times the batch-4 1024^2 preset and the
video preset in the same run (per-decode time, Mpixel/s, conv and norm
fractions).  `tiled_encode` times the tiled encode of the same preset's image size
(vaep_encode_tiled: the 2-D encoder on 32-latent tiles every 24, and as one
whole-image tile) with seeded encoder weights and image.

`--only-bands` runs nothing but the band decodes of the chosen preset (no
width, auto, tiled or other-preset decodes, no CPU baseline): the form used
under rocprofv3, so that per-kernel averages describe the band decode alone.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3] [--only-bands]
                       [--no-cpu-baseline] [--no-other-configs]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decoded Mpixel/s, 1024² bf16 VAE decode; conv MFMA util; GroupNorm GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=3, help="preset id (3 = the 1024^2 headline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true")
    ap.add_argument("--only-bands", action="store_true",
                    help="band decodes of --config only (for profiler runs)")
    ap.add_argument("--cpu-sample-latent", type=int, default=0,
                    help="latent side of a smaller oracle sample (0: the preset's own latent)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="only run a device-to-device copy of MB MiB (reference dispatch for HBM counters)")
    return ap.parse_args()


def aggregates(recs, steps):
    """Whole-decode figures: conv MFMA utilisation over every MFMA-bound conv (3x3 / 3x3x3 with
    K >= 1152 and >= 96 outputs, any kernel, algorithmic flops) and GroupNorm bandwidth over the
    tensors of at least 512 MiB (fp32 input; larger than the 256 MB last-level cache)."""
    import spatially_sharded_conv_amd._lib as L
    cf = cm = nb = nm = 0.0
    for r in recs:
        if r["step"] == L.STEP_CONV and r["ks"] == 3 and r["kt"] * 9 * r["cin"] >= 1152 and r["cout"] >= 96:
            cf += r["flops"]
            cm += r["ms"]
        if r["step"] == L.STEP_GROUPNORM and r["pixels"] * r["cin"] * 4 >= 512 << 20:
            nb += r["bytes"]
            nm += r["ms"]
    return {
        "conv_mfma_util": {"convs": "3x3 / 3x3x3, K >= 1152, N >= 96, all kernels",
                           "tflops": round(cf / (cm * 1e-3) / 1e12, 2) if cm else 0.0,
                           "frac": round(cf / (cm * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4) if cm else 0.0,
                           "ms_per_step": round(cm / steps, 4)},
        "groupnorm_large": {"tensors": ">= 512 MiB fp32",
                            "gbs": round(nb / (nm * 1e-3) / 1e9, 1) if nm else 0.0,
                            "frac": round(nb / (nm * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) if nm else 0.0,
                            "ms_per_step": round(nm / steps, 4)},
    }


def summarise(recs, steps):
    """Group per-launch records into the classes the roofline reports."""
    import spatially_sharded_conv_amd._lib as L
    out = {}

    def add(key, r):
        d = out.setdefault(key, {"launches": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0})
        d["launches"] += 1
        d["ms"] += r["ms"]
        d["flops"] += r["flops"]
        d["bytes"] += r["bytes"]

    for r in recs:
        if r["step"] == L.STEP_CONV:
            # the roofline kernel: the halo-tile kernel's 128-channel form (the 1024^2 stage's
            # plain 3x3 convs); its 256-channel form, its launches with a folded shortcut, the
            # wide kernel's launches (plain 3x3 at 256^2, sub-pixel upsample, split output), the
            # 128x128-tile kernel and the narrow conv_out are reported apart
            if r["kernel"] == L.KERNEL_CONV_HALO:
                # halo-tile kernel: 128 x (4 x 128) tiles for 128-channel outputs, 256 x (4 x 64) else
                add("conv_halo_128" if r["cout"] <= 128 else "conv_halo_256", r)
            elif r["kernel"] == L.KERNEL_CONV_HALO_X2:
                # the same kernel with a resnet's 1x1 shortcut folded in as extra K steps
                add("conv_halo_shortcut", r)
            elif r["kernel"] == L.KERNEL_CONV_WIDE256 and r["ks"] == 3 and r["ups"] == 0 and r["mode"] == 0:
                add("conv_wide_3x3", r)
            elif r["kernel"] == L.KERNEL_CONV_WIDE128X512:
                add("conv_wide_512px", r)
            elif r["kernel"] in (L.KERNEL_CONV_WIDE256, L.KERNEL_CONV_WIDE128):
                add("conv_wide_other", r)
            elif r["kernel"] == L.KERNEL_CONV_TILE128:
                add("conv_tile128", r)
            else:
                add("conv_other", r)
        elif r["step"] == L.STEP_GROUPNORM:
            add("groupnorm", r)
        elif r["step"] == L.STEP_RMSNORM:
            add("rmsnorm", r)
        elif r["step"] == L.STEP_ATTENTION:
            add("attention", r)
        else:
            add("other", r)
    total = sum(d["ms"] for d in out.values())
    for d in out.values():
        d["ms_per_step"] = d["ms"] / steps
        d["share"] = d["ms"] / total if total else 0.0
        d["tflops"] = d["flops"] / (d["ms"] * 1e-3) / 1e12 if d["ms"] else 0.0
        d["gbs"] = d["bytes"] / (d["ms"] * 1e-3) / 1e9 if d["ms"] else 0.0
        d["avg_launch_ms"] = d["ms"] / d["launches"]
    return out


def measured_traffic():
    """HBM bytes per launch of the roofline kernel from the committed rocprofv3 counter summary,
    if the kernel source is still the one the counters were taken on (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "conv_halo_128_1024_hbm_traffic.md")
    src = os.path.join(ROOT, "spatially_sharded_conv_amd", "csrc", "conv_halo.hip")
    try:
        fields = dict(l.split(": ", 1) for l in open(path).read().splitlines() if ": " in l and " " not in l.split(": ", 1)[0])
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if fields.get("conv_halo_source_sha256", "").strip() != sha:
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg_id, side):
    """The oracle as it stands, timed on the host cores: one full decode of the preset's own
    latent (side 0), or of a side x side latent of the same decoder."""
    import torch
    from oracle import Precision, decode_full
    from synth import make_latent, make_params, preset
    cfg = preset(cfg_id)
    if side:
        cfg = cfg.with_size(latent_h=side, latent_w=side, band_starts=(0, side))
    params = make_params(cfg)
    z = make_latent(cfg)
    t0 = time.perf_counter()
    y = decode_full(cfg, params, z, Precision("f32"))
    dt = time.perf_counter() - t0
    px = y.shape[0] * y.shape[-1] * y.shape[-2] * (y.shape[2] if y.dim() == 5 else 1)
    what = "the workload itself" if not side else f"a seeded {side}x{side} latent of the same decoder"
    return {"value": px / dt / 1e6, "unit": "Mpixel/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"one full decode by the oracle of {what} ({cfg.name}, latent "
                      f"{cfg.z_channels}x{cfg.latent_h}x{cfg.latent_w}, output {list(y.shape)}, {px} px) "
                      f"in {dt:.1f} s, float32 storage and float64 arithmetic",
            "seconds": round(dt, 2), "hardware_concurrency": os.cpu_count(),
            "torch_threads": torch.get_num_threads(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "cpu_model": _cpu_model()}


def build_decoder(cfg_id):
    import torch
    import spatially_sharded_conv_amd as vaep
    from synth import make_latent, make_params, preset
    cfg = preset(cfg_id)
    params = make_params(cfg)
    lc = vaep.make_config(cfg.family, cfg.dtype, cfg.z_channels, cfg.stage_channels,
                          cfg.resnets_per_stage, cfg.norm_groups, cfg.temporal_up_stages, cfg.eps)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    dev = [params[n].to(tdt).cuda() for n, _ in vaep.param_info(lc)]
    dec = vaep.Decoder(lc, dev)
    del dev, params
    latent = make_latent(cfg).to(tdt).cuda()
    out = torch.empty(cfg.output_shape(), dtype=torch.float32, device="cuda")
    ws = dec.workspace(cfg.batch, cfg.frames, cfg.latent_h, cfg.latent_w, len(cfg.band_starts) - 1)
    return cfg, dec, latent, out, ws


def timed_decodes(run, steps, warmup, stream):
    """W untimed calls, then K timed calls between stream synchronisations; each call also
    bracketed by its own events.  Returns (mean ms over the region, median ms per call, last result)."""
    import torch
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    res = None
    for k in range(steps):
        res = run()
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(steps))
    mean = ev[0].elapsed_time(ev[steps]) / steps
    med = per[steps // 2] if steps % 2 else 0.5 * (per[steps // 2 - 1] + per[steps // 2])
    return mean, med, res


def profiled_decodes(dec, run, steps, launches, stream):
    """K band decodes with every kernel launch bracketed by HIP events on the decode stream."""
    import torch
    import spatially_sharded_conv_amd as vaep
    vaep.profile_begin(dec, max_launches=steps * (launches + 8))
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        run()
    b.record(stream)
    torch.cuda.synchronize()
    recs = vaep.profile_end(dec)
    return recs, a.elapsed_time(b) / steps


def tiled_encode(cfg_id, steps, warmup, stream):
    """Time the tiled encode of preset cfg_id's image size: overlapping 32-latent tiles every 24
    and one whole-image tile; report image Mpixel/s and the distance between the two."""
    import torch
    import spatially_sharded_conv_amd as vaep
    from synth import make_encoder_params, make_image, preset
    cfg = preset(cfg_id)
    params = make_encoder_params(cfg)
    lc = vaep.make_config(cfg.family, cfg.dtype, cfg.z_channels, cfg.stage_channels,
                          cfg.resnets_per_stage, cfg.norm_groups, cfg.temporal_up_stages, cfg.eps)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    enc = vaep.Encoder(lc, [params[n].to(tdt).cuda() for n, _ in vaep.encoder_param_info(lc)])
    img = make_image(cfg).to(tdt).cuda()
    b, _, h, w = img.shape
    pixels = b * h * w
    res = {"image": list(img.shape)}
    outs = {}
    for name, tile, stride in (("tiles_32_every_24", 32, 24), ("whole_image", max(cfg.latent_h, cfg.latent_w),
                                                                  max(cfg.latent_h, cfg.latent_w))):
        out = torch.empty(cfg.moments_shape(), dtype=torch.float32, device="cuda")
        ws = enc.workspace(b, h, w, tile, stride)
        ms, med, (rc, info) = timed_decodes(lambda: enc.encode_tiled(img, tile, stride, out, ws, stream), steps,
                                            warmup, stream)
        res[name] = {"tiles": info.bands_used, "ms_per_step": round(ms, 4), "ms_median": round(med, 4),
                     "mpixel_s": round(pixels / (ms * 1e-3) / 1e6, 3)}
        outs[name] = out
        del ws
    d = outs["tiles_32_every_24"].double() - outs["whole_image"].double()
    res["rel_l2_tiles_vs_whole_image"] = round((d.norm() / outs["whole_image"].double().norm()).item(), 5)
    enc.close()
    del outs, img
    torch.cuda.empty_cache()
    return res


def other_config(cfg_id, steps, warmup, stream):
    """Per-decode time, throughput and the conv / norm fractions of another preset's band decode."""
    cfg, dec, latent, out, ws = build_decoder(cfg_id)
    starts = cfg.band_starts
    pixels = out.numel() // 3
    run = lambda: dec.decode_bands(latent, starts, out, ws, stream)
    mean, med, (rc, info) = timed_decodes(run, steps, warmup, stream)
    recs, _ = profiled_decodes(dec, run, steps, info.n_launches, stream)
    cls = summarise(recs, steps)
    agg = aggregates(recs, steps)
    nk = "groupnorm" if "groupnorm" in cls else "rmsnorm"
    norm = cls.get(nk, {"gbs": 0.0, "ms_per_step": 0.0})
    dec.close()
    return {"workload": f"{cfg.name}: band decode of a seeded {cfg.z_channels}x{cfg.latent_h}x{cfg.latent_w} latent "
                        f"(batch {cfg.batch}{', frames ' + str(cfg.frames) if cfg.is_video else ''}) on "
                        f"{len(starts) - 1} latent row bands {[b - a for a, b in zip(starts, starts[1:])]}, "
                        f"output {list(out.shape)}",
            "ms_per_step": round(mean, 4), "ms_per_step_median": round(med, 4),
            "mpixel_s": round(pixels / (mean * 1e-3) / 1e6, 3),
            "conv_mfma_util": agg["conv_mfma_util"],
            "norm": {"kernel": nk, "gbs": round(norm["gbs"], 1), "frac": round(norm["gbs"] / PEAK_HBM_GBS, 4),
                     "ms_per_step": round(norm["ms_per_step"], 4)},
            "breakdown_ms": {k: round(v["ms_per_step"], 4) for k, v in sorted(cls.items())}}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: every band of the decode runs on this device and there "
              f"is no multi-GPU path in this library (asked for --gpus {args.gpus}, WORLD_SIZE {world}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}), flush=True)
        return
    cfg, dec, latent, out, ws = build_decoder(args.config)
    starts = cfg.band_starts
    nb = len(starts) - 1
    stream = torch.cuda.current_stream()
    pixels = out.numel() // 3

    # plain timed region (value), with per-decode events for the median
    run = lambda: dec.decode_bands(latent, starts, out, ws, stream)
    ms, ms_med, (rc, info) = timed_decodes(run, args.steps, args.warmup, stream)
    value = pixels / (ms * 1e-3) / 1e6

    # event-bracketed region: per-launch kernel durations on the decode stream
    recs, ms_prof = profiled_decodes(dec, run, args.steps, info.n_launches, stream)
    cls = summarise(recs, args.steps)
    conv = cls.get("conv_halo_128", {"tflops": 0.0, "flops": 0.0, "bytes": 0.0, "launches": 1, "avg_launch_ms": 0.0})
    gn = cls.get("groupnorm") or cls.get("rmsnorm") or {"gbs": 0.0}

    roofline = {
        "kernel": "conv_halo<128, 128> (3x3 band conv of the 1024^2 stage: 128 output channels x 4 rows x 128 "
                  "pixels per workgroup, halo pixel tile and weights staged in LDS by buffer-to-LDS loads once per "
                  "32-channel block, 8 waves, v_mfma_f32_32x32x16_bf16, fp32 output with GroupNorm records)",
        "bound": "mfma",
        "achieved": round(conv["tflops"], 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(conv["tflops"] / PEAK_BF16_TFLOPS, 4),
        "traffic": measured_traffic() if args.config == 3 else None,
        "launches_per_step": conv["launches"] // args.steps,
        "avg_launch_ms": round(conv["avg_launch_ms"], 4),
        "flops_per_launch": conv["flops"] / max(1, conv["launches"]),
        "algorithmic_bytes_per_launch": conv.get("bytes", 0.0) / max(1, conv["launches"]),
    }
    axes, tiled, fold = {}, None, None
    if not args.only_bands and cfg.norm_groups > 0:
        # the GroupNorm apply folded into the operand load of the latent-resolution resnet
        # convs (vaep_model_set_norm_fold) beside the separate apply pass timed above
        dec.set_norm_fold(True)
        f_ms, f_med, (_, finfo) = timed_decodes(run, args.steps, args.warmup, stream)
        frecs, _ = profiled_decodes(dec, run, args.steps, finfo.n_launches, stream)
        dec.set_norm_fold(False)
        fcls = summarise(frecs, args.steps)
        pick = lambda c, k: round(c.get(k, {}).get("ms_per_step", 0.0), 4)
        fold = {"ms_per_step": round(f_ms, 4), "ms_per_step_median": round(f_med, 4),
                "mpixel_s": round(pixels / (f_ms * 1e-3) / 1e6, 3),
                "speedup_vs_separate_apply": round(ms / f_ms, 4),
                "groupnorm_ms": pick(fcls, "groupnorm"), "conv_tile128_ms": pick(fcls, "conv_tile128"),
                "separate_apply": {"groupnorm_ms": pick(cls, "groupnorm"), "conv_tile128_ms": pick(cls, "conv_tile128")}}
    if not args.only_bands:
        # the same workload sharded along the width (the row bands' sizes laid across the
        # columns when they fit) and with the per-request axis policy
        sizes = [b - a for a, b in zip(starts, starts[1:])]
        col = [0]
        for v in sizes:
            col.append(col[-1] + v)
        for name, st in (("width", tuple(col) if col[-1] == cfg.latent_w else None), ("auto", None)):
            a_ms, a_med, (_, ainfo) = timed_decodes(
                lambda: dec.decode_sharded(latent, name, nb, out, ws, st, stream), args.steps, args.warmup, stream)
            axes[name] = {"axis": {1: "height", 2: "width", 3: "dense", 4: "tile"}.get(ainfo.axis, ainfo.axis),
                          "bands": list(st) if st else ainfo.bands_used,
                          "ms_per_step": round(a_ms, 4), "mpixel_s": round(pixels / (a_ms * 1e-3) / 1e6, 3)}
    if not args.only_bands and not cfg.is_video:
        # the overlap-blending tile decode the sharded decode replaces (latent tiles of 32 with
        # stride 24: 256-pixel tiles every 192 output pixels at 8x upsampling), same latent
        tile, tstride = 32, 24
        band_out = torch.empty_like(out)
        dec.decode_bands(latent, starts, band_out, ws, stream)
        tws = dec.tiled_workspace(cfg.batch, cfg.frames, cfg.latent_h, cfg.latent_w, tile, tstride)
        tout = torch.empty_like(out)
        t_ms, t_med, _ = timed_decodes(lambda: dec.decode_tiled(latent, tile, tstride, tout, tws, stream),
                                       args.steps, args.warmup, stream)

        # seam diagnostic (validation page): mean absolute jump between adjacent rows of the
        # per-pixel RGB mean, 0-255 units; at the tiles' row boundaries and over all rows
        def row_jumps(y):
            m = (y.double().mean(dim=1) + 1.0) * 127.5
            return (m[:, 1:, :] - m[:, :-1, :]).abs().mean(dim=(0, 2))
        keep = tstride * (out.shape[-1] // cfg.latent_w)
        bnd = torch.arange(keep - 1, out.shape[-2] - 1, keep, device=out.device)
        jt, jb = row_jumps(tout), row_jumps(band_out)
        d = (tout.double() - band_out.double())
        del tws
        tiled = {"tile_latent": tile, "stride_latent": tstride, "ms_per_step": round(t_ms, 4),
                 "mpixel_s": round(pixels / (t_ms * 1e-3) / 1e6, 3),
                 "rel_l2_vs_band_decode": round((d.norm() / band_out.double().norm()).item(), 5),
                 "row_jump_at_tile_rows": round(jt[bnd].mean().item(), 4),
                 "row_jump_at_those_rows_band_decode": round(jb[bnd].mean().item(), 4),
                 "row_jump_all_rows": round(jt.mean().item(), 4)}
    dec.close()
    del ws, out, latent
    torch.cuda.empty_cache()
    encode = None
    if not args.only_bands and not cfg.is_video:
        encode = tiled_encode(args.config, max(3, min(args.steps, 8)), max(1, args.warmup), stream)
    others = {}
    if not args.only_bands and not args.no_other_configs:
        for cid in (4, 5):
            if cid != args.config:
                others[f"config{cid}"] = other_config(cid, max(5, min(args.steps, 8)), max(1, args.warmup), stream)
                torch.cuda.empty_cache()
    norm_key = "groupnorm" if "groupnorm" in cls else "rmsnorm"
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "Mpixel/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(ms_med, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: band decode of a seeded {cfg.z_channels}x{cfg.latent_h}x{cfg.latent_w} "
                        f"latent (batch {cfg.batch}{', frames ' + str(cfg.frames) if cfg.is_video else ''}) "
                        f"on {nb} latent row bands {[b - a for a, b in zip(starts, starts[1:])]}, "
                        f"output {list(cfg.output_shape())}",
            "batch": cfg.batch, "bands": list(starts), "random_init": True,
            "storage": "bf16 weights/latent/matrix operands, fp32 conv outputs and statistics",
        },
        "roofline": roofline,
        "norm": {
            "kernel": f"{norm_key} (stats -> merge -> apply + SiLU)" if norm_key == "groupnorm" else "rmsnorm + SiLU",
            "bound": "hbm", "achieved": round(gn.get("gbs", 0.0), 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gn.get("gbs", 0.0) / PEAK_HBM_GBS, 4),
        },
        "breakdown": {k: {"ms_per_step": round(v["ms_per_step"], 4), "share": round(v["share"], 4),
                          "launches_per_step": v["launches"] // args.steps,
                          "tflops": round(v["tflops"], 2), "gbs": round(v["gbs"], 1)}
                      for k, v in sorted(cls.items())},
        "profiled_ms_per_step": round(ms_prof, 4),
        "shard_axes": axes,
        "norm_fold": fold,
        "tiled_baseline": tiled,
        "tiled_encode": encode,
        **aggregates(recs, args.steps),
        "other_configs": others,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and not args.only_bands:
        line["cpu_baseline"] = cpu_baseline(args.config, args.cpu_sample_latent)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Batch-1 greedy decode benchmark of the MI355X persistent decode megakernel.

One step = one decode launch = one token of the whole model (every op of the decode step runs
inside that launch). Default workload: TinyLlama-1.1B shape, int8 W8A16 (per-output-channel
fp16 scales, bf16 activations and KV cache, fp32 accumulation), random init, KV cache rows
0..511 prefilled with N(0,1), greedy decode chained on the device from position 512.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--records PATH]

Prints one JSON line: tokens/s and ms/step over the timed region, the roofline of the kernel
(algorithmic HBM bytes per launch over the mean launch duration, both timed with HIP events on
the launch stream, against the 8 TB/s HBM peak), the CPU oracle timed on a bounded sample of
the same workload and, under "prefill", the prompt-prefill kernel on a 256-token prompt
(prompt tokens/s, and algorithmic FLOPs over the launch duration against the bf16 matrix-core
peak).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "batch-1 decode tokens/s + achieved HBM GB/s vs 8 TB/s peak, per model"

# name -> (start position = prefilled cache rows, description)
WORKLOADS = {
    "tinyllama_int8": (512, "TinyLlama-1.1B shape, int8 W8A16, batch-1 greedy decode from pos 512"),
    "smollm2_135m_bf16": (16, "SmolLM2-135M shape, bf16, batch-1 greedy decode from pos 16"),
    "llama7b_bf16": (2048, "Llama-7B shape, bf16, batch-1 greedy decode at context 2048"),
    "llama7b_int8": (2048, "Llama-7B shape, int8 W8A16, batch-1 greedy decode at context 2048"),
    "llama3_8b_int4": (4096, "Llama-3-8B shape, int4 g128, batch-1 greedy decode at context 4096"),
    "tiny_fp32": (8, "tiny Llama shape, fp32, batch-1 greedy decode from pos 8"),
}

# counters measured for the default workload by rocprofv3 (--pmc FETCH_SIZE, then WRITE_SIZE),
# scaled by the same counters on a device copy of known size; None until measured for the
# current kernel
TRAFFIC_BYTES_PER_LAUNCH = 1094293439
# the same for the prefill kernel on a 256-token prompt of the default workload
PREFILL_TRAFFIC_BYTES_PER_LAUNCH = 2993278682


def weight_bytes(shape) -> int:
    """Bytes of the model the step must read once: every projection in its stored format
    (int8 codes + one fp16 scale per output row; int4 nibbles + one fp16 scale per 128
    inputs), the norm gains and one embedding row in the activation type."""
    import amk_inputs as I
    H, I_, V, L = shape.hidden, shape.intermediate, shape.vocab, shape.n_layers
    qd, kd = shape.q_dim, shape.kv_dim
    mats = [(qd, H), (kd, H), (kd, H), (H, qd), (I_, H), (I_, H), (H, I_)]
    act = 4 if shape.act_f32 else 2

    def mbytes(rows, cols):
        if shape.wfmt == I.WF_F32:
            return 4 * rows * cols
        if shape.wfmt == I.WF_BF16:
            return 2 * rows * cols
        if shape.wfmt == I.WF_INT8:
            return rows * cols + 2 * rows
        return rows * cols // 2 + 2 * rows * (cols // 128)

    per_layer = sum(mbytes(r, c) for r, c in mats) + 2 * H * act
    return L * per_layer + mbytes(V, H) + H * act + H * act


def kv_bytes(shape, pos: int) -> int:
    """KV cache bytes of one step at position pos: rows [0, pos) read, row pos written."""
    act = 4 if shape.act_f32 else 2
    row = shape.n_layers * 2 * shape.n_kv_heads * shape.head_dim * act
    return row * pos + row


MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_flops(shape, n_tokens: int, pos0: int = 0) -> int:
    """Algorithmic FLOPs of one prefill of n_tokens tokens from pos0: every projection of every
    token (2 per weight), causal attention (q.k and p.v, 2 x 2 x head_dim per query head and
    visible position) and the LM head of the last token only."""
    H, I_, L = shape.hidden, shape.intermediate, shape.n_layers
    qd, kd = shape.q_dim, shape.kv_dim
    per_tok = L * (qd * H + 2 * kd * H + H * qd + 3 * I_ * H)
    vis = sum(pos0 + m + 1 for m in range(n_tokens))
    attn = 4 * shape.n_heads * shape.head_dim * vis * L
    return 2 * n_tokens * per_tok + attn + 2 * shape.vocab * H


def prefill_leg(dec, shape, n_tokens: int = 256, reps: int = 10, traffic=None) -> dict:
    """Prompt prefill (amk_prefill) of n_tokens synthetic tokens at position 0, timed with HIP
    events around each launch on the launch stream; roofline against the bf16 matrix-core peak
    (the projections run as bf16 MFMA GEMM tiles, int8 and int4 codes widened exactly)."""
    import torch
    import amk_inputs as I
    toks = torch.tensor(I.prompt_tokens(shape, n_tokens, stream=7), dtype=torch.int32, device="cuda")
    tout = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(3):   # the first call lowers, validates and uploads this chunk size's schedule
        dec.prefill(toks, 0, tout)
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
    for r in range(reps):
        marks[2 * r].record(stream)
        dec.prefill(toks, 0, tout)
        marks[2 * r + 1].record(stream)
    torch.cuda.synchronize()
    ms = sum(marks[2 * r].elapsed_time(marks[2 * r + 1]) for r in range(reps)) / reps
    fl = prefill_flops(shape, n_tokens)
    tf = fl / (ms * 1e-3) / 1e12
    return {"tokens": n_tokens, "launches": (n_tokens + 255) // 256, "value": round(n_tokens / (ms * 1e-3), 1),
            "unit": "prompt tokens/s", "ms_per_prefill": round(ms, 4),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 5), "flops_per_launch": fl, "traffic": traffic},
            "vs_decode": "one decode launch per prompt token at the timed decode rate"}


def cpu_baseline(shape, w, pos0: int, budget_s: float = 12.0):
    """The oracle (plain C, fp64, OpenMP over rows and heads) timed on the host's cores on
    consecutive greedy steps of the same workload from pos0, stopping after budget_s."""
    import amk_inputs as I
    import oracle
    ref = oracle.OracleModel(shape, w)
    if pos0:
        oracle.prefill_model(ref, shape, pos0)
    tok = int(I.prompt_tokens(shape, 1, stream=99)[0])
    times = []
    t_end = time.perf_counter() + budget_s
    pos = pos0
    while time.perf_counter() < t_end or len(times) < 2:
        t0 = time.perf_counter()
        _, _, tok = ref.step(tok, pos)
        times.append(time.perf_counter() - t0)
        pos += 1
        if pos >= ref.max_ctx:
            break
    ref.close()
    times.sort()
    med = times[len(times) // 2]
    cores = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    return {"value": round(1.0 / med, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(times)} greedy oracle steps from pos {pos0} (median step {med * 1e3:.1f} ms)"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="tinyllama_int8", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prompt-prefill leg")
    ap.add_argument("--prefill-tokens", type=int, default=256)
    ap.add_argument("--records", default=None, help="also append the JSON line to this file")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a device-to-device copy of this size (the traffic counters' calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU: --gpus must be 1 (the multi-GPU "
                                   "sharding is a design only)"}))
        return 2

    import torch
    import amk_inputs as I
    import persistent_megakernel_amd as M

    torch.cuda.set_device(0)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        a = torch.ones(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return 0

    pos0, desc = WORKLOADS[args.workload]
    base = I.SHAPES[args.workload]
    K, W = args.steps, args.warmup
    shape = base.replace(max_ctx=max(base.max_ctx, pos0 + W + K + 1))
    print(f"[bench] workload {args.workload}: generating weights", file=sys.stderr, flush=True)
    w = I.make_weights(shape)
    dec = M.Decoder(shape, w)
    if pos0:
        for l in range(shape.n_layers):
            dec.set_kv_prefix(l, I.kv_prefill(shape, pos0, l))
    tok0 = int(I.prompt_tokens(shape, 1, stream=99)[0])
    toks = torch.full((W + K + 1,), -1, dtype=torch.int32, device="cuda")
    toks[0] = tok0
    stream = torch.cuda.current_stream()
    print(f"[bench] warmup {W} steps", file=sys.stderr, flush=True)
    for s in range(W):
        dec.step(toks[s:s + 1], pos0 + s, toks[s + 1:s + 2])
    torch.cuda.synchronize()
    # events around the whole timed region (throughput) and around every launch (the kernel's own
    # duration, for the roofline), all on the launch stream
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(2 * K)]
    t0 = time.perf_counter()
    start.record(stream)
    for k, s in enumerate(range(W, W + K)):
        marks[2 * k].record(stream)
        dec.step(toks[s:s + 1], pos0 + s, toks[s + 1:s + 2])
        marks[2 * k + 1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = start.elapsed_time(stop)
    launch_ms = sum(marks[2 * k].elapsed_time(marks[2 * k + 1]) for k in range(K)) / K
    status = dec.status()
    pf = None
    if not args.no_prefill and not status:
        print(f"[bench] prefill {args.prefill_tokens} tokens", file=sys.stderr, flush=True)
        pf = prefill_leg(dec, shape, args.prefill_tokens,
                         traffic=PREFILL_TRAFFIC_BYTES_PER_LAUNCH
                         if args.workload == "tinyllama_int8" and args.prefill_tokens == 256 else None)
        status = dec.status()
    dec.close()
    if status:
        print(json.dumps({"error": f"device status {status}"}))
        return 1
    ms_step = ev_ms / K
    # algorithmic bytes per launch, averaged over the timed positions
    wb = weight_bytes(shape)
    kvb = sum(kv_bytes(shape, pos0 + s) for s in range(W, W + K)) / K
    per_launch = wb + kvb
    achieved = per_launch / (launch_ms * 1e-3) / 1e9
    rec = {
        "metric": METRIC, "value": round(1e3 / ms_step, 2), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {I.WF_F32: "f32", I.WF_BF16: "bf16", I.WF_INT8: "w8a16",
                                       I.WF_INT4: "w4a16"}[shape.wfmt],
        "data": "synthetic (seeded random-init weights, N(0,1) prefilled KV cache)",
        "config": {"workload": desc, "hidden": shape.hidden, "layers": shape.n_layers,
                   "heads": shape.n_heads, "kv_heads": shape.n_kv_heads, "intermediate": shape.intermediate,
                   "vocab": shape.vocab, "start_pos": pos0, "batch": 1},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": TRAFFIC_BYTES_PER_LAUNCH if args.workload == "tinyllama_int8" else None},
        "bytes_per_launch": int(per_launch),
        "us_per_token": round(ms_step * 1e3, 2),
        "us_per_launch": round(launch_ms * 1e3, 2),
        "wall_s_timed": round(wall, 4),
    }
    if pf is not None:
        pf["speedup_vs_decode_per_token"] = round(pf["value"] / rec["value"], 1)
        rec["prefill"] = pf
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(base.replace(max_ctx=max(base.max_ctx, pos0 + 64)), w, pos0)
    line = json.dumps(rec)
    print(line, flush=True)
    if args.records:
        with open(args.records, "a") as f:
            f.write(line + "\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())

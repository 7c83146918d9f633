"""Throughput of the paged-KV attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = one pass of the whole path at Qwen3-0.6B attention shapes (16 q /
8 kv heads, head_dim 128, bf16):
  * prefill  : pa_store_kv of a 4096-token prompt, then pa_prefill_varlen
               (1 sequence x 4096, causal, block_size 16);
  * decode   : for each of 28 layers, pa_store_kv of the 256 new tokens, then
               pa_decode over 256 sequences with contexts uniform in
               [100, 2048] (block_size 256, one KV pool per layer).
Inputs are synthetic (seeded) and resident in HBM before timing starts.

Prints ONE JSON line.  `value` is the decode KV read rate (GB/s: bytes of
every visible K and V row, once per KV head, over the decode calls' time);
`prefill.value` is the prefill rate (TFLOP/s: 4*d*Hq per visible causal
pair over the prefill call's time).  Both come from HIP events recorded on
the stream the kernels run on.  `roofline` is for the decode kernel (the
dominant cost), `prefill.roofline` for the prefill kernel.  `cpu_baseline`
times the fp64 CPU oracle on a bounded sample of the same decode workload.

Outside the timed step, the INT8 KV cache is measured on the same shapes:
`int8_decode` times pa_decode_int8 over INT8 pools quantized from four of
the decode layers (bytes: every visible row's int8 codes and fp16 scale,
K and V, once per KV head), `int8_store` times pa_store_kv_int8 of the
4096-token prompt and `int8_prefill` pa_prefill_varlen_int8 over it.
`prefill_mixed` times the 8192-token chunked-prefill batch in one call.
The fp16 legs (`f16_decode`, `f16_prefill`) run the same shapes over fp16
pools and queries, and `fork_microbench_decode` times fp16 against INT8
pools at the fork's microbenchmark shape (batch 8, 512 keys per row).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 MFMA


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--layers", type=int, default=28)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-int8", action="store_true", help="skip the INT8 KV-cache measurements")
    p.add_argument("--no-f16", action="store_true", help="skip the fp16 measurements")
    p.add_argument("--no-graph", action="store_true", help="skip the HIP graph replay measurements")
    p.add_argument("--no-small", action="store_true",
                   help="skip the small-shape timings (they launch the long prompt's prefill kernel too, "
                        "which would mix into a kernel trace's per-kernel statistics)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run one plain 1 GiB device copy (HBM counter calibration)")
    p.add_argument("--no-c5b", action="store_true", help="skip the 64 x 32768 long-context decode")
    p.add_argument("--only-c5b", action="store_true",
                   help="run only the 64 x 32768 long-context decode (for a kernel trace of that shape alone); "
                        "prints its JSON block")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only (the kernels run on one GPU's share); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_attention_mapping_amd as pa
    import workloads as W

    torch.cuda.set_device(0)
    dev = "cuda"
    if args.only_c5b:
        res = c5b_measure(pa, W, max(args.steps, 2))
        if args.calibrate_copy:
            src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
            torch.empty_like(src).copy_(src)
            torch.cuda.synchronize()
        print(json.dumps({"decode_c5b": res}), flush=True)
        return

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---------------- prefill input: 1 x 4096, block 16 ----------------------
    pf = W.c5a_long()
    pf_k, pf_v = (torch.zeros((pf.num_blocks, pf.block_size, pf.num_kv_heads, pf.head_dim),
                              dtype=torch.bfloat16, device=dev) for _ in range(2))
    pf_q, pf_kn, pf_vn = to_dev(pf.q), to_dev(pf.k_new), to_dev(pf.v_new)
    pf_slots = to_dev(pf.slot_new)
    pf_cuq, pf_cuk = to_dev(pf.cu_seqlens_q), to_dev(pf.cu_seqlens_k)
    pf_off, pf_bt = to_dev(np.asarray(pf.q_offsets, np.int32)), to_dev(pf.block_table)
    pf_out = torch.empty_like(pf_q)
    pf_ws_bytes = pa.pa_prefill_workspace_bytes(1, pf.total_q, pf.num_q_heads, pf.max_seqlen_q,
                                                pf.max_seqlen_k, pf_k)
    pf_ws = torch.empty(max(pf_ws_bytes, 1), dtype=torch.uint8, device=dev)
    pf_flops = 4.0 * pf.head_dim * pf.num_q_heads * pf.causal_pairs

    # ---------------- decode input: 256 x U[100,2048], 28 layer pools -------
    lay = W.c4_decode_layout()
    L = args.layers
    nb, bs, hkv, d, hq = lay.num_blocks, lay.block_size, lay.num_kv_heads, lay.head_dim, lay.num_q_heads
    k_pools, v_pools, qs, k_news, v_news = [], [], [], [], []
    for layer in range(L):
        k_pools.append(W.device_normal((nb, bs, hkv, d), 4100 + 2 * layer))
        v_pools.append(W.device_normal((nb, bs, hkv, d), 4101 + 2 * layer))
        qs.append(W.device_normal((lay.num_seqs, hq, d), 9000 + layer))
        k_news.append(W.device_normal((lay.num_seqs, hkv, d), 7000 + 2 * layer))
        v_news.append(W.device_normal((lay.num_seqs, hkv, d), 7001 + 2 * layer))
    ctx_d, bt_d, slot_d = to_dev(lay.context_lens), to_dev(lay.block_table), to_dev(lay.slot_new)
    dec_out = torch.empty((lay.num_seqs, hq, d), dtype=torch.bfloat16, device=dev)
    ws_bytes = pa.pa_decode_workspace_bytes(lay.num_seqs, hq, lay.max_context_len, k_pools[0])
    dec_ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    order_d = torch.empty(lay.num_seqs, dtype=torch.int32, device=dev)
    kv_bytes_layer = lay.kv_bytes()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(ev=None):
        # prefill: store the prompt's K/V, then causal varlen attention
        if ev is not None:
            ev["pf"][0].record(stream)
        pa.pa_store_kv(pf_kn, pf_vn, pf_slots, pf_k, pf_v)
        if ev is not None:
            ev["pf_attn"][0].record(stream)
        pa.pa_prefill_varlen(pf_q, pf_k, pf_v, pf_cuq, pf_cuk, pf_off, pf_bt, pf.max_seqlen_q,
                             pf.max_seqlen_k, pf.scale, out=pf_out, workspace=pf_ws)
        if ev is not None:
            ev["pf_attn"][1].record(stream)
            ev["pf"][1].record(stream)
        # decode: the longest-first row order once per step (same context
        # lengths in every layer), then every layer stores its new token and
        # attends
        if ev is not None:
            ev["order"][0].record(stream)
        pa.pa_decode_order(ctx_d, row_order=order_d)
        if ev is not None:
            ev["order"][1].record(stream)
        for layer in range(L):
            pa.pa_store_kv(k_news[layer], v_news[layer], slot_d, k_pools[layer], v_pools[layer])
            if ev is not None:
                ev["dec"][layer][0].record(stream)
            pa.pa_decode(qs[layer], k_pools[layer], v_pools[layer], ctx_d, bt_d, lay.max_context_len,
                         lay.scale, out=dec_out, workspace=dec_ws, row_order=order_d)
            if ev is not None:
                ev["dec"][layer][1].record(stream)

    def new_events():
        mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        return {"pf": (mk(), mk()), "pf_attn": (mk(), mk()), "order": (mk(), mk()),
                "dec": [(mk(), mk()) for _ in range(L)]}

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    per_step_events = [new_events() for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(per_step_events[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    ms_total = t_start.elapsed_time(t_end)
    ms_per_step = ms_total / args.steps
    dec_ms = [e["dec"][l][0].elapsed_time(e["dec"][l][1]) for e in per_step_events for l in range(L)]
    pf_attn_ms = [e["pf_attn"][0].elapsed_time(e["pf_attn"][1]) for e in per_step_events]
    pf_ms = [e["pf"][0].elapsed_time(e["pf"][1]) for e in per_step_events]
    order_ms = [e["order"][0].elapsed_time(e["order"][1]) for e in per_step_events]
    dec_call_ms = float(np.mean(dec_ms))
    # whole decode phase: the per-step order call is charged to the layers
    decode_gbps = kv_bytes_layer * L * args.steps / ((sum(dec_ms) + sum(order_ms)) * 1e-3) / 1e9
    pf_call_ms = float(np.mean(pf_attn_ms))
    prefill_tflops = pf_flops / (pf_call_ms * 1e-3) / 1e12

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    int8 = None if args.no_int8 else int8_measure(pa, W, lay, pf, k_pools, v_pools, qs, ctx_d, bt_d, order_d,
                                                  pf_kn, pf_vn, pf_slots, dec_call_ms, max(args.steps, 2),
                                                  (pf_q, pf_cuq, pf_cuk, pf_off, pf_bt, pf_flops, pf_call_ms))

    graph = None if args.no_graph else graph_measure(step, ms_per_step, max(args.steps, 2))
    mixed = mixed_prefill_measure(pa, W, max(args.steps, 2))
    d256 = d256_prefill_measure(pa, W, max(args.steps, 2))
    small = None if args.no_small else small_configs_measure(pa, W)

    f16 = None if args.no_f16 else f16_measure(pa, W, lay, ctx_d, bt_d, order_d, dec_call_ms, pf_call_ms,
                                               max(args.steps, 2))
    c5b = None if args.no_c5b else c5b_measure(pa, W, max(args.steps, 2))
    # the prompt's store alone (K and V rows read, then written into the
    # pool): 20 calls back to back between two events (per call: the kernel
    # and the gap to the next), and single calls each between two events
    # (which adds the event packets' own few microseconds to a 7 us kernel)
    store_call = lambda: pa.pa_store_kv(pf_kn, pf_vn, pf_slots, pf_k, pf_v)  # noqa: E731
    st_ms = _time_calls([lambda: [store_call() for _ in range(20)]], max(args.steps, 5)) / 20
    st1_ms = _time_calls([store_call], max(args.steps, 10))
    st_bytes = 2 * 2 * pf.total_q * pf.num_kv_heads * pf.head_dim * 2
    store = {"workload": f"pa_store_kv of {pf.total_q} tokens x {pf.num_kv_heads} KV heads x {pf.head_dim}, bf16, "
                         f"block {pf.block_size}",
             "avg_launch_us": round(st_ms * 1e3, 2), "bytes_per_launch": st_bytes,
             "achieved_gbps": round(st_bytes / (st_ms * 1e-3) / 1e9, 2),
             "frac_hbm": round(st_bytes / (st_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
             "single_call_us": round(st1_ms * 1e3, 2),
             "traffic": measured_traffic("store")}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(lay, k_pools[0], v_pools[0], qs[0], pf, pf_k, pf_v, pf_q)

    result = {
        "metric": "paged-attn decode KV GB/s + prefill TFLOP/s (Qwen3-0.6B shapes, 1 GPU)",
        "value": round(decode_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V/Q; seeded lengths and shuffled block tables)",
        "seeds": {
            "prefill_1x4096": {"lengths_table_values": pf.seed},
            "decode_256": {"lengths_table": lay.seed, "k_pool_layer_l": "4100+2l", "v_pool_layer_l": "4101+2l",
                           "q_layer_l": "9000+l", "new_k_layer_l": "7000+2l", "new_v_layer_l": "7001+2l"},
            "decode_64x32768": {"lengths_table": W.c5b_decode_layout().seed, "k_pool": 5330, "v_pool": 5331,
                                "q": 5332},
            "prefill_mixed_8192": {"lengths_table": W.c5a_mixed(with_values=False).seed, "k_pool": 5400,
                                   "v_pool": 5401, "q": 5402},
            "prefill_d256_1x4096": {"lengths_table": 5500, "k_pool": 5501, "v_pool": 5502, "q": 5503},
        },
        "config": {
            "workload": (f"qwen3-0.6b attention step: store+prefill 1x4096 causal (block 16) + "
                         f"{L} layers x (store 256 + decode 256 seqs, ctx U[100,2048], block 256)"),
            "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": d,
            "decode_seqs": lay.num_seqs, "decode_sum_ctx": int(lay.context_lens.sum()),
            "decode_layers": L, "prefill_tokens": pf.total_q,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("pa_decode (split-K kernel + log-sum-exp merge), one call per layer, rows in the "
                       "longest-first order of one pa_decode_order call per step"),
            "achieved": round(kv_bytes_layer / (dec_call_ms * 1e-3) / 1e9, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(kv_bytes_layer / (dec_call_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic("decode"),
            "bytes_per_launch": kv_bytes_layer,
            "avg_launch_us": round(dec_call_ms * 1e3, 2),
            "launch_us_median_min_max": [round(float(np.median(dec_ms)) * 1e3, 2), round(min(dec_ms) * 1e3, 2),
                                         round(max(dec_ms) * 1e3, 2)],
            "order_us_per_step": round(float(np.mean(order_ms)) * 1e3, 2),
        },
        "prefill": {
            "value": round(prefill_tflops, 2),
            "unit": "TFLOP/s",
            "flops_per_launch": pf_flops,
            "avg_launch_us": round(pf_call_ms * 1e3, 2),
            "launch_us_median_min_max": [round(float(np.median(pf_attn_ms)) * 1e3, 2),
                                         round(min(pf_attn_ms) * 1e3, 2), round(max(pf_attn_ms) * 1e3, 2)],
            "store_plus_prefill_us": round(float(np.mean(pf_ms)) * 1e3, 2),
            "roofline": {"bound": "mfma", "achieved": round(prefill_tflops, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(prefill_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("prefill")},
        },
        "cpu_baseline": cpu,
        "host_wall_s": round(wall, 3),
    }
    if int8 is not None:
        result.update(int8)
    if f16 is not None:
        result.update(f16)
    if c5b is not None:
        result["decode_c5b"] = c5b
    result["store"] = store
    if graph is not None:
        result["graph_step"] = graph
    result["prefill_mixed"] = mixed
    result["prefill_d256"] = d256
    gemm = gemm_reference()
    result["prefill"]["gemm_reference"] = gemm
    result["prefill"]["frac_of_gemm_reference"] = round(prefill_tflops / gemm["tflops"], 4)
    if small is not None:
        result["small_configs"] = small
    print(json.dumps(result), flush=True)


def int8_measure(pa, W, lay, pf, k_pools, v_pools, qs, ctx_d, bt_d, order_d, pf_kn, pf_vn, pf_slots,
                 bf16_call_ms, reps, pf_args, layers=4):
    """INT8 KV cache on the decode and prefill shapes (not part of the step)."""
    import torch
    dev = "cuda"
    stream = torch.cuda.current_stream()
    nb, bs, hkv, d, hq = lay.num_blocks, lay.block_size, lay.num_kv_heads, lay.head_dim, lay.num_q_heads
    layers = min(layers, len(k_pools))
    all_slots = torch.arange(nb * bs, dtype=torch.int32, device=dev)
    pools = []
    for i in range(layers):
        kq = torch.empty((nb, bs, hkv, d), dtype=torch.int8, device=dev)
        vq = torch.empty_like(kq)
        ks = torch.empty((nb, bs, hkv), dtype=torch.float16, device=dev)
        vs = torch.empty_like(ks)
        pa.pa_store_kv_int8(k_pools[i].view(nb * bs, hkv, d), v_pools[i].view(nb * bs, hkv, d), all_slots,
                            kq, vq, ks, vs)
        pools.append((kq, vq, ks, vs))
    out = torch.empty((lay.num_seqs, hq, d), dtype=torch.bfloat16, device=dev)
    wsb = pa.pa_decode_int8_workspace_bytes(lay.num_seqs, hq, lay.max_context_len, pools[0][0], pools[0][2])
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    tokens = int(lay.context_lens.astype(np.int64).sum()) * hkv
    i8_bytes = tokens * (d + 2) * 2

    def dec(i):
        pa.pa_decode_int8(qs[i], *pools[i], ctx_d, bt_d, lay.max_context_len, lay.scale, out=out, workspace=ws,
                          row_order=order_d)

    for i in range(layers):
        dec(i)
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(layers)]
          for _ in range(reps)]
    for r in range(reps):
        for i in range(layers):
            ev[r][i][0].record(stream)
            dec(i)
            ev[r][i][1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for row in ev for a, b in row]))
    gbps = i8_bytes / (ms * 1e-3) / 1e9

    # quantizing store of the 4096-token prompt into an INT8 pool of the prefill layout
    kq = torch.empty((pf.num_blocks, pf.block_size, pf.num_kv_heads, pf.head_dim), dtype=torch.int8, device=dev)
    vq = torch.empty_like(kq)
    ks = torch.empty((pf.num_blocks, pf.block_size, pf.num_kv_heads), dtype=torch.float16, device=dev)
    vs = torch.empty_like(ks)
    for _ in range(2):
        pa.pa_store_kv_int8(pf_kn, pf_vn, pf_slots, kq, vq, ks, vs)
    torch.cuda.synchronize()
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in sev:
        a.record(stream)
        pa.pa_store_kv_int8(pf_kn, pf_vn, pf_slots, kq, vq, ks, vs)
        b.record(stream)
    torch.cuda.synchronize()
    st_ms = float(np.mean([a.elapsed_time(b) for a, b in sev]))
    st_bytes = pf.total_q * pf.num_kv_heads * (pf.head_dim * 2 + pf.head_dim + 2) * 2  # read bf16, write int8+scale

    # prefill over the INT8 pool just filled (1 x 4096 causal, block 16)
    pf_q, pf_cuq, pf_cuk, pf_off, pf_bt, pf_flops, pf_bf16_ms = pf_args
    pf_out = torch.empty_like(pf_q)

    def pre():
        pa.pa_prefill_varlen_int8(pf_q, kq, vq, ks, vs, pf_cuq, pf_cuk, pf_off, pf_bt, pf.max_seqlen_q,
                                  pf.max_seqlen_k, pf.scale, out=pf_out)

    for _ in range(2):
        pre()
    torch.cuda.synchronize()
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in pev:
        a.record(stream)
        pre()
        b.record(stream)
    torch.cuda.synchronize()
    pf_ms = float(np.mean([a.elapsed_time(b) for a, b in pev]))
    pf_tflops = pf_flops / (pf_ms * 1e-3) / 1e12
    return {
        "int8_decode": {
            "value": round(gbps, 2), "unit": "GB/s",
            "workload": f"decode 256 seqs ctx U[100,2048], int8 codes + fp16 scales, {layers} layer pools",
            "avg_launch_us": round(ms * 1e3, 2), "bytes_per_launch": i8_bytes,
            "speedup_vs_bf16_decode": round(bf16_call_ms / ms, 3),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": measured_traffic("decode_int8")},
        },
        "int8_prefill": {
            "value": round(pf_tflops, 2), "unit": "TFLOP/s",
            "workload": "prefill 1x4096 causal over INT8 pools (block 16), bf16 queries",
            "avg_launch_us": round(pf_ms * 1e3, 2), "flops_per_launch": pf_flops,
            "time_vs_bf16_prefill": round(pf_ms / pf_bf16_ms, 3),
            "roofline": {"bound": "mfma", "achieved": round(pf_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(pf_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("prefill_int8")},
        },
        "int8_store": {
            "workload": "pa_store_kv_int8 of 4096 tokens x 8 KV heads x 128 (bf16 in, int8 + fp16 scale out)",
            "avg_launch_us": round(st_ms * 1e3, 2), "bytes_per_launch": st_bytes,
            "achieved_gbps": round(st_bytes / (st_ms * 1e-3) / 1e9, 2),
        },
    }


def _time_calls(fns, reps, queue_ahead=True):
    """Mean duration (ms) of each call in fns, from HIP events on the current
    stream, over reps rounds after two untimed rounds.  With queue_ahead a
    spin kernel of about a millisecond goes first, so the host has queued the
    timed calls before the GPU reaches them: for calls of a few microseconds
    the events would otherwise also time the host's launch work between them.
    Without it (eager launch sequences), that host work is what is timed."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(2):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
          for _ in range(reps)]
    if queue_ahead:
        torch.cuda._sleep(2_000_000)
    for r in range(reps):
        for i, fn in enumerate(fns):
            ev[r][i][0].record(stream)
            fn()
            ev[r][i][1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for row in ev for a, b in row]))


def mixed_prefill_measure(pa, W, reps):
    """The chunked-prefill batch (8192 new tokens: one sequence resuming after
    a cached prefix, then fresh prompts of U[100, 1024] tokens, block 16) in
    one pa_prefill_varlen call, bf16 (not part of the step)."""
    import torch
    dev = "cuda"
    mx = W.c5a_mixed(with_values=False)
    shape = (mx.num_blocks, mx.block_size, mx.num_kv_heads, mx.head_dim)
    kp, vp = W.device_normal(shape, 5400), W.device_normal(shape, 5401)
    q = W.device_normal((mx.total_q, mx.num_q_heads, mx.head_dim), 5402)
    out = torch.empty_like(q)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)  # noqa: E731
    args = (i32(mx.cu_seqlens_q), i32(mx.cu_seqlens_k), i32(mx.q_offsets), i32(mx.block_table))
    ms = _time_calls([lambda: pa.pa_prefill_varlen(q, kp, vp, *args, mx.max_seqlen_q, mx.max_seqlen_k, mx.scale,
                                                   out=out)], reps)
    flops = 4.0 * mx.head_dim * mx.num_q_heads * mx.causal_pairs
    tflops = flops / (ms * 1e-3) / 1e12
    return {"value": round(tflops, 2), "unit": "TFLOP/s",
            "workload": f"chunked prefill batch: {mx.num_seqs} sequences, {mx.total_q} new tokens, block 16, bf16",
            "avg_launch_us": round(ms * 1e3, 2), "flops_per_launch": flops,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("prefill_mixed")}}


def d256_prefill_measure(pa, W, reps):
    """head_dim 256 on the matrix cores: one 4096-token causal prompt, 8
    query heads over 4 KV heads, block 16, bf16 (not part of the step; the
    Qwen3 shapes have head_dim 128)."""
    import torch
    dev = "cuda"
    case = W.make_prefill("d256_1x4096", 5500, [4096], [0], 8, 4, 256, 16, "bf16", with_values=False)
    shape = (case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim)
    kp, vp = W.device_normal(shape, 5501), W.device_normal(shape, 5502)
    q = W.device_normal((case.total_q, case.num_q_heads, case.head_dim), 5503)
    out = torch.empty_like(q)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)  # noqa: E731
    args = (i32(case.cu_seqlens_q), i32(case.cu_seqlens_k), i32(case.q_offsets), i32(case.block_table))
    ms = _time_calls([lambda: pa.pa_prefill_varlen(q, kp, vp, *args, case.max_seqlen_q, case.max_seqlen_k,
                                                   case.scale, out=out)], reps)
    flops = 4.0 * case.head_dim * case.num_q_heads * case.causal_pairs
    tflops = flops / (ms * 1e-3) / 1e12
    return {"value": round(tflops, 2), "unit": "TFLOP/s",
            "workload": "prefill 1x4096 causal, head_dim 256, 8/4 heads, block 16, bf16",
            "avg_launch_us": round(ms * 1e3, 2), "flops_per_launch": flops,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("prefill_d256")}}


def c5b_measure(pa, W, reps):
    """Long-context decode: 64 sequences x 32768 keys (block 16, one layer
    pool, 8.59 GB of K/V), one pa_decode call per launch (not part of the
    step).  Bytes: every visible K and V row once per KV head."""
    import torch
    dev = "cuda"
    lay = W.c5b_decode_layout()
    nb, bs, hkv, d, hq = lay.num_blocks, lay.block_size, lay.num_kv_heads, lay.head_dim, lay.num_q_heads
    kp = W.device_normal((nb, bs, hkv, d), 5330)
    vp = W.device_normal((nb, bs, hkv, d), 5331)
    q = W.device_normal((lay.num_seqs, hq, d), 5332)
    out = torch.empty_like(q)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)  # noqa: E731
    ctx, bt = i32(lay.context_lens), i32(lay.block_table)
    ws = torch.empty(max(pa.pa_decode_workspace_bytes(lay.num_seqs, hq, lay.max_context_len, kp), 1),
                     dtype=torch.uint8, device=dev)
    order = pa.pa_decode_order(ctx)
    ms = _time_calls([lambda: pa.pa_decode(q, kp, vp, ctx, bt, lay.max_context_len, lay.scale, out=out,
                                           workspace=ws, row_order=order)], max(reps, 5))
    kv = lay.kv_bytes()
    gbps = kv / (ms * 1e-3) / 1e9
    del kp, vp
    torch.cuda.empty_cache()
    return {"value": round(gbps, 2), "unit": "GB/s",
            "workload": (f"decode {lay.num_seqs} seqs x {int(lay.context_lens[0])} keys, block {bs}, "
                         f"{hq}/{hkv} heads, d {d}, bf16, one layer pool"),
            "avg_launch_us": round(ms * 1e3, 2), "bytes_per_launch": kv,
            "roofline": {"bound": "hbm",
                         "kernel": "pa_decode (split-K kernel + log-sum-exp merge)",
                         "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": measured_traffic("decode_c5b")}}


def _time_in_graph(fn, calls=20, replays=5):
    """Mean duration (ms) of one call of fn, from `calls` calls captured in one
    HIP graph and replayed: for launches shorter than the host's own launch
    work, which per-call events would measure instead."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(replays):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (replays * calls)


def small_configs_measure(pa, W):
    """Per-call times of the small prefill shapes (not part of the step): the
    tiny fp32 batch (3 prompts of 5, 17, 40 tokens, d 32, block 16, and one
    decode step of its 3 rows), 8 prompts of 32, 128 and 256 tokens, and 2
    suffixes of 44 tokens after 256 cached (16/8 heads, d 128, bf16, block
    256).  These launches are latency-bound, shorter than the host's work to
    launch them, so each is timed inside a HIP graph of 20 calls."""
    import torch
    dev = "cuda"
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)  # noqa: E731
    res = {}

    def prefill_leg(name, case, seed):
        shape = (case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim)
        if case.dtype == "f32":
            kp = torch.randn(shape, generator=torch.Generator().manual_seed(seed)).to(dev)
            vp = torch.randn(shape, generator=torch.Generator().manual_seed(seed + 1)).to(dev)
            q = torch.from_numpy(np.ascontiguousarray(case.q)).to(dev)
        else:
            kp, vp = W.device_normal(shape, seed), W.device_normal(shape, seed + 1)
            q = W.device_normal((case.total_q, case.num_q_heads, case.head_dim), seed + 2)
        out = torch.empty_like(q)
        args = (i32(case.cu_seqlens_q), i32(case.cu_seqlens_k), i32(case.q_offsets), i32(case.block_table))
        ms = _time_in_graph(lambda: pa.pa_prefill_varlen(q, kp, vp, *args, case.max_seqlen_q, case.max_seqlen_k,
                                                         case.scale, out=out))
        flops = 4.0 * case.head_dim * case.num_q_heads * case.causal_pairs
        res[name] = {"tokens": case.total_q, "avg_launch_us": round(ms * 1e3, 2),
                     "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
        return kp, vp

    pre, dec = W.c1_tiny()
    kp, vp = prefill_leg("c1_prefill_fp32", pre, 6100)
    st = dec[0]
    q1 = torch.from_numpy(np.ascontiguousarray(st["q"])).to(dev)
    ctx1, bt1 = i32(st["context_lens"]), i32(pre.block_table)
    out1 = torch.empty_like(q1)
    ms = _time_in_graph(lambda: pa.pa_decode(q1, kp, vp, ctx1, bt1, int(st["context_lens"].max()), pre.scale,
                                             out=out1))
    res["c1_decode_fp32"] = {"rows": 3, "avg_launch_us": round(ms * 1e3, 2)}
    for n in (32, 128, 256):
        prefill_leg(f"c2_prefill_8x{n}", W.c2_varlen(n, with_values=False), 6200 + n)
    prefill_leg("c3_prefill_2x44_after_256", W.c3_prefix(with_values=False), 6300)
    return res


def gemm_reference(reps=10):
    """A second denominator for the prefill: the rate of a large plain bf16
    GEMM (8192^3, torch.mm on contiguous operands, hipBLASLt), i.e. what the
    matrix cores sustain on this machine in a library kernel."""
    import torch
    n = 8192
    g = torch.Generator(device="cuda")
    g.manual_seed(5600)
    a = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
    b = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16)
    c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    ms = _time_calls([lambda: torch.mm(a, b, out=c)], reps)
    del a, b, c
    torch.cuda.empty_cache()
    return {"tflops": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1), "shape": "8192 x 8192 x 8192 bf16, torch.mm",
            "avg_launch_us": round(ms * 1e3, 1)}


def graph_measure(step, eager_ms_per_step, reps):
    """The whole step captured once in a HIP graph (torch's CUDAGraph over the
    current stream) and replayed: same kernels, same buffers, no host launch
    work per kernel."""
    import torch
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    return {"workload": "the timed step (prefill + 28 decode layers, their stores and the row order) as one graph",
            "ms_per_step": round(ms, 4), "eager_ms_per_step": round(eager_ms_per_step, 4),
            "graph_over_eager_time": round(ms / eager_ms_per_step, 3)}


def f16_measure(pa, W, lay, ctx_d, bt_d, order_d, bf16_dec_ms, bf16_pf_ms, reps, layers=4):
    """fp16 pools and queries (not part of the step): the decode shape over
    `layers` fp16 layer pools, the 1 x 4096 prefill on the fp16 matrix cores,
    and the fork's fp16-versus-INT8 decode microbenchmark shape (batch 8,
    16 / 8 heads, head_dim 128, 512 keys per row)."""
    import torch
    dev = "cuda"
    nb, bs, hkv, d, hq = lay.num_blocks, lay.block_size, lay.num_kv_heads, lay.head_dim, lay.num_q_heads
    pools = [(W.device_normal((nb, bs, hkv, d), 4500 + 2 * i, dtype="f16"),
              W.device_normal((nb, bs, hkv, d), 4501 + 2 * i, dtype="f16"),
              W.device_normal((lay.num_seqs, hq, d), 9500 + i, dtype="f16")) for i in range(layers)]
    out = torch.empty((lay.num_seqs, hq, d), dtype=torch.float16, device=dev)
    wsb = pa.pa_decode_workspace_bytes(lay.num_seqs, hq, lay.max_context_len, pools[0][0])
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    dec_ms = _time_calls([lambda i=i: pa.pa_decode(pools[i][2], pools[i][0], pools[i][1], ctx_d, bt_d,
                                                   lay.max_context_len, lay.scale, out=out, workspace=ws,
                                                   row_order=order_d) for i in range(layers)], reps)
    dec_bytes = lay.kv_bytes()
    dec_gbps = dec_bytes / (dec_ms * 1e-3) / 1e9

    pf = W.c5a_long(dtype="f16", with_values=False)
    kp = W.device_normal((pf.num_blocks, pf.block_size, pf.num_kv_heads, pf.head_dim), 5300, dtype="f16")
    vp = W.device_normal((pf.num_blocks, pf.block_size, pf.num_kv_heads, pf.head_dim), 5301, dtype="f16")
    q = W.device_normal((pf.total_q, pf.num_q_heads, pf.head_dim), 5302, dtype="f16")
    pf_out = torch.empty_like(q)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)  # noqa: E731
    cuq, cuk, off, bt = i32(pf.cu_seqlens_q), i32(pf.cu_seqlens_k), i32(pf.q_offsets), i32(pf.block_table)
    pf_ms = _time_calls([lambda: pa.pa_prefill_varlen(q, kp, vp, cuq, cuk, off, bt, pf.max_seqlen_q,
                                                      pf.max_seqlen_k, pf.scale, out=pf_out)], reps)
    pf_flops = 4.0 * pf.head_dim * pf.num_q_heads * pf.causal_pairs
    pf_tflops = pf_flops / (pf_ms * 1e-3) / 1e12
    # the same prefill over INT8 pools quantized from the fp16 ones, fp16 queries
    pshape = (pf.num_blocks, pf.block_size, pf.num_kv_heads, pf.head_dim)
    pkq, pvq = torch.empty(pshape, dtype=torch.int8, device=dev), torch.empty(pshape, dtype=torch.int8, device=dev)
    pks = torch.empty(pshape[:3], dtype=torch.float16, device=dev)
    pvs = torch.empty_like(pks)
    pflat = (pf.num_blocks * pf.block_size, pf.num_kv_heads, pf.head_dim)
    pa.pa_store_kv_int8(kp.view(pflat), vp.view(pflat),
                        torch.arange(pflat[0], dtype=torch.int32, device=dev), pkq, pvq, pks, pvs)
    pf8_ms = _time_calls([lambda: pa.pa_prefill_varlen_int8(q, pkq, pvq, pks, pvs, cuq, cuk, off, bt,
                                                            pf.max_seqlen_q, pf.max_seqlen_k, pf.scale,
                                                            out=pf_out)], reps)

    mb = W.fork_microbench_decode(with_values=False)
    mk = W.device_normal((mb.num_blocks, mb.block_size, mb.num_kv_heads, mb.head_dim), 8600, dtype="f16")
    mv = W.device_normal((mb.num_blocks, mb.block_size, mb.num_kv_heads, mb.head_dim), 8601, dtype="f16")
    mq = W.device_normal((mb.num_seqs, mb.num_q_heads, mb.head_dim), 8602, dtype="f16")
    mctx, mbt = i32(mb.context_lens), i32(mb.block_table)
    slots = torch.arange(mb.num_blocks * mb.block_size, dtype=torch.int32, device=dev)
    shape = (mb.num_blocks, mb.block_size, mb.num_kv_heads, mb.head_dim)
    kq, vq = torch.empty(shape, dtype=torch.int8, device=dev), torch.empty(shape, dtype=torch.int8, device=dev)
    ks = torch.empty(shape[:3], dtype=torch.float16, device=dev)
    vs = torch.empty_like(ks)
    flat = (mb.num_blocks * mb.block_size, mb.num_kv_heads, mb.head_dim)
    pa.pa_store_kv_int8(mk.view(flat), mv.view(flat), slots, kq, vq, ks, vs)
    mout = torch.empty_like(mq)
    mws = torch.empty(max(pa.pa_decode_workspace_bytes(mb.num_seqs, mb.num_q_heads, mb.max_context_len, mk),
                          pa.pa_decode_int8_workspace_bytes(mb.num_seqs, mb.num_q_heads, mb.max_context_len, kq,
                                                            ks), 1), dtype=torch.uint8, device=dev)
    mb_f16 = _time_calls([lambda: pa.pa_decode(mq, mk, mv, mctx, mbt, mb.max_context_len, mb.scale, out=mout,
                                               workspace=mws)], max(reps, 20))
    mb_i8 = _time_calls([lambda: pa.pa_decode_int8(mq, kq, vq, ks, vs, mctx, mbt, mb.max_context_len, mb.scale,
                                                   out=mout, workspace=mws)], max(reps, 20))
    mb_tokens = int(mb.context_lens.sum()) * mb.num_kv_heads
    # the small decode as a model step would issue it: 28 calls back to back,
    # eager and as one captured graph
    layers28 = lambda: [pa.pa_decode(mq, mk, mv, mctx, mbt, mb.max_context_len, mb.scale, out=mout,  # noqa: E731
                                     workspace=mws) for _ in range(28)]
    eager28 = _time_calls([layers28], max(reps, 10), queue_ahead=False) / 28
    layers28()
    torch.cuda.synchronize()
    g28 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g28):
        layers28()
    torch.cuda.synchronize()
    graph28 = _time_calls([g28.replay], max(reps, 10), queue_ahead=False) / 28
    return {
        "f16_decode": {
            "value": round(dec_gbps, 2), "unit": "GB/s",
            "workload": f"decode 256 seqs ctx U[100,2048], fp16 pools and queries, {layers} layer pools",
            "avg_launch_us": round(dec_ms * 1e3, 2), "bytes_per_launch": dec_bytes,
            "time_vs_bf16_decode": round(dec_ms / bf16_dec_ms, 3),
            "roofline": {"bound": "hbm", "achieved": round(dec_gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "traffic": measured_traffic("decode_f16")},
        },
        "f16_prefill": {
            "value": round(pf_tflops, 2), "unit": "TFLOP/s",
            "workload": "prefill 1x4096 causal (block 16), fp16 pools and queries, fp16 MFMA",
            "avg_launch_us": round(pf_ms * 1e3, 2), "flops_per_launch": pf_flops,
            "time_vs_bf16_prefill": round(pf_ms / bf16_pf_ms, 3),
            "roofline": {"bound": "mfma", "achieved": round(pf_tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(pf_tflops / MFMA_F16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("prefill_f16")},
        },
        "int8_prefill_f16q": {
            "value": round(pf_flops / (pf8_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "workload": "prefill 1x4096 causal over INT8 pools (block 16), fp16 queries, fp16 MFMA",
            "avg_launch_us": round(pf8_ms * 1e3, 2), "time_vs_f16_prefill": round(pf8_ms / pf_ms, 3),
        },
        "fork_microbench_decode": {
            "workload": ("decode batch 8 x 512 keys, 16 q / 8 kv heads, head_dim 128, block 256: fp16 pools "
                         "against INT8 pools (fp16 queries)"),
            "f16_us": round(mb_f16 * 1e3, 2), "int8_us": round(mb_i8 * 1e3, 2),
            "int8_over_f16_time": round(mb_i8 / mb_f16, 3),
            "f16_us_per_call_28_back_to_back": round(eager28 * 1e3, 2),
            "f16_us_per_call_28_in_graph": round(graph28 * 1e3, 2),
            "f16_cache_bytes": mb_tokens * mb.head_dim * 2 * 2,
            "int8_cache_bytes": mb_tokens * (mb.head_dim + 2) * 2,
        },
    }


def measured_traffic(which):
    """HBM bytes per launch (read + write) of the decode or prefill kernel, from
    the rocprofv3 FETCH_SIZE / WRITE_SIZE runs summarised in profiles/ (scaled by
    the plain-copy calibration there).  None when the kernel source changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(which)
    if not rec:
        return None
    src = os.path.join(ROOT, rec["source"])
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["sha256"]:
        return None
    return int(rec["read_bytes"] + rec["write_bytes"])


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(lay, k_pool, v_pool, q, pf, pf_k, pf_v, pf_q, target_s=10.0):
    """The fp64 CPU oracle on the host cores, over bounded samples of the
    same workloads (a reported baseline, not a target):
      * decode layer 0 (all 256 sequences, all 16 query heads), repeated
        until about target_s seconds of host work have run on all threads,
        then once on a single thread over its first 32 sequences;
      * the 1 x 4096 prefill over every 4th query row on all threads, and
        over every 64th row on a single thread.
    Rates are in the metric's units (decode: KV bytes per second; prefill:
    4*d*Hq FLOP per visible causal pair per second, fp64)."""
    import torch

    import oracle

    def bits(t):
        return t.cpu().view(torch.int16).numpy().view(np.uint16)

    threads = oracle.num_threads()
    kp, vp, qh = bits(k_pool), bits(v_pool), bits(q)
    reps, t_total = 0, 0.0
    while t_total < target_s and reps < 1000:
        t0 = time.perf_counter()
        oracle.decode(qh, kp, vp, lay.context_lens, lay.block_table, lay.scale)
        t_total += time.perf_counter() - t0
        reps += 1
    kv = lay.kv_bytes() * reps
    d, hq, hkv = lay.head_dim, lay.num_q_heads, lay.num_kv_heads
    dec_flops = 4.0 * d * hq * float(lay.context_lens.astype(np.int64).sum()) * reps
    seqs1 = np.arange(32, dtype=np.int32)
    oracle.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.decode(qh, kp, vp, lay.context_lens, lay.block_table, lay.scale, seqs=seqs1)
        t1_dec = time.perf_counter() - t0
        kv1 = int(lay.context_lens[:32].astype(np.int64).sum()) * hkv * d * 2 * 2

        pkp, pvp, pqh = bits(pf_k), bits(pf_v), bits(pf_q)
        rows1 = np.arange(0, pf.total_q, 64, dtype=np.int32)
        t0 = time.perf_counter()
        _, pairs1 = oracle.prefill(pqh, pkp, pvp, pf.cu_seqlens_q, pf.cu_seqlens_k, pf.q_offsets, pf.block_table,
                                   pf.scale, rows=rows1, return_pairs=True)
        t1_pf = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(threads)
    rows = np.arange(0, pf.total_q, 4, dtype=np.int32)
    t0 = time.perf_counter()
    _, pairs = oracle.prefill(pqh, pkp, pvp, pf.cu_seqlens_q, pf.cu_seqlens_k, pf.q_offsets, pf.block_table,
                              pf.scale, rows=rows, return_pairs=True)
    t_pf = time.perf_counter() - t0
    pf_flops, pf_flops1 = 4.0 * d * hq * pairs, 4.0 * d * hq * pairs1
    return {"value": round(kv / t_total / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"decode layer 0 ({lay.num_seqs} sequences, {hq} query heads, "
                       f"{lay.kv_bytes()} KV bytes) x {reps} repetitions, {t_total:.1f} s fp64 on {threads} threads"),
            "cpu_model": _cpu_model(),
            "decode_fp64_gflops": round(dec_flops / t_total / 1e9, 3),
            "decode_one_thread": {"value": round(kv1 / t1_dec / 1e9, 4), "unit": "GB/s",
                                  "sample": f"decode layer 0, sequences 0..31 ({kv1} KV bytes), {t1_dec:.1f} s"},
            "prefill": {"value": round(pf_flops / t_pf / 1e9, 3), "unit": "GFLOP/s", "cores": threads,
                        "sample": (f"prefill 1x4096 causal, every 4th query row ({len(rows)} rows x {hq} heads, "
                                   f"{pairs} causal pairs), {t_pf:.1f} s fp64"),
                        "full_prefill_s_estimate": round(t_pf * 4.0, 2)},
            "prefill_one_thread": {"value": round(pf_flops1 / t1_pf / 1e9, 3), "unit": "GFLOP/s",
                                   "sample": (f"prefill 1x4096 causal, every 64th query row ({len(rows1)} rows, "
                                              f"{pairs1} causal pairs), {t1_pf:.1f} s fp64")}}


if __name__ == "__main__":
    main()

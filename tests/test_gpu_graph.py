"""A mixed attention step under HIP graph capture.

One step = a chunked-prefill batch (store its new tokens, then prefill over
cached prefixes) and a decode batch with padding rows (store each row's new
token, order the rows, decode), all on torch's current stream.  The step is
captured once, with every size planned for a capacity (decode rows x table
width x block size keys, prefill tokens and chunk lengths), and replayed with
new lengths, block tables and values written into the same device buffers.
The decode split count per row is chosen on the device from its own length,
so the one graph serves every length up to the capacity.

Each replay is checked against the eager calls on the same inputs (bit for
bit: same kernels, same plan) and against the oracle (every row), with eager
work and synchronisations between the replays.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_attention_mapping_amd as pa
import workloads as W
from helpers import max_abs_err, say, to_dev, to_host_bits, tol

pytestmark = pytest.mark.gpu

HQ, HKV, D, BS = 16, 8, 128, 16
B, WIDTH = 32, 256                  # decode rows, table width (blocks): 4096 keys per row
PF_SEQS, PF_TOKENS, PF_MAX_Q = 3, 384, 256
CAP_K = WIDTH * BS
NB_DEC = B * WIDTH + 2
NB_PF = PF_SEQS * WIDTH + 2


def _decode_case(seed):
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1, CAP_K, size=B, endpoint=True).astype(np.int32)
    ctx[rng.choice(np.arange(1, B), 3, replace=False)] = 0      # padding rows
    ctx[0] = CAP_K if seed % 2 else int(rng.integers(1, 64))    # a full row, or no row past 4032 keys
    if seed % 2 == 0:
        ctx = np.minimum(ctx, CAP_K - 64)
    return W.make_decode("graph_dec", seed, ctx, HQ, HKV, D, BS, "bf16", num_spare=2)


def _prefill_case(seed):
    rng = np.random.default_rng(seed)
    q_lens = rng.integers(1, PF_MAX_Q, size=PF_SEQS, endpoint=True)
    while q_lens.sum() > PF_TOKENS:
        q_lens = (q_lens * 3) // 4 + 1
    q_offs = [int(rng.integers(0, CAP_K - int(n), endpoint=True)) for n in q_lens]
    return W.make_prefill("graph_pf", seed, [int(n) for n in q_lens], q_offs, HQ, HKV, D, BS, "bf16",
                          num_spare=2)


def _padded_table(table, spare, rows, width=WIDTH):
    out = np.full((rows, width), spare, np.int32)
    out[:table.shape[0], :table.shape[1]] = table
    return out


class Step:
    """Static device buffers of one step and the calls that use them."""

    def __init__(self):
        dev = "cuda"
        bf = torch.bfloat16
        self.kd = torch.empty((NB_DEC, BS, HKV, D), dtype=bf, device=dev)
        self.vd = torch.empty_like(self.kd)
        self.q_dec = torch.empty((B, HQ, D), dtype=bf, device=dev)
        self.kn_dec = torch.empty((B, HKV, D), dtype=bf, device=dev)
        self.vn_dec = torch.empty_like(self.kn_dec)
        self.slot_dec = torch.empty(B, dtype=torch.int32, device=dev)
        self.ctx = torch.empty(B, dtype=torch.int32, device=dev)
        self.bt_dec = torch.empty((B, WIDTH), dtype=torch.int32, device=dev)
        self.order = torch.empty(B, dtype=torch.int32, device=dev)
        self.out_dec = torch.empty((B, HQ, D), dtype=bf, device=dev)
        self.ws_dec = torch.empty(max(pa.pa_decode_workspace_bytes(B, HQ, CAP_K, self.kd), 1), dtype=torch.uint8,
                                  device=dev)
        self.kp = torch.empty((NB_PF, BS, HKV, D), dtype=bf, device=dev)
        self.vp = torch.empty_like(self.kp)
        self.q_pf = torch.empty((PF_TOKENS, HQ, D), dtype=bf, device=dev)
        self.kn_pf = torch.empty((PF_TOKENS, HKV, D), dtype=bf, device=dev)
        self.vn_pf = torch.empty_like(self.kn_pf)
        self.slot_pf = torch.empty(PF_TOKENS, dtype=torch.int32, device=dev)
        self.cu_q = torch.empty(PF_SEQS + 1, dtype=torch.int32, device=dev)
        self.cu_k = torch.empty_like(self.cu_q)
        self.q_off = torch.empty(PF_SEQS, dtype=torch.int32, device=dev)
        self.bt_pf = torch.empty((PF_SEQS, WIDTH), dtype=torch.int32, device=dev)
        self.out_pf = torch.empty((PF_TOKENS, HQ, D), dtype=bf, device=dev)
        self.ws_pf = torch.empty(max(pa.pa_prefill_workspace_bytes(PF_SEQS, PF_TOKENS, HQ, PF_MAX_Q, CAP_K,
                                                                   self.kp), 1), dtype=torch.uint8, device=dev)
        self.scale = 1.0 / np.sqrt(D)

    def run(self):
        pa.pa_store_kv(self.kn_pf, self.vn_pf, self.slot_pf, self.kp, self.vp)
        pa.pa_prefill_varlen(self.q_pf, self.kp, self.vp, self.cu_q, self.cu_k, self.q_off, self.bt_pf, PF_MAX_Q,
                             CAP_K, self.scale, out=self.out_pf, workspace=self.ws_pf)
        pa.pa_store_kv(self.kn_dec, self.vn_dec, self.slot_dec, self.kd, self.vd)
        pa.pa_decode_order(self.ctx, row_order=self.order)
        pa.pa_decode(self.q_dec, self.kd, self.vd, self.ctx, self.bt_dec, CAP_K, self.scale, out=self.out_dec,
                     workspace=self.ws_dec, row_order=self.order)

    def load(self, dec, pf):
        """Write one step's inputs into the buffers; the pools get the cached
        history (by the oracle's store on the host) and NaN everywhere else."""
        kp_h, vp_h = W.poisoned_pool(NB_DEC, BS, HKV, D, "bf16"), W.poisoned_pool(NB_DEC, BS, HKV, D, "bf16")
        oracle.store_kv(dec.k_hist, dec.v_hist, dec.slot_hist, kp_h, vp_h)
        self.kd.copy_(to_dev(kp_h))
        self.vd.copy_(to_dev(vp_h))
        self.q_dec.copy_(to_dev(dec.q))
        self.kn_dec.copy_(to_dev(dec.k_new))
        self.vn_dec.copy_(to_dev(dec.v_new))
        self.slot_dec.copy_(to_dev(dec.slot_new))
        self.ctx.copy_(to_dev(dec.context_lens))
        self.bt_dec.copy_(to_dev(_padded_table(dec.block_table, dec.spare_blocks[0], B)))
        kq_h, vq_h = W.poisoned_pool(NB_PF, BS, HKV, D, "bf16"), W.poisoned_pool(NB_PF, BS, HKV, D, "bf16")
        if len(pf.slot_cached):
            oracle.store_kv(pf.k_cached, pf.v_cached, pf.slot_cached, kq_h, vq_h)
        self.kp.copy_(to_dev(kq_h))
        self.vp.copy_(to_dev(vq_h))
        tq = pf.total_q
        pad = lambda a, n, fill: np.concatenate([a, np.full((n - len(a),) + a.shape[1:], fill, a.dtype)])  # noqa
        self.q_pf.copy_(to_dev(pad(pf.q, PF_TOKENS, 0)))
        self.kn_pf.copy_(to_dev(pad(pf.k_new, PF_TOKENS, 0)))
        self.vn_pf.copy_(to_dev(pad(pf.v_new, PF_TOKENS, 0)))
        self.slot_pf.copy_(to_dev(pad(pf.slot_new.astype(np.int32), PF_TOKENS, -1)))
        self.cu_q.copy_(to_dev(pf.cu_seqlens_q))
        self.cu_k.copy_(to_dev(pf.cu_seqlens_k))
        self.q_off.copy_(to_dev(np.asarray(pf.q_offsets, np.int32)))
        self.bt_pf.copy_(to_dev(_padded_table(pf.block_table, pf.spare_blocks[0], PF_SEQS)))
        self.out_pf.zero_()
        self.out_dec.zero_()
        self.host = (kp_h, vp_h, kq_h, vq_h)
        return tq

    def outputs(self, tq):
        return to_host_bits(self.out_dec), to_host_bits(self.out_pf[:tq])


def test_mixed_step_graph_replays_match_eager_and_oracle():
    step = Step()
    first_dec, first_pf = _decode_case(9100), _prefill_case(9200)
    step.load(first_dec, first_pf)
    torch.cuda.synchronize()
    step.run()                                  # warm up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run()
    torch.cuda.synchronize()

    for r in range(4):
        dec, pf = _decode_case(9101 + r), _prefill_case(9201 + r)
        say(f"[graph] replay {r}: decode ctx max {int(dec.context_lens.max())}, "
            f"prefill q {list(np.diff(pf.cu_seqlens_q))} off {list(pf.q_offsets)}")
        tq = step.load(dec, pf)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        g_dec, g_pf = step.outputs(tq)
        g_pools = to_host_bits(step.kd), to_host_bits(step.kp)

        step.load(dec, pf)                      # eager calls on the same inputs
        torch.cuda.synchronize()
        step.run()
        torch.cuda.synchronize()
        e_dec, e_pf = step.outputs(tq)
        assert g_dec.tobytes() == e_dec.tobytes(), "decode: replay differs from the eager call"
        assert g_pf.tobytes() == e_pf.tobytes(), "prefill: replay differs from the eager call"
        assert g_pools[0].tobytes() == to_host_bits(step.kd).tobytes()
        assert g_pools[1].tobytes() == to_host_bits(step.kp).tobytes()

        kp_h, vp_h, kq_h, vq_h = step.host
        oracle.store_kv(dec.k_new, dec.v_new, dec.slot_new, kp_h, vp_h)
        assert g_pools[0].tobytes() == kp_h.tobytes(), "decode store differs from the oracle's"
        ref_dec = oracle.decode(dec.q, kp_h, vp_h, dec.context_lens, dec.block_table, step.scale)
        err_dec = max_abs_err(g_dec, ref_dec)
        oracle.store_kv(pf.k_new, pf.v_new, pf.slot_new, kq_h, vq_h)
        ref_pf = oracle.prefill(pf.q, kq_h, vq_h, pf.cu_seqlens_q, pf.cu_seqlens_k, pf.q_offsets, pf.block_table,
                                step.scale)
        err_pf = max_abs_err(g_pf, ref_pf)
        say(f"  max-abs decode {err_dec:.2e}, prefill {err_pf:.2e}")
        assert err_dec <= tol("bf16") and err_pf <= tol("bf16")
        pad_rows = np.nonzero(dec.context_lens == 0)[0]
        assert (g_dec[pad_rows] == 0).all()


# ---------------------------------------------------------------- INT8 pools, fp16 queries

I8_B, I8_WIDTH = 16, 128            # 2048 keys per decode row
I8_CAP = I8_WIDTH * BS
I8_NB_DEC = I8_B * I8_WIDTH + 2
I8_NB_PF = PF_SEQS * I8_WIDTH + 2


def _i8_pools(nb):
    kq = np.full((nb, BS, HKV, D), -128, np.int8)
    ks = np.full((nb, BS, HKV), np.float16(np.nan), np.float16)
    return [kq, kq.copy(), ks, ks.copy()]


def test_int8_fp16_step_graph_replays_match_eager_and_oracle():
    """The same capture-once, replay-with-new-lengths check over INT8 pools
    with fp16 rows and queries (the fork's fp16 model with an INT8 cache):
    quantizing stores, the INT8 prefill on the fp16 matrix cores and the
    INT8 decode with device-chosen splits."""
    from oracle import int8 as Q
    dev = "cuda"
    f16 = torch.float16
    dpools = [torch.from_numpy(a).to(dev) for a in _i8_pools(I8_NB_DEC)]
    ppools = [torch.from_numpy(a).to(dev) for a in _i8_pools(I8_NB_PF)]
    q_dec = torch.empty((I8_B, HQ, D), dtype=f16, device=dev)
    kn_dec, vn_dec = (torch.empty((I8_B, HKV, D), dtype=f16, device=dev) for _ in range(2))
    slot_dec, ctx_d = (torch.empty(I8_B, dtype=torch.int32, device=dev) for _ in range(2))
    bt_dec = torch.empty((I8_B, I8_WIDTH), dtype=torch.int32, device=dev)
    out_dec = torch.empty((I8_B, HQ, D), dtype=f16, device=dev)
    ws_dec = torch.empty(max(pa.pa_decode_int8_workspace_bytes(I8_B, HQ, I8_CAP, dpools[0], dpools[2]), 1),
                         dtype=torch.uint8, device=dev)
    q_pf = torch.empty((PF_TOKENS, HQ, D), dtype=f16, device=dev)
    kn_pf, vn_pf = (torch.empty((PF_TOKENS, HKV, D), dtype=f16, device=dev) for _ in range(2))
    slot_pf = torch.empty(PF_TOKENS, dtype=torch.int32, device=dev)
    cu_q, cu_k = (torch.empty(PF_SEQS + 1, dtype=torch.int32, device=dev) for _ in range(2))
    q_off = torch.empty(PF_SEQS, dtype=torch.int32, device=dev)
    bt_pf = torch.empty((PF_SEQS, I8_WIDTH), dtype=torch.int32, device=dev)
    out_pf = torch.empty((PF_TOKENS, HQ, D), dtype=f16, device=dev)
    import ctypes
    nb_pf = pa.load().pa_prefill_int8_workspace_bytes(PF_SEQS, PF_TOKENS, HQ, I8_CAP,
                                                       ctypes.byref(pa.pool_desc_int8(ppools[0], ppools[2])))
    ws_pf = torch.empty(max(int(nb_pf), 1), dtype=torch.uint8, device=dev)
    scale = 1.0 / np.sqrt(D)

    def run():
        pa.pa_store_kv_int8(kn_pf, vn_pf, slot_pf, *ppools)
        pa.pa_prefill_varlen_int8(q_pf, *ppools, cu_q, cu_k, q_off, bt_pf, PF_MAX_Q, I8_CAP, scale, out=out_pf,
                                  workspace=ws_pf)
        pa.pa_store_kv_int8(kn_dec, vn_dec, slot_dec, *dpools)
        pa.pa_decode_int8(q_dec, *dpools, ctx_d, bt_dec, I8_CAP, scale, out=out_dec, workspace=ws_dec)

    def cases(seed):
        rng = np.random.default_rng(seed)
        ctx = rng.integers(1, I8_CAP, size=I8_B, endpoint=True).astype(np.int32)
        ctx[rng.choice(np.arange(1, I8_B), 2, replace=False)] = 0
        dec = W.make_decode("graph_i8", seed, ctx, HQ, HKV, D, BS, "f16", num_spare=2)
        q_lens = rng.integers(1, PF_MAX_Q, size=PF_SEQS, endpoint=True)
        while q_lens.sum() > PF_TOKENS:
            q_lens = (q_lens * 3) // 4 + 1
        q_offs = [int(rng.integers(0, I8_CAP - int(n), endpoint=True)) for n in q_lens]
        pf = W.make_prefill("graph_i8_pf", seed + 1, [int(n) for n in q_lens], q_offs, HQ, HKV, D, BS, "f16",
                            num_spare=2)
        return dec, pf

    def load(dec, pf):
        hd = _i8_pools(I8_NB_DEC)
        Q.store_kv(dec.k_hist, dec.v_hist, dec.slot_hist, *hd)
        hp = _i8_pools(I8_NB_PF)
        if len(pf.slot_cached):
            Q.store_kv(pf.k_cached, pf.v_cached, pf.slot_cached, *hp)
        for d_, h_ in zip(dpools + ppools, hd + hp):
            d_.copy_(torch.from_numpy(h_))
        q_dec.copy_(to_dev(dec.q))
        kn_dec.copy_(to_dev(dec.k_new))
        vn_dec.copy_(to_dev(dec.v_new))
        slot_dec.copy_(to_dev(dec.slot_new))
        ctx_d.copy_(to_dev(dec.context_lens))
        bt_dec.copy_(to_dev(_padded_table(dec.block_table, dec.spare_blocks[0], I8_B, I8_WIDTH)))
        pad = lambda a, n, fill: np.concatenate([a, np.full((n - len(a),) + a.shape[1:], fill, a.dtype)])  # noqa
        q_pf.copy_(to_dev(pad(pf.q, PF_TOKENS, 0)))
        kn_pf.copy_(to_dev(pad(pf.k_new, PF_TOKENS, 0)))
        vn_pf.copy_(to_dev(pad(pf.v_new, PF_TOKENS, 0)))
        slot_pf.copy_(to_dev(pad(pf.slot_new.astype(np.int32), PF_TOKENS, -1)))
        cu_q.copy_(to_dev(pf.cu_seqlens_q))
        cu_k.copy_(to_dev(pf.cu_seqlens_k))
        q_off.copy_(to_dev(np.asarray(pf.q_offsets, np.int32)))
        bt_pf.copy_(to_dev(_padded_table(pf.block_table, pf.spare_blocks[0], PF_SEQS, I8_WIDTH)))
        out_dec.zero_()
        out_pf.zero_()
        return hd, hp

    first_dec, first_pf = cases(9300)
    load(first_dec, first_pf)
    torch.cuda.synchronize()
    run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for r in range(3):
        dec, pf = cases(9301 + 7 * r)
        say(f"[graph int8] replay {r}: decode ctx max {int(dec.context_lens.max())}, "
            f"prefill q {list(np.diff(pf.cu_seqlens_q))}")
        hd, hp = load(dec, pf)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        tq = pf.total_q
        g_dec, g_pf = to_host_bits(out_dec), to_host_bits(out_pf[:tq])
        g_pools = [t.cpu().numpy() for t in dpools + ppools]
        load(dec, pf)
        torch.cuda.synchronize()
        run()
        torch.cuda.synchronize()
        assert g_dec.tobytes() == to_host_bits(out_dec).tobytes(), "decode: replay differs from the eager call"
        assert g_pf.tobytes() == to_host_bits(out_pf[:tq]).tobytes(), "prefill: replay differs from the eager call"
        Q.store_kv(dec.k_new, dec.v_new, dec.slot_new, *hd)
        Q.store_kv(pf.k_new, pf.v_new, pf.slot_new, *hp)
        for g_, h_ in zip(g_pools, hd + hp):
            assert g_.view(np.uint8).tobytes() == h_.view(np.uint8).tobytes(), "INT8 store differs from the oracle's"
        err_dec = max_abs_err(g_dec, Q.decode(dec.q, *hd, dec.context_lens, dec.block_table, scale))
        err_pf = max_abs_err(g_pf, Q.prefill(pf.q, *hp, pf.cu_seqlens_q, pf.cu_seqlens_k, pf.q_offsets,
                                            pf.block_table, scale))
        say(f"  max-abs decode {err_dec:.2e}, prefill {err_pf:.2e}")
        assert err_dec <= tol("f16") and err_pf <= tol("f16")

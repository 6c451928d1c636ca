"""Test/benchmark plumbing: put one seeded hybrid step on the GPU through the
C ABI, and give the oracle the same inputs.

The GPU side uses only the library (scheduler, upload, append, attention);
the oracle side uses only ``oracle/`` plus the shared input generators.  The
two meet only in the generator's bf16 tensors.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

import workloads as W


def load_native_sched(inst: W.Instance, free_pages=None):
    from chunked_prefill_decode_amd import native as N
    s = N.Scheduler(inst.token_budget, inst.max_blocks_per_seq,
                    inst.free_pages if free_pages is None else free_pages)
    for r in inst.injected:
        s.add_request(r.req_id, r.prompt_len, r.max_new_tokens, r.num_computed, r.num_generated)
    for r in inst.waiting:
        s.add_request(r.req_id, r.prompt_len, r.max_new_tokens)
    return s


def load_oracle_sched(inst: W.Instance, free_pages=None):
    from oracle import scheduler as OS
    s = OS.Scheduler(inst.token_budget, inst.max_blocks_per_seq,
                     (inst.free_pages if free_pages is None else free_pages).tolist())
    for r in inst.injected:
        s.add_request(r.req_id, r.prompt_len, r.max_new_tokens, r.num_computed, r.num_generated)
    for r in inst.waiting:
        s.add_request(r.req_id, r.prompt_len, r.max_new_tokens)
    return s


def requests_by_id(inst: W.Instance) -> Dict[int, W.Req]:
    return {r.req_id: r for r in inst.injected + inst.waiting}


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


class GpuStep:
    """One layer's hybrid step for a workload instance, resident on the GPU."""

    def __init__(self, inst: W.Instance, device="cuda:0", gen_device="cpu", fill: float = 1024.0,
                 free_pages: Optional[np.ndarray] = None, keep_before: bool = False, window: int = 0):
        from chunked_prefill_decode_amd import native as N
        self.N, self.inst, self.device, self.fill, self.window = N, inst, device, fill, window
        Hq, Hkv, d, P = inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages
        self.sched = load_native_sched(inst, free_pages)
        cap = len(inst.injected) + len(inst.waiting) + 1
        self.batch = self.sched.build_batch(cap_seqs=cap)
        b = self.batch
        self.S, self.D, self.T = b.num_seqs, b.num_decodes, b.num_tokens
        kshape, vshape = N.kv_cache_shapes(P, Hkv, d)
        self.k_cache = torch.full(kshape, fill, dtype=torch.bfloat16, device=device)
        self.v_cache = torch.full(vshape, fill, dtype=torch.bfloat16, device=device)

        # history rows, in batch order
        reqs = requests_by_id(inst)
        self.hist: Dict[int, Tuple[torch.Tensor, torch.Tensor]] = {}
        ks, vs = [], []
        for s in range(self.S):
            r = reqs[int(b.req_ids[s])]
            k, v = W.history_kv(inst, r, device=gen_device)
            assert k.shape[0] == int(b.context_lens[s])
            self.hist[r.req_id] = (k, v)
            ks.append(k)
            vs.append(v)
        hslots = N.sa_history_slots(b)
        if len(hslots):
            hk = torch.cat(ks).to(device)
            hv = torch.cat(vs).to(device)
            hs = torch.from_numpy(hslots).to(device)
            N.sa_kv_append(hk, hv, self.k_cache, self.v_cache, hs, len(hslots), Hkv, d, P)
            del hk, hv, hs

        q, kn, vn = W.step_qkv(inst, self.T, device=gen_device)
        self.q_gen, self.k_new_gen, self.v_new_gen = q, kn, vn
        self.q, self.k_new, self.v_new = q.to(device), kn.to(device), vn.to(device)

        nbytes = N.sa_batch_upload_size(b, Hq, Hkv, d, window)
        self.staging = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        self.meta = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.dev = N.sa_batch_upload(b, Hq, Hkv, d, P, self.staging, self.meta, window=window)
        ws = N.sa_hybrid_attn_workspace_size(self.dev)
        self.ws = torch.zeros(max(ws, 256), dtype=torch.uint8, device=device)
        self.out = torch.empty(self.T, Hq, d, dtype=torch.bfloat16, device=device)
        torch.cuda.synchronize(device)
        if keep_before:
            self.k_before, self.v_before = self.k_cache.clone(), self.v_cache.clone()

    def append(self, stream=None):
        i = self.inst
        self.N.sa_kv_append(self.k_new, self.v_new, self.k_cache, self.v_cache, self.dev.slot_mapping, self.T,
                            i.num_kv_heads, i.head_dim, i.num_pages, stream)

    def attend(self, stream=None):
        self.N.sa_hybrid_attn(self.q, self.k_cache, self.v_cache, self.dev, self.inst.softmax_scale, self.out,
                              self.ws, stream=stream)

    def run(self, stream=None) -> torch.Tensor:
        self.append(stream)
        self.attend(stream)
        return self.out

    # cache as logical slots [num_slots, Hkv, d], whatever the physical layout
    @staticmethod
    def slots_view(k_cache: torch.Tensor, v_cache: torch.Tensor):
        P, Hkv, _, d = k_cache.shape
        k = k_cache.permute(0, 2, 1, 3).reshape(P * 16, Hkv, d)
        v = v_cache.permute(0, 3, 1, 2).reshape(P * 16, Hkv, d)
        return k, v

    def kv_bit_exact(self) -> bool:
        """After run(): the cache equals the oracle's append expectation."""
        from oracle import kvcache as OK
        ob = load_oracle_sched(self.inst).build_batch()
        # expected before-image: fill everywhere, history at the oracle's slots
        P, Hkv, _, d = self.k_cache.shape
        from oracle import scheduler as OS
        fill_bits = bf16_bits(torch.tensor([self.fill], dtype=torch.bfloat16))[0]
        kb = np.full((P * 16, Hkv, d), fill_bits, np.uint16)
        vb = kb.copy()
        for rid, ctx, bt in zip(ob.req_ids, ob.context_lens, ob.block_tables):
            hk, hv = self.hist[rid]
            sl = OS.slots_of(bt, range(ctx))
            kb = OK.append_expected(kb, bf16_bits(hk), sl)
            vb = OK.append_expected(vb, bf16_bits(hv), sl)
        ke = OK.append_expected(kb, bf16_bits(self.k_new_gen), ob.slot_mapping)
        ve = OK.append_expected(vb, bf16_bits(self.v_new_gen), ob.slot_mapping)
        kg, vg = self.slots_view(self.k_cache, self.v_cache)
        return np.array_equal(bf16_bits(kg), ke) and np.array_equal(bf16_bits(vg), ve)


def oracle_inputs(inst: W.Instance, step: GpuStep, seq_subset: Optional[Sequence[int]] = None):
    """The oracle's view: (ctx, q_len) from the ORACLE's batch builder, fp64 q
    rows and contiguous per-sequence K/V from the generator's tensors.

    With seq_subset, only those sequences are returned (in that order) and
    the third value lists the packed q rows they cover."""
    ob = load_oracle_sched(inst).build_batch()
    cu = ob.cu_seqlens_q
    idx = range(len(ob.req_ids)) if seq_subset is None else seq_subset
    seqs, qs, kv, rows = [], [], [], []
    q_all = step.q_gen
    for s in idx:
        rid, ctx, n = ob.req_ids[s], ob.context_lens[s], ob.q_lens[s]
        hk, hv = step.hist[rid]
        k = torch.cat([hk.cpu(), step.k_new_gen[cu[s]:cu[s + 1]].cpu()]).to(torch.float64).numpy()
        v = torch.cat([hv.cpu(), step.v_new_gen[cu[s]:cu[s + 1]].cpu()]).to(torch.float64).numpy()
        seqs.append((ctx, n))
        kv.append((k, v))
        qs.append(q_all[cu[s]:cu[s + 1]].cpu().to(torch.float64).numpy())
        rows.extend(range(cu[s], cu[s + 1]))
    q64 = np.concatenate(qs) if qs else np.zeros((0, inst.num_q_heads, inst.head_dim))
    if seq_subset is None:
        return seqs, q64, kv
    return seqs, q64, kv, rows


class ChunkingStudy:
    """One prompt of L tokens prefilled through the paged path unchunked or in
    chunks of C (each chunk attends its prompt's earlier chunks again through
    the cache), optionally with D single-token decodes of dec_ctx cached tokens
    riding in every iteration.  All K/V rows are placed once at set-up; every
    iteration re-appends its own rows (idempotent) and runs the attention."""

    def __init__(self, L: int, Hq: int, Hkv: int, d: int, decodes: int = 0, dec_ctx: int = 2000,
                 seed: int = 5000, device="cuda:0"):
        from chunked_prefill_decode_amd import native as N
        self.N, self.L, self.Hq, self.Hkv, self.d, self.D, self.dec_ctx = N, L, Hq, Hkv, d, decodes, dec_ctx
        self.device = device
        self.scale = 1.0 / float(np.sqrt(d))
        rng = np.random.default_rng(seed)
        npp, npd = -(-L // 16), -(-(dec_ctx + 1) // 16)
        self.P = npp + decodes * npd
        perm = rng.permutation(self.P).astype(np.int32)
        self.W = max(npp, npd)
        self.bt_prompt = perm[:npp]
        self.bt_dec = [perm[npp + j * npd: npp + (j + 1) * npd] for j in range(decodes)]
        self.q = W.normal_bf16((L, Hq, d), seed + 1)
        self.k = W.normal_bf16((L, Hkv, d), seed + 2)
        self.v = W.normal_bf16((L, Hkv, d), seed + 3)
        # decodes: history rows and the new token (key dec_ctx) of each
        self.dq = W.normal_bf16((decodes, Hq, d), seed + 4)
        self.dk = W.normal_bf16((decodes, dec_ctx + 1, Hkv, d), seed + 5)
        self.dv = W.normal_bf16((decodes, dec_ctx + 1, Hkv, d), seed + 6)
        kshape, vshape = N.kv_cache_shapes(self.P, Hkv, d)
        self.k_cache = torch.full(kshape, 1024.0, dtype=torch.bfloat16, device=device)
        self.v_cache = torch.full(vshape, 1024.0, dtype=torch.bfloat16, device=device)
        slots = [int(self.bt_prompt[p // 16]) * 16 + p % 16 for p in range(L)]
        for j in range(decodes):
            slots += [int(self.bt_dec[j][p // 16]) * 16 + p % 16 for p in range(dec_ctx + 1)]
        ks = torch.cat([self.k] + [self.dk[j] for j in range(decodes)]).to(device)
        vs = torch.cat([self.v] + [self.dv[j] for j in range(decodes)]).to(device)
        N.sa_kv_append(ks, vs, self.k_cache, self.v_cache, torch.tensor(slots, dtype=torch.int32, device=device),
                       len(slots), Hkv, d, self.P)
        torch.cuda.synchronize(device)

    def _slot(self, bt, p):
        return int(bt[p // 16]) * 16 + p % 16

    def iteration(self, c0: int, C: int, with_decodes: bool, with_chunk: bool = True):
        """Device state of one iteration: decodes (optional) + prompt rows c0 .. c0+C-1."""
        N, D = self.N, (self.D if with_decodes else 0)
        rows = C if with_chunk else 0
        q_lens = [1] * D + ([C] if with_chunk else [])
        ctx = [self.dec_ctx] * D + ([c0] if with_chunk else [])
        bt = np.full((len(q_lens), self.W), -1, np.int32)
        for j in range(D):
            bt[j, :len(self.bt_dec[j])] = self.bt_dec[j]
        if with_chunk:
            n = -(-(c0 + C) // 16)
            bt[D, :n] = self.bt_prompt[:n]
        slots = [self._slot(self.bt_dec[j], self.dec_ctx) for j in range(D)]
        slots += [self._slot(self.bt_prompt, p) for p in range(c0, c0 + rows)]
        batch = N.HostBatch.from_arrays(q_lens, ctx, bt, slots, num_decodes=D)
        it = type("Iteration", (), {})()
        it.T = D + rows
        it.q = torch.cat([self.dq[:D], self.q[c0:c0 + rows]]).to(self.device)
        it.k_new = torch.cat([self.dk[:D, self.dec_ctx], self.k[c0:c0 + rows]]).to(self.device)
        it.v_new = torch.cat([self.dv[:D, self.dec_ctx], self.v[c0:c0 + rows]]).to(self.device)
        nbytes = N.sa_batch_upload_size(batch, self.Hq, self.Hkv, self.d)
        it.staging = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        it.meta = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        it.dev = N.sa_batch_upload(batch, self.Hq, self.Hkv, self.d, self.P, it.staging, it.meta)
        it.ws = torch.zeros(max(N.sa_hybrid_attn_workspace_size(it.dev), 256), dtype=torch.uint8, device=self.device)
        it.out = torch.empty(it.T, self.Hq, self.d, dtype=torch.bfloat16, device=self.device)
        it.D, it.c0, it.C = D, c0, rows
        return it

    def schedule(self, C: int, with_decodes: bool):
        return [self.iteration(c0, min(C, self.L - c0), with_decodes) for c0 in range(0, self.L, C)]

    def append(self, it, stream=None):
        self.N.sa_kv_append(it.k_new, it.v_new, self.k_cache, self.v_cache, it.dev.slot_mapping, it.T, self.Hkv,
                            self.d, self.P, stream)

    def attend(self, it, stream=None):
        self.N.sa_hybrid_attn(it.q, self.k_cache, self.v_cache, it.dev, self.scale, it.out, it.ws, stream=stream)

    def prompt_rows(self, its) -> torch.Tensor:
        """The prompt's output rows [L, Hq, d] gathered from a schedule's iterations."""
        return torch.cat([it.out[it.D:] for it in its])


class PolicyTrace:
    """A request trace driven through the scheduler under one batch-building
    policy, every iteration's append + attention timed on the GPU; simulated
    time advances by the measured kernel time, and requests join the waiting
    queue once their arrival time has passed."""

    def __init__(self, Hq: int, Hkv: int, d: int, num_pages: int, max_len: int = 8192,
                 max_tokens: int = 8192, device="cuda:0", seed: int = 7000):
        from chunked_prefill_decode_amd import native as N
        self.N, self.Hq, self.Hkv, self.d, self.P, self.device = N, Hq, Hkv, d, num_pages, device
        self.W = -(-max_len // 16)
        self.scale = 1.0 / float(np.sqrt(d))
        kshape, vshape = N.kv_cache_shapes(num_pages, Hkv, d)
        self.k_cache = torch.full(kshape, 0.5, dtype=torch.bfloat16, device=device)
        self.v_cache = torch.full(vshape, 0.5, dtype=torch.bfloat16, device=device)
        self.q = W.normal_bf16((max_tokens, Hq, d), seed + 1, device)
        self.k = W.normal_bf16((max_tokens, Hkv, d), seed + 2, device)
        self.v = W.normal_bf16((max_tokens, Hkv, d), seed + 3, device)
        self.out = torch.empty(max_tokens, Hq, d, dtype=torch.bfloat16, device=device)
        self.meta_bytes = 32 << 20
        self.staging = torch.empty(self.meta_bytes, dtype=torch.uint8, pin_memory=True)
        self.meta = torch.empty(self.meta_bytes, dtype=torch.uint8, device=device)
        self.ws = torch.zeros(256 << 20, dtype=torch.uint8, device=device)
        self.max_tokens = max_tokens
        self.pages = np.random.default_rng(seed).permutation(num_pages).astype(np.int32)

    def run(self, policy: int, budget: int, limit: int, arrivals, max_iters: int = 100000):
        """arrivals: list of (time_us, prompt_len, max_new_tokens) sorted by time."""
        N = self.N
        sched = N.Scheduler(budget, self.W, self.pages)
        if policy:
            sched.set_policy(policy, limit)
        stream = torch.cuda.current_stream()
        t, nxt, it = 0.0, 0, 0
        arrive, first, token_times, done = {}, {}, {}, {}
        iters = []
        live = 0
        while it < max_iters:
            while nxt < len(arrivals) and arrivals[nxt][0] <= t:
                rid = nxt + 1
                sched.add_request(rid, arrivals[nxt][1], arrivals[nxt][2])
                arrive[rid] = arrivals[nxt][0]
                nxt += 1
                live += 1
            b = sched.build_batch(cap_seqs=4096, cap_tokens=self.max_tokens)
            if b.num_tokens == 0:
                if nxt >= len(arrivals) and live == 0:
                    break
                t = max(t, arrivals[nxt][0]) if nxt < len(arrivals) else t
                sched.commit(b)
                continue
            T = b.num_tokens
            dev = N.sa_batch_upload(b, self.Hq, self.Hkv, self.d, self.P, self.staging, self.meta)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            N.sa_kv_append(self.k[:T], self.v[:T], self.k_cache, self.v_cache, dev.slot_mapping, T, self.Hkv, self.d,
                           self.P)
            N.sa_hybrid_attn(self.q[:T], self.k_cache, self.v_cache, dev, self.scale, self.out[:T], self.ws)
            e1.record(stream)
            e1.synchronize()
            dt = e0.elapsed_time(e1) * 1e3
            t += dt
            v = b.view()
            D = v["num_decodes"]
            iters.append((t, dt, D, T))
            cu = v["cu_seqlens_q"]
            for s, rid in enumerate(v["req_ids"]):
                rid = int(rid)
                if s < D:                               # a decode's token
                    token_times[rid].append(t)
                else:                                   # a chunk; its prompt's last yields the first token
                    done[rid] = done.get(rid, 0) + (cu[s + 1] - cu[s])
                    if done[rid] == arrivals[rid - 1][1]:
                        first[rid] = t
                        token_times[rid] = [t]
            live -= len(sched.commit(b))
            it += 1
        return self._summary(iters, arrive, first, token_times, t)

    @staticmethod
    def _summary(iters, arrive, first, token_times, t_end):
        tbt = []
        for rid, ts in token_times.items():
            tbt += list(np.diff(ts))
        ttft = [first[r] - arrive[r] for r in first]
        dts = np.array([x[1] for x in iters]) if iters else np.zeros(1)
        stalls = sum(1 for x in iters if x[2] == 0 and x[3] > 0)
        pct = lambda a, q: float(np.percentile(a, q)) if len(a) else None
        return {"iterations": len(iters), "time_us": round(t_end, 1),
                "tokens": int(sum(x[3] for x in iters)), "decode_tokens": int(sum(x[2] for x in iters)),
                "requests_done": len(first), "iteration_us_p50": round(pct(dts, 50), 1),
                "iteration_us_max": round(float(dts.max()), 1), "prompt_only_iterations": stalls,
                "tbt_us_p50": None if not tbt else round(pct(tbt, 50), 1),
                "tbt_us_p99": None if not tbt else round(pct(tbt, 99), 1),
                "tbt_us_max": None if not tbt else round(float(max(tbt)), 1),
                "ttft_us_p50": None if not ttft else round(pct(ttft, 50), 1)}

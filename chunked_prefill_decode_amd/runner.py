"""Driving the hybrid step on the GPU through the C ABI.

Plumbing around ``native`` for the benchmark and the tests: it allocates the
paged caches and the metadata / workspace buffers with PyTorch, places the
synthetic history rows, and strings the library's calls together in the
order of one serving iteration (build -> upload -> append -> attention ->
commit).  It holds no arithmetic of the method: every step of the path runs
in libsarathi_attn.  Inputs come from ``workloads`` (seeded generators); the
CPU oracle is not used here.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

import workloads as W
from chunked_prefill_decode_amd import native as N


def batch_from_arrays(q_lens, context_lens, block_tables, slot_mapping, num_decodes: int,
                      req_ids=None) -> N.HostBatch:
    """A host batch given directly (not built by the scheduler), for studies
    and hand-made cases: q_lens per sequence, decodes first."""
    block_tables = np.asarray(block_tables, np.int32)
    S, Wd = block_tables.shape
    T = int(np.sum(q_lens))
    b = N.HostBatch(S, T, Wd)
    b.cu_seqlens_q[1:] = np.cumsum(q_lens)
    b.context_lens[:] = context_lens
    b.block_tables[:] = block_tables
    b.slot_mapping[:T] = slot_mapping
    b.req_ids[:] = np.arange(S) if req_ids is None else req_ids
    b.c.num_seqs, b.c.num_decodes, b.c.num_prefill_chunks = S, num_decodes, S - num_decodes
    b.c.num_tokens = T
    b.c.max_kv_len = int(max((np.asarray(context_lens) + np.asarray(q_lens)).tolist() or [0]))
    return b


def load_scheduler(inst: W.Instance, free_pages=None) -> N.Scheduler:
    """A native scheduler holding the instance's running and waiting requests."""
    s = N.Scheduler(inst.token_budget, inst.max_blocks_per_seq,
                    inst.free_pages if free_pages is None else free_pages)
    for r in inst.injected:
        s.add_request(r.req_id, r.prompt_len, r.max_new_tokens, r.num_computed, r.num_generated)
    for r in inst.waiting:
        s.add_request(r.req_id, r.prompt_len, r.max_new_tokens)
    return s


def requests_by_id(inst: W.Instance) -> Dict[int, W.Req]:
    return {r.req_id: r for r in inst.injected + inst.waiting}


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """Attention workspace filled with 0xFF bytes (fp32 NaN): the library
    needs no initialisation, and a partial that were read without having been
    written would show up as a non-finite output."""
    return torch.full((max(nbytes, 256),), 0xFF, dtype=torch.uint8, device=device)


def place_history(inst: W.Instance, batch: N.HostBatch, k_cache, v_cache, gen_device, device):
    """Generate every cached row of the batch's sequences and store them at
    their slots (sa_history_slots, then sa_kv_append).  Returns the rows per
    request id, as generated."""
    reqs = requests_by_id(inst)
    hist: Dict[int, Tuple[torch.Tensor, torch.Tensor]] = {}
    ks, vs = [], []
    for s in range(batch.num_seqs):
        r = reqs.get(int(batch.req_ids[s]))
        ctx = int(batch.context_lens[s])
        if r is None or r.cached_tokens == 0:
            assert ctx == 0
            continue
        k, v = W.history_kv(inst, r, device=gen_device)
        assert k.shape[0] == ctx
        hist[r.req_id] = (k, v)
        ks.append(k)
        vs.append(v)
    hslots = N.sa_history_slots(batch)
    if len(hslots):
        hk = torch.cat(ks).to(device)
        hv = torch.cat(vs).to(device)
        hs = torch.from_numpy(hslots).to(device)
        N.sa_kv_append(hk, hv, k_cache, v_cache, hs, len(hslots), inst.num_kv_heads, inst.head_dim,
                       inst.num_pages)
        del hk, hv, hs
    return hist


class GpuStep:
    """One layer's hybrid step for a workload instance, resident on the GPU:
    the scheduler's first batch, the paged caches with every cached row in
    place, this step's q / k / v rows, the uploaded metadata and workspace."""

    def __init__(self, inst: W.Instance, device="cuda:0", gen_device="cpu", fill: float = 1024.0,
                 free_pages: Optional[np.ndarray] = None, window: int = 0):
        self.inst, self.device, self.fill, self.window = inst, device, fill, window
        Hq, Hkv, d, P = inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages
        self.free_pages = inst.free_pages if free_pages is None else free_pages
        self.sched = load_scheduler(inst, self.free_pages)
        self.cap_seqs = len(inst.injected) + len(inst.waiting) + 1
        self.batch = self.sched.build_batch(cap_seqs=self.cap_seqs)
        b = self.batch
        self.S, self.D, self.T = b.num_seqs, b.num_decodes, b.num_tokens
        kshape, vshape = N.kv_cache_shapes(P, Hkv, d)
        self.k_cache = torch.full(kshape, fill, dtype=torch.bfloat16, device=device)
        self.v_cache = torch.full(vshape, fill, dtype=torch.bfloat16, device=device)
        self.hist = place_history(inst, b, self.k_cache, self.v_cache, gen_device, device)

        q, kn, vn = W.step_qkv(inst, self.T, device=gen_device)
        self.q_gen, self.k_new_gen, self.v_new_gen = q, kn, vn
        self.q, self.k_new, self.v_new = q.to(device), kn.to(device), vn.to(device)

        nbytes = N.sa_batch_upload_size(b, Hq, Hkv, d, window)
        self.staging = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        self.meta = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.dev = N.sa_batch_upload(b, Hq, Hkv, d, P, self.staging, self.meta, window=window)
        self.ws = new_workspace(N.sa_hybrid_attn_workspace_size(self.dev), device)
        self.out = torch.empty(self.T, Hq, d, dtype=torch.bfloat16, device=device)
        torch.cuda.synchronize(device)

    def append(self, stream=None):
        i = self.inst
        N.sa_kv_append(self.k_new, self.v_new, self.k_cache, self.v_cache, self.dev.slot_mapping, self.T,
                       i.num_kv_heads, i.head_dim, i.num_pages, stream)

    def attend(self, stream=None):
        N.sa_hybrid_attn(self.q, self.k_cache, self.v_cache, self.dev, self.inst.softmax_scale, self.out,
                         self.ws, stream=stream)

    def run(self, stream=None) -> torch.Tensor:
        self.append(stream)
        self.attend(stream)
        return self.out


def slots_view(k_cache: torch.Tensor, v_cache: torch.Tensor):
    """The caches as logical slots [num_slots, Hkv, d], whatever the physical layout."""
    P, Hkv, _, d = k_cache.shape
    k = k_cache.permute(0, 2, 1, 3).reshape(P * 16, Hkv, d)
    v = v_cache.permute(0, 3, 1, 2).reshape(P * 16, Hkv, d)
    return k, v


class StepLoop:
    """The whole per-iteration path of one layer, as a serving loop runs it:
    build the batch (host), pack the metadata and upload it together with
    the append of the new K/V (sa_batch_upload_append: one kernel copies the
    pinned staging buffer and scatters the rows), run the attention, commit
    the batch (host).  Every step starts from its own copy of the same
    scheduler state, so every step runs the same batch.  The host work of
    later steps (build, pack, commit) proceeds while the GPU runs earlier
    ones.  Staging and metadata buffers form a ring of RING; an event pair
    around the attention is recorded every SAMPLE steps (each record sits
    between kernels on the GPU, so the other steps carry none), and before a
    ring slot is packed again the host waits for the latest such event that
    follows the slot's previous use."""

    RING, SAMPLE = 8, 4

    def __init__(self, step: GpuStep, steps: int, stream=None):
        self.step = step
        self.stream = torch.cuda.current_stream() if stream is None else stream
        nbytes = step.staging.numel()
        self.staging = [torch.empty(nbytes, dtype=torch.uint8, pin_memory=True) for _ in range(self.RING)]
        self.meta = [torch.empty(nbytes, dtype=torch.uint8, device=step.device) for _ in range(self.RING)]
        self.done = []                      # (step index, event recorded after that step's attention)
        self.clones = [step.sched.clone() for _ in range(steps)]
        self.batches = [N.HostBatch(step.cap_seqs, step.inst.token_budget, step.inst.max_blocks_per_seq)
                        for _ in range(self.RING)]

    def _wait_for_slot(self, i: int):
        """Ring slot i % RING was last packed for step i - RING: wait until
        that step's upload has run, i.e. for the earliest event recorded
        after the attention of a step k with i - RING <= k < i (steps that
        are multiples of RING always record one, so it exists)."""
        if i < self.RING:
            return
        while self.done and self.done[0][0] < i - self.RING:
            self.done.pop(0)
        assert self.done and self.done[0][0] < i
        self.done[0][1].synchronize()

    def run(self, i: int, timing: bool = False, before=None):
        """Step i (steps in increasing order, each at most once).  Returns
        (tokens, event after the upload + append or None, event after the
        attention or None).  The event pair is recorded when `timing` is set
        (the attention's duration is their difference; callers time every
        SAMPLE-th step) and when `before` is given: that one is recorded
        ahead of the upload (to time the upload + append launch).  Every
        RING-th step records the event after the attention in any case, to
        guard the ring."""
        st, inst = self.step, self.step.inst
        j = i % self.RING
        sched, b = self.clones[i], self.batches[j]
        N.sa_build_batch(sched.h, b)
        self._wait_for_slot(i)
        pair = timing or before is not None
        if before is not None:
            before.record(self.stream)
        dev = N.sa_batch_upload_append(b, inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages,
                                       self.staging[j], self.meta[j], st.k_new, st.v_new, st.k_cache, st.v_cache,
                                       stream=self.stream, window=st.window)
        ev = end = None
        if pair:
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(self.stream)
        N.sa_hybrid_attn(st.q, st.k_cache, st.v_cache, dev, inst.softmax_scale, st.out, st.ws,
                         stream=self.stream)
        if pair or i % self.RING == 0:
            end = torch.cuda.Event(enable_timing=pair)
            end.record(self.stream)
            self.done.append((i, end))
        sched.commit(b)
        self.clones[i] = None
        return b.num_tokens, ev, end


class ScheduleRun:
    """A request trace driven through the whole path on one persistent paged
    cache: each iteration adds that iteration's arrivals, builds the batch,
    uploads it and appends the new rows (sa_batch_upload_append), runs the
    attention and (on commit()) advances the scheduler.  Pages freed by finished requests are handed out
    again with whatever their slots held, as in a serving loop."""

    def __init__(self, inst: W.Instance, arrivals: List[List[W.Req]], device="cuda:0", gen_device="cuda",
                 fill: float = 1024.0, window: int = 0):
        self.inst, self.arrivals, self.device, self.gen_device = inst, arrivals, device, gen_device
        self.fill, self.window = fill, window
        self.sched = load_scheduler(inst)
        kshape, vshape = N.kv_cache_shapes(inst.num_pages, inst.num_kv_heads, inst.head_dim)
        self.k_cache = torch.full(kshape, fill, dtype=torch.bfloat16, device=device)
        self.v_cache = torch.full(vshape, fill, dtype=torch.bfloat16, device=device)
        self.cap_seqs = len(inst.injected) + len(inst.waiting) + sum(len(a) for a in arrivals) + 1
        self.hist: Dict[int, Tuple[torch.Tensor, torch.Tensor]] = {}
        self.staging = self.meta = None
        self.ws = None
        self.it = 0

    def _buffers(self, nbytes: int):
        if self.staging is None or self.staging.numel() < nbytes:
            self.staging = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
            self.meta = torch.empty(nbytes, dtype=torch.uint8, device=self.device)

    def iteration(self):
        """Runs iteration self.it up to the attention (not committed yet).
        Returns an object with the batch, this step's generated rows, the
        device metadata and the output."""
        inst, it = self.inst, self.it
        for r in self.arrivals[it]:
            self.sched.add_request(r.req_id, r.prompt_len, r.max_new_tokens)
        b = self.sched.build_batch(cap_seqs=self.cap_seqs, cap_tokens=inst.token_budget)
        if it == 0:
            self.hist = place_history(inst, b, self.k_cache, self.v_cache, self.gen_device, self.device)
        T = b.num_tokens
        q, kn, vn = W.step_qkv(inst, T, step=it, device=self.gen_device)
        x = type("Iteration", (), {})()
        x.it, x.batch, x.T = it, b, T
        x.q_gen, x.k_new_gen, x.v_new_gen = q, kn, vn
        Hq, Hkv, d, P = inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages
        x.out = torch.empty(T, Hq, d, dtype=torch.bfloat16, device=self.device)
        if T == 0:
            return x
        self._buffers(N.sa_batch_upload_size(b, Hq, Hkv, d, self.window))
        x.dev = N.sa_batch_upload_append(b, Hq, Hkv, d, P, self.staging, self.meta, kn.to(self.device),
                                         vn.to(self.device), self.k_cache, self.v_cache, window=self.window)
        need = N.sa_hybrid_attn_workspace_size(x.dev)
        if self.ws is None or self.ws.numel() < need:
            self.ws = new_workspace(need, self.device)
        N.sa_hybrid_attn(q.to(self.device), self.k_cache, self.v_cache, x.dev, inst.softmax_scale, x.out, self.ws)
        return x

    def commit(self, x) -> List[int]:
        fin = self.sched.commit(x.batch)
        self.it += 1
        return fin


class ChunkingStudy:
    """One prompt of L tokens prefilled through the paged path unchunked or in
    chunks of C (each chunk attends its prompt's earlier chunks again through
    the cache), optionally with D single-token decodes of dec_ctx cached tokens
    riding in every iteration.  All K/V rows are placed once at set-up; every
    iteration re-appends its own rows (idempotent) and runs the attention."""

    def __init__(self, L: int, Hq: int, Hkv: int, d: int, decodes: int = 0, dec_ctx: int = 2000,
                 seed: int = 5000, device="cuda:0"):
        self.L, self.Hq, self.Hkv, self.d, self.D, self.dec_ctx = L, Hq, Hkv, d, decodes, dec_ctx
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
        slots = [self._slot(self.bt_prompt, p) for p in range(L)]
        for j in range(decodes):
            slots += [self._slot(self.bt_dec[j], p) for p in range(dec_ctx + 1)]
        ks = torch.cat([self.k] + [self.dk[j] for j in range(decodes)]).to(device)
        vs = torch.cat([self.v] + [self.dv[j] for j in range(decodes)]).to(device)
        N.sa_kv_append(ks, vs, self.k_cache, self.v_cache, torch.tensor(slots, dtype=torch.int32, device=device),
                       len(slots), Hkv, d, self.P)
        torch.cuda.synchronize(device)

    @staticmethod
    def _slot(bt, p):
        return int(bt[p // 16]) * 16 + p % 16

    def iteration(self, c0: int, C: int, with_decodes: bool, with_chunk: bool = True):
        """Device state of one iteration: decodes (optional) + prompt rows c0 .. c0+C-1."""
        D = self.D if with_decodes else 0
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
        batch = batch_from_arrays(q_lens, ctx, bt, slots, num_decodes=D)
        it = type("Iteration", (), {})()
        it.T = D + rows
        it.q = torch.cat([self.dq[:D], self.q[c0:c0 + rows]]).to(self.device)
        it.k_new = torch.cat([self.dk[:D, self.dec_ctx], self.k[c0:c0 + rows]]).to(self.device)
        it.v_new = torch.cat([self.dv[:D, self.dec_ctx], self.v[c0:c0 + rows]]).to(self.device)
        nbytes = N.sa_batch_upload_size(batch, self.Hq, self.Hkv, self.d)
        it.staging = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        it.meta = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        it.dev = N.sa_batch_upload(batch, self.Hq, self.Hkv, self.d, self.P, it.staging, it.meta)
        it.ws = new_workspace(N.sa_hybrid_attn_workspace_size(it.dev), self.device)
        it.out = torch.empty(it.T, self.Hq, self.d, dtype=torch.bfloat16, device=self.device)
        it.D, it.c0, it.C = D, c0, rows
        return it

    def schedule(self, C: int, with_decodes: bool):
        return [self.iteration(c0, min(C, self.L - c0), with_decodes) for c0 in range(0, self.L, C)]

    def append(self, it, stream=None):
        N.sa_kv_append(it.k_new, it.v_new, self.k_cache, self.v_cache, it.dev.slot_mapping, it.T, self.Hkv,
                       self.d, self.P, stream)

    def attend(self, it, stream=None):
        N.sa_hybrid_attn(it.q, self.k_cache, self.v_cache, it.dev, self.scale, it.out, it.ws, stream=stream)

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
        self.Hq, self.Hkv, self.d, self.P, self.device = Hq, Hkv, d, num_pages, device
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
        self.ws = new_workspace(256 << 20, device)
        self.max_tokens = max_tokens
        self.pages = np.random.default_rng(seed).permutation(num_pages).astype(np.int32)

    def run(self, policy: int, budget: int, limit: int, arrivals, max_iters: int = 100000):
        """arrivals: list of (time_us, prompt_len, max_new_tokens) sorted by time."""
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

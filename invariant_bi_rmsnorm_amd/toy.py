"""Toy greedy-decode engine on top of bi_toy_step (include/bi_toy.h).

The experiment (page "la température zéro n'est pas déterministe",
introduction; post 論文／ブログ「Defeating Nondeterminism in LLM Inference」の
技術的なポイント, section 実装上の工夫：ツールとライブラリ): one prompt decoded
greedily many times while the server's load changes from run to run; count the
distinct completions.

`ToyEngine` owns the device buffers (weights, per-layer paged KV caches, the
rotary table, the workspace) and a host-side block allocator; `step()` packs
one mixed batch (decode tokens first, then prefill chunks) into a
bi_toy_step_desc and runs the C driver.  `run_load_experiment()` is the
continuous-batching load generator: target requests (the fixed prompt) and
random other requests arrive and leave at random, prefill is chunked at random
sizes, and the batch order is shuffled every step.  All arithmetic runs in
libbi.so; this module only schedules and marshals.
"""
from __future__ import annotations

import ctypes
import hashlib
from dataclasses import dataclass, field

import numpy as np
import torch

from . import ops
from .inputs import BLOCK


class _Cfg(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("mlp", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("max_pos", ctypes.c_int32), ("eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float)]


class _Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("layer", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int64), ("rope_table", ctypes.c_void_p)]


class _Step(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("S", ctypes.c_int32), ("n_decode", ctypes.c_int32),
                ("max_q_len", ctypes.c_int32), ("max_kv_len", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32),
                ("ids", ctypes.c_void_p), ("pos", ctypes.c_void_p), ("slots", ctypes.c_void_p),
                ("q_start", ctypes.c_void_p), ("kv_lens", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("logit_rows", ctypes.c_void_p),
                ("n_logit_rows", ctypes.c_int32), ("fp32_head_margin", ctypes.c_float)]


def _dev16(bits: np.ndarray, device) -> torch.Tensor:
    a = np.array(bits, dtype=np.uint16, copy=True).view(np.int16)
    return torch.from_numpy(a).to(device).view(torch.bfloat16)


@dataclass
class Request:
    rid: int
    prompt: np.ndarray
    max_new: int
    target: bool = False
    seed: int = 0                         # sampling key (T > 0); targets share one
    length: int = 0                       # tokens already in the cache
    pending: list = field(default_factory=list)
    generated: list = field(default_factory=list)
    blocks: list = field(default_factory=list)

    def __post_init__(self):
        self.pending = [int(t) for t in self.prompt]

    @property
    def decoding(self) -> bool:
        return self.length >= len(self.prompt)

    @property
    def done(self) -> bool:
        return len(self.generated) >= self.max_new


class ToyEngine:
    def __init__(self, cfg: dict, weights: dict, num_blocks: int, max_tokens: int, max_seqs: int,
                 max_kv_len: int, device: str = "cuda"):
        self.cfg = cfg
        self.device = device
        self.L = ops.lib()          # the library current at construction serves every call
        self.max_tokens, self.max_seqs, self.max_kv_len = max_tokens, max_seqs, max_kv_len
        self.max_blocks = -(-max_kv_len // BLOCK)
        L, H, D = cfg["layers"], cfg["hidden"], cfg["head_dim"]
        Hkv = cfg["kv_heads"]
        self.c = _Cfg(L, H, cfg["heads"], Hkv, D, cfg["mlp"], cfg["vocab"], max_kv_len,
                      float(cfg["eps"]), float(cfg["rope_theta"]))
        self.t = {"embed": _dev16(weights["embed"], device),
                  "final_norm": _dev16(weights["final_norm"], device),
                  "lm_head": _dev16(weights["lm_head"], device)}
        self.layers = []
        ptrs = []
        for lw in weights["layers"]:
            d = {k: _dev16(lw[k], device) for k in ("attn_norm", "wqkv", "wo", "mlp_norm", "wgu", "wd")}
            self.layers.append(d)
            ptrs += [d[k].data_ptr() for k in ("attn_norm", "wqkv", "wo", "mlp_norm", "wgu", "wd")]
        self._layer_ptrs = (ctypes.c_void_p * len(ptrs))(*ptrs)
        self.kc = [torch.zeros((num_blocks, Hkv, BLOCK, D), dtype=torch.bfloat16, device=device) for _ in range(L)]
        self.vc = [torch.zeros((num_blocks, Hkv, D, BLOCK), dtype=torch.bfloat16, device=device) for _ in range(L)]
        self._kp = (ctypes.c_void_p * L)(*[t.data_ptr() for t in self.kc])
        self._vp = (ctypes.c_void_p * L)(*[t.data_ptr() for t in self.vc])
        self.rope = ops.bi_rope_table(max_kv_len, D, cfg["rope_theta"])
        self.w = _Weights(self.t["embed"].data_ptr(), self.t["final_norm"].data_ptr(),
                          self.t["lm_head"].data_ptr(), ctypes.cast(self._layer_ptrs, ctypes.c_void_p),
                          ctypes.cast(self._kp, ctypes.c_void_p), ctypes.cast(self._vp, ctypes.c_void_p),
                          num_blocks, self.rope.data_ptr())
        nbytes = int(self.L.bi_toy_workspace_bytes(ctypes.byref(self.c), max_tokens, max_seqs, max_kv_len))
        if nbytes == 0:
            raise ValueError("unsupported toy configuration")
        self.ws = torch.empty((nbytes,), dtype=torch.uint8, device=device)
        self.next_ids = torch.empty((max_seqs,), dtype=torch.int32, device=device)
        self.logits = torch.empty((max_seqs, cfg["vocab"]), dtype=torch.float32, device=device)
        self.sampled = torch.empty((max_seqs,), dtype=torch.int32, device=device)
        self.free = list(range(num_blocks))[::-1]
        self.num_blocks = num_blocks
        self.tokens_processed = 0       # tokens fed through step(), all requests

    @classmethod
    def sharing(cls, other: "ToyEngine") -> "ToyEngine":
        """An engine over the same weights, KV caches and block pool as `other`
        (the same objects, so either engine's steps extend the same requests),
        bound to the library current now, e.g. another build of the same ABI."""
        e = cls.__new__(cls)
        e.__dict__.update(other.__dict__)
        e.L = ops.lib()
        nbytes = int(e.L.bi_toy_workspace_bytes(ctypes.byref(e.c), e.max_tokens, e.max_seqs, e.max_kv_len))
        if nbytes == 0:
            raise ValueError("unsupported toy configuration")
        e.ws = torch.empty((nbytes,), dtype=torch.uint8, device=e.device)
        e.next_ids = torch.empty_like(other.next_ids)
        e.logits = torch.empty_like(other.logits)
        e.sampled = torch.empty_like(other.sampled)
        e.tokens_processed = 0
        return e

    # ---------------------------------------------------------------- blocks
    def _ensure_blocks(self, r: Request, new_len: int):
        need = -(-new_len // BLOCK)
        while len(r.blocks) < need:
            if not self.free:
                raise RuntimeError("KV block pool exhausted")
            r.blocks.append(self.free.pop())

    def release(self, r: Request):
        self.free.extend(r.blocks)
        r.blocks = []

    def hidden_states(self, T: int) -> torch.Tensor:
        """The residual stream after the last layer of the latest step: bf16
        [T, hidden] at the start of the workspace, row t for token t of the
        step (include/bi_toy.h); a view, overwritten by the next step."""
        H = self.cfg["hidden"]
        return self.ws[:T * H * 2].view(torch.bfloat16).view(T, H)

    # ---------------------------------------------------------------- one step
    def step(self, work, want_logits: bool = False, temperature: float = 0.0, all_rows=(),
             fp32_head_margin: float = 0.0):
        """work: list of (request, n_tokens) with all decode entries (n == 1 and
        request decoding) first.  Returns next ids (numpy [S]) and optionally
        logits (numpy [S, vocab]).  temperature 0 takes the argmax; T > 0 draws
        with bi_sample, keyed by each request's seed, counter = the position of
        the token drawn.  all_rows: indices s of work entries that also get the
        argmax after every one of their tokens (greedy only); with it the
        result has a third member, {s: numpy [n_tokens]}.  fp32_head_margin > 0
        recomputes, in fp32 from the unrounded final norm, the logits of rows
        whose top-2 margin is below it (bi_lm_head_f32) before the token is
        taken."""
        if all_rows and temperature > 0.0:
            raise ValueError("all_rows is for greedy steps")
        S = len(work)
        n_decode = 0
        while n_decode < S and work[n_decode][0].decoding and work[n_decode][1] == 1:
            n_decode += 1
        ids, pos, slots, q_start, kv_lens, rows = [], [], [], [0], [], []
        table = np.zeros((S, self.max_blocks), dtype=np.int32)
        max_q = 1
        for s, (r, n) in enumerate(work):
            toks = r.pending[:n]
            new_len = r.length + n
            if new_len > self.max_kv_len:
                raise RuntimeError("sequence longer than max_kv_len")
            self._ensure_blocks(r, new_len)
            p = np.arange(r.length, new_len)
            bl = np.asarray(r.blocks, dtype=np.int32)
            ids += toks
            pos.append(p)
            slots.append(bl[p // BLOCK] * BLOCK + p % BLOCK)
            q_start.append(q_start[-1] + n)
            kv_lens.append(new_len)
            rows.append(q_start[-1] - 1)
            table[s, :len(bl)] = bl
            max_q = max(max_q, n)
        T = q_start[-1]
        self.tokens_processed += T
        extra = {}                      # s -> positions (rows) of its tokens before the last
        for s in sorted(set(all_rows)):
            first, last = q_start[s], q_start[s + 1] - 1
            extra[s] = list(range(first, last))
            rows += extra[s]
        R = len(rows)
        if T > self.max_tokens or R > self.max_seqs:
            raise RuntimeError("step larger than the workspace")
        dev = self.device
        host = np.concatenate([np.asarray(ids, np.int32), np.concatenate(pos).astype(np.int32),
                               np.concatenate(slots).astype(np.int32), np.asarray(q_start, np.int32),
                               np.asarray(kv_lens, np.int32), np.asarray(rows, np.int32), table.ravel()])
        buf = torch.from_numpy(host).to(dev)
        o = 0
        def take(n):
            nonlocal o
            t = buf[o:o + n]
            o += n
            return t
        d_ids, d_pos, d_slots = take(T), take(T), take(T)
        d_qs, d_kv, d_rows = take(S + 1), take(S), take(R)
        d_tab = take(S * self.max_blocks)
        st = _Step(T, S, n_decode, max_q, self.max_kv_len, self.max_blocks,
                   d_ids.data_ptr(), d_pos.data_ptr(), d_slots.data_ptr(), d_qs.data_ptr(),
                   d_kv.data_ptr(), d_tab.data_ptr(), d_rows.data_ptr(), R, float(fp32_head_margin))
        stream = torch.cuda.current_stream().cuda_stream
        sampling = temperature > 0.0
        rc = self.L.bi_toy_step(ctypes.byref(self.c), ctypes.byref(self.w), ctypes.byref(st),
                                   self.ws.data_ptr(), self.ws.numel(), self.next_ids.data_ptr(),
                                   self.logits.data_ptr() if (want_logits or sampling) else None, stream)
        if rc != 0:
            raise ops.BiError(rc, "bi_toy_step")
        if sampling:
            keys = np.array([[r.seed & (2 ** 64 - 1) for (r, n) in work],
                             [r.length + n for (r, n) in work]], np.uint64)
            d_keys = torch.from_numpy(keys.view(np.int64)).to(dev)        # [2, S]: seeds, offsets
            rc = self.L.bi_sample(self.logits.data_ptr(), self.cfg["vocab"], S, self.cfg["vocab"],
                                  float(temperature), d_keys[0].data_ptr(), d_keys[1].data_ptr(),
                                  self.sampled.data_ptr(), stream)
            if rc != 0:
                raise ops.BiError(rc, "bi_sample")
            nxt = self.sampled[:S].cpu().numpy()
        else:
            allnext = self.next_ids[:R].cpu().numpy()
            nxt = allnext[:S]
        lg = self.logits[:S].cpu().numpy() if want_logits else None
        rows_next = {}
        o = S
        for s in sorted(extra):
            n = len(extra[s])
            rows_next[s] = np.concatenate([allnext[o:o + n], allnext[s:s + 1]])
            o += n
        for s, (r, n) in enumerate(work):
            r.length += n
            del r.pending[:n]
            if not r.pending:                 # the step consumed the last pending token
                r.generated.append(int(nxt[s]))
                r.pending = [int(nxt[s])]
        if all_rows:
            return nxt, lg, rows_next
        return nxt, lg


def completion_hash(tokens) -> str:
    return hashlib.sha256(np.asarray(tokens, dtype=np.int32).tobytes()).hexdigest()[:16]


def run_load_experiment(engine: ToyEngine, prompt: np.ndarray, n_runs: int, n_new: int, seed: int,
                        max_active: int = 64, max_step_tokens: int = 1024, other_prompt=(1, 512),
                        other_new=(1, 256), chunk=(16, 512), progress=None, temperature: float = 0.0,
                        target_seed: int = 0x5EED, tokens_out: list | None = None,
                        fp32_head_margin: float = 0.0):
    """Decode `prompt` n_runs times (n_new tokens each) inside a randomly
    varying continuous batch, greedily (temperature 0) or by seeded sampling
    (every run of the prompt uses target_seed; other requests random seeds);
    fp32_head_margin > 0 recomputes the head in fp32 for rows whose top-2
    margin is below it (ToyEngine.step).
    Returns (list of completion hashes, stats); with tokens_out, the token lists
    of the runs are appended there too.  Each run of the prompt is one
    request; it shares every step with 0..max_active-1 other requests (other
    runs of the prompt and random requests), arriving and leaving at random, in
    shuffled order."""
    g = np.random.default_rng(seed)
    V = engine.cfg["vocab"]
    active: list[Request] = []
    results = []
    targets_started = 0
    rid = 0
    cap = int(g.integers(1, max_active + 1))
    steps = 0
    co_load = []
    while len(results) < n_runs:
        if g.random() < 0.02:                  # the server's load level drifts
            cap = 1 if g.random() < 0.25 or max_active < 2 else int(g.integers(2, max_active + 1))
        while len(active) < cap and g.random() < 0.7:
            if targets_started < n_runs and g.random() < 0.5:
                active.append(Request(rid, prompt, n_new, target=True, seed=target_seed))
                targets_started += 1
            else:
                lp = int(g.integers(other_prompt[0], other_prompt[1] + 1))
                active.append(Request(rid, g.integers(0, V, lp).astype(np.int32),
                                      int(g.integers(other_new[0], other_new[1] + 1)),
                                      seed=int(g.integers(0, 2 ** 62))))
            rid += 1
        if not any(r.target for r in active) and targets_started < n_runs and len(active) < max_active:
            active.append(Request(rid, prompt, n_new, target=True, seed=target_seed))
            targets_started += 1
            rid += 1
        dec = [r for r in active if r.decoding]
        pre = [r for r in active if not r.decoding]
        g.shuffle(dec)
        g.shuffle(pre)
        work = [(r, 1) for r in dec]
        budget = max_step_tokens - len(work)
        for r in pre:
            if budget <= 0:
                break
            n = min(len(r.pending), int(g.integers(chunk[0], chunk[1] + 1)), budget)
            work.append((r, n))
            budget -= n
        engine.step(work, temperature=temperature, fp32_head_margin=fp32_head_margin)
        steps += 1
        co_load.append(len(work) - 1)
        for r in list(active):
            if r.done:
                if r.target:
                    results.append(completion_hash(r.generated[:n_new]))
                    if tokens_out is not None:
                        tokens_out.append(list(r.generated[:n_new]))
                engine.release(r)
                active.remove(r)
        if progress and steps % 500 == 0:
            progress(f"steps={steps} finished_runs={len(results)} active={len(active)} cap={cap}")
    for r in active:
        engine.release(r)
    return results, {"steps": steps, "co_load_min": int(min(co_load)), "co_load_max": int(max(co_load)),
                     "co_load_mean": float(np.mean(co_load))}


def run_verify_rollback(bi: ToyEngine, nb: ToyEngine, prompt: np.ndarray, n_runs: int, n_new: int, seed: int,
                        k: int = 8, max_active: int = 32, max_step_tokens: int = 1024, other_prompt=(1, 512),
                        other_new=(1, 256), chunk=(16, 512), progress=None, tokens_out: list | None = None,
                        perturb=None):
    """Selective determinism by verify-and-rollback (page "la température zéro
    n'est pas déterministe", sections "Le prix d'une sortie bit à bit
    identique" and "Déterminisme sélectif" and its comparison table): a fast
    path that is not batch-invariant proposes tokens, the invariant path checks
    them, and the output is rolled back to the first token the invariant path
    disagrees with.

    `bi` and `nb` share weights, KV caches and the block pool
    (ToyEngine.sharing).  Each run of `prompt` is a target request: its prompt
    is prefilled by `bi` in random chunks; then it alternates up to k draft
    tokens decoded by `nb`, in the same nb steps as a random load of other
    requests (which run on nb only), with one `bi` step that feeds the tokens
    drafted since the last commit again, with a logit row per token: the
    drafts are kept up to the first one bi's argmax disagrees with, bi's token
    is taken there, and the cache length rolls back to the kept prefix (the bi
    step rewrote those positions' K and V).  Every committed token is thus bi's
    argmax over a cache written by bi, so each completion equals the invariant
    engine's greedy completion whatever the drafts were.  perturb(position,
    token) -> token, if given, replaces each draft token (a test hook that
    forces rollbacks).  Returns (completion hashes, stats)."""
    g = np.random.default_rng(seed)
    V = bi.cfg["vocab"]
    active: list[Request] = []
    results = []
    targets_started = 0
    rid = 0
    cap = int(g.integers(1, max_active + 1))
    st = {"nb_steps": 0, "bi_steps": 0, "verifies": 0, "rollbacks": 0, "drafted": 0, "accepted": 0}
    phase, commit = {}, {}              # target rid -> phase; -> (length, n_generated, next token)

    def start_target():
        nonlocal targets_started, rid
        r = Request(rid, prompt, n_new, target=True)
        phase[rid] = "prefill"
        active.append(r)
        targets_started += 1
        rid += 1

    while len(results) < n_runs:
        if g.random() < 0.02:
            cap = 1 if g.random() < 0.25 or max_active < 2 else int(g.integers(2, max_active + 1))
        while len(active) < cap and g.random() < 0.7:
            if targets_started < n_runs and g.random() < 0.5:
                start_target()
            else:
                lp = int(g.integers(other_prompt[0], other_prompt[1] + 1))
                active.append(Request(rid, g.integers(0, V, lp).astype(np.int32),
                                      int(g.integers(other_new[0], other_new[1] + 1))))
                rid += 1
        if not any(r.target for r in active) and targets_started < n_runs and len(active) < max_active:
            start_target()

        # ---- fast path: load requests and drafting targets
        dec = [r for r in active if (not r.target and r.decoding) or (r.target and phase[r.rid] == "draft")]
        pre = [r for r in active if not r.target and not r.decoding]
        g.shuffle(dec)
        g.shuffle(pre)
        work = [(r, 1) for r in dec]
        budget = max_step_tokens - len(work)
        for r in pre:
            if budget <= 0:
                break
            n = min(len(r.pending), int(g.integers(chunk[0], chunk[1] + 1)), budget)
            work.append((r, n))
            budget -= n
        if work:
            nb.step(work)
            st["nb_steps"] += 1
            for r in dec:
                if r.target:
                    if perturb is not None:
                        t = int(perturb(r.length, r.generated[-1]))
                        r.generated[-1] = t
                        r.pending = [t]
                    c_len, c_gen, _ = commit[r.rid]
                    drafted = len(r.generated) - c_gen
                    if drafted >= k or c_gen + drafted > n_new:
                        phase[r.rid] = "verify"

        # ---- invariant path: target prompts and verifications
        tg = [r for r in active if r.target and phase[r.rid] in ("prefill", "verify")]
        if tg:
            g.shuffle(tg)
            work, ver, budget, rows_left = [], [], max_step_tokens, bi.max_seqs
            for r in tg:                       # a verify entry of d tokens takes d logit rows
                if phase[r.rid] == "verify":
                    c_len, c_gen, c_next = commit[r.rid]
                    drafts = r.generated[c_gen:]
                    if len(drafts) > budget or len(drafts) > rows_left:
                        continue
                    r.length = c_len
                    r.pending = [c_next] + drafts[:-1]
                    ver.append((r, drafts))
                    budget -= len(drafts)
                    rows_left -= len(drafts)
                else:
                    if budget <= 0 or rows_left <= 0:
                        continue
                    n = min(len(r.pending), int(g.integers(chunk[0], chunk[1] + 1)), budget)
                    work.append((r, n))
                    budget -= n
                    rows_left -= 1
            entries = [(r, len(d)) for (r, d) in ver] + work
            entries.sort(key=lambda e: not (e[0].decoding and e[1] == 1))      # decode entries first
            if entries:
                idx = {id(e[0]): i for i, e in enumerate(entries)}
                vidx = [idx[id(r)] for (r, _) in ver]
                _, _, rows = bi.step(entries, all_rows=vidx) if vidx else (*bi.step(entries), {})
                st["bi_steps"] += 1
                for (r, drafts) in ver:
                    c_len, c_gen, c_next = commit[r.rid]
                    b = rows[idx[id(r)]]               # bi's token after each fed token
                    a = 0
                    while a < len(drafts) - 1 and drafts[a] == int(b[a]):
                        a += 1
                    st["verifies"] += 1
                    st["rollbacks"] += a < len(drafts) - 1          # a draft bi disagrees with
                    st["drafted"] += len(drafts)
                    st["accepted"] += a
                    nxt = int(b[a])
                    r.generated = r.generated[:c_gen] + drafts[:a] + [nxt]
                    r.length = c_len + a + 1
                    r.pending = [nxt]
                    commit[r.rid] = (r.length, len(r.generated), nxt)
                    phase[r.rid] = "draft"
                for (r, n) in work:
                    if r.decoding and phase[r.rid] == "prefill":     # the prompt is in: first token is bi's
                        commit[r.rid] = (r.length, len(r.generated), r.generated[-1])
                        phase[r.rid] = "draft"

        for r in list(active):
            fin = (r.target and r.rid in commit and commit[r.rid][1] >= n_new) or (not r.target and r.done)
            if fin:
                if r.target:
                    toks = r.generated[:n_new]
                    results.append(completion_hash(toks))
                    if tokens_out is not None:
                        tokens_out.append(list(toks))
                    phase.pop(r.rid), commit.pop(r.rid)
                bi.release(r)
                active.remove(r)
        if progress and (st["nb_steps"] + st["bi_steps"]) % 500 == 0:
            progress(f"steps={st['nb_steps'] + st['bi_steps']} finished_runs={len(results)} active={len(active)}")
    for r in active:
        bi.release(r)
    return results, st
